"""Plain, slow, obviously-correct CPU oracle for the TurboQuant hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``kv_cache_compression_04_amd``) never imports it, and this module imports
nothing from the product: the two share no code.

Everything is float64 numpy.  Library primitives used as single steps: matrix
products, ``numpy.linalg.qr``, ``numpy.polynomial.legendre.leggauss``.

Sources (the pages are cited by title and section):
  [P5]  "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破" (王艺), section
        "2.TurboQuant到底做了什么？": sub-sections 第一阶段 (random rotation +
        MSE-optimal Lloyd-Max scalar quantiser on the Beta coordinate law) and
        第二阶段 (b-1 MSE bits + 1-bit QJL on the residual), and the
        distortion-bound paragraph after them.
  [P3]  "TurboQuant 与 AI 效率革命：当旧数学遇到新智能" (雨轩), section 三
        (JL 变换; 非对称估计器 -- the estimator sqrt(pi/2)/m*||k||*<Sq, sign(Sk)>;
        零开销的秘密 -- sign bits plus one 32-bit norm) and section 四 (三段论:
        random preconditioning P, then sign(S * residual) with S in R^{m x d}).
  [P1]  the yeyulingfeng.com bilingual explainer, section "TurboQuant：6倍压缩，
        零损失" (rotate, then quantise with a precomputed Lloyd-Max codebook).

Readings taken where the pages are silent (numbered; tests and comments refer to them):
  R1  random numbers: SplitMix64 (Steele, Lea & Flood 2014), counter-addressable;
      Gaussians by Box-Muller.  Exact recipe in ``splitmix64`` / ``gaussian``.
  R2  Pi = Q of the QR factorisation of a seeded Gaussian d x d matrix, with
      diag(R) > 0 (unique); rotation is y = Pi x.
  R3  S has i.i.d. N(0,1) entries (the sqrt(pi/2)/m constant of [P3] needs unit
      variance).
  R4  codebook: Lloyd-Max for the density of one coordinate of a uniformly
      random unit vector, f_d(x) ∝ (1-x^2)^((d-3)/2) on [-1,1]; the exchanged
      codebook is float32 centroids c (ascending) and float32 boundaries
      t_j = fp32((c_j + c_{j+1}) / 2).
  R5  quantisation index idx_i = #{j : fp32(u_i) >= t_j}, u = Pi x / ||x||
      (decision taken in float32, ties go to the upper bucket).
  R6  the residual is taken in the original domain, r = x - ||x|| Pi^T c[idx];
      sign bit_j = [fp32((S r)_j) >= 0]; norms stored as float32.
  R7  zero vector: u = 0, r = 0, all sign bits 1, both norms 0.
  R8  prod mode: B = b-1 MSE bits + QJL; mse mode: B = b MSE bits, no QJL.
      prod with b = 1 has no MSE bits (r = x).
  R9  the logit is unscaled: nu*<Pi q, c[idx]> + sqrt(pi/2)/m * rnorm * <S q, s>
      with the stored float32 norms; attention uses softmax(logit / sqrt(d)).
"""
from __future__ import annotations

import functools
import math

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
MODE_PROD = 0
MODE_MSE = 1


# ---------------------------------------------------------------------------
# R1: random numbers
# ---------------------------------------------------------------------------
def splitmix64(seed: int, k) -> np.ndarray:
    """k-th output word(s) of SplitMix64 started at ``seed`` (k = 0, 1, ...).

    SplitMix64 advances its state by the golden gamma and returns a mixed copy
    of the new state, so word k is mix(seed + (k+1)*gamma) and any word can be
    addressed directly.  Mixer: xor-shift 30, multiply, xor-shift 27,
    multiply, xor-shift 31 (Steele, Lea & Flood 2014; constants of the
    published generator).
    """
    k = np.asarray(k, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & MASK64) + (k + np.uint64(1)) * np.uint64(GOLDEN_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def gaussian(seed: int, rows: int, cols: int) -> np.ndarray:
    """rows x cols matrix of N(0,1) draws, element (i, j) at counter c = i*cols + j.

    Box-Muller on pairs: pair p = c // 2 uses u1 from word 2p and u2 from word
    2p + 1 (top 53 bits; u1 in (0,1], u2 in [0,1)); even c takes the cosine
    branch, odd c the sine branch.
    """
    c = np.arange(rows * cols, dtype=np.uint64)
    p = c // np.uint64(2)
    w1 = splitmix64(seed, np.uint64(2) * p)
    w2 = splitmix64(seed, np.uint64(2) * p + np.uint64(1))
    u1 = ((w1 >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    u2 = (w2 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * math.pi * u2
    even = (c % np.uint64(2)) == 0
    z = np.where(even, rad * np.cos(ang), rad * np.sin(ang))
    return z.reshape(rows, cols)


# ---------------------------------------------------------------------------
# R2, R3: the random rotation Pi and the JL matrix S   ([P3] section 四)
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=64)
def rotation(d: int, seed: int) -> np.ndarray:
    """Pi = Q of G = QR, G a seeded d x d Gaussian, with diag(R) > 0."""
    g = gaussian(seed, d, d)
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    pi = q * s[None, :]
    pi.setflags(write=False)
    return pi


def jl_matrix(m: int, d: int, seed: int) -> np.ndarray:
    """S in R^{m x d}, i.i.d. N(0,1)."""
    return gaussian(seed, m, d)


# ---------------------------------------------------------------------------
# R4: Lloyd-Max codebook for the rotated-coordinate law   ([P5] 第一阶段)
# ---------------------------------------------------------------------------
def coord_log_density(d: int, x: np.ndarray) -> np.ndarray:
    """log f_d(x), f_d(x) = G(d/2) / (sqrt(pi) G((d-1)/2)) * (1-x^2)^((d-3)/2)."""
    x = np.asarray(x, dtype=np.float64)
    logc = math.lgamma(d / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2.0)
    alpha = (d - 3) / 2.0
    with np.errstate(divide="ignore"):
        one_m = np.log1p(-x * x)
    if alpha == 0.0:
        return np.full_like(x, logc)
    return logc + alpha * one_m


def coord_density(d: int, x: np.ndarray) -> np.ndarray:
    return np.exp(coord_log_density(d, x))


_GL_X, _GL_W = np.polynomial.legendre.leggauss(24)


def _breakpoints(d: int, a: float, b: float) -> np.ndarray:
    """Sub-interval ends for composite Gauss-Legendre on [a, b] (a >= 0).

    Pieces are at most a quarter of the coordinate's standard deviation wide;
    near x = 1 a geometric grading resolves the (1-x^2)^alpha endpoint
    behaviour of small d.
    """
    sigma = 1.0 / math.sqrt(d)
    n = max(1, int(math.ceil((b - a) / (sigma / 4.0))))
    pts = list(np.linspace(a, b, n + 1))
    if b == 1.0:
        for k in range(1, 60):
            e = 1.0 - 2.0 ** -k
            if a < e < b:
                pts.append(e)
    return np.unique(np.asarray(pts))


def _integrate(fn, d: int, a: float, b: float) -> float:
    if b <= a:
        return 0.0
    pts = _breakpoints(d, a, b)
    lo, hi = pts[:-1], pts[1:]
    half = 0.5 * (hi - lo)
    mid = 0.5 * (hi + lo)
    x = mid[:, None] + half[:, None] * _GL_X[None, :]
    return float(np.sum(half[:, None] * _GL_W[None, :] * fn(x)))


def lloyd_max(d: int, nbits: int, tol: float = 1e-15, max_iter: int = 100000):
    """Lloyd-Max quantiser with 2^nbits levels for f_d, in float64.

    Lloyd-Max is 1-D k-means on the known density ([P5] 第一阶段): alternate
    (i) boundaries = midpoints of neighbouring centroids and (ii) centroids =
    conditional means of the density over their cells, until the centroids no
    longer move.  f_d is symmetric, so the iteration runs on the positive half
    (cells between 0 and 1) and the result is mirrored.  Returns
    (centroids[2^nbits], boundaries[2^nbits - 1]) ascending.
    """
    if nbits == 0:
        return np.zeros(0), np.zeros(0)
    L = 1 << nbits
    half = L // 2
    sigma = 1.0 / math.sqrt(d)
    f = lambda x: coord_density(d, x)
    xf = lambda x: x * coord_density(d, x)
    # start from equally spaced points over [0, min(3 sigma, 1))
    c = (np.arange(half) + 0.5) * (min(3.0 * sigma, 1.0) / half)
    for it in range(max_iter):
        edges = np.concatenate([[0.0], 0.5 * (c[:-1] + c[1:]), [1.0]])
        new = np.empty_like(c)
        for j in range(half):
            mass = _integrate(f, d, edges[j], edges[j + 1])
            mom = _integrate(xf, d, edges[j], edges[j + 1])
            new[j] = mom / mass
        delta = np.max(np.abs(new - c))
        c = new
        if delta <= tol * c[-1]:
            break
    full = np.concatenate([-c[::-1], c])
    bounds = 0.5 * (full[:-1] + full[1:])
    bounds[half - 1] = 0.0
    return full, bounds


def mse_bits(b: int, mode: int) -> int:
    """Number of Lloyd-Max bits B: b-1 in prod mode ([P5] 第二阶段), b in mse mode."""
    return b - 1 if mode == MODE_PROD else b


@functools.lru_cache(maxsize=64)
def codebook_fp32(d: int, nbits: int):
    """The exchanged codebook (R4): fp32 centroids and fp32 midpoint boundaries."""
    c, _ = lloyd_max(d, nbits)
    c32 = c.astype(np.float32)
    t = (0.5 * (c32[:-1].astype(np.float64) + c32[1:].astype(np.float64))).astype(np.float32)
    c32.setflags(write=False)
    t.setflags(write=False)
    return c32, t


# ---------------------------------------------------------------------------
# Parameters and matrices
# ---------------------------------------------------------------------------
class Params:
    """d, b, m, mode and the two seeds; matrices and codebook derived lazily."""

    def __init__(self, d, b, m, mode=MODE_PROD, seed_pi=2, seed_s=3):
        self.d, self.b, self.m, self.mode = int(d), int(b), int(m), int(mode)
        self.seed_pi, self.seed_s = int(seed_pi), int(seed_s)
        self.B = mse_bits(self.b, self.mode)
        self._pi = self._s = self._cb = None

    @property
    def pi(self):
        if self._pi is None:
            self._pi = rotation(self.d, self.seed_pi)
        return self._pi

    @property
    def s(self):
        if self._s is None:
            self._s = jl_matrix(self.m, self.d, self.seed_s)
        return self._s

    @property
    def codebook(self):
        if self._cb is None:
            self._cb = codebook_fp32(self.d, self.B)
        return self._cb

    @property
    def prod(self):
        return self.mode == MODE_PROD


# ---------------------------------------------------------------------------
# Encode   ([P5] 第一阶段 + 第二阶段, [P3] section 四)
# ---------------------------------------------------------------------------
def encode(x: np.ndarray, p: Params) -> dict:
    """Encode rows of x (n x d).  Returns unpacked codes and diagnostics.

    idx   int  [n, d]  bucket index per rotated coordinate (absent when B = 0)
    sign  bool [n, m]  QJL sign bits of the residual (prod mode only)
    knorm f32  [n]     ||x||
    rnorm f32  [n]     ||r|| (prod mode only)
    u, z  float64 diagnostics: rotated unit coordinates, raw S r.
    """
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    assert d == p.d
    nu = np.sqrt(np.sum(x * x, axis=1))
    out = {"knorm": nu.astype(np.float32)}
    safe = np.where(nu > 0, nu, 1.0)
    u = (x @ p.pi.T) / safe[:, None]
    u[nu == 0] = 0.0
    out["u"] = u
    if p.B > 0:
        c32, t32 = p.codebook
        u32 = u.astype(np.float32)
        idx = np.sum(u32[:, :, None] >= t32[None, None, :], axis=2)
        out["idx"] = idx
        recon = nu[:, None] * (c32.astype(np.float64)[idx] @ p.pi)
    else:
        recon = np.zeros_like(x)
    if p.prod:
        r = x - recon
        r[nu == 0] = 0.0
        z = r @ p.s.T
        out["z"] = z
        out["sign"] = z.astype(np.float32) >= 0
        out["rnorm"] = np.sqrt(np.sum(r * r, axis=1)).astype(np.float32)
    return out


def dequantize(codes: dict, p: Params) -> np.ndarray:
    """MSE reconstruction x~ = ||x|| Pi^T c[idx] (the first stage alone)."""
    nu = codes["knorm"].astype(np.float64)
    if p.B == 0:
        return np.zeros((nu.shape[0], p.d))
    c32, _ = p.codebook
    return nu[:, None] * (c32.astype(np.float64)[codes["idx"]] @ p.pi)


def residual_signs(x: np.ndarray, idx: np.ndarray, p: Params) -> dict:
    """Sign bits and residual norm for given MSE indices (used to check the
    QJL stage independently of the bucket decisions)."""
    x = np.asarray(x, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    c32, _ = p.codebook
    recon = nu[:, None] * (c32.astype(np.float64)[idx] @ p.pi) if p.B > 0 else 0.0 * x
    r = x - recon
    r[nu == 0] = 0.0
    z = r @ p.s.T
    return {"z": z, "sign": z.astype(np.float32) >= 0,
            "rnorm": np.sqrt(np.sum(r * r, axis=1)).astype(np.float32)}


# ---------------------------------------------------------------------------
# Packed layout (a format, defined here and in include/tq.h)
# ---------------------------------------------------------------------------
def _coord_word_bit(d: int):
    """Word and bit of each coordinate c in a d-bit plane (d % 128 == 0).

    c = 128 q + 16 t + 4 k + i  (t < 8, k < 4, i < 4)  ->  word 4 q + k, bit 4 t + i.
    """
    c = np.arange(d)
    q, rem = c // 128, c % 128
    t, k, i = rem // 16, (rem // 4) % 4, rem % 4
    return 4 * q + k, 4 * t + i


def pack(codes: dict, p: Params) -> dict:
    """Unpacked codes -> packed arrays.

    idx  uint32 [n, d/32, B]   plane j of word w holds bit j of idx
    sgn  uint32 [n, m/32]      bit set <=> sign bit 1 (z >= 0)
    knorm, rnorm float32 [n]
    """
    n = codes["knorm"].shape[0]
    out = {"knorm": codes["knorm"].astype(np.float32)}
    if p.B > 0:
        assert p.d % 128 == 0
        w, bit = _coord_word_bit(p.d)
        idx = codes["idx"].astype(np.uint64)
        words = np.zeros((n, p.d // 32, p.B), dtype=np.uint64)
        for j in range(p.B):
            plane = (idx >> np.uint64(j)) & np.uint64(1)
            for c in range(p.d):
                words[:, w[c], j] |= plane[:, c] << np.uint64(bit[c])
        out["idx"] = words.astype(np.uint32)
    if p.prod:
        assert p.m % 128 == 0
        w, bit = _coord_word_bit(p.m)
        sg = codes["sign"].astype(np.uint64)
        words = np.zeros((n, p.m // 32), dtype=np.uint64)
        for r in range(p.m):
            words[:, w[r]] |= sg[:, r] << np.uint64(bit[r])
        out["sgn"] = words.astype(np.uint32)
        out["rnorm"] = codes["rnorm"].astype(np.float32)
    return out


def unpack(packed: dict, p: Params) -> dict:
    n = packed["knorm"].shape[0]
    out = {"knorm": np.asarray(packed["knorm"], dtype=np.float32)}
    if p.B > 0:
        w, bit = _coord_word_bit(p.d)
        words = np.asarray(packed["idx"]).astype(np.uint64).reshape(n, p.d // 32, p.B)
        idx = np.zeros((n, p.d), dtype=np.int64)
        for j in range(p.B):
            idx |= (((words[:, w, j] >> bit.astype(np.uint64)) & np.uint64(1)).astype(np.int64) << j)
        out["idx"] = idx
    if p.prod:
        w, bit = _coord_word_bit(p.m)
        words = np.asarray(packed["sgn"]).astype(np.uint64).reshape(n, p.m // 32)
        out["sign"] = ((words[:, w] >> bit.astype(np.uint64)) & np.uint64(1)).astype(bool)
        out["rnorm"] = np.asarray(packed["rnorm"], dtype=np.float32)
    return out


# ---------------------------------------------------------------------------
# Decode-time logit estimation   ([P3] 非对称估计器, [P5] 第二阶段)
# ---------------------------------------------------------------------------
def score(q: np.ndarray, codes: dict, p: Params, n_kv: int, g: int, seq: int) -> np.ndarray:
    """Logits [n_kv*g, seq] from unpacked codes of n_kv*seq keys.

    Query head h uses KV head h // g; keys of KV head k are rows k*seq ... .
    logit = knorm * <Pi q, c[idx]> + sqrt(pi/2)/m * rnorm * <S q, s>, s = +-1.
    """
    q = np.asarray(q, dtype=np.float64).reshape(n_kv * g, p.d)
    knorm = codes["knorm"].astype(np.float64).reshape(n_kv, seq)
    out = np.zeros((n_kv * g, seq))
    qt = q @ p.pi.T
    if p.B > 0:
        c32, _ = p.codebook
        vals = c32.astype(np.float64)[codes["idx"]].reshape(n_kv, seq, p.d)
        for h in range(n_kv * g):
            out[h] += knorm[h // g] * (vals[h // g] @ qt[h])
    if p.prod:
        qs = q @ p.s.T
        s = np.where(codes["sign"], 1.0, -1.0).reshape(n_kv, seq, p.m)
        rn = codes["rnorm"].astype(np.float64).reshape(n_kv, seq)
        const = math.sqrt(math.pi / 2.0) / p.m
        for h in range(n_kv * g):
            out[h] += const * rn[h // g] * (s[h // g] @ qs[h])
    return out


def attend(q, kcodes, vcodes, kp: Params, vp: Params, batch, n_kv, g, seq, scale=None):
    """Decode attention over compressed K and V: out [batch, n_kv*g, d].

    Logits from the K codes (``score``), scaled by 1/sqrt(d), max-subtracted
    softmax over all seq positions, weighted sum of the MSE reconstructions of
    the values v~ = ||v|| Pi_V^T c_V[idx], each reconstructed per key in the
    original domain.
    """
    d = kp.d
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q = np.asarray(q, dtype=np.float64).reshape(batch, n_kv * g, d)
    out = np.zeros((batch, n_kv * g, vp.d))
    per_b = n_kv * seq
    for bi in range(batch):
        ks = {k: v[bi * per_b:(bi + 1) * per_b] for k, v in kcodes.items()}
        vs = {k: v[bi * per_b:(bi + 1) * per_b] for k, v in vcodes.items()}
        logits = score(q[bi], ks, kp, n_kv, g, seq) * scale
        vrec = dequantize(vs, vp).reshape(n_kv, seq, vp.d)
        for h in range(n_kv * g):
            z = logits[h] - np.max(logits[h])
            w = np.exp(z)
            w /= np.sum(w)
            out[bi, h] = w @ vrec[h // g]
    return out


# ---------------------------------------------------------------------------
# Quality metrics (bit-width sweep)
# ---------------------------------------------------------------------------
def mse_distortion(x: np.ndarray, p: Params) -> float:
    """Mean ||x - x~||^2 / ||x||^2 of the MSE stage."""
    codes = encode(x, p)
    xr = dequantize(codes, p)
    x = np.asarray(x, dtype=np.float64)
    return float(np.mean(np.sum((x - xr) ** 2, axis=1) / np.sum(x * x, axis=1)))


def ip_error(x: np.ndarray, q: np.ndarray, p: Params):
    """Bias and RMSE of the logit vs <q, x>, normalised by ||q|| ||x||."""
    codes = encode(x, p)
    n = x.shape[0]
    est = score(q, codes, p, 1, q.shape[0], n)
    true = np.asarray(q, np.float64) @ np.asarray(x, np.float64).T
    norm = np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(x, axis=1)[None, :]
    err = (est - true) / norm
    return float(np.mean(err)), float(np.sqrt(np.mean(err * err)))
