"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: every check is a known-answer
value, a closed form, an independent library routine (scipy), an invariant or
a brute-force search on a tiny case.
"""
import math
import os

import numpy as np
import pytest
from scipy import integrate, optimize, special, stats

from oracle import tq_oracle as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def _page_constant(name):
    for row in _golden_rows("page_constants.txt"):
        parts = row.split()
        if parts[0] == name:
            return float(parts[1]), float(parts[2])
    raise KeyError(name)


# --------------------------------------------------------------------------- RNG
def test_splitmix64_known_answers():
    for row in _golden_rows("splitmix64_seed0.txt"):
        k, word = row.split()
        assert int(o.splitmix64(0, int(k))) == int(word, 16)


def test_gaussian_moments_and_pairing():
    z = o.gaussian(12345, 1000, 1000).ravel()
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n)
    assert abs(np.mean(z ** 4) - 3.0) < 5 * math.sqrt(96.0 / n)
    # cosine/sine members of one Box-Muller pair are uncorrelated
    pairs = z.reshape(-1, 2)
    assert abs(np.mean(pairs[:, 0] * pairs[:, 1])) < 5 / math.sqrt(n / 2)
    # element (i, j) is counter i*cols + j: a 1 x N draw equals the flattened R x C draw
    assert np.array_equal(o.gaussian(7, 1, 600).ravel(), o.gaussian(7, 20, 30).ravel())


def test_gaussian_ks():
    z = o.gaussian(99, 200, 500).ravel()
    assert stats.kstest(z, "norm").pvalue > 1e-3


# --------------------------------------------------------------------------- Pi, S
@pytest.mark.parametrize("d", [4, 32, 128])
def test_rotation_is_the_unique_positive_qr_factor(d):
    pi = o.rotation(d, 5)
    g = o.gaussian(5, d, d)
    assert np.max(np.abs(pi.T @ pi - np.eye(d))) < 1e-12
    r = pi.T @ g                     # must be R of G = Pi R
    assert np.max(np.abs(np.tril(r, -1))) < 1e-10 * np.max(np.abs(r))
    assert np.all(np.diag(r) > 0)


def test_rotation_preserves_norms_and_inner_products():
    # The preconditioning rotation keeps inner products: "TurboQuant 与 AI 效率革命：当旧数学遇到新智能", section 四.
    pi = o.rotation(128, 2)
    rng = np.random.default_rng(0)
    x, y = rng.standard_normal((2, 50, 128))
    assert np.allclose(np.linalg.norm(x @ pi.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    assert np.allclose(np.sum((x @ pi.T) * (y @ pi.T), 1), np.sum(x * y, 1), atol=1e-11)


def test_jl_matrix_shape_and_law():
    s = o.jl_matrix(64, 128, 3)
    assert s.shape == (64, 128)
    assert np.array_equal(s, o.gaussian(3, 64, 128))


def _coord_cdf(d, x):
    # (X+1)/2 ~ Beta((d-1)/2, (d-1)/2) for one coordinate of a uniform unit vector
    a = (d - 1) / 2.0
    return special.betainc(a, a, (np.asarray(x) + 1.0) / 2.0)


def test_rotated_coordinates_follow_the_beta_law():
    # After a random rotation each coordinate of a unit vector follows a fixed
    # Beta law: "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破", 第一阶段.
    # Fixed x with heavy outliers, many seeds.
    d = 32
    x = np.ones(d)
    x[:3] = 40.0
    coords = []
    for seed in range(300):
        pi = o.rotation(d, 1000 + seed)
        u = pi @ x / np.linalg.norm(x)
        coords.append(u[seed % d])
    res = stats.kstest(np.array(coords), lambda v: _coord_cdf(d, v))
    assert res.pvalue > 1e-3


# --------------------------------------------------------------------------- codebook
@pytest.mark.parametrize("d", [3, 4, 128, 1024])
def test_one_bit_codebook_closed_form(d):
    c, t = o.lloyd_max(d, 1)
    exact = math.exp(math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d + 1) / 2))
    assert abs(c[1] - exact) < 1e-13 and abs(c[0] + exact) < 1e-13
    assert t[0] == 0.0
    if d == 3:
        assert abs(exact - 0.5) < 1e-15
    if d == 4:
        assert abs(exact - 4 / (3 * math.pi)) < 1e-15


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_d3_is_the_uniform_quantiser(B):
    # d = 3: f is uniform on [-1, 1] (Archimedes), so Lloyd-Max is the uniform quantiser.
    c, t = o.lloyd_max(3, B)
    L = 1 << B
    assert np.allclose(c, -1 + (2 * np.arange(L) + 1) / L, atol=1e-12)


def _cell_mass(d, a, b):
    return _coord_cdf(d, b) - _coord_cdf(d, a)


def _cell_moment(d, a, b):
    # int x f_d(x) dx = -C (1-x^2)^((d-1)/2) / (d-1)
    logc = math.lgamma(d / 2) - 0.5 * math.log(math.pi) - math.lgamma((d - 1) / 2)
    F = lambda x: -math.exp(logc) * (1 - x * x) ** ((d - 1) / 2) / (d - 1)
    return F(b) - F(a)


@pytest.mark.parametrize("d", [16, 128, 1024])
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_codebook_lloyd_max_conditions_independent_quadrature(d, B):
    c, t = o.lloyd_max(d, B)
    L = 1 << B
    assert np.allclose(c, -c[::-1], atol=0)                       # symmetry
    assert np.all(np.diff(c) > 0)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-17)      # midpoint condition
    edges = np.concatenate([[-1.0], t, [1.0]])
    for j in range(L):
        mean = _cell_moment(d, edges[j], edges[j + 1]) / _cell_mass(d, edges[j], edges[j + 1])
        assert abs(mean - c[j]) < 1e-11 * max(1.0, abs(c[j]) * math.sqrt(d))  # centroid condition


def test_codebook_gaussian_limit_matches_max_1960():
    d = 1_000_000
    for row in _golden_rows("gaussian_lloyd_max.txt"):
        parts = row.split()
        B, levels = int(parts[0]), np.array([float(v) for v in parts[2:]])
        c, _ = o.lloyd_max(d, B)
        pos = c[len(c) // 2:] * math.sqrt(d)
        assert np.allclose(pos, levels, atol=1.5e-3, rtol=1e-3), (B, pos, levels)


@pytest.mark.parametrize("B", [1, 2])
def test_d4_codebook_by_brute_force_threshold_search(B):
    # d = 4: f is the semicircle law 2/pi sqrt(1-x^2).  Search the symmetric
    # thresholds directly (MSE with scipy.integrate.quad) and compare.
    f = lambda x: 2 / math.pi * math.sqrt(max(0.0, 1 - x * x))

    def mse_for(thr):
        edges = [-1.0] + list(thr) + [1.0]
        tot = 0.0
        for a, b in zip(edges[:-1], edges[1:]):
            m0 = integrate.quad(f, a, b, epsabs=1e-13)[0]
            m1 = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-13)[0]
            m2 = integrate.quad(lambda x: x * x * f(x), a, b, epsabs=1e-13)[0]
            tot += m2 - m1 * m1 / m0
        return tot

    c, t = o.lloyd_max(4, B)
    if B == 1:
        # only symmetric threshold is 0; centroid is E[x | x > 0] = 4/(3 pi)
        assert abs(c[1] - 4 / (3 * math.pi)) < 1e-9
        return
    grid = np.linspace(0.05, 0.95, 181)
    best = grid[np.argmin([mse_for([-g, 0.0, g]) for g in grid])]
    res = optimize.minimize_scalar(lambda g: mse_for([-g, 0.0, g]),
                                   bracket=(best - 0.005, best, best + 0.005), tol=1e-10)
    assert abs(res.x - t[2]) < 2e-6


def _analytic_distortion(d, B):
    """d * E[(u - c[idx(u)])^2] = 1 - d * sum_j P_j c_j^2 (centroid condition)."""
    c, t = o.lloyd_max(d, B)
    edges = np.concatenate([[-1.0], t, [1.0]])
    p = _cell_mass(d, edges[:-1], edges[1:])
    return 1.0 - d * float(np.sum(p * c * c))


def test_distortion_bounds_printed_on_the_pages():
    lo_c, _ = _page_constant("mse_lower_constant")
    hi_c, tol = _page_constant("mse_upper_constant")
    assert abs(math.sqrt(3) * math.pi / 2 - hi_c) < tol
    prev = 1.0
    for B in (1, 2, 3, 4):
        D = _analytic_distortion(128, B)
        assert lo_c * 4.0 ** -B <= D <= math.sqrt(3) * math.pi / 2 * 4.0 ** -B
        assert D < prev
        prev = D
    ratio, tol = _page_constant("one_bit_ratio")
    gauss_1bit = 1 - 2 / math.pi                      # Gaussian limit of the 1-bit MSE
    assert abs(gauss_1bit / 0.25 - ratio) < tol
    assert abs(_analytic_distortion(128, 1) - 0.3609) < 5e-4


def test_gaussian_limit_distortion_matches_max_1960():
    for row in _golden_rows("gaussian_lloyd_max.txt"):
        parts = row.split()
        B, mse = int(parts[0]), float(parts[1])
        assert abs(_analytic_distortion(1_000_000, B) - mse) < 2e-3 * max(1, mse * 100)


# --------------------------------------------------------------------------- encode
def _params(d=128, b=3, m=128, mode=o.MODE_PROD, seed_pi=2, seed_s=3):
    return o.Params(d, b, m, mode, seed_pi, seed_s)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_measured_distortion_matches_analytic(b):
    # isotropic directions with log-normal norms: for any fixed Pi, Pi x / ||x||
    # is uniform on the sphere, so the mean distortion is the analytic one
    p = _params(b=b, mode=o.MODE_MSE)
    rng = np.random.default_rng(b)
    x = rng.standard_normal((20000, 128)) * np.exp(0.5 * rng.standard_normal((20000, 1)))
    codes = o.encode(x, p)
    per = np.sum((x - o.dequantize(codes, p)) ** 2, 1) / np.sum(x * x, 1)
    Da = _analytic_distortion(128, b)
    assert abs(per.mean() - Da) < 5 * per.std() / math.sqrt(len(per))
    assert abs(o.mse_distortion(x[:100], p) - per[:100].mean()) < 1e-12


def test_one_bit_inner_product_bias():
    # A 1-bit MSE-optimal quantiser shrinks inner products by about 2/pi:
    # "谷歌TurboQuant如何绕过内存墙？重新审视它的技术突破", 第二阶段.
    # With q = x, E<q, x~>/<q, x> = d c^2 exactly for the 1-bit codebook; -> 2/pi as d grows.
    d = 128
    p = _params(d=d, b=1, mode=o.MODE_MSE)
    x = np.random.default_rng(1).standard_normal((40000, d))
    codes = o.encode(x, p)
    xr = o.dequantize(codes, p)
    ratio = np.sum(x * xr, 1) / np.sum(x * x, 1)
    c1 = p.codebook[0][1].astype(np.float64)
    assert abs(ratio.mean() - d * c1 * c1) < 6 * ratio.std() / math.sqrt(len(ratio))
    bias, tol = _page_constant("one_bit_ip_bias")
    assert abs(2 / math.pi - bias) < tol
    assert abs(d * c1 * c1 - 2 / math.pi) < 0.003


def test_qjl_estimator_is_unbiased_over_draws_of_S():
    # The asymmetric QJL estimator is unbiased: "TurboQuant 与 AI 效率革命：当旧数学遇到新智能",
    # section 三, 非对称估计器.
    d = m = 32
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, d)) * 3
    q = rng.standard_normal((1, d))
    est = []
    for s in range(10000):
        p = _params(d=d, b=3, m=m, seed_s=100000 + s)
        codes = o.encode(x, p)
        est.append(o.score(q, codes, p, 1, 1, 1)[0, 0])
    est = np.array(est)
    p = _params(d=d, b=3, m=m)
    r = x - o.dequantize(o.encode(x, p), p)
    qn, rn, qr = np.sum(q * q), np.sum(r * r), float(np.sum(q * r))
    var = (math.pi / 2 * qn * rn - qr * qr) / m
    truth = float(np.sum(q * x))
    assert abs(est.mean() - truth) < 3 * math.sqrt(var / len(est))
    assert abs(est.var() / var - 1) < 0.06


def test_mse_score_equals_inner_product_with_reconstruction():
    p = _params(b=3, mode=o.MODE_MSE)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 128))
    q = rng.standard_normal((3, 128))
    codes = o.encode(x, p)
    assert np.allclose(o.score(q, codes, p, 1, 3, 64), q @ o.dequantize(codes, p).T, atol=1e-11)


def test_zero_vector_codes():
    p = _params(b=3)
    x = np.zeros((1, 128))
    codes = o.encode(x, p)
    assert np.all(codes["idx"] == 2) and np.all(codes["sign"])
    assert codes["knorm"][0] == 0 and codes["rnorm"][0] == 0
    assert o.score(np.ones((1, 128)), codes, p, 1, 1, 1)[0, 0] == 0.0


@pytest.mark.parametrize("B", [1, 2])
def test_d4_encode_is_nearest_codeword_and_sign_is_best_pattern(B):
    d, m = 4, 10
    p = _params(d=d, b=B + 1, m=m)
    c32, _ = p.codebook
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, d))
    codes = o.encode(x, p)
    L = 1 << B
    words = np.array(np.meshgrid(*[np.arange(L)] * d, indexing="ij")).reshape(d, -1).T
    cw = c32.astype(np.float64)[words]                      # all L^d codewords
    for n in range(len(x)):
        u = codes["u"][n].astype(np.float32).astype(np.float64)
        best = words[np.argmin(np.sum((cw - u) ** 2, axis=1))]
        assert np.array_equal(best, codes["idx"][n])
    pats = ((np.arange(1 << m)[:, None] >> np.arange(m)) & 1).astype(bool)
    s = np.where(pats, 1.0, -1.0)
    for n in range(len(x)):
        best = pats[np.argmax(s @ codes["z"][n])]
        assert np.array_equal(best, codes["sign"][n])


def test_residual_signs_agree_with_encode():
    p = _params()
    x = np.random.default_rng(6).standard_normal((32, 128))
    codes = o.encode(x, p)
    rs = o.residual_signs(x, codes["idx"], p)
    assert np.array_equal(rs["sign"], codes["sign"]) and np.array_equal(rs["rnorm"], codes["rnorm"])


# --------------------------------------------------------------------------- layout
def test_layout_word_and_bit_examples():
    w, bit = o._coord_word_bit(256)
    for c, (ww, bb) in {0: (0, 0), 1: (0, 1), 3: (0, 3), 4: (1, 0), 15: (3, 3), 16: (0, 4),
                        127: (3, 31), 128: (4, 0), 200: (6, 16)}.items():
        assert (w[c], bit[c]) == (ww, bb), c
    # a bijection onto the d/32 words x 32 bits
    assert len(set(zip(w.tolist(), bit.tolist()))) == 256


@pytest.mark.parametrize("b,mode", [(1, o.MODE_PROD), (3, o.MODE_PROD), (4, o.MODE_PROD), (2, o.MODE_MSE)])
def test_pack_roundtrip(b, mode):
    p = _params(d=256, m=128, b=b, mode=mode)
    x = np.random.default_rng(7).standard_normal((9, 256))
    codes = o.encode(x, p)
    pk = o.pack(codes, p)
    back = o.unpack(pk, p)
    if p.B:
        assert pk["idx"].shape == (9, 8, p.B) and np.array_equal(back["idx"], codes["idx"])
    if p.prod:
        assert pk["sgn"].shape == (9, 4) and np.array_equal(back["sign"], codes["sign"])


# --------------------------------------------------------------------------- attend
def test_attend_with_zero_query_is_mean_of_reconstructed_values():
    kp = _params(b=3, seed_pi=2)
    vp = _params(b=3, mode=o.MODE_MSE, seed_pi=4)
    rng = np.random.default_rng(8)
    n_kv, g, seq = 2, 2, 50
    k = rng.standard_normal((n_kv * seq, 128))
    v = rng.standard_normal((n_kv * seq, 128))
    kc, vc = o.encode(k, kp), o.encode(v, vp)
    out = o.attend(np.zeros((n_kv * g, 128)), kc, vc, kp, vp, 1, n_kv, g, seq)
    vr = o.dequantize(vc, vp).reshape(n_kv, seq, 128)
    for h in range(n_kv * g):
        assert np.allclose(out[0, h], vr[h // g].mean(0), atol=1e-12)


def test_attend_with_a_dominant_key_returns_its_value():
    kp = _params(b=3, seed_pi=2)
    vp = _params(b=3, mode=o.MODE_MSE, seed_pi=4)
    rng = np.random.default_rng(9)
    seq = 40
    k = rng.standard_normal((seq, 128))
    k[17] *= 200.0
    v = rng.standard_normal((seq, 128))
    q = k[17:18] / np.linalg.norm(k[17]) * 50
    kc, vc = o.encode(k, kp), o.encode(v, vp)
    out = o.attend(q, kc, vc, kp, vp, 1, 1, 1, seq)
    assert np.allclose(out[0, 0], o.dequantize(vc, vp)[17], atol=1e-9)


def _temperature_case(kp, vp, nus, vnus):
    """Hand-built codes whose logits are known in closed form.

    Query q = Pi^T 1, so Pi q is the all-ones vector.  Key j has every index in
    the top bucket, knorm nus[j] and rnorm 0, so its logit is
    nus[j] * c_top * d exactly (the QJL term vanishes with rnorm = 0).  Value j
    has every index in the top bucket and knorm vnus[j], so its
    reconstruction is vnus[j] * c_top_V * Pi_V^T 1.
    """
    d, n = kp.d, len(nus)
    ctop_k = float(kp.codebook[0][-1])
    ctop_v = float(vp.codebook[0][-1])
    kc = {"idx": np.full((n, d), (1 << kp.B) - 1), "knorm": np.asarray(nus, np.float32),
          "sign": np.ones((n, kp.m), bool), "rnorm": np.zeros(n, np.float32)}
    vc = {"idx": np.full((n, d), (1 << vp.B) - 1), "knorm": np.asarray(vnus, np.float32)}
    q = (kp.pi.T @ np.ones(d))[None, :]
    logits = np.asarray(nus, np.float32).astype(np.float64) * ctop_k * d
    return q, kc, vc, logits, ctop_v


@pytest.mark.parametrize("scale", [None, 0.37, 0.05])
def test_attend_temperature_closed_form(scale):
    """softmax(scale * logit) with scale = 1/sqrt(d) by default, checked on 2
    and 3 keys against the closed form: with Pi_V out = w . vnus * c_top * 1,
    so each weight is read off one value at a time."""
    kp = _params(b=3, seed_pi=2)
    vp = _params(b=3, mode=o.MODE_MSE, seed_pi=4)
    d = kp.d
    s = 1.0 / math.sqrt(d) if scale is None else scale
    ctop_k = float(kp.codebook[0][-1])
    for gaps in ([0.0, 1.3], [0.0, 0.8, 2.1]):
        # knorms chosen so that the scaled logits are close to `gaps`
        nus = [gp / (s * ctop_k * d) for gp in gaps]
        n = len(nus)
        for j in range(n):
            vnus = [1.0 if i == j else 0.0 for i in range(n)]
            q, kc, vc, logits, ctop_v = _temperature_case(kp, vp, nus, vnus)
            out = o.attend(q, kc, vc, kp, vp, 1, 1, 1, n, scale=scale)[0, 0]
            e = np.exp(s * logits - np.max(s * logits))
            w = e / e.sum()
            rot = vp.pi @ out                     # Pi_V out = w_j * c_top_V * 1
            assert np.allclose(rot, w[j] * ctop_v, rtol=1e-12, atol=1e-15), (gaps, j)
        # a wrong temperature would move the weights: the check above has teeth
        e_wrong = np.exp(logits / d - np.max(logits / d))
        assert abs(e_wrong[-1] / e_wrong.sum() - w[-1]) > 1e-3


def test_ip_error_bias_of_one_bit_mse_on_aligned_queries():
    """mse mode, b = 1: for q = x/||x|| the normalised estimate is
    <u, c[idx]> = c_1 ||u||_1, whose mean is d c_1^2 (the 1-bit shrinkage of
    the MSE quantiser, 2/pi in the Gaussian limit); so the bias of ip_error is
    d c_1^2 - 1 = -0.3609 at d = 128, with c_1 from the closed form
    Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))."""
    d = 128
    p = _params(d=d, b=1, mode=o.MODE_MSE, seed_pi=21)
    c1 = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    rng = np.random.default_rng(31)
    biases = []
    for _ in range(200):
        x = rng.standard_normal((1, d)) * rng.uniform(0.5, 3.0)
        bias, rmse = o.ip_error(x, x / np.linalg.norm(x), p)
        assert abs(abs(bias) - rmse) < 1e-12          # one pair: |bias| = rmse
        biases.append(bias)
    # the spread of c_1 ||u||_1 over random directions is ~ c_1 sqrt(d (1 - 2/pi)) / sqrt(d) ~ 0.04
    assert abs(np.mean(biases) - (d * c1 * c1 - 1.0)) < 0.01


def test_ip_error_rmse_of_pure_qjl_matches_closed_form_variance():
    """prod mode, b = 1 (no MSE bits, r = x): for fixed q, x and S ~ N(0,1)^{m x d},
    the estimator has mean <q, x> and variance ((pi/2) ||q||^2 ||x||^2 - <q,x>^2) / m,
    so the normalised error has E[err^2] = (pi/2 - cos^2) / m.  Averaged over
    independent draws of S (seeds) and pairs, ip_error's RMSE^2 matches the
    mean of that closed form, and its bias is zero within sampling error."""
    d, m = 128, 128
    rng = np.random.default_rng(41)
    x = rng.standard_normal((48, d)) * np.exp(0.5 * rng.standard_normal((48, 1)))
    q = rng.standard_normal((24, d))
    q[:6] = x[:6] + 0.3 * rng.standard_normal((6, d))          # a few correlated pairs
    cos = (q @ x.T) / np.linalg.norm(q, axis=1)[:, None] / np.linalg.norm(x, axis=1)[None, :]
    expect = float(np.mean((math.pi / 2 - cos ** 2) / m))
    ms, bs = [], []
    for seed in range(40):
        p = _params(d=d, b=1, m=m, seed_s=1000 + seed)
        bias, rmse = o.ip_error(x, q, p)
        ms.append(rmse ** 2)
        bs.append(bias)
    # 40 draws of S x 1152 pairs: relative standard error of the mean square ~1-2%
    assert abs(np.mean(ms) / expect - 1.0) < 0.06, (np.mean(ms), expect)
    assert abs(np.mean(bs)) < 3 * math.sqrt(expect / (40 * 48))
    # a dropped sqrt(pi/2) (or an m in place of sqrt(m)) is far outside that band
    assert abs((2 / math.pi) * np.mean(ms) / expect - 1.0) > 0.2
