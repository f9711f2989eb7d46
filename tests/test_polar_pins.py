"""Pins of the PolarQuant oracle against closed forms, invariants and
independent computations (CPU only)."""
import math

import numpy as np
import pytest
from scipy import integrate, stats

from oracle import polar_oracle as po
from oracle import tq_oracle as tqo


def test_transform_hand_example():
    # y = (1, 0, 0, 1): psi = (0, pi/2), radii (1, 1), theta = pi/4, radius sqrt 2
    r, ang = po.polar_transform(np.array([[1.0, 0.0, 0.0, 1.0]]))
    assert r[0] == pytest.approx(math.sqrt(2.0), abs=1e-15)
    assert np.allclose(ang[0][0], [0.0, math.pi / 2], atol=1e-15)
    assert ang[1][0, 0] == pytest.approx(math.pi / 4, abs=1e-15)
    # (-1, 0, 0, -1): level-1 angles pi and 3 pi / 2 (atan2 taken mod 2 pi)
    _, ang = po.polar_transform(np.array([[-1.0, 0.0, 0.0, -1.0]]))
    assert np.allclose(ang[0][0], [math.pi, 1.5 * math.pi], atol=1e-15)


@pytest.mark.parametrize("d", [4, 16, 128, 1024])
def test_transform_inverts(d):
    y = np.random.default_rng(d).standard_normal((40, d)) * np.exp(np.random.default_rng(1).standard_normal((40, 1)))
    r, ang = po.polar_transform(y)
    assert len(ang) == int(math.log2(d)) and sum(a.shape[1] for a in ang) == d - 1
    assert np.allclose(r, np.linalg.norm(y, axis=1), rtol=1e-14)
    back = po.polar_inverse(r, ang)
    assert np.max(np.abs(back - y)) <= 1e-13 * np.max(np.abs(y))
    assert np.all((ang[0] >= 0) & (ang[0] < 2 * math.pi))
    for a in ang[1:]:
        assert np.all((a >= 0) & (a <= math.pi / 2))


@pytest.mark.parametrize("k", [2, 4, 8, 16, 32, 64])
def test_angle_law_closed_forms(k):
    f = lambda t: po.angle_density(k, t)
    mass, _ = integrate.quad(f, 0.0, math.pi / 2, epsabs=1e-13, limit=200)
    mean, _ = integrate.quad(lambda t: t * f(t), 0.0, math.pi / 2, epsabs=1e-13, limit=200)
    assert mass == pytest.approx(1.0, abs=1e-11)
    assert mean == pytest.approx(math.pi / 4, abs=1e-11)   # the pages' E[Theta] = pi/4
    # the density is the derivative of the Beta-law CDF (an independent closed form)
    for t in (0.3, 0.7, math.pi / 4, 1.1):
        h = 1e-6
        fd = (po.angle_cdf(k, t + h) - po.angle_cdf(k, t - h)) / (2 * h)
        assert fd == pytest.approx(float(f(t)), rel=1e-6, abs=1e-9)
    assert float(po.angle_cdf(k, math.pi / 4)) == pytest.approx(0.5, abs=1e-14)
    # k = 2: sin(2 theta) exactly
    if k == 2:
        t = np.linspace(0.01, 1.5, 7)
        assert np.allclose(f(t), np.sin(2 * t), rtol=1e-14)


def test_angle_laws_of_rotated_gaussian_vectors():
    """Levels >= 2 follow the k = 2^(l-1) law; level 1 is uniform on [0, 2 pi)."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3000, 128)) * np.exp(rng.standard_normal((3000, 1)))
    y = x @ tqo.rotation(128, 2).T
    _, ang = po.polar_transform(y)
    assert stats.kstest(ang[0].reshape(-1)[::7], stats.uniform(0, 2 * math.pi).cdf).pvalue > 1e-3
    for lev in range(2, 8):
        k = 1 << (lev - 1)
        sample = ang[lev - 1][:, ::max(1, ang[lev - 1].shape[1] // 8)].reshape(-1)
        assert stats.kstest(sample, lambda t: po.angle_cdf(k, t)).pvalue > 1e-3, lev
    # concentration at 45 degrees grows with the level
    sd = [np.std(a) for a in ang[1:]]
    assert all(sd[i + 1] < sd[i] for i in range(len(sd) - 1))


def test_level1_codebook_is_the_uniform_grid():
    c, t = po.angle_codebook(1, 4)
    step = math.pi / 8
    assert np.allclose(c, (np.arange(16) + 0.5) * step, atol=1e-15)
    assert np.allclose(t, np.arange(1, 16) * step, atol=1e-15)


def test_one_bit_k2_codebook_closed_form():
    # density sin(2t): two cells split at pi/4; E[t | t < pi/4] = (1/4) / (1/2) = 1/2
    c, t = po.angle_codebook(2, 1)
    assert t[0] == pytest.approx(math.pi / 4, abs=1e-13)
    assert c[0] == pytest.approx(0.5, abs=1e-12)
    assert c[1] == pytest.approx(math.pi / 2 - 0.5, abs=1e-12)


@pytest.mark.parametrize("level", [2, 3, 4, 5, 6, 7])
def test_lloyd_max_conditions_by_independent_quadrature(level):
    k = 1 << (level - 1)
    c, t = po.angle_codebook(level, 2)
    assert np.all(np.diff(c) > 0)
    assert np.allclose(c + c[::-1], math.pi / 2, atol=1e-12)          # symmetric about pi/4
    assert t[1] == pytest.approx(math.pi / 4, abs=1e-12)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15)         # boundaries = midpoints
    edges = np.concatenate([[0.0], t, [math.pi / 2]])
    f = lambda s: float(po.angle_density(k, s))
    for j in range(4):
        m0, _ = integrate.quad(f, edges[j], edges[j + 1], epsabs=1e-14, limit=200)
        m1, _ = integrate.quad(lambda s: s * f(s), edges[j], edges[j + 1], epsabs=1e-14, limit=200)
        assert c[j] == pytest.approx(m1 / m0, abs=1e-10)               # centroids = conditional means


def _keys(n, d=128, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)) * np.exp(rng.standard_normal((1, d)))
    x[:, 5] *= 20.0
    return x


def test_distortion_falls_with_bits():
    x = _keys(300)
    errs = []
    for b1, b in ((4, 2), (5, 3), (6, 4)):
        p = po.PolarParams(128, b1, b, 2)
        xh = po.decode(po.encode(x, p), p)
        errs.append(float(np.mean(np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1))))
    # each extra bit per angle cuts the error by about 4 (high-resolution rate)
    assert errs[0] > 2.5 * errs[1] > 6.0 * errs[2]


def test_codes_are_buckets_of_the_angles():
    p = po.PolarParams()
    c = po.encode(_keys(50), p)
    for lev in range(1, 8):
        _, bnd = p.codebook(lev)
        th = c["angles"][lev - 1]
        idx = c[f"level{lev}"]
        lo = np.concatenate([[-np.inf], bnd])[idx]
        hi = np.concatenate([bnd, [np.inf]])[idx]
        assert np.all((th >= lo) & (th < hi))
    # level 1 with a uniform grid: code = floor(psi / (pi / 8))
    assert np.array_equal(c["level1"], np.floor(c["angles"][0] / (math.pi / 8)).astype(int))


def test_score_equals_dot_with_decoded_vector():
    """<Pi q, y^> computed in the rotated domain equals q . (Pi^T y^)."""
    p = po.PolarParams()
    x = _keys(2 * 37)
    codes = po.encode(x, p)
    q = np.random.default_rng(9).standard_normal((2 * 3, 128))
    got = po.score(q, codes, p, 2, 3, 37)
    xh = po.decode(codes, p).reshape(2, 37, 128)
    for h in range(6):
        assert np.allclose(got[h], xh[h // 3] @ q[h], rtol=1e-12, atol=1e-12)


def test_zero_vector():
    p = po.PolarParams()
    c = po.encode(np.zeros((2, 128)), p)
    assert np.all(c["radius"] == 0)
    for lev in range(1, 8):
        assert np.all(c[f"level{lev}"] == 0)
    assert np.all(po.decode(c, p) == 0)


def test_pack_layout_is_a_bijection():
    slots = po._slots_128()
    bits = set()
    for (lev, j), (w, b) in slots.items():
        nb = 4 if lev == 1 else 2
        for i in range(nb):
            assert (w, b + i) not in bits
            bits.add((w, b + i))
    assert len(slots) == 127 and len(bits) == 64 * 4 + 63 * 2 == 382      # about 3 bits per coordinate
    assert all(0 <= w < 12 and 0 <= b < 32 for w, b in bits)
    p = po.PolarParams()
    c = po.encode(_keys(64), p)
    u = po.unpack(po.pack(c, p), p)
    for lev in range(1, 8):
        assert np.array_equal(u[f"level{lev}"], c[f"level{lev}"])
