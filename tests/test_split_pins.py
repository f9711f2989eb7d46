"""Pins of the mixed bit-width (outlier-channel split) oracle (CPU only)."""
import math

import numpy as np
import pytest

from oracle import split_oracle as so
from oracle import tq_oracle as tqo


def _keys(n, seed=1, outliers=(3, 40, 77, 120)):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)) * np.exp(0.5 * rng.standard_normal((1, 128)))
    for c in outliers:
        x[:, c] *= 20.0
    return x


def test_average_bits_are_the_pages_figures():
    ch = np.arange(128)
    assert so.SplitParams(ch, 3, 2).bits_per_coordinate == 2.5
    assert so.SplitParams(ch, 4, 3).bits_per_coordinate == 3.5
    p = so.SplitParams(ch, 3, 2)
    assert so.words_per_vector(p) == 2 * (2 + 1 + 1 + 1)     # 2 + 1 index planes, 2 sign planes
    assert so.words_per_vector(so.SplitParams(ch, 4, 3)) == 2 * (3 + 1 + 2 + 1)


def test_outlier_channels_come_first():
    x = _keys(500)
    ch = so.outlier_channels(x, 64)
    assert sorted(ch.tolist()) == list(range(128))
    assert {3, 40, 77, 120} <= set(ch[:64].tolist())
    ms = np.mean(x ** 2, axis=0)
    assert ms[ch[:64]].min() >= ms[ch[64:]].max()


def test_relabelling_the_channels_gives_the_same_codes():
    """Permuting the channels of x and relabelling the channel list the same
    way leaves every code unchanged (the split follows the channel list)."""
    x = _keys(50)
    ch = so.outlier_channels(x, 64)
    perm = np.random.default_rng(4).permutation(128)      # new position of old channel c is inv[c]
    inv = np.argsort(perm)
    a = so.encode(x, so.SplitParams(ch, 3, 2))
    b = so.encode(x[:, perm], so.SplitParams(inv[ch], 3, 2))
    for g in range(2):
        for k in ("idx", "sign", "knorm", "rnorm"):
            assert np.array_equal(a[g][k], b[g][k])


def test_estimator_is_unbiased_over_the_random_matrices():
    """Averaged over independent rotations and JL matrices, the split estimate
    is the exact inner product (each group's estimator is unbiased)."""
    x = _keys(1, seed=5)
    q = np.random.default_rng(6).standard_normal((1, 128))
    ch = so.outlier_channels(_keys(300, seed=7), 64)
    exact = float(q[0] @ x[0])
    est = []
    for s in range(300):
        p = so.SplitParams(ch, 3, 2, seed_pi=1000 + 2 * s, seed_s=5000 + 2 * s)
        est.append(so.score(q, so.encode(x, p), p, 1, 1, 1)[0, 0])
    est = np.asarray(est)
    sem = est.std(ddof=1) / math.sqrt(est.size)
    assert abs(est.mean() - exact) <= 4.0 * sem


def test_split_equals_the_sum_of_two_64_dimensional_instances():
    """Closed check against TurboQuant of each group alone: a key living only
    in the outlier channels scores exactly as group 0 scores its part."""
    x = np.zeros((3, 128))
    ch = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])   # even channels are the outliers
    x[:, 0::2] = np.random.default_rng(8).standard_normal((3, 64))
    q = np.random.default_rng(9).standard_normal((2, 128))
    p = so.SplitParams(ch, 3, 2)
    codes = so.encode(x, p)
    assert np.all(codes[1]["knorm"] == 0)                    # the rest of the key is zero
    got = so.score(q, codes, p, 1, 2, 3)
    g0 = tqo.score(q[:, 0::2], tqo.encode(x[:, 0::2], p.groups[0]), p.groups[0], 1, 2, 3)
    assert np.allclose(got, g0, rtol=0, atol=1e-12)


def test_more_bits_on_outliers_beats_two_bits_everywhere():
    """At 2.5 bits the inner-product error falls below that of uniform 2-bit
    TurboQuant of the whole head on outlier-heavy keys (the purpose of the split)."""
    x = _keys(2000, seed=11)
    q = np.random.default_rng(12).standard_normal((8, 128))
    ch = so.outlier_channels(x[:500], 64)
    p = so.SplitParams(ch, 3, 2)
    e_split = so.score(q, so.encode(x, p), p, 1, 8, 2000) - q @ x.T
    u = tqo.Params(128, 2, 128, tqo.MODE_PROD, 2, 3)
    e_uni = tqo.score(q, tqo.encode(x, u), u, 1, 8, 2000) - q @ x.T
    assert np.sqrt(np.mean(e_split ** 2)) < np.sqrt(np.mean(e_uni ** 2))


@pytest.mark.parametrize("b_out,b_rest", [(3, 2), (4, 3)])
def test_pack_roundtrip(b_out, b_rest):
    x = _keys(40, seed=13)
    p = so.SplitParams(so.outlier_channels(x, 64), b_out, b_rest)
    codes = so.encode(x, p)
    pk = so.pack(codes, p)
    assert pk["words"].shape == (40, so.words_per_vector(p)) and pk["norms"].shape == (40, 4)
    u = so.unpack(pk, p)
    for g in range(2):
        for k in ("idx", "sign", "knorm", "rnorm"):
            assert np.array_equal(u[g][k], codes[g][k])


# ---------------------------------------------------------------- outlier count
@pytest.mark.parametrize("n_out,b_out,b_rest,bits,words", [
    (32, 3, 2, 2.25, 3 * 1 + 2 * 3),      # a few outliers: 32 of 128 at 3 bits, 96 at 2
    (96, 3, 2, 2.75, 3 * 3 + 2 * 1),
    (32, 4, 3, 3.25, 4 * 1 + 3 * 3),
    (64, 3, 2, 2.5, 2 * (2 + 1 + 1 + 1)),
])
def test_outlier_count_sets_the_average_and_the_record(n_out, b_out, b_rest, bits, words):
    p = so.SplitParams(np.arange(128), b_out, b_rest, n_out=n_out)
    assert p.dims == (n_out, 128 - n_out)
    assert p.bits_per_coordinate == bits
    assert so.words_per_vector(p) == words
    assert p.groups[0].d == p.groups[0].m == n_out and p.groups[1].d == p.groups[1].m == 128 - n_out


@pytest.mark.parametrize("dg", [32, 64, 96])
def test_plane_layout_is_a_bijection_with_the_stated_positions(dg):
    pos = [so._plane_pos(dg, c) for c in range(dg)]
    assert sorted(pos) == list(range(dg))
    # coordinate 16 t + 4 k + i sits at bit k dg / 4 + 4 t + i of the plane
    t, k, i = dg // 16 - 1, 3, 3
    assert so._plane_pos(dg, 16 * t + 4 * k + i) == dg - 1
    assert so._plane_pos(dg, 16) == 4 and so._plane_pos(dg, 4) == dg // 4
    if dg == 64:  # the two-word form: word k // 2, bit 16 (k % 2) + 4 t + i
        for c in range(64):
            tt, kk, ii = c // 16, (c // 4) % 4, c % 4
            assert so._plane_pos(64, c) == 32 * (kk // 2) + 16 * (kk % 2) + 4 * tt + ii


@pytest.mark.parametrize("n_out", [32, 96])
def test_pack_round_trips_for_any_outlier_count(n_out):
    x = _keys(40, seed=11)
    p = so.SplitParams(so.outlier_channels(x, n_out), 3, 2, n_out=n_out)
    codes = so.encode(x, p)
    pk = so.pack(codes, p)
    assert pk["words"].shape == (40, so.words_per_vector(p))
    back = so.unpack(pk, p)
    for g in range(2):
        assert np.array_equal(back[g]["idx"], codes[g]["idx"])
        assert np.array_equal(back[g]["sign"], codes[g]["sign"])
    # a single set index bit lands in the word and bit the layout states
    one = [{k: np.zeros_like(v) for k, v in c.items()} for c in codes]
    dg = 128 - n_out
    t = dg // 16 - 1                                     # group 1's last t, k = 1, i = 3
    one[1]["idx"][0, 16 * t + 4 * 1 + 3] = 1
    w = so.pack(one, p)["words"][0]
    j = 1 * dg // 4 + 4 * t + 3
    at = (p.groups[0].B + 1) * n_out // 32 + j // 32
    assert w[at] == 1 << (j % 32) and np.count_nonzero(w) == 1


def test_few_outliers_split_equals_group_zero_for_a_key_in_the_outlier_channels():
    x = np.zeros((3, 128))
    ch = np.concatenate([np.arange(0, 128, 4), np.setdiff1d(np.arange(128), np.arange(0, 128, 4))])
    x[:, 0::4] = np.random.default_rng(12).standard_normal((3, 32))
    q = np.random.default_rng(13).standard_normal((2, 128))
    p = so.SplitParams(ch, 3, 2, n_out=32)
    codes = so.encode(x, p)
    assert np.all(codes[1]["knorm"] == 0)
    got = so.score(q, codes, p, 1, 2, 3)
    g0 = tqo.score(q[:, 0::4], tqo.encode(x[:, 0::4], p.groups[0]), p.groups[0], 1, 2, 3)
    assert np.allclose(got, g0, rtol=0, atol=1e-12)


def test_few_outliers_estimator_is_unbiased():
    x = _keys(1, seed=14)
    q = np.random.default_rng(15).standard_normal((1, 128))
    ch = so.outlier_channels(_keys(300, seed=16), 32)
    exact = float(q[0] @ x[0])
    est = []
    for s in range(300):
        p = so.SplitParams(ch, 3, 2, seed_pi=2000 + 2 * s, seed_s=7000 + 2 * s, n_out=32)
        est.append(so.score(q, so.encode(x, p), p, 1, 1, 1)[0, 0])
    est = np.asarray(est)
    sem = est.std(ddof=1) / math.sqrt(est.size)
    assert abs(est.mean() - exact) <= 4.0 * sem
