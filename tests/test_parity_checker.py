"""The parity checker must reject planted mistakes (planted in oracle codes, on the CPU)."""
import numpy as np
import pytest

from oracle import tq_oracle as o
from tests.parity import check_encode, check_logits


def _case(b=3):
    p = o.Params(128, b, 128)
    x = np.random.default_rng(0).standard_normal((64, 128)) * 3
    return p, x, o.pack(o.encode(x, p), p)


def test_checker_accepts_the_oracle_itself():
    p, x, pk = _case()
    rep = {}
    check_encode(x, pk, p, rep)
    assert rep["idx_mismatch"] == 0 and rep["sign_mismatch"] == 0


@pytest.mark.parametrize("field,word", [("idx", (5, 2, 1)), ("sgn", (7, 3)), ("idx", (63, 0, 0))])
def test_checker_rejects_a_flipped_bit(field, word):
    p, x, pk = _case()
    pk[field] = pk[field].copy()
    pk[field][word] ^= np.uint32(1 << 9)
    with pytest.raises(AssertionError):
        check_encode(x, pk, p)


def test_checker_rejects_a_wrong_norm():
    p, x, pk = _case()
    pk["rnorm"] = pk["rnorm"] * np.float32(1.001)
    with pytest.raises(AssertionError):
        check_encode(x, pk, p)


def test_logit_checker_rejects_small_errors():
    p, x, _ = _case()
    codes = o.encode(x, p)
    q = np.random.default_rng(1).standard_normal((2, 128))
    ref = o.score(q, codes, p, 1, 2, 64)
    check_logits(ref, ref, q, codes["knorm"], 1, 2, 64, 128)
    bad = ref.copy()
    bad[1, 7] += 3e-4 * max(abs(ref[1, 7]), np.linalg.norm(q[1]) * codes["knorm"][7] / np.sqrt(128))
    with pytest.raises(AssertionError):
        check_logits(bad, ref, q, codes["knorm"], 1, 2, 64, 128)


def test_sign_window_is_on_the_raw_projection_scale():
    """A sign mismatch is allowed only where |(S r)_j| < 1e-5 ||x|| on the raw
    S r scale (no division by ||S_j||, which is ~sqrt(d))."""
    from tests.parity import check_sign_codes
    n, m = 20000, 128
    rng = np.random.default_rng(3)
    kn = rng.uniform(0.5, 2.0, n)
    z = rng.standard_normal((n, m)) * kn[:, None]
    ref = z >= 0
    z[5, 7] = 5e-6 * kn[5]
    ref[5, 7] = True
    got = ref.copy()
    got[5, 7] = ~got[5, 7]
    st = {}
    check_sign_codes(z, got, ref, kn, st)
    assert st["sign_mismatch"] == 1 and st["sign_max_mis_zk"] < 1e-5
    # 5e-5 ||x|| lies inside a window normalised by ||S_j|| ~ 11 but outside the raw one
    z[5, 7] = 5e-5 * kn[5]
    with pytest.raises(AssertionError):
        check_sign_codes(z, got, ref, kn, {})


def test_index_window_and_fraction():
    from tests.parity import check_index_codes
    t32 = np.array([-0.1, 0.0, 0.1], np.float32)
    u = np.full((1000, 128), 0.05)
    ref = np.full((1000, 128), 2)
    got = ref.copy()
    u[3, 4] = 0.1 - 3e-6
    got[3, 4] = 3
    st = {}
    check_index_codes(u, got, ref, t32, st)
    assert st["idx_mismatch"] == 1
    u[3, 4] = 0.1 - 3e-5
    with pytest.raises(AssertionError):
        check_index_codes(u, got, ref, t32, {})
    # too many mismatches, even inside the window
    u[:, 4] = 0.1 - 1e-6
    got[:, 4] = 3
    with pytest.raises(AssertionError):
        check_index_codes(u, got, ref, t32, {})
