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
