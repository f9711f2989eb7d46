"""Comparison helpers for the GPU-vs-oracle parity tests (test code only).

Tolerances (readings of the stated parity bar):
  * index planes and sign bits are bit-exact, except where the decided value
    lies within 1e-5 * ||x|| of its decision boundary: for an index, the
    rotated coordinate y_i = ||x|| u_i against ||x|| t_j; for a sign bit, the
    raw projection z_j = (S r)_j against 0 (z on the S r scale, S with
    N(0,1) entries, no normalisation by ||S_j||).  The fraction of
    mismatched codes must stay below 1e-4.  Both the mismatch count and the
    population of the window are reported, with the largest
    distance-to-boundary / ||x|| among the mismatches.
  * logits computed from identical codes agree within
    1e-4 * max(|logit_ref|, ||q|| * knorm / sqrt(d)).
  * norms: knorm within 2e-6 relative.  rnorm = ||x|| ||u - c[idx]|| inherits
    the error of the rotated coordinates (|du| <= ~1e-6 with the bf16 hi/lo
    split products), so |d rnorm| <= sqrt(d) * 1e-6 * ||x||: the bar is
    2e-5 * knorm + 1e-6 * rnorm.
"""
import math

import numpy as np

from oracle import tq_oracle as o

WINDOW = 1e-5
MAX_MISMATCH_FRACTION = 1e-4
LOGIT_TOL = 1e-4


def to_numpy_codes(codes: dict) -> dict:
    out = {}
    for k, v in codes.items():
        if v is None:
            continue
        a = v.detach().cpu().numpy()
        out[k] = a.view(np.uint32) if a.dtype == np.int32 else a
    return out


def check_index_codes(u: np.ndarray, got_idx: np.ndarray, ref_idx: np.ndarray, t32: np.ndarray,
                      stats: dict):
    """Index codes: every mismatch within WINDOW (in units of ||x||) of a
    boundary, mismatch fraction below MAX_MISMATCH_FRACTION."""
    mism = got_idx != ref_idx
    dist = np.min(np.abs(u[:, :, None] - t32.astype(np.float64)[None, None, :]), axis=2)
    stats["idx_mismatch"] = int(mism.sum())
    stats["idx_window"] = int((dist < WINDOW).sum())
    stats["idx_codes"] = int(mism.size)
    stats["idx_max_mis_dist"] = float(dist[mism].max()) if mism.any() else 0.0
    bad = mism & (dist >= WINDOW)
    assert not bad.any(), (f"{int(bad.sum())} index mismatches outside the boundary window "
                           f"(largest distance {stats['idx_max_mis_dist']:.3e} x ||x||)")
    assert mism.mean() < MAX_MISMATCH_FRACTION, f"index mismatch fraction {mism.mean()}"
    return ~mism.any(axis=1)


def check_sign_codes(z: np.ndarray, got_sign: np.ndarray, ref_sign: np.ndarray, knorm: np.ndarray,
                     stats: dict):
    """Sign bits: every mismatch has |z_j| < WINDOW * ||x|| (raw S r scale),
    mismatch fraction below MAX_MISMATCH_FRACTION."""
    smis = got_sign != ref_sign
    zk = np.abs(z) / np.where(knorm > 0, knorm, 1.0)[:, None]
    stats["sign_mismatch"] = int(smis.sum())
    stats["sign_window"] = int((zk < WINDOW).sum())
    stats["sign_codes"] = int(smis.size)
    stats["sign_max_mis_zk"] = float(zk[smis].max()) if smis.any() else 0.0
    bad = smis & (zk >= WINDOW)
    assert not bad.any(), (f"{int(bad.sum())} sign mismatches outside the window "
                           f"(largest |z|/||x|| {stats['sign_max_mis_zk']:.3e})")
    assert smis.mean() < MAX_MISMATCH_FRACTION, f"sign mismatch fraction {smis.mean()}"


def check_encode(x: np.ndarray, gpu_packed: dict, p: o.Params, report: dict = None):
    """Compare GPU-packed codes of the rows of x with the oracle's."""
    x = np.asarray(x, dtype=np.float64)
    ref = o.encode(x, p)
    got = o.unpack(gpu_packed, p)
    n = x.shape[0]
    kn_ref = ref["knorm"].astype(np.float64)
    kn = got["knorm"].astype(np.float64)
    assert np.all(np.abs(kn - kn_ref) <= 2e-6 * kn_ref + 1e-30), "knorm"
    stats = {"n": n, "idx_mismatch": 0, "idx_window": 0, "sign_mismatch": 0}
    idx_rows_ok = np.ones(n, dtype=bool)
    if p.B > 0:
        _, t32 = p.codebook
        idx_rows_ok = check_index_codes(ref["u"], got["idx"], ref["idx"], t32, stats)
    if p.prod:
        # the QJL stage of rows whose indices differ is checked against the
        # oracle's residual for the GPU's indices
        z = ref["z"].copy()
        sign_ref = ref["sign"].copy()
        rn_ref = ref["rnorm"].astype(np.float64).copy()
        if p.B > 0 and not idx_rows_ok.all():
            rows = np.nonzero(~idx_rows_ok)[0]
            rs = o.residual_signs(x[rows], got["idx"][rows], p)
            z[rows], sign_ref[rows], rn_ref[rows] = rs["z"], rs["sign"], rs["rnorm"]
        check_sign_codes(z, got["sign"], sign_ref, kn_ref, stats)
        rn = got["rnorm"].astype(np.float64)
        tol = 2e-5 * kn_ref + 1e-6 * rn_ref
        assert np.all(np.abs(rn - rn_ref) <= tol), \
            f"rnorm error up to {np.max(np.abs(rn - rn_ref) / np.maximum(tol, 1e-30)):.3f} x tolerance"
    if report is not None:
        report.update(stats)
    return ref


def check_logits(got: np.ndarray, ref: np.ndarray, q: np.ndarray, knorm: np.ndarray,
                 n_kv: int, g: int, seq: int, d: int):
    got = np.asarray(got, dtype=np.float64).reshape(n_kv * g, seq)
    ref = np.asarray(ref, dtype=np.float64).reshape(n_kv * g, seq)
    qn = np.linalg.norm(np.asarray(q, np.float64).reshape(n_kv * g, -1), axis=1)
    kn = np.asarray(knorm, np.float64).reshape(n_kv, seq)
    floor = qn[:, None] * kn[np.arange(n_kv * g) // g] / math.sqrt(d)
    tol = LOGIT_TOL * np.maximum(np.abs(ref), floor)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0
    assert np.all(err <= tol), f"logit error up to {worst:.3f} x tolerance"
    return worst


def check_attend(got, ref):
    """max_i |o_gpu - o_ref| <= 1e-4 * max_i |o_ref| for every query head."""
    got = np.asarray(got, np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    err = np.max(np.abs(got - ref), axis=1)
    scale = np.max(np.abs(ref), axis=1)
    worst = float(np.max(err / (1e-4 * scale)))
    assert np.all(err <= 1e-4 * scale), f"attend error up to {worst:.3f} x tolerance"
    return worst
