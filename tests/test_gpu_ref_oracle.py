"""GPU parity against the plain C++ oracle (oracle/tq_oracle_ref.cpp), the
second, independent CPU implementation beside the numpy oracle that the other
GPU tests use.  The HIP path is called through the C ABI; the C++ oracle's
codes are packed into the library's layout by the numpy oracle's packer (a
bit permutation, pinned on its own) and fed to the score, attention and
search kernels, so those compare the kernels' arithmetic with the C++
oracle's on identical codes.  The bars are the ones every GPU parity test
uses: codes inside the decision windows, logits and attention outputs within
1e-4, top-k sets up to swaps within the logit tolerance.
"""
import numpy as np
import pytest

from oracle import ref
from oracle import tq_oracle as o
from tests.parity import check_attend, check_index_codes, check_logits, check_sign_codes, to_numpy_codes

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - the CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from kv_cache_compression_04_amd import synth, tq  # noqa: E402
from tests.gpu_helpers import DEV, _gpu_encode, _oparams, _report, _upload, check_search  # noqa: E402


def _ref_of(p: tq.Params) -> ref.Ref:
    return ref.Ref(p.d, p.b, p.m, 0 if p.mode == tq.MODE_PROD else 1, p.seed_pi, p.seed_s)


@pytest.mark.parametrize("b,mode", [(3, tq.MODE_PROD), (4, tq.MODE_PROD), (3, tq.MODE_MSE)])
def test_encode_against_cpp_oracle(b, mode):
    p = tq.Params(128, b, 128, mode, 2, 3)
    op, r = _oparams(p), _ref_of(p)
    n = 4096 + 37
    x = synth.llama_keys(heads=1, seq=n, seed=61, dtype=torch.float32)
    got = o.unpack(to_numpy_codes(_gpu_encode(p, x.to(DEV))), op)
    xs = x.double().numpy()
    want = r.encode(xs)
    kn = want["knorm"].astype(np.float64)
    assert np.all(np.abs(got["knorm"].astype(np.float64) - kn) <= 2e-6 * kn + 1e-30)
    stats = {}
    rows_ok = np.ones(n, dtype=bool)
    if op.B > 0:
        pi, _, _, t32 = r.matrices()
        u = (xs @ pi.T) / np.where(kn > 0, kn, 1.0)[:, None]
        rows_ok = check_index_codes(u, got["idx"], want["idx"], t32, stats)
    if op.prod:
        # signs of rows whose indices agree (a differing index changes the
        # residual; the numpy-oracle tests check such rows against the
        # residual of the GPU's indices)
        stats["rows_idx_differ"] = int((~rows_ok).sum())
        check_sign_codes(want["z"][rows_ok], got["sign"][rows_ok], want["sign"][rows_ok], kn[rows_ok], stats)
        rn = want["rnorm"].astype(np.float64)[rows_ok]
        assert np.all(np.abs(got["rnorm"].astype(np.float64)[rows_ok] - rn) <= 2e-5 * kn[rows_ok] + 1e-6 * rn)
    _report(f"C++ oracle encode b={b} mode={mode}", stats)


@pytest.mark.parametrize("n_kv,g,seq", [(2, 4, 1000), (1, 3, 77)])
def test_score_against_cpp_oracle(n_kv, g, seq):
    p = tq.Params(128, 3, 128, tq.MODE_PROD, 2, 3)
    op, r = _oparams(p), _ref_of(p)
    x = synth.llama_keys(heads=n_kv, seq=seq, seed=62, dtype=torch.float32).double().numpy()
    c = r.encode(x)
    q = synth.queries(n_kv * g, seed=63).numpy().astype(np.float64)
    want = r.score(q, c, n_kv, g, seq)
    logits = torch.empty((n_kv * g, seq), device=DEV)
    ws = torch.empty(tq.score_workspace_bytes(p, n_kv, g), dtype=torch.uint8, device=DEV)
    tq.score(p, torch.from_numpy(q.astype(np.float32)).to(DEV), _upload(o.pack(c, op)), n_kv, g, seq, logits, ws)
    torch.cuda.synchronize()
    worst = check_logits(logits.cpu().numpy(), want, q, c["knorm"], n_kv, g, seq, 128)
    print(f"[parity] C++ oracle score n_kv={n_kv} g={g} seq={seq}: worst/tol={worst:.4f}", flush=True)


@pytest.mark.parametrize("batch,n_kv,g,seq,scale", [(2, 2, 4, 1000, None), (1, 1, 4, 513, 0.37)])
def test_attend_against_cpp_oracle(batch, n_kv, g, seq, scale):
    kp = tq.Params(128, 3, 128, tq.MODE_PROD, 2, 3)
    vp = tq.Params(128, 3, 128, tq.MODE_MSE, 4, 0)
    kr, vr = _ref_of(kp), _ref_of(vp)
    k = synth.llama_keys(heads=n_kv, seq=seq, seed=64, dtype=torch.float32, batch=batch).double().numpy()
    v = synth.llama_keys(heads=n_kv, seq=seq, seed=65, dtype=torch.float32, batch=batch).double().numpy()
    q = synth.queries(batch * n_kv * g, seed=66).numpy().astype(np.float64).reshape(batch, n_kv * g, 128)
    kc, vc = kr.encode(k), vr.encode(v)
    want = kr.attend(vr, q, kc, vc, batch, n_kv, g, seq, scale=scale)
    out = torch.full((batch, n_kv * g, 128), float("nan"), device=DEV)
    ws = torch.empty(tq.attend_workspace_bytes(kp, vp, batch, n_kv, g, seq), dtype=torch.uint8, device=DEV)
    tq.attend(kp, vp, torch.from_numpy(q.astype(np.float32)).to(DEV), batch, n_kv, g,
              _upload(o.pack(kc, _oparams(kp))), _upload(o.pack(vc, _oparams(vp))), seq, out, ws,
              scale=0.0 if scale is None else scale)
    torch.cuda.synchronize()
    worst = check_attend(out.cpu().numpy(), want)
    print(f"[parity] C++ oracle attend batch={batch} n_kv={n_kv} g={g} seq={seq} scale={scale}: "
          f"worst/tol={worst:.4f}", flush=True)


@pytest.mark.parametrize("nq,n,k", [(16, 4096, 10), (5, 300, 32)])
def test_search_against_cpp_oracle(nq, n, k):
    p = tq.Params(128, 3, 128, tq.MODE_PROD, 41, 42)
    op, r = _oparams(p), _ref_of(p)
    x = synth.sweep_keys(n=n, seed=67).double().numpy()
    q = synth.queries(nq, seed=68).numpy().astype(np.float64)
    c = r.encode(x)
    want_idx, _ = r.search(q, c, n, k)
    rows = r.score(q, c, 1, nq, n)
    out_idx = torch.empty((nq, k), dtype=torch.int64, device=DEV)
    out_val = torch.empty((nq, k), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.search_workspace_bytes(p, nq, n, k), dtype=torch.uint8, device=DEV)
    tq.search(p, torch.from_numpy(q.astype(np.float32)).to(DEV), _upload(o.pack(c, op)), n, k, out_idx, out_val, ws)
    torch.cuda.synchronize()
    gi = out_idx.cpu().numpy()
    check_search(gi, out_val.cpu().numpy(), rows, q, c["knorm"].astype(np.float64), k)
    same = sum(set(gi[i].tolist()) == set(want_idx[i].tolist()) for i in range(nq))
    print(f"[parity] C++ oracle search nq={nq} n={n} k={k}: {same}/{nq} sets identical to the oracle's", flush=True)
