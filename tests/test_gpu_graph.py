"""The device entry points can be captured in a HIP graph: they allocate
nothing and record no memset.  Each graph is replayed several times with
eager work and synchronisations in between, and every replay is compared with
the eager result."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - the CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from kv_cache_compression_04_amd import synth, tq  # noqa: E402
from tests.gpu_helpers import DEV  # noqa: E402


def _poison(o):
    o.fill_(-7) if not o.dtype.is_floating_point else o.fill_(float("nan"))


def _replays_match(run, outputs, reps=3, rows=None):
    """outputs: tensors every run writes in full.  rows: (tensor, index) pairs
    of which a run writes only the indexed rows."""
    rows = rows or []
    run()                                   # eager: builds the library's caches
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    ref_rows = [t[i].clone() for t, i in rows]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for r in range(reps):
        for o in outputs:
            _poison(o)
        for t, i in rows:
            t[i] = -7 if not t.dtype.is_floating_point else float("nan")
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, ref):
            assert torch.equal(o, e), f"replay {r} differs from the eager result"
        for (t, i), e in zip(rows, ref_rows):
            assert torch.equal(t[i], e), f"replay {r}: written rows differ from the eager result"
        run()                               # eager work between replays
        torch.cuda.synchronize()


def test_graph_encode_score_attend_search():
    kp = tq.Params(128, 3, 128, tq.MODE_PROD, 2, 3)
    vp = tq.Params(128, 3, 128, tq.MODE_MSE, 4, 0)
    n_kv, g, seq = 2, 4, 1500
    k = synth.llama_keys(heads=n_kv, seq=seq, seed=3, device=DEV)
    v = synth.llama_keys(heads=n_kv, seq=seq, seed=4, device=DEV)
    q = synth.queries(n_kv * g, seed=5, device=DEV)
    kc, vc = tq.alloc_codes(kp, n_kv * seq, DEV), tq.alloc_codes(vp, n_kv * seq, DEV)
    logits = torch.empty((n_kv * g, seq), device=DEV)
    sws = torch.empty(tq.score_workspace_bytes(kp, n_kv, g), dtype=torch.uint8, device=DEV)
    out = torch.empty((1, n_kv * g, 128), device=DEV)
    aws = torch.empty(tq.attend_workspace_bytes(kp, vp, 1, n_kv, g, seq), dtype=torch.uint8, device=DEV)
    idx = torch.empty((n_kv * g, 10), dtype=torch.int64, device=DEV)
    val = torch.empty((n_kv * g, 10), device=DEV)
    hws = torch.empty(tq.search_workspace_bytes(kp, n_kv * g, n_kv * seq, 10), dtype=torch.uint8, device=DEV)

    def run():
        tq.encode(kp, k, kc)
        tq.encode(vp, v, vc)
        tq.score(kp, q, kc, n_kv, g, seq, logits, sws)
        tq.attend(kp, vp, q.reshape(1, n_kv * g, 128), 1, n_kv, g, kc, vc, seq, out, aws)
        tq.search(kp, q, kc, n_kv * seq, 10, idx, val, hws)

    outs = [kc["idx"], kc["sgn"], kc["knorm"], kc["rnorm"], vc["idx"], vc["knorm"], logits, out, idx, val]
    _replays_match(run, outs)
    print("[parity] graph replays of encode/score/attend/search equal the eager results", flush=True)


def test_graph_paged_polar_and_split():
    kp = tq.Params(128, 3, 128, tq.MODE_PROD, 2, 3)
    vp = tq.Params(128, 3, 128, tq.MODE_MSE, 4, 0)
    n_kv, g, npg = 2, 4, 3
    cap = npg * n_kv * tq.PAGE_POSITIONS
    kc, vc = tq.alloc_codes(kp, cap, DEV), tq.alloc_codes(vp, cap, DEV)
    x = synth.llama_keys(heads=1, seq=cap, seed=9, device=DEV)
    tq.encode(kp, x, kc)
    tq.encode(vp, x, vc)
    newk = synth.llama_keys(heads=1, seq=n_kv, seed=10, device=DEV)
    slots = torch.tensor([5, cap - 1], dtype=torch.int64, device=DEV)
    bt = torch.tensor([[2, 0, 1]], dtype=torch.int32, device=DEV)
    lens = torch.tensor([1100], dtype=torch.int32, device=DEV)
    q = synth.queries(n_kv * g, seed=11, device=DEV).reshape(1, n_kv * g, 128)
    out = torch.empty((1, n_kv * g, 128), device=DEV)
    ws = torch.empty(tq.attend_paged_workspace_bytes(kp, vp, 1, n_kv, g, npg), dtype=torch.uint8, device=DEV)
    pp = tq.PolarParams()
    pc = tq.alloc_polar_codes(700, DEV)
    px = synth.llama_keys(heads=1, seq=700, seed=12, device=DEV)
    plog = torch.empty((4, 700), device=DEV)
    pws = torch.empty(tq.polar_score_workspace_bytes(pp, 1, 4), dtype=torch.uint8, device=DEV)
    pq = synth.queries(4, seed=13, device=DEV)
    sp = tq.SplitParams(list(range(64, 128)) + list(range(64)), 3, 2)
    sc = tq.alloc_split_codes(sp, 700, DEV)
    slog = torch.empty((4, 700), device=DEV)
    sws = torch.empty(tq.split_score_workspace_bytes(sp, 1, 4), dtype=torch.uint8, device=DEV)

    def run():
        tq.encode_slots(kp, newk, slots, cap, kc)
        tq.attend_paged(kp, vp, q, 1, n_kv, g, kc, vc, npg, bt, lens, out, ws)
        tq.polar_encode(pp, px, pc)
        tq.polar_score(pp, pq, pc, 1, 4, 700, plog, pws)
        tq.split_encode(sp, px, sc)
        tq.split_score(sp, pq, sc, 1, 4, 700, slog, sws)

    _replays_match(run, [out, pc["pq"], pc["radius"], plog, sc["words"], sc["norms"], slog],
                   rows=[(kc["idx"], slots), (kc["sgn"], slots), (kc["knorm"], slots), (kc["rnorm"], slots)])
    print("[parity] graph replays of slot encode/paged attend/polar/split equal the eager results", flush=True)
