"""Benchmark of the TurboQuant hot path on one MI355X.

One step = the whole hot path on the Llama-3.1-8B-shaped decode layer:
  tq_encode of all 8 KV heads x 32768 positions x d 128 bf16 keys (b = 3:
  2-bit Lloyd-Max + 1-bit QJL, m = 128), then tq_score of one decode step
  (32 query heads, grouped 4:1) from the packed codes.
Inputs are resident in HBM before the timed region; the K timed steps are
captured once as a HIP graph (replays checked equal to the eager step) and
one replay is timed, bracketed by torch.cuda.synchronize(); the same K steps
issued eagerly are reported beside it (eager_ms_per_step).

Reported on one JSON line:
  value        keys encoded + scored per second through the whole step (Mvectors/s)
  encode_*     the encode kernel alone (HIP events around its launch)
  score_*      the score share of the step on the same layer (codes 14.7 MB: they
               sit in the 256 MB last-level cache) and, separately timed, the
               score call streaming 32 such layers' codes (470 MB) from HBM, as
               a fraction of the nominal peak and of a plain 1 GiB device copy
               (hbm_stream_reference)
  roofline     the dominant kernel (encode, a bf16 MFMA contraction)
  roofline_score  the score kernel on the 32-layer stream (HBM-bound)
  cpu_baseline the CPU oracle (numpy float64) on a bounded sample of the step
Further sections (each can be switched off): long-context attention (plain
and through a paged block table), the PolarQuant variant and the
outlier-channel mixed bit widths (2.5 / 3.5 bits) on the same layer,
the bit-width sweep, high-dimensional batched search (d = m = 1024, 1M
vectors, 1024 queries, top-10) and search at database scale (2^26 vectors of
d = 128, 3.76 GB of codes, 1024 queries, top-10).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROFILE = os.path.join(ROOT, "profiles", "bench_kernels_d128_b3.md")
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0

N_KV, SEQ, D, M, G = 8, 32768, 128, 128, 4
LAYERS = 32


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--b", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hbm-score", action="store_true")
    ap.add_argument("--no-attend", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-highdim", action="store_true")
    ap.add_argument("--no-searchdb", action="store_true")
    ap.add_argument("--no-polar", action="store_true")
    ap.add_argument("--no-split", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=8)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for scaling PMC byte counters)")
    return ap.parse_args()


def profiled_traffic(kernel_prefix: str, grid: int = None):
    """HBM bytes per launch of a kernel from the committed rocprofv3 summary
    (the launch with `grid` threads, else the largest one), or None when the
    summary is missing or the kernel source changed since it was taken."""
    from kv_cache_compression_04_amd.rocprof_summary import kernel_source_hash
    try:
        text = open(PROFILE, encoding="utf-8").read()
    except OSError:
        return None
    if f"`{kernel_source_hash()}`" not in text:
        return None
    best = None
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:"):
            parts = line.split()
            name, g, val = " ".join(parts[1:-2]), int(parts[-2]), float(parts[-1])
            if name.startswith(kernel_prefix) and (grid is None or g == grid):
                if best is None or g > best[0]:
                    best = (g, int(val))
    return None if best is None else best[1]


def cpu_baseline(b, heads):
    """The oracle as it stands on `heads` KV heads of the same layer recipe."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from kv_cache_compression_04_amd import synth
    from oracle import tq_oracle as o

    p = o.Params(D, b, M, o.MODE_PROD, 2, 3)
    _ = p.pi, p.s, p.codebook          # set-up outside the timed region
    x = synth.llama_keys(heads=heads, seq=SEQ, seed=1).double().numpy()
    q = synth.queries(heads * G, seed=5).double().numpy()
    t0 = time.perf_counter()
    codes = o.encode(x, p)
    o.pack(codes, p)
    o.score(q, codes, p, heads, G, SEQ)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    n = heads * SEQ
    return {"value": round(n / dt / 1e6, 4), "unit": "Mvectors/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{heads} of {N_KV} KV heads x {SEQ} positions (encode + pack + score of "
                      f"{heads * G} query heads), float64 numpy, {dt:.1f} s"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the hot path is per-GPU and needs no collectives)", file=sys.stderr)
        sys.exit(2)
    import torch

    from kv_cache_compression_04_amd import synth, tq

    if args.copy_calibration:
        # a plain copy: 512 MiB read + 512 MiB written per launch
        nbytes = 512 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                          "launches": 5}), flush=True)
        return

    dev = "cuda:0"
    torch.cuda.set_device(0)
    p = tq.Params(D, args.b, M, tq.MODE_PROD, 2, 3)
    n = N_KV * SEQ
    x = synth.llama_keys(heads=N_KV, seq=SEQ, seed=1, device=dev)
    q = synth.queries(N_KV * G, seed=5, device=dev)
    codes = tq.alloc_codes(p, n, dev)
    logits = torch.empty((N_KV * G, SEQ), device=dev)
    ws = torch.empty(tq.score_workspace_bytes(p, N_KV, G), dtype=torch.uint8, device=dev)
    code_bytes = sum(tq.codes_bytes(p, 1))
    stream = torch.cuda.current_stream()

    def step():
        tq.encode(p, x, codes)
        tq.score(p, q, codes, N_KV, G, SEQ, logits, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref_logits = logits.clone()
    ref_codes = {k: v.clone() for k, v in codes.items() if v is not None}
    # The K timed steps are captured once as a HIP graph (one launch for the
    # whole sequence of kernels, so the host's per-call marshalling does not
    # pace the GPU), and so are K encodes alone for the encode share.
    graph, enc_graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    with torch.cuda.graph(enc_graph):
        for _ in range(args.steps):
            tq.encode(p, x, codes)
    # every replay reproduces the eager step exactly (eager work in between)
    for _ in range(2):
        logits.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(logits, ref_logits) and all(torch.equal(codes[k], v) for k, v in ref_codes.items())
        if not same:
            raise RuntimeError("graph replay differs from the eager step")
        step()
        torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    graph.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    enc_graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    enc_ms = e0.elapsed_time(e1) / args.steps
    sc_ms = ms_step - enc_ms
    # the same K steps issued eagerly, one library call at a time (reference)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / args.steps
    enc_flops = (2 * D * D + 2 * D * M) * n
    enc_tflops = enc_flops / (enc_ms * 1e-3) / 1e12
    score_bytes_layer = code_bytes * n + 4 * N_KV * G * SEQ
    out = {
        "metric": "tq_score packed-KV GB/s (% of HBM peak) + tq_encode Mvectors/s, d=128 b=3",
        "value": round(n / (ms_step * 1e-3) / 1e6, 3),
        "unit": "Mvectors/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 MFMA (hi/lo split, fp32 accumulate) + int8 MFMA (int32 accumulate)",
        "data": "synthetic (seeded Llama-3.1-8B-shaped keys: N(0,1) x per-channel log-normal, 2% outlier channels x20)",
        "config": {"workload": f"Llama-3.1-8B-shaped decode layer: {N_KV} KV heads x seq {SEQ} x d {D} bf16 keys, "
                               f"{N_KV * G} query heads (GQA {G}:1), b={args.b}, m={M}; encode all keys + score one decode step",
                   "b": args.b, "d": D, "m": M, "n_keys": n, "query_heads": N_KV * G},
        "encode_ms": round(enc_ms, 5),
        "encode_mvectors_per_s": round(n / (enc_ms * 1e-3) / 1e6, 2),
        "score_ms_one_layer": round(sc_ms, 5),
        "step_timing": "K steps captured as one HIP graph, timed with HIP events around one replay (replays "
                       "checked equal to the eager step); encode share from a graph of K encodes; score = "
                       "step - encode",
        "eager_ms_per_step": round(eager_ms, 5),
        "score_gbps_one_layer_cache_resident": round(score_bytes_layer / (sc_ms * 1e-3) / 1e9, 1),
        "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "mfma", "achieved": round(enc_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(enc_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": profiled_traffic(f"tq::encode128_kernel<{args.b - 1}, true, true>",
                                                 256 * 1024),
                     "kernel": "encode128_kernel", "algorithmic_per_launch": f"{enc_flops} flop "
                     "((2 d^2 + 2 d m) per key; the hi/lo split executes 5 bf16 passes of the two GEMMs)"},
    }

    # A plain streaming kernel for reference: a 1 GiB device copy (torch),
    # counted as bytes read + bytes written.
    cp_src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cp_dst = torch.empty_like(cp_src)
    for _ in range(3):
        cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        cp_dst.copy_(cp_src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * cp_src.numel() * 4 / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
    del cp_src, cp_dst
    out["hbm_stream_reference"] = {"kernel": "1 GiB device copy (torch)", "GBps": round(copy_gbps, 1),
                                   "frac_hbm_peak": round(copy_gbps / HBM_PEAK_GBPS, 4)}

    if not args.no_hbm_score:
        # 32 layers' codes of the same shape streamed by one launch (n_kv = 256)
        nL = N_KV * LAYERS
        big = tq.alloc_codes(p, nL * SEQ, dev)
        for layer in range(LAYERS):
            sl = slice(layer * n, (layer + 1) * n)
            xl = synth.llama_keys(heads=N_KV, seq=SEQ, seed=100 + layer, device=dev)
            tq.encode(p, xl, {k: (v[sl] if v is not None else None) for k, v in big.items()})
        del xl
        qb = synth.queries(nL * G, seed=6, device=dev)
        lb = torch.empty((nL * G, SEQ), device=dev)
        wsb = torch.empty(tq.score_workspace_bytes(p, nL, G), dtype=torch.uint8, device=dev)
        for _ in range(3):
            tq.score(p, qb, big, nL, G, SEQ, lb, wsb)
        torch.cuda.synchronize()
        reps = max(5, args.steps // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            tq.score(p, qb, big, nL, G, SEQ, lb, wsb)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        bytes_ = code_bytes * nL * SEQ + 4 * nL * G * SEQ
        gbps = bytes_ / (ms * 1e-3) / 1e9
        out["score_hbm"] = {"workload": f"{LAYERS} layers x {N_KV} KV heads x {SEQ} positions, one launch",
                            "ms": round(ms, 4), "GBps": round(gbps, 1),
                            "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                            "frac_measured_copy": round(gbps / copy_gbps, 4),
                            "bytes_per_launch": bytes_}
        out["roofline_score"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                                 "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                                 # the launch of this workload: one 64-thread wave per 256 keys of each
                                 # (KV head, group of 4 query heads)
                                 "traffic": profiled_traffic(f"tq::score128_kernel<{args.b - 1}, true>",
                                                             nL * ((G + 3) // 4) * ((SEQ + 255) // 256) * 64),
                                 "kernel": "score128_kernel (+ qprep128_kernel)",
                                 "algorithmic_per_launch": f"{bytes_} B ({code_bytes} B of codes per key + 4 B per logit)"}
        del big, lb

    if not args.no_attend:
        # long-context decode attention: batch 4 x 8 KV heads x 131072 positions, d 128,
        # keys prod b=3 (m=128), values mse b=3; 32 query heads
        ab, akv, aseq = 4, 8, 131072
        kp = tq.Params(D, 3, M, tq.MODE_PROD, 2, 3)
        vp = tq.Params(D, 3, M, tq.MODE_MSE, 4, 0)
        kc = tq.alloc_codes(kp, ab * akv * aseq, dev)
        vc = tq.alloc_codes(vp, ab * akv * aseq, dev)
        # encoded in pieces of one layer's size (262 144 vectors), so that every
        # launch of the layer's encode kernel in a profile has the same work
        piece = N_KV * SEQ
        for b in range(ab):
            kx = synth.llama_keys(heads=akv, seq=aseq, seed=200 + b, device=dev)
            vx = synth.llama_keys(heads=akv, seq=aseq, seed=300 + b, device=dev)
            for o in range(0, akv * aseq, piece):
                sl = slice(b * akv * aseq + o, b * akv * aseq + o + piece)
                tq.encode(kp, kx[o:o + piece], {k: (v[sl] if v is not None else None) for k, v in kc.items()})
                tq.encode(vp, vx[o:o + piece], {k: (v[sl] if v is not None else None) for k, v in vc.items()})
        del kx, vx
        aq = synth.queries(ab * akv * G, seed=7, device=dev).reshape(ab, akv * G, D)
        aout = torch.empty((ab, akv * G, D), device=dev)
        aws = torch.empty(tq.attend_workspace_bytes(kp, vp, ab, akv, G, aseq), dtype=torch.uint8, device=dev)
        for _ in range(3):
            tq.attend(kp, vp, aq, ab, akv, G, kc, vc, aseq, aout, aws)
        torch.cuda.synchronize()
        reps = max(5, args.steps // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            tq.attend(kp, vp, aq, ab, akv, G, kc, vc, aseq, aout, aws)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nb = (sum(tq.codes_bytes(kp, 1)) + sum(tq.codes_bytes(vp, 1))) * ab * akv * aseq
        gbps = nb / (ms * 1e-3) / 1e9
        out["attend_hbm"] = {"workload": f"batch {ab} x {akv} KV heads x {aseq} positions x d {D}, "
                                         f"{akv * G} query heads; K prod b=3 m={M}, V mse b=3",
                             "ms": round(ms, 4), "GBps": round(gbps, 1),
                             "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                             "frac_measured_copy": round(gbps / copy_gbps, 4), "bytes_per_call": nb}
        # the same code arrays read as a paged store (512-position pages, vector
        # (page * n_kv + head) * 512 + offset) through a shuffled block table
        npg = aseq // tq.PAGE_POSITIONS
        perm = torch.randperm(ab * npg, generator=torch.Generator().manual_seed(11))
        bt = perm.reshape(ab, npg).to(torch.int32).to(dev)
        lens = torch.full((ab,), aseq, dtype=torch.int32, device=dev)
        pws = torch.empty(tq.attend_paged_workspace_bytes(kp, vp, ab, akv, G, npg), dtype=torch.uint8, device=dev)
        for _ in range(3):
            tq.attend_paged(kp, vp, aq, ab, akv, G, kc, vc, ab * npg, bt, lens, aout, pws)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            tq.attend_paged(kp, vp, aq, ab, akv, G, kc, vc, ab * npg, bt, lens, aout, pws)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbps = nb / (ms * 1e-3) / 1e9
        out["attend_paged_hbm"] = {"workload": f"as attend_hbm, the codes as {ab * npg} pages of "
                                               f"{tq.PAGE_POSITIONS} positions in a shuffled block table",
                                   "ms": round(ms, 4), "GBps": round(gbps, 1),
                                   "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                                   "frac_measured_copy": round(gbps / copy_gbps, 4), "bytes_per_call": nb}
        del kc, vc

    if not args.no_polar:
        # PolarQuant variant (4 bits at level 1, 2 bits above: 52 B per key) on the
        # same Llama-shaped layer: encode of 8 x 32768 bf16 keys, and the score of
        # 32 query heads streaming 32 such layers' codes from HBM
        pp = tq.PolarParams(D, 4, 2, 2)
        px = synth.llama_keys(heads=N_KV, seq=SEQ, seed=1, device=dev)
        pc = tq.alloc_polar_codes(N_KV * SEQ, dev)
        nL = LAYERS * N_KV
        pbig = tq.alloc_polar_codes(nL * SEQ, dev)
        for layer in range(LAYERS):
            xl = synth.llama_keys(heads=N_KV, seq=SEQ, seed=100 + layer, device=dev)
            sl = slice(layer * N_KV * SEQ, (layer + 1) * N_KV * SEQ)
            tq.polar_encode(pp, xl, {k: v[sl] for k, v in pbig.items()})
        del xl
        pq_ = synth.queries(nL * G, seed=6, device=dev)
        plg = torch.empty((nL * G, SEQ), device=dev)
        pws = torch.empty(tq.polar_score_workspace_bytes(pp, nL, G), dtype=torch.uint8, device=dev)
        for _ in range(3):
            tq.polar_encode(pp, px, pc)
            tq.polar_score(pp, pq_, pbig, nL, G, SEQ, plg, pws)
        torch.cuda.synchronize()
        reps = max(5, args.steps // 2)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        for _ in range(reps):
            tq.polar_encode(pp, px, pc)
        e[1].record(stream)
        for _ in range(reps):
            tq.polar_score(pp, pq_, pbig, nL, G, SEQ, plg, pws)
        e[2].record(stream)
        torch.cuda.synchronize()
        enc_ms = e[0].elapsed_time(e[1]) / reps
        sc_ms = e[1].elapsed_time(e[2]) / reps
        n1 = N_KV * SEQ
        enc_exec = 2 * (2 * D * D) * n1                      # Pi x in 2 bf16 passes (hi, lo of Pi)
        sbytes = 52 * nL * SEQ + 4 * nL * G * SEQ
        out["polar"] = {
            "workload": f"PolarQuant d {D} (level 1: 4 bits, levels 2..7: 2 bits; 52 B per key); encode "
                        f"{N_KV} x {SEQ} bf16 Llama-shaped keys; score {nL * G} query heads over "
                        f"{LAYERS} layers x {N_KV} KV heads x {SEQ} positions",
            "encode_us": round(enc_ms * 1e3, 2), "encode_mvectors_per_s": round(n1 / (enc_ms * 1e-3) / 1e6, 1),
            "encode_frac_bf16_peak_executed": round(enc_exec / (enc_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "score_ms": round(sc_ms, 4), "score_GBps": round(sbytes / (sc_ms * 1e-3) / 1e9, 1),
            "score_frac_hbm_peak": round(sbytes / (sc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        }
        del px, pc, pbig, plg, pws

    if not args.no_split:
        # outlier-channel mixed bit widths (2.5 and 3.5 bits) on the same layer:
        # the 64 channels of largest mean square in head 0's keys form the
        # outlier group (one channel list for the layer; a list per head is a
        # launch per head); encode of the 8 x 32768 bf16 keys, and the score of
        # 1024 query heads over 32 such layers' codes
        sx = synth.llama_keys(heads=N_KV, seq=SEQ, seed=1, device=dev)
        ms = (sx[:SEQ].float() ** 2).mean(dim=0)
        order = torch.argsort(-ms, stable=True).cpu()
        chans = torch.cat([torch.sort(order[:64]).values, torch.sort(order[64:]).values]).tolist()
        nL = LAYERS * N_KV
        sq_ = synth.queries(nL * G, seed=6, device=dev)
        slg = torch.empty((nL * G, SEQ), device=dev)
        res = []
        for b_rest in (2, 3):
            sp_ = tq.SplitParams(chans, b_rest + 1, b_rest, 2, 3)
            sc1 = tq.alloc_split_codes(sp_, N_KV * SEQ, dev)
            sbig = tq.alloc_split_codes(sp_, nL * SEQ, dev)
            for layer in range(LAYERS):
                xl = synth.llama_keys(heads=N_KV, seq=SEQ, seed=100 + layer, device=dev)
                sl = slice(layer * N_KV * SEQ, (layer + 1) * N_KV * SEQ)
                tq.split_encode(sp_, xl, {k: v[sl] for k, v in sbig.items()})
            del xl
            sws = torch.empty(tq.split_score_workspace_bytes(sp_, nL, G), dtype=torch.uint8, device=dev)
            for _ in range(2):
                tq.split_encode(sp_, sx, sc1)
                tq.split_score(sp_, sq_, sbig, nL, G, SEQ, slg, sws)
            torch.cuda.synchronize()
            reps = max(3, args.steps // 10)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            for _ in range(reps):
                tq.split_encode(sp_, sx, sc1)
            e[1].record(stream)
            for _ in range(reps):
                tq.split_score(sp_, sq_, sbig, nL, G, SEQ, slg, sws)
            e[2].record(stream)
            torch.cuda.synchronize()
            enc_ms = e[0].elapsed_time(e[1]) / reps
            sc_ms = e[1].elapsed_time(e[2]) / reps
            rec = 4 * tq.split_words(sp_) + 16
            sbytes = rec * nL * SEQ + 4 * nL * G * SEQ
            res.append({"bits": b_rest + 0.5, "bytes_per_key": rec, "encode_us": round(enc_ms * 1e3, 2),
                        "encode_mvectors_per_s": round(N_KV * SEQ / (enc_ms * 1e-3) / 1e6, 1),
                        "score_ms": round(sc_ms, 4), "score_GBps": round(sbytes / (sc_ms * 1e-3) / 1e9, 1),
                        "score_frac_hbm_peak": round(sbytes / (sc_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)})
            del sc1, sbig, sws
        out["split"] = {"workload": f"outlier-channel split (64 + 64 channels) of {N_KV} x {SEQ} bf16 Llama-shaped "
                                    f"keys; score {nL * G} query heads over {LAYERS} layers",
                        "rows": res}
        del sx, slg

    if not args.no_sweep:
        # bit-width sweep: 65536 unit-direction x log-normal-norm float32 vectors, 1024 queries
        sn, snq = 65536, 1024
        sx = synth.sweep_keys(n=sn, seed=1, device=dev)
        sq = synth.queries(snq, seed=5, device=dev)
        true_ip = sq @ sx.T
        qn = torch.linalg.vector_norm(sq, dim=1, keepdim=True)
        xn = torch.linalg.vector_norm(sx, dim=1, keepdim=True).T
        rows = []
        for b in (1, 2, 3, 4):
            pp = tq.Params(D, b, M, tq.MODE_PROD, 2, 3)
            pm = tq.Params(D, b, M, tq.MODE_MSE, 2, 3)
            cp = tq.alloc_codes(pp, sn, dev)
            cm = tq.alloc_codes(pm, sn, dev)
            lg = torch.empty((snq, sn), device=dev)
            sws = torch.empty(tq.score_workspace_bytes(pp, 1, snq), dtype=torch.uint8, device=dev)
            xr = torch.empty_like(sx)
            tq.encode(pp, sx, cp)
            tq.score(pp, sq, cp, 1, snq, sn, lg, sws)
            torch.cuda.synchronize()
            reps = 5
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            for _ in range(reps):
                tq.encode(pp, sx, cp)
            e[1].record(stream)
            for _ in range(reps):
                tq.score(pp, sq, cp, 1, snq, sn, lg, sws)
            e[2].record(stream)
            tq.encode(pm, sx, cm)
            tq.decode(pm, cm, sn, xr)
            torch.cuda.synchronize()
            enc_ms = e[0].elapsed_time(e[1]) / reps
            sc_ms = e[1].elapsed_time(e[2]) / reps
            dist = (torch.sum((sx - xr) ** 2, dim=1) / torch.sum(sx * sx, dim=1)).mean().item()
            err = (lg - true_ip) / (qn * xn)
            rows.append({"b": b, "encode_ms": round(enc_ms, 4),
                         "encode_mvectors_per_s": round(sn / (enc_ms * 1e-3) / 1e6, 1),
                         "score_ms_1024q": round(sc_ms, 4),
                         "score_glogits_per_s": round(snq * sn / (sc_ms * 1e-3) / 1e9, 1),
                         "mse_distortion_mse_mode": round(dist, 6),
                         "ip_bias_prod": round(err.mean().item(), 7),
                         "ip_rmse_prod": round(err.pow(2).mean().sqrt().item(), 6)})
            del cp, cm, lg, sws, xr
        out["bit_width_sweep"] = {"workload": f"{sn} x d {D} float32 (unit direction x log-normal norm), "
                                              f"{snq} N(0,1) queries, m={M}", "rows": rows}

    if not args.no_highdim:
        # high-dimensional batched scoring: 1,048,576 x d 1024 float32 vectors
        # (N(0,1), 1% channels x10), b = 3, m = 1024; 1024 queries, top-10
        hn, hq, hd, hk = 1 << 20, 1024, 1024, 10
        hp = tq.Params(hd, 3, hd, tq.MODE_PROD, 2, 3)
        hx = synth.highdim_keys(hn, d=hd, seed=1, device=dev)
        hc = tq.alloc_codes(hp, hn, dev)
        hws = tq.alloc_workspace(tq.encode_workspace_bytes(hp, hn), dev)
        hqv = synth.queries(hq, d=hd, seed=5, device=dev)
        hidx = torch.empty((hq, hk), dtype=torch.int64, device=dev)
        hval = torch.empty((hq, hk), device=dev)
        hsws = torch.empty(tq.search_workspace_bytes(hp, hq, hn, hk), dtype=torch.uint8, device=dev)
        tq.encode(hp, hx, hc, workspace=hws)
        tq.search(hp, hqv, hc, hn, hk, hidx, hval, hsws)
        torch.cuda.synchronize()
        reps = 3
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        for _ in range(reps):
            tq.encode(hp, hx, hc, workspace=hws)
        e[1].record(stream)
        for _ in range(reps):
            tq.search(hp, hqv, hc, hn, hk, hidx, hval, hsws)
        e[2].record(stream)
        torch.cuda.synchronize()
        enc_ms = e[0].elapsed_time(e[1]) / reps
        se_ms = e[1].elapsed_time(e[2]) / reps
        enc_alg = (2 * hd * hd + 2 * hd * hd) * hn          # Pi x and S' r per vector
        enc_exec = 3 * enc_alg                                # hi/lo split: 3 bf16 products each
        pairs = hq * hn
        sc_alg = 2 * (hd + hd) * pairs                        # 2 (d + m) per (query, code)
        sc_exec = 2 * 4 * 3 * hd * pairs                      # 4 int8 limbs x 3 parts (2 planes + signs)
        out["highdim"] = {
            "workload": f"{hn} x d {hd} float32 vectors (N(0,1), 1% channels x10), b=3, m={hd}; "
                        f"{hq} N(0,1) queries, top-{hk}",
            "encode_ms": round(enc_ms, 3), "encode_mvectors_per_s": round(hn / (enc_ms * 1e-3) / 1e6, 2),
            "encode_tflops_algorithmic": round(enc_alg / (enc_ms * 1e-3) / 1e12, 1),
            "encode_tflops_executed_bf16": round(enc_exec / (enc_ms * 1e-3) / 1e12, 1),
            "encode_frac_bf16_peak_executed": round(enc_exec / (enc_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "search_ms": round(se_ms, 3),
            "search_gpairs_per_s": round(pairs / (se_ms * 1e-3) / 1e9, 1),
            "search_tops_algorithmic": round(sc_alg / (se_ms * 1e-3) / 1e12, 1),
            "search_tops_executed_int8": round(sc_exec / (se_ms * 1e-3) / 1e12, 1),
            "search_frac_int8_peak_executed": round(sc_exec / (se_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "codes_mb": round(sum(tq.codes_bytes(hp, hn)) / 1e6, 1),
        }
        del hx, hc, hws, hsws

    if not args.no_searchdb:
        # many-query search at database scale: 2^26 vectors of d = m = 128
        # (N(0,1), 1% channels x10, generated and encoded in 8 chunks), b = 3,
        # 3.76 GB of codes; 1024 queries, top-10, no logit matrix
        dn, dch, dnq, dk = 1 << 26, 1 << 23, 1024, 10
        dp = tq.Params(D, 3, M)
        dc = tq.alloc_codes(dp, dn, dev)
        for c in range(dn // dch):
            sl = slice(c * dch, (c + 1) * dch)
            dx = synth.highdim_keys(dch, d=D, seed=100 + c, device=dev)
            tq.encode(dp, dx, {k: (v[sl] if v is not None else None) for k, v in dc.items()})
            del dx
        dqv = synth.queries(dnq, d=D, seed=5, device=dev)
        didx = torch.empty((dnq, dk), dtype=torch.int64, device=dev)
        dval = torch.empty((dnq, dk), device=dev)
        dws = torch.empty(tq.search_workspace_bytes(dp, dnq, dn, dk), dtype=torch.uint8, device=dev)
        tq.search(dp, dqv, dc, dn, dk, didx, dval, dws)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            tq.search(dp, dqv, dc, dn, dk, didx, dval, dws)
        e1.record(stream)
        torch.cuda.synchronize()
        se_ms = e0.elapsed_time(e1) / reps
        pairs = dnq * dn
        sc_exec = 2 * 4 * 3 * D * pairs                      # 4 int8 limbs x 3 parts (2 planes + signs)
        nb = sum(tq.codes_bytes(dp, dn))
        out["search_db"] = {
            "workload": f"{dn} x d {D} float32 vectors (N(0,1), 1% channels x10), b=3, m={M}; "
                        f"{dnq} N(0,1) queries, top-{dk}",
            "codes_gb": round(nb / 1e9, 3),
            "search_ms": round(se_ms, 3),
            "search_gpairs_per_s": round(pairs / (se_ms * 1e-3) / 1e9, 1),
            "search_tops_executed_int8": round(sc_exec / (se_ms * 1e-3) / 1e12, 1),
            "search_frac_int8_peak_executed": round(sc_exec / (se_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
            "codes_read_gbps_once": round(nb / (se_ms * 1e-3) / 1e9, 1),
        }
        del dc, dws

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.b, args.cpu_sample_heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
