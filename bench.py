#!/usr/bin/env python3
"""Benchmark: causal bf16 attention forward + backward on one MI355X.

One step = one forward (attn_fwd) and one backward (attn_bwd) of causal
exact attention over the Llama-7B-shaped 16K workload (B=1, H=Hkv=32,
N=16384, d=128, bf16, iid N(0,1) synthetic inputs resident in HBM). Prints
one JSON line. FLOPs: forward 4*B*H*N^2*d halved for the causal mask,
backward 2.5x the forward. The line also carries the other workloads, each
against its own roofline: "configs" (the GPT-2 and BERT shapes, the 16K
sequence as 4 chunks and the 64K GQA sequence as 8 chunks), the sliding-
window, packed variable-length and block-sparse variants, the key/value-
cache forward on a decode and a chunked-prefill workload, and the causal
forward at the FlashAttention-2 ablation shape (context only).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published)

# HBM traffic of one bwd_dkdv_kernel launch on the 16K workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; calibrated against a plain
# 1 GiB device copy in the same process), valid only for the kernel sources
# and build flags whose SHA-1 is recorded with it (profiles/llama16k_causal_bf16_traffic.md).
DKDV_TRAFFIC = {"sources_sha1": "ac08606f580ebb709b7c85ceb88dcae38c0dda24", "bytes": 2849822628}   # fetch 2.581 GB + write 0.269 GB
DKDV_SOURCES = ("exact_attention_37_amd/csrc/bwd_mfma.hip", "exact_attention_37_amd/csrc/mfma_common.h",
                "exact_attention_37_amd/csrc/common.h", "exact_attention_37_amd/build.py")


def sources_sha1():
    import hashlib
    h = hashlib.sha1()
    for rel in DKDV_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline leg")
    ap.add_argument("--main-only", action="store_true",
                    help="time only the main step (for profiler runs): no secondary workloads")
    ap.add_argument("--workload", default="llama16k")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="after timing, run 3 plain device copies of MIB MiB (a known-size "
                         "reference for the HBM traffic counters)")
    return ap.parse_args()


def cpu_baseline(workload, heads=3):
    """The float64 oracle, untouched, on a bounded sample of the workload:
    `heads` query heads at the full sequence length, forward + backward."""
    import numpy as np
    import oracle
    from workloads import draw, as_f64, flops
    w = workload
    q, k, v, do = draw(1, heads, heads, w.N, w.d, seed=w.seed, dtype=w.torch_dtype)
    qq, kk, vv, dd = (as_f64(t) for t in (q, k, v, do))
    scale = w.d ** -0.5
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threads = os.cpu_count()
    t0 = time.perf_counter()
    oracle.forward(qq, kk, vv, True, scale)
    oracle.backward(qq, kk, vv, dd, True, scale)
    dt = time.perf_counter() - t0
    ff, fb = flops(1, heads, w.N, w.d, True)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), model)
    except OSError:
        pass
    return {"value": round((ff + fb) / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(dt, 2), "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": "%d query heads (B=1, N=%d, d=%d, causal) fwd+bwd in float64; "
                      "FLOPs counted as for the GPU" % (heads, w.N, w.d)}


def bench_cache(mi, torch, name, reps=20):
    """Key/value-cache forward (attn_fwd_kvcache) on one cache workload:
    event-timed average over `reps` calls, against the HBM roofline.
    Algorithmic bytes: the valid K and V cache rows once, Q and O once, LSE."""
    from workloads import CACHE_WORKLOADS, draw_cache_workload
    w = CACHE_WORKLOADS[name]
    q, k, v, lens = [t.to("cuda:0") for t in draw_cache_workload(w)]
    scale = w.d ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=q.device)
    for _ in range(3):
        mi.fwd_kvcache(q, k, v, lens, True, scale, 0, out=o, out_lse=lse)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mi.fwd_kvcache(q, k, v, lens, True, scale, 0, out=o, out_lse=lse)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    L = [int(x) for x in lens.tolist()]
    kv_bytes = 2.0 * sum(L) * w.Hkv * w.d * 2
    qo_bytes = 2.0 * w.B * w.Nq * w.H * w.d * 2 + w.B * w.H * w.Nq * 4
    nbytes = kv_bytes + qo_bytes
    # visible (query, key) pairs: row i sees L - Nq + i + 1 keys
    pairs = sum(sum(max(0, Lb - w.Nq + i + 1) for i in range(w.Nq)) for Lb in L) * w.H
    nflops = 4.0 * w.d * pairs
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfs = nflops / (ms * 1e-3) / 1e12
    del q, k, v, lens, o, lse
    # the bound follows from the arithmetic intensity against the ridge point
    if nflops / nbytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tfs, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tfs / PEAK_BF16_TFLOPS, 4)}
    return {"workload": "%s: B=%d H=%d Hkv=%d Nq=%d cache=%d d=%d causal, lens %d..%d" % (
                w.name, w.B, w.H, w.Hkv, w.Nq, w.Nk, w.d, min(L), max(L)),
            "ms": round(ms, 4), "bytes": int(nbytes), "flops": nflops, "GB_per_s": round(gbs, 1),
            "tflops": round(tfs, 2), "roofline": roof}


def bench_window(mi, torch, q, k, v, do, w, window, reps=10):
    """Causal sliding-window fwd+bwd (attn_fwd_window / attn_bwd_window) on
    the main workload's tensors. FLOPs count the visible pairs only: row i
    sees min(i + 1, window) keys; backward 2.5x forward."""
    scale = w.d ** -0.5
    for _ in range(2):
        o, lse = mi.fwd(q, k, v, True, scale, window=window)
        mi.bwd(q, k, v, o, lse, do, True, scale, window=window)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    f_ms = b_ms = 0.0
    for _ in range(reps):
        e[0].record()
        o, lse = mi.fwd(q, k, v, True, scale, window=window)
        e[1].record()
        mi.bwd(q, k, v, o, lse, do, True, scale, window=window)
        e[2].record()
        torch.cuda.synchronize()
        f_ms += e[0].elapsed_time(e[1]) / reps
        b_ms += e[1].elapsed_time(e[2]) / reps
    W, N = window, w.N
    pairs = (W * (W + 1) // 2 + (N - W) * W) if N > W else N * (N + 1) // 2
    ff = 4.0 * w.B * w.H * w.d * pairs
    fb = 2.5 * ff
    tf = (ff + fb) / ((f_ms + b_ms) * 1e-3) / 1e12
    return {"workload": "%s with a causal sliding window of %d keys" % (w.name, W),
            "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "tflops": round(tf, 2),
            "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2)}


def bench_varlen(mi, torch, reps=10):
    """Causal fwd+bwd over the packed variable-length workload
    (attn_fwd_varlen / attn_bwd_varlen). FLOPs count the visible pairs of
    each sequence, L (L + 1) / 2; backward 2.5x forward."""
    from workloads import VARLEN_WORKLOADS, draw_varlen_workload
    w = VARLEN_WORKLOADS["packed16k"]
    q, k, v, do, cu = draw_varlen_workload(w)
    lengths = (cu[1:] - cu[:-1]).tolist()
    q, k, v, do, cu = (t.to("cuda:0") for t in (q, k, v, do, cu))
    scale, L = w.d ** -0.5, max(lengths)
    for _ in range(2):
        o, lse = mi.fwd_varlen(q, k, v, cu, L, True, scale)
        mi.bwd_varlen(q, k, v, o, lse, do, cu, L, True, scale)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    f_ms = b_ms = 0.0
    for _ in range(reps):
        e[0].record()
        o, lse = mi.fwd_varlen(q, k, v, cu, L, True, scale)
        e[1].record()
        mi.bwd_varlen(q, k, v, o, lse, do, cu, L, True, scale)
        e[2].record()
        torch.cuda.synchronize()
        f_ms += e[0].elapsed_time(e[1]) / reps
        b_ms += e[1].elapsed_time(e[2]) / reps
    pairs = sum(n * (n + 1) // 2 for n in lengths)
    ff = 4.0 * w.H * w.d * pairs
    tf = 3.5 * ff / ((f_ms + b_ms) * 1e-3) / 1e12
    return {"workload": "%s: %d tokens packed as sequences of %s, %d heads, d=%d, causal"
                        % (w.name, w.total, lengths, w.H, w.d),
            "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "tflops": round(tf, 2),
            "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2)}


def visible_pairs_blocksparse(mask, N, causal, rows=256, cols=128):
    """(query, key) pairs a block mask keeps (and the causal mask allows)."""
    import numpy as np
    total = 0
    i = np.arange(N)
    for r, c in zip(*np.nonzero(mask)):
        ii = i[r * rows:min(N, (r + 1) * rows)]
        c0, c1 = c * cols, min(N, (c + 1) * cols)
        total += int(np.sum(np.clip(np.minimum(ii, c1 - 1) - c0 + 1, 0, c1 - c0))) if causal else len(ii) * (c1 - c0)
    return total


def bench_blocksparse(mi, torch, q, k, v, do, w, density=0.25, reps=10):
    """Causal block-sparse fwd+bwd (attn_fwd_blocksparse / attn_bwd_blocksparse)
    on the main workload's tensors with a quarter of the 256 x 128 blocks kept
    plus the diagonal. FLOPs count the kept, visible pairs; backward 2.5x."""
    from workloads import draw_block_mask
    mask = draw_block_mask(w.N, density, seed=9)
    md = mask.to("cuda:0")
    scale = w.d ** -0.5
    for _ in range(2):
        o, lse = mi.fwd_blocksparse(q, k, v, md, True, scale)
        mi.bwd_blocksparse(q, k, v, o, lse, do, md, True, scale)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    f_ms = b_ms = 0.0
    for _ in range(reps):
        e[0].record()
        o, lse = mi.fwd_blocksparse(q, k, v, md, True, scale)
        e[1].record()
        mi.bwd_blocksparse(q, k, v, o, lse, do, md, True, scale)
        e[2].record()
        torch.cuda.synchronize()
        f_ms += e[0].elapsed_time(e[1]) / reps
        b_ms += e[1].elapsed_time(e[2]) / reps
    pairs = visible_pairs_blocksparse(mask.numpy(), w.N, True)
    ff = 4.0 * w.B * w.H * w.d * pairs
    tf = 3.5 * ff / ((f_ms + b_ms) * 1e-3) / 1e12
    dense = w.N * (w.N + 1) // 2
    return {"workload": "%s causal, block mask of 256 x 128 blocks, %d of %d kept (density %.2f + diagonal, "
                        "seed 9): %.1f%% of the causal pairs" % (w.name, int(mask.sum()), mask.numel(), density,
                                                                  100.0 * pairs / dense),
            "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "tflops": round(tf, 2),
            "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2)}


def time_fwd_bwd(torch, fwd, bwd, reps, flush=None):
    """Average event-timed forward and backward (ms) over `reps` calls. With
    `flush` (a device tensor), it is overwritten before every rep, outside the
    timed events, so that the inputs are not served from the caches."""
    # all reps are enqueued before one synchronisation, so the host's call
    # overhead overlaps the device work instead of landing between events
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in evs:
        if flush is not None:
            flush.fill_(1)
        e[0].record()
        out = fwd()
        e[1].record()
        bwd(*out)
        e[2].record()
    torch.cuda.synchronize()
    f_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / reps
    b_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / reps
    return f_ms, b_ms


def algorithmic_bytes(w):
    """Bytes of the forward and the backward with every tensor touched once:
    forward reads Q, K, V and writes O, LSE; backward reads Q, K, V, O, dO,
    LSE, writes dQ, dK, dV and writes and reads the rowsum vector D."""
    e = 4 if w.dtype == "f32" else 2
    nq = w.B * w.N * w.H * w.d * e
    nk = w.B * w.N * w.Hkv * w.d * e
    nl = w.B * w.H * w.N * 4
    return 2 * nq + 2 * nk + nl, 4 * nq + 4 * nk + 3 * nl


def bench_workload(mi, torch, name, reps=20):
    """fwd+bwd on a whole small workload (GPT-2 or BERT shape): TFLOP/s against
    the bf16 peak and against its own roofline min(peak, intensity x HBM
    bandwidth). These working sets (150-400 MB) fit largely in the 256 MB
    last-level cache, so a second timing overwrites a 1 GiB buffer before
    every rep."""
    from workloads import WORKLOADS, draw_workload, flops
    w = WORKLOADS[name]
    causal = w.causal[0]
    q, k, v, do = [t.to("cuda:0") for t in draw_workload(w)]
    scale = w.d ** -0.5
    o, lse = torch.empty_like(q), torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fwd = lambda: mi.fwd(q, k, v, causal, scale, out=o, out_lse=lse)
    bwd = lambda o_, l_: mi.bwd(q, k, v, o_, l_, do, causal, scale, dq=dq, dk=dk, dv=dv)
    time_fwd_bwd(torch, fwd, bwd, 3)
    f_ms, b_ms = time_fwd_bwd(torch, fwd, bwd, reps)
    # the throughput: steps back to back, one event pair around all of them
    # (an event between two kernels costs a few microseconds of device time,
    # much of a 0.1 ms step)
    steps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        bwd(*fwd())
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=q.device)
    fc_ms, bc_ms = time_fwd_bwd(torch, fwd, bwd, reps, flush=flush)
    del flush
    ff, fb = flops(w.B, w.H, w.N, w.d, causal)
    bf_, bb = algorithmic_bytes(w)
    ridge_tf = (ff + fb) / (bf_ + bb) * PEAK_HBM_GBS / 1e3        # intensity x bandwidth, TFLOP/s
    roof_tf = min(PEAK_BF16_TFLOPS, ridge_tf)
    tf = (ff + fb) / (step_ms * 1e-3) / 1e12
    tfc = (ff + fb) / ((fc_ms + bc_ms) * 1e-3) / 1e12
    return {"workload": "%s: B=%d H=%d Hkv=%d N=%d d=%d %s, fwd+bwd" % (
                w.name, w.B, w.H, w.Hkv, w.N, w.d, "causal" if causal else "non-causal"),
            "step_ms": round(step_ms, 4),
            "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "split_note": "fwd_ms, bwd_ms: each phase between its own events; tflops from step_ms (%d steps back to back)" % steps,
            "tflops": round(tf, 2),
            "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
            "roofline": {"bound": "mfma" if roof_tf >= PEAK_BF16_TFLOPS else "hbm", "achieved": round(tf, 2),
                         "peak": round(roof_tf, 1), "unit": "TFLOP/s", "frac": round(tf / roof_tf, 4),
                         "algorithmic_bytes": int(bf_ + bb)},
            "cold": {"fwd_ms": round(fc_ms, 4), "bwd_ms": round(bc_ms, 4), "tflops": round(tfc, 2),
                     "note": "1 GiB buffer overwritten before every rep"}}


def bench_chunked(mi, torch, name, reps=3):
    """The chunk-pair driver (attn_fwd_chunked / attn_bwd_chunked) on a
    chunked workload; FLOPs counted as for the whole problem."""
    from workloads import WORKLOADS, draw_workload, flops
    w = WORKLOADS[name]
    q, k, v, do = [t.to("cuda:0") for t in draw_workload(w)]
    scale = w.d ** -0.5
    fwd = lambda: mi.fwd_chunked(q, k, v, w.chunks, scale)
    bwd = lambda o_, l_: mi.bwd_chunked(q, k, v, o_, l_, do, w.chunks, scale)
    time_fwd_bwd(torch, fwd, bwd, 2)
    f_ms, b_ms = time_fwd_bwd(torch, fwd, bwd, reps)
    ff, fb = flops(w.B, w.H, w.N, w.d, True)
    tf = (ff + fb) / ((f_ms + b_ms) * 1e-3) / 1e12
    out = {"workload": "%s: B=%d H=%d Hkv=%d N=%d d=%d causal, %d chunks of %d rows in balanced rounds, fwd+bwd" % (
               w.name, w.B, w.H, w.Hkv, w.N, w.d, w.chunks, w.N // w.chunks),
           "fwd_ms": round(f_ms, 3), "bwd_ms": round(b_ms, 3), "tflops": round(tf, 2),
           "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}
    del q, k, v, do
    return out


def bench_fa2_ablation_shape(mi, torch, reps=20):
    """Causal forward at the shape of the FlashAttention-2 authors' ablation
    table (B = 8 and 1, H = 16, N = 2048, d = 128): context only, next to
    their A100 figures."""
    from workloads import draw, flops
    out = {}
    for B in (8, 1):
        q, k, v, _ = [t.to("cuda:0") for t in draw(B, 16, 16, 2048, 128, seed=10 + B)]
        o, lse = torch.empty_like(q), torch.empty((B, 16, 2048), dtype=torch.float32, device=q.device)
        for _ in range(3):
            mi.fwd(q, k, v, True, 128 ** -0.5, out=o, out_lse=lse)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            mi.fwd(q, k, v, True, 128 ** -0.5, out=o, out_lse=lse)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        ff, _ = flops(B, 16, 2048, 128, True)
        out["B%d" % B] = {"fwd_ms": round(ms, 4), "tflops": round(ff / (ms * 1e-3) / 1e12, 2)}
    out["workload"] = "causal forward, H=16, N=2048, d=128, bf16 (the FlashAttention-2 ablation shape; context only)"
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: libmiattn has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import exact_attention_37_amd as mi
    from workloads import WORKLOADS, draw_workload, flops

    w = WORKLOADS[args.workload]
    causal = w.causal[0]
    scale = w.d ** -0.5
    q, k, v, do = [t.to("cuda:0") for t in draw_workload(w)]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    torch.cuda.synchronize()

    def step(ev=None):
        # events (all on torch's current stream, which is the stream the
        # library launches on): before fwd | after fwd | after the dQ kernel
        # (which also forms the rowsum D) | after the dK/dV kernel | after bwd
        if ev is not None:
            ev[0].record()
        mi.fwd(q, k, v, causal, scale, out=o, out_lse=lse)
        if ev is not None:
            ev[1].record()
        mi.bwd(q, k, v, o, lse, do, causal, scale, dq=dq, dk=dk, dv=dv,
               marks=None if ev is None else (ev[2], ev[3]))
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    def avg(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in evs) / args.steps
    fwd_ms, bwd_ms = avg(0, 1), avg(1, 4)
    dq_ms, dkdv_ms = avg(1, 2), avg(2, 3)
    ms = wall * 1e3 / args.steps

    ff, fb = flops(w.B, w.H, w.N, w.d, causal)
    value = (ff + fb) / (ms * 1e-3) / 1e12
    fwd_tf = ff / (fwd_ms * 1e-3) / 1e12
    bwd_tf = fb / (bwd_ms * 1e-3) / 1e12
    # Dominant kernel: bwd_dkdv_kernel (the largest share of the step). Its
    # algorithmic work is 4 of the backward's 5 counted products (S, dP,
    # dV^T, dK^T: 8 d FLOPs per visible (query, key) pair) = 2 x the forward
    # count; the dQ kernel's recomputed S and dP are not algorithmic.
    dkdv_flops = 2.0 * ff
    dkdv_tf = dkdv_flops / (dkdv_ms * 1e-3) / 1e12
    traffic = None
    if DKDV_TRAFFIC is not None and args.workload == "llama16k" and DKDV_TRAFFIC["sources_sha1"] == sources_sha1():
        traffic = DKDV_TRAFFIC["bytes"]
    out = {
        "metric": "causal bf16 attention fwd+bwd TFLOP/s on 1 GPU and % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: B=%d H=%d Hkv=%d N=%d d=%d %s, fwd+bwd" % (w.name, w.B, w.H, w.Hkv, w.N, w.d, "causal" if causal else "non-causal"),
                   "global_batch": w.B, "seq_len": w.N, "parallelism": "none (1 GPU)"},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "fwd_tflops": round(fwd_tf, 2), "bwd_tflops": round(bwd_tf, 2),
        "kernel_ms": {"fwd_mfma": round(fwd_ms, 4), "bwd_dq": round(dq_ms, 4), "bwd_dkdv": round(dkdv_ms, 4)},
        "roofline": {"bound": "mfma", "kernel": "bwd_dkdv_kernel", "achieved": round(dkdv_tf, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dkdv_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if not args.main_only:
        out["window"] = bench_window(mi, torch, q, k, v, do, w, 4096)
        out["varlen"] = bench_varlen(mi, torch)
        out["blocksparse"] = bench_blocksparse(mi, torch, q, k, v, do, w)
        out["kvcache"] = {name: bench_cache(mi, torch, name) for name in ("decode16k", "prefill16k")}
        del q, k, v, do, o, lse, dq, dk, dv
        out["configs"] = {
            "gpt2": bench_workload(mi, torch, "gpt2"),
            "bert": bench_workload(mi, torch, "bert"),
            "llama16k_chunked4": bench_chunked(mi, torch, "llama16k"),
            "gqa64k_chunked8": bench_chunked(mi, torch, "gqa64k"),
        }
        out["fa2_ablation_shape"] = bench_fa2_ablation_shape(mi, torch)
    if args.calib_copy:
        nbytes = args.calib_copy << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = nbytes
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
