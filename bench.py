"""Benchmark of the transposable 2:4 FFN hot path on one MI355X.

Workload: one GPT-2-1.5B-shaped FFN layer (d = 1600, 4d = 6400, 16384
tokens) run as the noisy re-search loop: at step s the weights are
W_s = fp16(f32(W_{s-1}) + N(0, 1e-3)) (precomputed and resident in HBM before
timing), and each step runs

    search+compress(W1_s and W2_s, one launch)         (sp24_search_compress_batch)
        with the flip count of each weight fused in: each weight's index
        buffer is updated in place and the entries that changed are counted
    Y1  = X   W1s^T,  dX1 = dY1 W1s                     (one sp24_spmm_group launch
    Y2  = H   W2s^T,  dX2 = dY2 W2s                      for all four products)

Prints one JSON line.  ``value`` is dense-equivalent GEMM TFLOP/s over the
whole step (2*T*N*K summed over the four GEMMs, divided by the wall time of
the step including the search+compress launch).  The line also carries the
search+compress GB/s (4.375 algorithmic bytes per weight element), the GEMM
kernel's roofline fraction, the per-step flip rates and the CPU oracle
baseline.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 60] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from structured_sparse_transformer_amd import workloads as WL  # noqa: E402

HBM_PEAK_GBPS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0      # dense fp16 matrix-core peak of MI355X
SC_BYTES_PER_ELEM = 4.375           # read W 2 and previous idx 1/16; write idx 1/16, two 2:4 forms 2 x (1 + 1/8)
COUNTERS = os.path.join(ROOT, "profiles", "spmm_group_gpt2-1.5b_counters.json")
DECAY = 2e-4                         # masked decay factor of the weight-gradient leg
GEGLU_GROUP = 16                     # GEGLU column layout: blocks of 16 values, then their 16 gates
TRIALS = 5                           # repeated timings behind each reported median
ROTATE_BYTES = 512 * 1024 * 1024     # rotating input sets exceed L2 and the 256 MB last-level cache
WARM_VERSIONS = 20                   # distinct weight versions the warm-up steps cycle through


def mvue_uniforms(torch, dev, cfg):
    """One fp32 uniform per group of 4 entries of dY1 [T, 4d], drawn on the
    device with a fixed torch seed."""
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed + 1)
    return torch.rand(cfg.tokens, cfg.dff // 4, generator=g, device=dev, dtype=torch.float32)


def geglu_inputs(torch, dev, cfg):
    """GEGLU input of a gated FFN of the same width: U [T, 2 * 4d] (values and
    gates in blocks of GEGLU_GROUP), dOut [T, 4d]; N(0, 1) draws made on the
    device (a fixed torch seed) to keep the host side short."""
    g = torch.Generator(device=dev)
    g.manual_seed(cfg.seed)
    U = torch.randn(cfg.tokens, 2 * cfg.dff, generator=g, device=dev).half()
    gd = torch.randn(cfg.tokens, cfg.dff, generator=g, device=dev).half()
    return U, gd
GEMM_SRC = os.path.join(ROOT, "structured_sparse_transformer_amd", "csrc", "sp24_spmm.hip")
SC_SRC = os.path.join(ROOT, "structured_sparse_transformer_amd", "csrc", "sp24_search.hip")
SC_COUNTERS = os.path.join(ROOT, "profiles", "search_compress_gpt2-1.5b_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_counters():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when the summary is missing or the kernel source changed since."""
    try:
        c = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if c.get("source_sha256_16") != src_hash(GEMM_SRC):
        return None
    return c.get("hbm_bytes_per_launch")


def sc_traffic_from_counters():
    """HBM bytes per batched search+compress launch (both 1.5B weights) from the
    committed counter summary, or None when missing or stale."""
    try:
        c = json.load(open(SC_COUNTERS))
    except (OSError, ValueError):
        return None
    if c.get("source_sha256_16") != src_hash(SC_SRC):
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, inp, sample_tokens: int, steps: int = 3):
    """The CPU oracle on a bounded sample of the loop (its first `steps`
    steps), scaled to TFLOP/s."""
    from oracle import sp24_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = os.cpu_count() or 1
    # the loop's first weight versions and the masks before step 0 (untimed)
    w1s = [w for _, w in WL.noisy_weights(cfg, inp.w1, 1, steps)]
    w2s = [w for _, w in WL.noisy_weights(cfg, inp.w2, 2, steps)]
    prev = [O.mask_search(inp.w1), O.mask_search(inp.w2)]
    Ts = sample_tokens if 0 < sample_tokens < cfg.tokens else cfg.tokens
    d, f = cfg.d, cfg.dff
    t_sc = t_gemm = 0.0
    for s in range(steps):
        t0 = time.perf_counter()
        forms = []
        for k, W in enumerate((w1s[s], w2s[s])):
            idx = O.mask_search(W)
            O.flip_count(prev[k], idx)
            forms.append(O.compress(W, idx))
            prev[k] = idx
        t_sc += time.perf_counter() - t0
        t0 = time.perf_counter()
        (f1, f2) = forms
        O.spmm_fwd(inp.x[:Ts], f1["vals_row"], f1["meta_row"], f, d)
        O.spmm_bwd_input(inp.dy1[:Ts], f1["vals_col"], f1["meta_col"], f, d)
        O.spmm_fwd(inp.h[:Ts], f2["vals_row"], f2["meta_row"], d, f)
        O.spmm_bwd_input(inp.dy2[:Ts], f2["vals_col"], f2["meta_col"], d, f)
        t_gemm += time.perf_counter() - t0
    step_s = (t_sc + t_gemm * cfg.tokens / Ts) / steps
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu_model)
    except OSError:
        pass
    return {
        "value": round(cfg.dense_equiv_flops() / step_s / 1e12, 4),
        "unit": "TFLOP/s",
        "cores": int(blas_threads),
        "cpu_model": cpu_model,
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": (f"the first {steps} steps of the 1.5B loop: mask search + flip count + compress of W1 and W2 "
                   f"in full (NumPy, single thread, {t_sc:.1f} s) and the four float64 GEMMs "
                   + (f"on all {cfg.tokens} tokens" if Ts == cfg.tokens else
                      f"on the first {Ts} of {cfg.tokens} tokens, time scaled linearly to all tokens")
                   + f" (BLAS, {blas_threads} threads, {t_gemm:.1f} s)"),
        "search_compress_GBps": round(SC_BYTES_PER_ELEM * (inp.w1.size + inp.w2.size) * steps / t_sc / 1e9, 4),
    }


def profile_only(args, sp24, torch, dev, cfg, F1, F2, FL, W1s, W2s, X, dY1, H, dY2, Y1, dX1, Y2, dX2):
    """Runs one kernel family alone so that counter passes see only it."""
    d, f = cfg.d, cfg.dff
    n = args.steps
    if args.profile_kernel == "copy":
        # plain copy of a known size: calibrates FETCH_SIZE / WRITE_SIZE
        src = torch.empty(256 * 1024 * 1024, dtype=torch.float16, device=dev)      # 512 MiB
        dst = torch.empty_like(src)
        for _ in range(n):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy: {n} x 512 MiB")
        return
    if args.profile_kernel == "ffn_layer":
        # the gated FFN layer step of the ffn_layer_step object, alone
        from structured_sparse_transformer_amd.ffn import SparseGegluFFN
        layer = SparseGegluFFN(W1s[0], W2s[0][:, :f // 2].contiguous(), DECAY)
        layer.refresh()
        for _ in range(args.warmup + n):    # the clocks ramp over the first steps
            layer.refresh()
            _, saved = layer.forward(X)
            layer.backward(dY2, saved)
        torch.cuda.synchronize()
        log(f"ffn_layer: {args.warmup} + {n} steps")
        return
    if args.profile_kernel == "mvue":
        Um = mvue_uniforms(torch, dev, cfg)
        for _ in range(n):
            sp24.sp24_mvue(dY1, Um)
        torch.cuda.synchronize()
        log(f"mvue: {n} rounds")
        return
    if args.profile_kernel == "geglu":
        U, gd = geglu_inputs(torch, dev, cfg)
        out, dU = torch.empty_like(gd), torch.empty_like(U)
        for _ in range(n):
            sp24.sp24_geglu_fwd(U, GEGLU_GROUP, out=out)
            sp24.sp24_geglu_bwd(U, gd, GEGLU_GROUP, dU=dU)
        torch.cuda.synchronize()
        log(f"geglu: {n} rounds")
        return
    if args.profile_kernel == "weight_grad":
        sp24.sp24_search_compress_batch([W1s[0], W2s[0]], outs=[F1, F2])
        dW1 = torch.empty(d * 4, d, dtype=torch.float32, device=dev)
        dW2 = torch.empty(d, d * 4, dtype=torch.float32, device=dev)
        for _ in range(n):
            sp24.sp24_weight_grad(dY1, X, W1s[0], F1["idx"], DECAY, dW=dW1)
            sp24.sp24_weight_grad(dY2, H, W2s[0], F2["idx"], DECAY, dW=dW2)
        torch.cuda.synchronize()
        log(f"weight_grad: {n} rounds")
        return
    if args.profile_kernel == "flip_count":
        prev = F1["idx"].clone()
        sp24.sp24_search_compress_batch([W1s[0], W2s[0]], outs=[F1, F2])
        for _ in range(n):
            sp24.sp24_flip_count(prev, F1["idx"], FL[0, 0:1])
        torch.cuda.synchronize()
        log(f"flip_count: {n} calls")
        return
    for s in range(len(W1s)):
        sp24.sp24_search_compress_batch([W1s[s], W2s[s]], outs=[F1, F2], prev=[F1["idx"], F2["idx"]],
                                        flips=[FL[s, 0:1], FL[s, 1:2]])
        if args.profile_kernel == "search_compress" and s + 1 >= n:
            break
    torch.cuda.synchronize()
    if args.profile_kernel == "gemm":
        prods = [(X, F1["vals_row"], F1["meta_row"], Y1), (dY1, F1["vals_col"], F1["meta_col"], dX1),
                 (H, F2["vals_row"], F2["meta_row"], Y2), (dY2, F2["vals_col"], F2["meta_col"], dX2)]
        for _ in range(n):
            sp24.sp24_spmm_group(prods)
        torch.cuda.synchronize()
    if args.profile_kernel == "gemm_single":
        for _ in range(n):
            sp24.sp24_spmm_fwd(X, F1["vals_row"], F1["meta_row"], f, d, Y=Y1)
            sp24.sp24_spmm_bwd_input(dY1, F1["vals_col"], F1["meta_col"], f, d, dX=dX1)
            sp24.sp24_spmm_fwd(H, F2["vals_row"], F2["meta_row"], d, f, Y=Y2)
            sp24.sp24_spmm_bwd_input(dY2, F2["vals_col"], F2["meta_col"], d, f, dX=dX2)
        torch.cuda.synchronize()
    log(f"{args.profile_kernel}: {n} rounds")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the oracle's GEMMs in the CPU baseline, scaled to all tokens (0: all of them)")
    ap.add_argument("--no-context", action="store_true", help="skip the dense-matmul and copy context numbers")
    ap.add_argument("--no-layer-step", action="store_true",
                    help="skip the gated FFN layer step (its GEMMs have other shapes than the step's)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the 355M and 774M shapes (their launches would mix into a kernel trace's averages)")
    ap.add_argument("--profile-kernel", choices=["gemm", "gemm_single", "search_compress", "flip_count", "weight_grad",
                                                 "geglu", "ffn_layer", "mvue", "copy"],
                    help="run only this kernel --steps times (for rocprofv3 counter passes); prints no JSON")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the transposable 2:4 hot path here has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from structured_sparse_transformer_amd import sp24
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a HIP device")
    sp24.lib()
    dev = torch.device("cuda:0")
    cfg = WL.GPT2_1P5B
    d, f, T = cfg.d, cfg.dff, cfg.tokens
    # weight versions: the warm-up cycles through the first nwv (ending on the
    # last of them), the timed steps take the next --steps, so the first timed
    # step counts its flips against its true predecessor
    nwv = min(args.warmup, WARM_VERSIONS)
    nsteps = nwv + args.steps

    t0 = time.perf_counter()
    inp = WL.ffn_inputs(cfg)
    to = lambda a: torch.from_numpy(a).to(dev)  # noqa: E731
    X, H, dY1, dY2 = to(inp.x), to(inp.h), to(inp.dy1), to(inp.dy2)
    W1s = [to(w) for _, w in WL.noisy_weights(cfg, inp.w1, 1, nsteps)]
    W2s = [to(w) for _, w in WL.noisy_weights(cfg, inp.w2, 2, nsteps)]
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")

    def forms(R, C):
        return {"idx": torch.empty(R // 4, C // 4, dtype=torch.uint8, device=dev),
                "vals_row": torch.empty(R, C // 2, dtype=torch.float16, device=dev),
                "meta_row": torch.empty(R, C // 16, dtype=torch.int16, device=dev),
                "vals_col": torch.empty(C, R // 2, dtype=torch.float16, device=dev),
                "meta_col": torch.empty(C, R // 16, dtype=torch.int16, device=dev)}
    F1, F2 = forms(f, d), forms(d, f)
    # masks of the initial weights: the "previous" masks of step 0
    sp24.sp24_search_compress_batch([to(inp.w1), to(inp.w2)], outs=[F1, F2])
    FL = torch.zeros(nsteps, 2, dtype=torch.int64, device=dev)     # flips of W1, W2 per step
    FLb = torch.zeros(nsteps, 2, dtype=torch.int64, device=dev)    # the breakdown pass's own counters
    Y1 = torch.empty(T, f, dtype=torch.float16, device=dev)
    dX1 = torch.empty(T, d, dtype=torch.float16, device=dev)
    Y2 = torch.empty(T, d, dtype=torch.float16, device=dev)
    dX2 = torch.empty(T, f, dtype=torch.float16, device=dev)

    step_products = [(X, F1["vals_row"], F1["meta_row"], Y1), (dY1, F1["vals_col"], F1["meta_col"], dX1),
                     (H, F2["vals_row"], F2["meta_row"], Y2), (dY2, F2["vals_col"], F2["meta_col"], dX2)]

    def step(s, ev=None, fl=FL, marks=(0, 1, 5)):
        # ev[i] is recorded at mark i when i is in `marks`: 0 before the search,
        # 1 after it, 5 after the grouped launch of the four GEMMs
        def mark(i):
            if ev is not None and i in marks:
                ev[i].record()
        mark(0)
        sp24.sp24_search_compress_batch([W1s[s], W2s[s]], outs=[F1, F2], prev=[F1["idx"], F2["idx"]],
                                        flips=[fl[s, 0:1], fl[s, 1:2]])
        mark(1)
        sp24.sp24_spmm_group(step_products)
        mark(5)

    def step_single(s, ev, fl):
        # the same step with the four GEMMs as single launches and events
        # between them (the per-GEMM breakdown): ev[0] before the search, ev[1]
        # after it, ev[2..4] between the GEMMs, ev[5] after the last one
        ev[0].record()
        sp24.sp24_search_compress_batch([W1s[s], W2s[s]], outs=[F1, F2], prev=[F1["idx"], F2["idx"]],
                                        flips=[fl[s, 0:1], fl[s, 1:2]])
        ev[1].record()
        sp24.sp24_spmm_fwd(X, F1["vals_row"], F1["meta_row"], f, d, Y=Y1)
        ev[2].record()
        sp24.sp24_spmm_bwd_input(dY1, F1["vals_col"], F1["meta_col"], f, d, dX=dX1)
        ev[3].record()
        sp24.sp24_spmm_fwd(H, F2["vals_row"], F2["meta_row"], d, f, Y=Y2)
        ev[4].record()
        sp24.sp24_spmm_bwd_input(dY2, F2["vals_col"], F2["meta_col"], d, f, dX=dX2)
        ev[5].record()

    if args.profile_kernel:
        profile_only(args, sp24, torch, dev, cfg, F1, F2, FL, W1s, W2s, X, dY1, H, dY2, Y1, dX1, Y2, dX2)
        return

    # The step time settles only after about 40 steps from the idle set-up (the
    # first 20 steps after 20 warm-up steps ran 0.857-0.872 ms, the next 100
    # 0.830-0.842 ms), so the default warm-up is 60 steps
    for i in range(args.warmup):
        step((i - (args.warmup - nwv)) % nwv)
    torch.cuda.synchronize()

    # timed region: exactly --steps steps, synchronised on both sides.  Two
    # events per step (after the search and after the four GEMMs; about 5 us
    # of the step) time the GEMM launches and the search within this region.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    for k, s in enumerate(range(nwv, nsteps)):
        step(s, tev[k], marks=(1, 5))
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    ms_total = start.elapsed_time(end)
    ms_per_step = ms_total / args.steps
    log(f"timed {args.steps} steps: {ms_total:.3f} ms on events, {wall_ms:.3f} ms wall")
    # the same --steps steps timed again in TRIALS more blocks, each between its
    # own synchronised pair of events (flips into scratch counters), for the
    # median beside the contract's single timing above
    trial_ms = []
    for _ in range(TRIALS):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for s in range(nwv, nsteps):
            step(s, fl=FLb)
        t1.record()
        torch.cuda.synchronize()
        trial_ms.append(t0.elapsed_time(t1) / args.steps)
    # search: from the previous step's last GEMM (or the start) to the end of
    # the search; GEMMs: the four calls of each step
    sc_ms = float(np.mean([(start if k == 0 else tev[k - 1][5]).elapsed_time(tev[k][1]) for k in range(args.steps)]))
    group_ms = float(np.mean([tev[k][1].elapsed_time(tev[k][5]) for k in range(args.steps)]))

    # per-GEMM breakdown: the same steps again with events between every
    # call, all enqueued before a single synchronisation so that host-side
    # call overhead never sits between two events of an idle GPU
    seg_trials = []
    for _ in range(TRIALS):
        evs = []
        for s in range(nwv, nsteps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
            step_single(s, ev, FLb)
            evs.append(ev)
        torch.cuda.synchronize()
        seg = np.zeros(5)
        for ev in evs:
            seg += [ev[i].elapsed_time(ev[i + 1]) for i in range(5)]
        seg_trials.append(seg / args.steps)
    seg_trials = np.array(seg_trials)
    gemm_ms = np.median(seg_trials[:, 1:], axis=0)
    gemm_ms_mean = seg_trials[:, 1:].mean(axis=0)
    gemm_shapes = cfg.gemm_shapes()
    sc_bytes = SC_BYTES_PER_ELEM * 2 * d * f
    sc_gbps = sc_bytes / (sc_ms * 1e-3) / 1e9
    gemm_dense_tflops = [2 * Tt * N * K / (ms * 1e-3) / 1e12 for (_, Tt, N, K), ms in zip(gemm_shapes, gemm_ms)]
    # roofline of the GEMM kernel: executed (non-zero) flops T*N*K per launch
    launch_flops = sum(Tt * N * K for (_, Tt, N, K) in gemm_shapes)     # one grouped launch: all four
    achieved = launch_flops / (group_ms * 1e-3) / 1e12
    single_achieved = launch_flops / (float(np.sum(gemm_ms)) * 1e-3) / 1e12
    traffic = traffic_from_counters()

    flips = FL[nwv:].cpu().numpy().astype(np.float64) / np.array([f * d, d * f], dtype=np.float64)

    # search+compress per weight: single-weight launches over every weight
    # version of the run (2 x 40 x 20.5 MB, more than L2 and the 256 MB
    # last-level cache hold), back to back, each counting its flips as in the
    # step
    pw_ctr = FLb[0, 1:2]
    def per_weight_us(Ws, F):
        sp24.sp24_search_compress_batch([Ws[0]], outs=[F], prev=[F["idx"]], flips=[pw_ctr])
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for Wk in Ws:
            sp24.sp24_search_compress_batch([Wk], outs=[F], prev=[F["idx"]], flips=[pw_ctr])
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / len(Ws)
    pw_trials = [[per_weight_us(W1s, F1) for _ in range(TRIALS)], [per_weight_us(W2s, F2) for _ in range(TRIALS)]]
    pw_us = [float(np.median(t)) for t in pw_trials]
    pw_gbps = [SC_BYTES_PER_ELEM * d * f / (us * 1e-6) / 1e9 for us in pw_us]

    # the step's batched launch (both weights, flips counted) back to back over
    # every weight version: one pair of events around all of them, so no
    # event's cost falls on a launch
    bb_ctr = torch.zeros(2, dtype=torch.int64, device=dev)
    def both_weights_us():
        run = lambda a, b: sp24.sp24_search_compress_batch(  # noqa: E731
            [a, b], outs=[F1, F2], prev=[F1["idx"], F2["idx"]], flips=[bb_ctr[0:1], bb_ctr[1:2]])
        run(W1s[0], W2s[0])
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for a, b in zip(W1s, W2s):
            run(a, b)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / len(W1s)
    bb_trials = [both_weights_us() for _ in range(TRIALS)]
    bb_us = float(np.median(bb_trials))
    bb_gbps = sc_bytes / (bb_us * 1e-6) / 1e9
    sc_traffic = sc_traffic_from_counters()

    # the standalone flip count (two index arrays of W1, 640000 blocks each),
    # back-to-back calls: launch-bound at this size
    fl_prev, fl_ctr, fl_calls = torch.roll(F1["idx"], 1, 0).contiguous(), FLb[0, 0:1], 50
    sp24.sp24_flip_count(fl_prev, F1["idx"], fl_ctr)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(fl_calls):
        sp24.sp24_flip_count(fl_prev, F1["idx"], fl_ctr)
    e1.record()
    torch.cuda.synchronize()
    fl_us = e0.elapsed_time(e1) * 1e3 / fl_calls
    fl_bytes = 2 * F1["idx"].numel()

    def timed_ms(fn, reps, warm=1):
        """Average ms per call over `reps` back-to-back calls between two events.
        `warm` untimed calls go first, so the GPU is busy while the timed calls
        are enqueued and host launch latency stays outside the events."""
        for _ in range(warm):
            fn()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    # next row: GEGLU forward and backward at the FFN width (HBM-bound)
    U, gd = geglu_inputs(torch, dev, cfg)
    g_out, g_dU = torch.empty_like(gd), torch.empty_like(U)
    geglu_ms = np.array([timed_ms(lambda: sp24.sp24_geglu_fwd(U, GEGLU_GROUP, out=g_out), 10),
                         timed_ms(lambda: sp24.sp24_geglu_bwd(U, gd, GEGLU_GROUP, dU=g_dU), 10)])
    units = T * f
    geglu_gbps = [6 * units / (geglu_ms[0] * 1e-3) / 1e9, 10 * units / (geglu_ms[1] * 1e-3) / 1e9]
    del U, gd, g_out, g_dU

    # GEGLU fused into the forward GEMM: W1 (6400 x 1600) read as a gated
    # layer with h = 3200 (rows in blocks of 16 values then 16 gates), against
    # the same GEMM followed by the GEGLU kernel
    Uf = torch.empty(T, f, dtype=torch.float16, device=dev)
    gf = torch.empty(T, f // 2, dtype=torch.float16, device=dev)
    fused_variants = {
        "gemm_then_geglu": lambda: (sp24.sp24_spmm_fwd(X, F1["vals_row"], F1["meta_row"], f, d, Y=Uf),
                                    sp24.sp24_geglu_fwd(Uf, 16, out=gf)),
        "fused_storing_U": lambda: sp24.sp24_spmm_fwd_geglu(X, F1["vals_row"], F1["meta_row"], f, d, out=gf, U=Uf),
        "fused_without_U": lambda: sp24.sp24_spmm_fwd_geglu(X, F1["vals_row"], F1["meta_row"], f, d, out=gf),
    }
    fused_us = {name: round(timed_ms(fn, 5) * 1e3, 1) for name, fn in fused_variants.items()}
    del Uf, gf

    # next row: MVUE 2:4 estimate of the output gradient dY1 [T, 4d] (HBM-bound)
    Um = mvue_uniforms(torch, dev, cfg)
    mv_out = sp24.sp24_mvue(dY1, Um)
    mvue_ms = timed_ms(lambda: sp24.sp24_mvue(dY1, Um, out=mv_out), 10)
    mvue_gbps = 4.125 * T * f / (mvue_ms * 1e-3) / 1e9
    del Um, mv_out

    # next row: the weight gradients of both linears with the masked decay
    # term (dense fp16 MFMA, fp32 out), timed back to back after the step.
    # After the memory-bound kernels above, the first 20 ms or so of these
    # launches run slower (a dW launch fell from about 410 to 345 us over
    # them), so 40 untimed calls (about 15 ms) of both go first
    dW1 = torch.empty(f, d, dtype=torch.float32, device=dev)
    dW2 = torch.empty(d, f, dtype=torch.float32, device=dev)
    wg_calls = [lambda: sp24.sp24_weight_grad(dY1, X, W1s[-1], F1["idx"], DECAY, dW=dW1),
                lambda: sp24.sp24_weight_grad(dY2, H, W2s[-1], F2["idx"], DECAY, dW=dW2)]
    for _ in range(20):
        for fn in wg_calls:
            fn()
    wg_ms = np.array([timed_ms(fn, 20) for fn in wg_calls])
    wg_flops = 2 * T * f * d
    wg_tflops = [wg_flops / (ms * 1e-3) / 1e12 for ms in wg_ms]
    wg_achieved = wg_flops / (float(np.mean(wg_ms)) * 1e-3) / 1e12
    del dW1, dW2

    # a whole training step of one gated FFN layer through the entry points
    # (structured_sparse_transformer_amd/ffn.py): W1 (6400 x 1600) read as a
    # gated layer with h = 3200 and W2 its 1600 x 3200 partner; refresh (both
    # searches), forward (GEGLU fused into the first GEMM), backward (two
    # input-gradient GEMMs, two weight gradients, the GEGLU backward)
    h = f // 2
    layer_obj = None
    if not args.no_layer_step:
        from structured_sparse_transformer_amd.ffn import SparseGegluFFN
        layer = SparseGegluFFN(W1s[-1], W2s[-1][:, :h].contiguous(), DECAY)
        layer.refresh()
        fwd_out = {}

        def layer_fwd():
            fwd_out["y"], fwd_out["saved"] = layer.forward(X)

        layer_fwd()
        layer_parts = {
            "refresh": layer.refresh,
            "forward": layer_fwd,
            "backward": lambda: layer.backward(dY2, fwd_out["saved"]),
        }
        layer_us = {name: round(timed_ms(fn, 5) * 1e3, 1) for name, fn in layer_parts.items()}
        layer_ms = timed_ms(lambda: (layer.refresh(), layer_fwd(), layer.backward(dY2, fwd_out["saved"])), 5)
        # dense-equivalent flops: forward and input-gradient GEMMs (2:4) plus
        # the dense weight gradients, each 2*T*N*K
        layer_flops = 3 * (2 * T * f * d + 2 * T * d * h)
        del layer, fwd_out
        layer_obj = {"definition": "one training step of a gated 2:4 FFN layer (SparseGegluFFN): refresh both "
                                   "weights' masks and forms, forward with GEGLU fused into the first GEMM, "
                                   "backward with both input gradients, both weight gradients (masked decay) "
                                   "and the GEGLU backward",
                     "shape": {"tokens": T, "d": d, "h": h, "W1": [f, d], "W2": [d, h]},
                     "ms": round(layer_ms, 4), "us_parts": layer_us,
                     "TFLOPs_dense_equiv": round(layer_flops / (layer_ms * 1e-3) / 1e12, 1),
                     "note": "dense-equivalent flops 2*T*N*K of the two forward GEMMs, the two input-gradient "
                             "GEMMs and the two weight gradients, over the whole step's time"}
    # the other GPT-2 FFN shapes of the same path (355M, 774M): one
    # search+compress launch for both weights (no flip count), back to back
    # over distinct weight pairs and output sets totalling more than
    # ROTATE_BYTES of inputs, so the caches cannot serve them; and each of the
    # four sparse GEMMs, warm.  Device-generated N(0, 0.02) weights and N(0, 1)
    # activations.
    def rotating_us(run, sets):
        """Median over TRIALS of the average µs per call of run(set) over all
        sets back to back between one pair of events."""
        run(sets[0])
        out = []
        for _ in range(TRIALS):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for st in sets:
                run(st)
            t1.record()
            torch.cuda.synchronize()
            out.append(t0.elapsed_time(t1) * 1e3 / len(sets))
        return float(np.median(out)), out

    other = {}
    for oc in () if args.no_other_configs else (WL.GPT2_355M, WL.GPT2_774M):
        og = torch.Generator(device=dev)
        og.manual_seed(oc.seed)
        od, of, oT = oc.d, oc.dff, oc.tokens
        rnd = lambda *shape, sd=1.0: (torch.randn(*shape, generator=og, device=dev) * sd).half()  # noqa: E731
        n_rot = -(-ROTATE_BYTES // (2 * 2 * of * od)) + 8
        pairs = [(rnd(of, od, sd=0.02), rnd(od, of, sd=0.02)) for _ in range(n_rot)]
        pair_forms = [sp24.sp24_search_compress_batch(list(wp)) for wp in pairs]
        sc_us, sc_trials = rotating_us(lambda k: sp24.sp24_search_compress_batch(list(pairs[k]), outs=pair_forms[k]),
                                       list(range(n_rot)))
        Wa, Wb = pairs[0]
        fa, fb = pair_forms[0]
        del pairs, pair_forms
        Xa, Ha, dYa, dYb = rnd(oT, od), rnd(oT, of), rnd(oT, of), rnd(oT, od)
        Ya, dXa = torch.empty(oT, of, dtype=torch.float16, device=dev), torch.empty(oT, od, dtype=torch.float16, device=dev)
        Yb, dXb = torch.empty(oT, od, dtype=torch.float16, device=dev), torch.empty(oT, of, dtype=torch.float16, device=dev)
        calls = {
            "fwd1": lambda: sp24.sp24_spmm_fwd(Xa, fa["vals_row"], fa["meta_row"], of, od, Y=Ya),
            "bwd1": lambda: sp24.sp24_spmm_bwd_input(dYa, fa["vals_col"], fa["meta_col"], of, od, dX=dXa),
            "fwd2": lambda: sp24.sp24_spmm_fwd(Ha, fb["vals_row"], fb["meta_row"], od, of, Y=Yb),
            "bwd2": lambda: sp24.sp24_spmm_bwd_input(dYb, fb["vals_col"], fb["meta_col"], od, of, dX=dXb),
        }
        g_ms = {name: float(np.median([timed_ms(fn, 5) for _ in range(TRIALS)])) for name, fn in calls.items()}
        g_flops = {name: 2 * t * n * k for name, t, n, k in oc.gemm_shapes()}
        executed = sum(g_flops.values()) / 2 / (sum(g_ms.values()) * 1e-3) / 1e12
        sc_gbps_o = 4.3125 * 2 * of * od / (sc_us * 1e-6) / 1e9
        other[oc.name] = {
            "d": od, "d_ff": of, "tokens": oT,
            "search_compress_us_both_weights": round(sc_us, 1),
            "search_compress_GBps": round(sc_gbps_o, 1),
            "search_compress_frac_hbm": round(sc_gbps_o / HBM_PEAK_GBPS, 4),
            "search_compress_trials_us": [round(x, 1) for x in sc_trials],
            "search_compress_rotation": f"{n_rot} distinct weight pairs and output sets, "
                                        f"{n_rot * 4 * of * od / 1e6:.0f} MB of weights",
            "gemm_us": {k: round(v * 1e3, 1) for k, v in g_ms.items()},
            "gemm_TFLOPs_dense_equiv": {k: round(g_flops[k] / (g_ms[k] * 1e-3) / 1e12, 1) for k in g_ms},
            "gemm_frac_of_dense_mfma_peak": round(executed / FP16_MFMA_PEAK_TFLOPS, 4),
        }
        del Wa, Wb, Xa, Ha, dYa, dYb, fa, fb, Ya, dXa, Yb, dXb, calls
    if not args.no_other_configs:
        # the 4096 x 4096 stress weight (integer rows, a constant band across
        # the seam, N(0, 0.02) rows): search and compression only, over
        # distinct copies and output sets
        Wst0 = torch.from_numpy(WL.stress_weight(WL.STRESS_SEED)).to(dev)
        n_rot = -(-ROTATE_BYTES // (2 * Wst0.numel())) + 8
        Wst = [Wst0.clone() for _ in range(n_rot)]
        Fst = [sp24.sp24_search_compress_batch([w]) for w in Wst]
        st_us, st_trials = rotating_us(lambda k: sp24.sp24_search_compress_batch([Wst[k]], outs=Fst[k]),
                                       list(range(n_rot)))
        st_gbps = 4.3125 * Wst0.numel() / (st_us * 1e-6) / 1e9
        other["stress-4096"] = {"shape": list(Wst0.shape), "search_compress_us": round(st_us, 1),
                                "search_compress_GBps": round(st_gbps, 1),
                                "search_compress_frac_hbm": round(st_gbps / HBM_PEAK_GBPS, 4),
                                "search_compress_trials_us": [round(x, 1) for x in st_trials],
                                "search_compress_rotation": f"{n_rot} distinct copies and output sets, "
                                                            f"{n_rot * 2 * Wst0.numel() / 1e6:.0f} MB of weights"}
        del Wst0, Wst, Fst
    flops_step = cfg.dense_equiv_flops()
    value = flops_step / (ms_per_step * 1e-3) / 1e12

    context = None
    if not args.no_context:
        context = {}
        # dense fp16 library GEMMs (hipBLASLt through torch) of the four shapes
        # of the step, on the dense weights: the MI355X sparse/dense ratio
        Wd1, Wd2 = W1s[0], W2s[0]
        dense = {"fwd1": lambda: torch.matmul(X, Wd1.t()), "bwd1": lambda: torch.matmul(dY1, Wd1),
                 "fwd2": lambda: torch.matmul(H, Wd2.t()), "bwd2": lambda: torch.matmul(dY2, Wd2)}
        dense_ms = {k: float(np.median([timed_ms(fn, 10) for _ in range(TRIALS)])) for k, fn in dense.items()}
        context["dense_torch_matmul_fp16_TFLOPs"] = {
            n: round(2 * Tt * N * K / (dense_ms[n] * 1e-3) / 1e12, 1) for n, Tt, N, K in gemm_shapes}
        context["dense_torch_matmul_us"] = {k: round(v * 1e3, 1) for k, v in dense_ms.items()}
        context["sparse_over_dense_speedup"] = {n: round(dense_ms[n] / gemm_ms[i], 3)
                                                for i, (n, *_) in enumerate(gemm_shapes)}
        # the library's dense weight-gradient product, dY1^T X, fp16 out
        dYt = dY1.t()
        ms = float(np.median([timed_ms(lambda: torch.matmul(dYt, X), 10) for _ in range(TRIALS)]))
        context["dense_torch_matmul_dYT_X_fp16_TFLOPs"] = round(2 * T * f * d / (ms * 1e-3) / 1e12, 1)
        # a 512 MiB device copy: the achievable HBM rate at a large size
        src = torch.empty(512 * 1024 * 1024 // 2, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        ms = float(np.median([timed_ms(lambda: dst.copy_(src), 5) for _ in range(TRIALS)]))
        context["copy_512MiB_GBps"] = round(2 * src.numel() * 2 / (ms * 1e-3) / 1e9, 1)
        del src, dst
        # the streaming floor at search+compress's own size: device copies that
        # move the same bytes as one launch (one weight: 20.5 MB read + 23.7 MB
        # written; both weights: twice that), each copy half reads and half
        # writes, rotating over distinct buffer sets beyond the caches
        floor = {}
        for name, nbytes in (("one_weight", SC_BYTES_PER_ELEM * d * f), ("both_weights", sc_bytes)):
            half = int(nbytes / 2) // 256 * 256
            n_rot = -(-ROTATE_BYTES // half) + 8
            bufs = [(torch.empty(half // 2, dtype=torch.float16, device=dev),
                     torch.empty(half // 2, dtype=torch.float16, device=dev)) for _ in range(n_rot)]
            us, tr = rotating_us(lambda k: bufs[k][1].copy_(bufs[k][0]), list(range(n_rot)))
            gbps = 2 * half / (us * 1e-6) / 1e9
            floor[name] = {"bytes": 2 * half, "us": round(us, 2), "GBps": round(gbps, 1),
                           "frac_hbm": round(gbps / HBM_PEAK_GBPS, 4), "rotation": n_rot}
            del bufs
        context["streaming_floor_same_traffic"] = floor

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline ...")
        cpu = cpu_baseline(cfg, inp, args.cpu_sample_tokens)

    line = {
        "metric": "mask-search+compress GB/s; 2:4 FFN GEMM TFLOP/s (dense-equiv), GPT-2 shapes",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_trials": {"median": round(float(np.median(trial_ms)), 4),
                               "mean": round(float(np.mean(trial_ms)), 4),
                               "all": [round(x, 4) for x in trial_ms],
                               "note": f"{TRIALS} more timings of the same --steps steps after the one above"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": "gpt2-1.5b-ffn noisy 20-step loop: search+compress W1,W2 (flip counts fused) then "
                               "4 sparse GEMMs per step",
                   "d": d, "d_ff": f, "tokens": T, "weights": [[f, d], [d, f]], "seed": cfg.seed},
        "value_definition": "dense-equivalent GEMM flops per step (sum of 2*T*N*K) / step wall time incl. search+compress",
        "search_compress_GBps": round(sc_gbps, 1),
        "search_compress_frac_hbm": round(sc_gbps / HBM_PEAK_GBPS, 4),
        "search_compress_us_both_weights": round(sc_ms * 1e3, 2),
        "search_compress_per_weight": {"W1_us": round(pw_us[0], 2), "W2_us": round(pw_us[1], 2),
                                       "W1_GBps": round(pw_gbps[0], 1), "W2_GBps": round(pw_gbps[1], 1),
                                       "note": "one launch per weight over all weight versions of the run "
                                               "(distinct buffers, 4.375 B per element with the flip count)"},
        "search_compress_back_to_back": {"us_both_weights": round(bb_us, 2), "GBps": round(bb_gbps, 1),
                                         "frac_hbm": round(bb_gbps / HBM_PEAK_GBPS, 4),
                                         "note": "the step's batched launch for both weights over all weight "
                                                 "versions of the run, back to back between one pair of events; "
                                                 "search_compress_GBps above times each launch inside the step, "
                                                 "between the step's own events"},
        "search_compress_roofline": {
            "kernel": "search_compress_kernel (one sp24_search_compress_batch launch for W1 and W2, flips counted)",
            "bound": "hbm", "achieved": round(bb_gbps, 1), "launch_us": round(bb_us, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(bb_gbps / HBM_PEAK_GBPS, 4), "traffic": sc_traffic,
            "trials_us": [round(x, 2) for x in bb_trials],
            "note": "4.375 algorithmic bytes per weight element over the median back-to-back launch time; traffic is "
                    "FETCH_SIZE + WRITE_SIZE per launch from the committed counter summary (null when stale)"},
        "flip_rate": {"definition": "mask entries changed since the previous step's search / entries",
                      "w1_mean": float(f"{flips[:, 0].mean():.4g}"), "w2_mean": float(f"{flips[:, 1].mean():.4g}"),
                      "w1_first_last": [float(f"{flips[0, 0]:.4g}"), float(f"{flips[-1, 0]:.4g}")],
                      "w2_first_last": [float(f"{flips[0, 1]:.4g}"), float(f"{flips[-1, 1]:.4g}")],
                      "standalone_sp24_flip_count_us": round(fl_us, 2),
                      "standalone_GBps": round(fl_bytes / (fl_us * 1e-6) / 1e9, 1)},
        "gemm_TFLOPs_dense_equiv": {n: round(v, 1) for (n, *_), v in zip(gemm_shapes, gemm_dense_tflops)},
        "gemm_us": {n: round(ms * 1e3, 1) for (n, *_), ms in zip(gemm_shapes, gemm_ms)},
        "gemm_us_mean": {n: round(ms * 1e3, 1) for (n, *_), ms in zip(gemm_shapes, gemm_ms_mean)},
        "gemm_breakdown_note": f"gemm_us (median) and gemm_us_mean over {TRIALS} more passes of the same steps with "
                               "the four GEMMs as single launches and events between every call; "
                               "gemm_TFLOPs_dense_equiv from the medians; roofline and search_compress from events in "
                               "the timed region (after each search and after each step's grouped GEMM launch)",
        "roofline": {"kernel": "spmm_group_kernel (one sp24_spmm_group launch: the step's four sparse GEMMs)",
                     "bound": "mfma", "achieved": round(achieved, 1), "launch_us": round(group_ms * 1e3, 1),
                     "single_launches": {"achieved": round(single_achieved, 1),
                                         "frac": round(single_achieved / FP16_MFMA_PEAK_TFLOPS, 4),
                                         "note": "the same four GEMMs as sp24_spmm_fwd / sp24_spmm_bwd_input calls "
                                                 "(gemm_us)"},
                     "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "note": "executed non-zero flops T*N*K of the four GEMMs per launch (half the dense-equivalent "
                             "2*T*N*K) over the dense fp16 MFMA peak; equal to dense-equivalent flops over the 2:4 "
                             "sparse peak"},
        "weight_grad": {"definition": "dW = dY^T X + decay * (1 - M) * W, fp16 in, fp32 out (sp24_weight_grad)",
                        "decay": DECAY, "us": {"dW1": round(wg_ms[0] * 1e3, 1), "dW2": round(wg_ms[1] * 1e3, 1)},
                        "TFLOPs": {"dW1": round(wg_tflops[0], 1), "dW2": round(wg_tflops[1], 1)},
                        "roofline": {"bound": "mfma", "achieved": round(wg_achieved, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(wg_achieved / FP16_MFMA_PEAK_TFLOPS, 4),
                                     "note": "2*T*R*C flops per launch (dense product) over the dense fp16 MFMA peak"}},
        "geglu": {"definition": "out = value * GELU(gate) (exact erf GELU), and its backward; U [T, 2h] in blocks "
                             "of 16 values then 16 gates (sp24_geglu_fwd / _bwd)",
                  "shape": {"tokens": T, "h": f, "group": GEGLU_GROUP},
                  "us": {"fwd": round(geglu_ms[0] * 1e3, 1), "bwd": round(geglu_ms[1] * 1e3, 1)},
                  "fused_forward_gemm_us": fused_us,
                  "fused_note": "W1 (6400 x 1600) as a gated layer, h = 3200, 16384 tokens: sp24_spmm_fwd_geglu "
                                "against sp24_spmm_fwd + sp24_geglu_fwd",
                  "GBps": {"fwd": round(geglu_gbps[0], 1), "bwd": round(geglu_gbps[1], 1)},
                  "roofline": {"bound": "hbm", "achieved": round(geglu_gbps[1], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                               "frac": round(geglu_gbps[1] / HBM_PEAK_GBPS, 4),
                               "note": "backward kernel: 10 B per hidden unit and token (read value, gate, dOut; "
                                       "write both gradients); forward moves 6 B"}},
        "ffn_layer_step": layer_obj,
        "other_configs": None if args.no_other_configs else {
            "definition": "the same path at the other GPT-2 FFN shapes, timed warm outside the step: one "
                          "search+compress launch for both weights (4.3125 B per element, no flip count) and each "
                          "sparse GEMM; executed flops over the dense fp16 MFMA peak; and search+compress alone "
                          "on the 4096 x 4096 stress weight",
            **other},
        "mvue": {"definition": "MVUE 2:4 estimate of dY1 [T, 4d] with one caller-supplied uniform per group, "
                            "row-form output (sp24_mvue)",
                 "us": round(mvue_ms * 1e3, 1), "GBps": round(mvue_gbps, 1),
                 "roofline": {"bound": "hbm", "achieved": round(mvue_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(mvue_gbps / HBM_PEAK_GBPS, 4),
                              "note": "4.125 B per entry: read 2 (gradient) + 1 (uniforms), write 1.125 (2:4 row form)"}},
        "cpu_baseline": cpu,
        "context": context,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
