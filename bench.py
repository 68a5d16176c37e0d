"""Benchmark of the FP8 training hot path on one MI355X.

One step is one pass of every stage of the path over one batch of synthetic
input, in the shapes of the MLP up-projection of a 768-wide GPT at 64 x 1024
tokens plus a fine-grained block-scaled projection:

  forward   quantize X [65536,768] -> E4M3 (per-tensor amax scale, + X^T copy)
            y  = X W^T            [65536,3072]   (W from the FP8 weight cache)
  backward  quantize dY [65536,3072] -> E5M2 (per-tensor, + dY^T copy)
            dX = dY W             [65536,768]    (E5M2 x E4M3, W^T cache copy)
            dW = dY^T X           [3072,768]     (K = 65536, split K)
  update    the weight-cache refresh after the optimizer step (amax + cast +
            transposed copy of W [3072,768]); the step alternates between the
            master before and after one update W <- bf16(W + N(0,1e-4)),
            both prepared beforehand, so every refresh sees a changed master
  fine      quantize A [16384,7168] in 1x128 row tiles, B [2048,7168] in
            128x128 blocks, block-scaled GEMM [16384,2048]

value = all GEMM flops of the step / step time (TFLOP/s, inputs resident in
HBM).  Outside the timed region, the other workloads are measured too: the
256x3072x768 up-projection (one call and a loop of 1000 calls), the 8192 x
8192 quantize-only pass (amax, per-tensor and 1x128 quantize in E4M3 and
E5M2, the 256 MB last-level cache flushed before every rep), and the batched
refresh of a 12-layer model's up-projection caches.  A breakdown pass before the timed region brackets every stage with
HIP events (each stage's average duration); the timed region records events
only around the dominant kernel, whose average launch duration gives the
roofline entry.  The CPU oracle is timed on a bounded sample of the same
work (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-GEMM TFLOP/s (% of FP8 MFMA peak) + quantize GB/s (% HBM)"
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

TOK, D, F = 65536, 768, 3072   # tokens, d_model, 4 d_model
LD_PAD = 256                   # bytes of padding per row of the transposed FP8 copies
FA_M, FA_N, FA_K = 16384, 2048, 7168
COPY_BYTES = 1 << 30           # calibration copy


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-rows", type=int, default=65536)
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path has no multi-GPU form (one GPU's share is the "
              "whole workload). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_scaled_matmul_amd as fm
    import synth

    torch.cuda.set_device(0)
    dev = "cuda"

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    t_gen = time.time()
    x = to_dev(synth.normal_bf16(3, 0, (TOK, D), 1.0))
    w_bits = synth.normal_bf16(3, 1, (F, D), 0.02)
    # the master before and after one optimizer update (the step refreshes
    # the cache from each in turn)
    w_masters = [to_dev(w_bits), to_dev(synth.apply_update_bf16(w_bits, synth.update_noise_f32(3, (F, D))))]
    w_master = w_masters[0]
    dy = to_dev(synth.normal_bf16(5, 0, (TOK, F), 1e-3))
    a_fine = to_dev(synth.channel_scaled_bf16(4, 0, 3, (FA_M, FA_K)))
    b_fine = to_dev(synth.channel_scaled_bf16(4, 1, 4, (FA_N, FA_K)))
    gen_s = time.time() - t_gen

    # outputs and caches, allocated once
    # The transposed FP8 copies (the dW operands) have 65536-byte rows; their
    # leading dimension is padded by 256 bytes so that the rows of a tile do
    # not all fall on the same HBM channel (measured: dW 216 -> 165 us).
    xq = torch.empty((TOK, D), dtype=torch.uint8, device=dev)
    xqt = torch.empty((D, TOK + LD_PAD), dtype=torch.uint8, device=dev)[:, :TOK]
    xs = torch.empty(1, dtype=torch.float32, device=dev)
    dyq = torch.empty((TOK, F), dtype=torch.uint8, device=dev)
    dyqt = torch.empty((F, TOK + LD_PAD), dtype=torch.uint8, device=dev)[:, :TOK]
    dys = torch.empty(1, dtype=torch.float32, device=dev)
    y = torch.empty((TOK, F), dtype=torch.bfloat16, device=dev)
    dx = torch.empty((TOK, D), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((F, D), dtype=torch.bfloat16, device=dev)
    aq = torch.empty((FA_M, FA_K), dtype=torch.uint8, device=dev)
    sa = torch.empty((FA_M, FA_K // 128), dtype=torch.float32, device=dev)
    bq = torch.empty((FA_N, FA_K), dtype=torch.uint8, device=dev)
    sb = torch.empty((FA_N // 128, FA_K // 128), dtype=torch.float32, device=dev)
    yf = torch.empty((FA_M, FA_N), dtype=torch.bfloat16, device=dev)
    ctr = fm.Counters(dev)
    cache = fm.WeightCache(F, D, fm.E4M3, fm.TENSOR, with_t=True, counters=ctr, device=dev)
    fm.requant_weights([cache], [w_master])
    dw_ws = torch.empty(max(fm.lib().fp8_scaled_mm_workspace_size(F, D, TOK, 0, 0), 1),
                        dtype=torch.uint8, device=dev)
    # a plain copy of known size (1 GiB read, 1 GiB written) outside the timed
    # region: the HBM byte counters of the dominant kernel are scaled by what
    # the same counters read for it, and its rate is this board's copy speed
    csrc = torch.zeros(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    cdst = torch.empty_like(csrc)
    torch.neg(csrc, out=cdst)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        torch.neg(csrc, out=cdst)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * COPY_BYTES * 5 / (c0.elapsed_time(c1) / 1e3) / 1e9
    del csrc, cdst
    torch.cuda.synchronize()

    refresh_state = [0]
    # one prepared refresh per master (the caches and masters stay put)
    refresh_plans = [fm.RequantPlan([cache], [wm]) for wm in w_masters]

    def refresh(c):
        refresh_plans[refresh_state[0] & 1]()
        refresh_state[0] += 1

    # (name, flops, algorithmic HBM bytes, callable)
    stages = [
        ("quantize_x_e4m3_tensor_t", 0, TOK * D * (2 + 2 + 1 + 1),
         lambda: fm.quantize(x, fm.E4M3, fm.TENSOR, want_t=True, counters=ctr, scale=xs, out=xq, out_t=xqt)),
        ("gemm_fwd_65536x3072x768", 2 * TOK * F * D, TOK * D + F * D + TOK * F * 2,
         lambda: fm.scaled_mm(xq, fm.E4M3, xs, fm.TENSOR, cache.q, fm.E4M3, cache.scale, fm.TENSOR,
                              out=y, counters=ctr)),
        ("quantize_dy_e5m2_tensor_t", 0, TOK * F * (2 + 2 + 1 + 1),
         lambda: fm.quantize(dy, fm.E5M2, fm.TENSOR, want_t=True, counters=ctr, scale=dys, out=dyq, out_t=dyqt)),
        ("gemm_dx_65536x768x3072", 2 * TOK * D * F, TOK * F + D * F + TOK * D * 2,
         lambda: fm.scaled_mm(dyq, fm.E5M2, dys, fm.TENSOR, cache.q_t, fm.E4M3, cache.scale, fm.TENSOR,
                              out=dx, counters=ctr)),
        ("gemm_dw_3072x768x65536", 2 * F * D * TOK, F * TOK + D * TOK + F * D * 2,
         lambda: fm.scaled_mm(dyqt, fm.E5M2, dys, fm.TENSOR, xqt, fm.E4M3, xs, fm.TENSOR,
                              out=dw, counters=ctr, workspace=dw_ws)),
        ("requant_w_cache", 0, F * D * (2 + 2 + 1 + 1),
         lambda: refresh(cache)),
        ("quantize_a_1x128", 0, FA_M * FA_K * 3 + FA_M * (FA_K // 128) * 4,
         lambda: fm.quantize(a_fine, fm.E4M3, fm.ROW_1x128, scale=sa, out=aq, counters=ctr)),
        ("quantize_b_128x128", 0, FA_N * FA_K * 3 + (FA_N // 128) * (FA_K // 128) * 4,
         lambda: fm.quantize(b_fine, fm.E4M3, fm.BLOCK_128x128, scale=sb, out=bq, counters=ctr)),
        ("gemm_block_16384x2048x7168", 2 * FA_M * FA_N * FA_K, FA_M * FA_K + FA_N * FA_K + FA_M * FA_N * 2
         + FA_M * (FA_K // 128) * 4,
         lambda: fm.scaled_mm(aq, fm.E4M3, sa, fm.ROW_1x128, bq, fm.E4M3, sb, fm.BLOCK_128x128,
                              out=yf, counters=ctr)),
    ]
    step_flops = sum(s[1] for s in stages)
    # Measured in the breakdown pass only, not part of the step: the same dY
    # quantization with delayed scaling (scale from a 16-step amax history,
    # one read of dY instead of two).
    dy_hist = fm.AmaxHistory(16, device=dev)
    dy_ws = torch.empty(fm.lib().fp8_quantize_delayed_workspace_size(TOK, F), dtype=torch.uint8, device=dev)
    # The fine-grained leg with power-of-two scales, which the MFMA applies
    # itself (E8M0): the same A and B, quantized with the power-of-two rule.
    aq2 = torch.empty_like(aq)
    sa2 = torch.empty_like(sa)
    bq2 = torch.empty_like(bq)
    sb2 = torch.empty_like(sb)
    # The forward with X quantized inside the GEMM's operand load: one amax
    # pass over X, then the A-stationary GEMM casting each block of X rows into
    # LDS and writing X^T's codes (the dW operand) on the way.  Compared with
    # the two stages quantize_x + gemm_fwd above (same outputs: y, X^T codes,
    # scale).  Algorithmic bytes: X read twice (4 B/elt), X^T written (1), W,
    # y written.
    fused_ws = torch.empty(fm.lib().fp8_quantize_scaled_mm_workspace_size(TOK, F, D), dtype=torch.uint8, device=dev)
    xs_f = torch.empty(1, dtype=torch.float32, device=dev)
    extra = [
        ("quantize_gemm_fwd_fused_65536x3072x768", 2 * TOK * F * D, TOK * D * (2 + 2 + 1) + F * D + TOK * F * 2,
         lambda: fm.quantize_scaled_mm(x, fm.E4M3, cache.q, fm.E4M3, cache.scale, out=y, counters=ctr, scale_a=xs_f,
                                       out_t=xqt, workspace=fused_ws)),
        ("quantize_dy_e5m2_delayed_t", 0, TOK * F * (2 + 1 + 1),
         lambda: fm.quantize_delayed(dy, fm.E5M2, dy_hist, scale=dys, want_t=True, counters=ctr, out=dyq,
                                     out_t=dyqt, workspace=dy_ws)),
        ("quantize_a_1x128_pow2", 0, FA_M * FA_K * 3 + FA_M * (FA_K // 128) * 4,
         lambda: fm.quantize(a_fine, fm.E4M3, fm.ROW_1x128, fm.FROM_AMAX_POW2, scale=sa2, out=aq2, counters=ctr)),
        ("quantize_b_128x128_pow2", 0, FA_N * FA_K * 3 + (FA_N // 128) * (FA_K // 128) * 4,
         lambda: fm.quantize(b_fine, fm.E4M3, fm.BLOCK_128x128, fm.FROM_AMAX_POW2, scale=sb2, out=bq2,
                             counters=ctr)),
        ("gemm_block_pow2_16384x2048x7168", 2 * FA_M * FA_N * FA_K, FA_M * FA_K + FA_N * FA_K + FA_M * FA_N * 2
         + FA_M * (FA_K // 128) * 4,
         lambda: fm.scaled_mm(aq2, fm.E4M3, sa2, fm.ROW_1x128_POW2, bq2, fm.E4M3, sb2, fm.BLOCK_128x128_POW2,
                              out=yf, counters=ctr)),
    ]

    def step(dom_events=None, dom=None):
        for name, _, _, fn in stages:
            timed = dom_events is not None and name == dom
            if timed:
                dom_events[0].record()
            fn()
            if timed:
                dom_events[1].record()

    def new_events():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    for _ in range(args.warmup):
        step()
        for _, _, _, fn in extra:   # also fills the delayed-scaling history
            fn()
    torch.cuda.synchronize()

    # Stage breakdown, outside the timed region: every stage bracketed by
    # events (an event record between two kernels costs the stream a gap of
    # several microseconds, so the timed region below records only around
    # the dominant kernel).
    stage_ms = {name: 0.0 for name, _, _, _ in stages + extra}
    evs = [[new_events() for _ in stages + extra] for _ in range(args.steps)]
    for k in range(args.steps):
        for i, (name, _, _, fn) in enumerate(stages + extra):
            evs[k][i][0].record()
            fn()
            evs[k][i][1].record()
    torch.cuda.synchronize()
    for k in range(args.steps):
        for i, (name, _, _, _) in enumerate(stages + extra):
            stage_ms[name] += evs[k][i][0].elapsed_time(evs[k][i][1]) / args.steps
    kernels = {}
    for name, flops, nbytes, _ in stages + extra:
        ms = stage_ms[name]
        d = {"ms": round(ms, 4)}
        if flops:
            d["tflops"] = round(flops / ms / 1e9, 1)
            d["frac_fp8_peak"] = round(flops / ms / 1e9 / PEAK_FP8_TFLOPS, 4)
        d["gbs"] = round(nbytes / ms / 1e6, 1)
        d["frac_hbm"] = round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)
        if name in [e[0] for e in extra]:
            d["in_step"] = False
        kernels[name] = d
    # dominant kernel: the single-kernel GEMM stage with the largest share
    single_kernel_gemms = ["gemm_fwd_65536x3072x768", "gemm_dx_65536x768x3072", "gemm_block_16384x2048x7168"]
    dom = max(single_kernel_gemms, key=lambda n: stage_ms[n])

    # timed region: K whole steps; events only around the dominant kernel
    dom_ev = [new_events() for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        step(dom_ev[k], dom)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    dom_ms = sum(a.elapsed_time(b) for a, b in dom_ev) / args.steps

    dflops = [s[1] for s in stages if s[0] == dom][0]
    achieved = dflops / dom_ms / 1e9
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                "launch_ms": round(dom_ms, 4), "traffic": measured_traffic(dom)}

    counters = ctr.read()
    value = step_flops / (ms_per_step / 1e3) / 1e12
    bf16 = bf16_matched(torch, x, w_master, dy, stage_ms, args.steps)
    other = other_workloads(torch, fm, synth, np, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_sample_rows, stage_ms)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (e4m3/e5m2) x fp8 -> fp32 accumulate -> bf16",
        "data": "synthetic (seeded; bf16 N(0,1)/N(0,0.02)/N(0,1e-3), 1% channels x100 for the block-scaled GEMM)",
        "config": {
            "workload": "FP8 MLP up-projection training step, 64 seqs x 1024 tokens, d_model 768 -> 3072 "
                        "(forward, E5M2 backward dX/dW, weight-cache refresh) + block-scaled "
                        "16384x2048x7168 GEMM with 1x128 / 128x128 scales",
            "tokens": TOK, "d_model": D, "d_ff": F,
            "block_scaled_mnk": [FA_M, FA_N, FA_K],
            "step_gemm_gflop": round(step_flops / 1e9, 2),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "counters": counters,
        "hbm_copy_gbs": round(copy_gbs, 1),
        "bf16_matched": bf16,
        "workloads": other,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(out))


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def _rate(nbytes, ms):
    return {"ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1),
            "frac_hbm": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}


def other_workloads(torch, fm, synth, np, dev):
    """The workloads that are not part of the training step, each timed on its
    own with HIP events on the current stream (outside the timed region):

    - the 256x3072x768 up-projection (X [256,768] N(0,1), W [3072,768]
      N(0,0.02), E4M3 per-tensor): median of 50 single calls of each stage,
      and the average over a loop of 1000 calls (quantize X, quantize W,
      GEMM), eager and replayed from captured HIP graphs -- a latency-bound
      shape (12 output tiles for 256 CUs);
    - the quantize-only pass over bf16 [8192,8192] N(0,1) with 0.1% outliers
      +-U(500,5000): amax (2 B/elt), per-tensor quantize from amax (two
      kernels: 3 B/elt useful, 5 B/elt moved), per-tensor cast with a given
      scale (3 B/elt), 1x128 tile quantize (3 + 4/128 B/elt), in E4M3 and
      E5M2; before every rep a 1 GiB buffer is read so that the input is not
      served from the 256 MB last-level cache; median of 15 reps;
    - the weight-cache refresh of a 12-layer model's up-projection weights
      (12 x [3072,768] bf16 -> E4M3 per-tensor with transposed copies; 6 B
      per element algorithmic), one batched call (a prepared RequantPlan,
      as a training loop holds it) against 12 single calls."""
    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def time_calls(fn, reps, flush=None):
        out = []
        for _ in range(reps):
            if flush is not None:
                flush()
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b))
        return out

    res = {}
    # ---- 256x3072x768 up-projection
    x1 = to_dev(synth.normal_bf16(1, 0, synth.SMALL_UP_PROJ["x"], 1.0))
    w1 = to_dev(synth.normal_bf16(1, 1, synth.SMALL_UP_PROJ["w"], 0.02))
    m, k = x1.shape
    n = w1.shape[0]
    xq1 = torch.empty((m, k), dtype=torch.uint8, device=dev)
    wq1 = torch.empty((n, k), dtype=torch.uint8, device=dev)
    xs1 = torch.empty(1, dtype=torch.float32, device=dev)
    ws1 = torch.empty(1, dtype=torch.float32, device=dev)
    y1 = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    # workspaces allocated once, as a training loop would hold them
    wsx1 = torch.empty(max(fm.lib().fp8_quantize_workspace_size(m, k, fm.TENSOR, fm.FROM_AMAX), 1),
                       dtype=torch.uint8, device=dev)
    wsw1 = torch.empty(max(fm.lib().fp8_quantize_workspace_size(n, k, fm.TENSOR, fm.FROM_AMAX), 1),
                       dtype=torch.uint8, device=dev)
    fq_x = lambda: fm.quantize(x1, fm.E4M3, scale=xs1, out=xq1, workspace=wsx1)
    fq_w = lambda: fm.quantize(w1, fm.E4M3, scale=ws1, out=wq1, workspace=wsw1)
    fg = lambda: fm.scaled_mm(xq1, fm.E4M3, xs1, fm.TENSOR, wq1, fm.E4M3, ws1, fm.TENSOR, out=y1)
    for _ in range(20):
        fq_x(), fq_w(), fg()
    torch.cuda.synchronize()
    flops1 = 2 * m * n * k
    single = {name: _median(time_calls(fn, 50)) for name, fn in
              (("quantize_x", fq_x), ("quantize_w", fq_w), ("gemm", fg))}
    a, b = ev(), ev()
    a.record()
    for _ in range(1000):
        fg()
    b.record()
    torch.cuda.synchronize()
    loop_gemm = a.elapsed_time(b) / 1000
    a, b = ev(), ev()
    a.record()
    for _ in range(1000):
        fq_x(), fq_w(), fg()
    b.record()
    torch.cuda.synchronize()
    loop_all = a.elapsed_time(b) / 1000
    # The same loops replayed from captured HIP graphs (100 iterations per
    # graph, 10 replays): the launch cost leaves the host.  The library
    # allocates nothing and never synchronizes, so a whole iteration
    # captures; the replayed outputs are checked against the eager ones.
    y_eager, xq_eager, wq_eager = y1.clone(), xq1.clone(), wq1.clone()

    def graph_loop(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(100):
                body()
        g.replay()
        torch.cuda.synchronize()
        a_, b_ = ev(), ev()
        a_.record()
        for _ in range(10):
            g.replay()
        b_.record()
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / 1000

    graph_gemm = graph_loop(fg)
    graph_all = graph_loop(lambda: (fq_x(), fq_w(), fg()))
    graph_ok = bool(torch.equal(y1, y_eager) and torch.equal(xq1, xq_eager) and torch.equal(wq1, wq_eager))
    res["up_projection_256x3072x768"] = {
        "single_call_us": {k_: round(v * 1e3, 2) for k_, v in single.items()},
        "gemm_tflops_single": round(flops1 / single["gemm"] / 1e9, 1),
        "loop_1000_gemm_us": round(loop_gemm * 1e3, 2),
        "loop_1000_gemm_tflops": round(flops1 / loop_gemm / 1e9, 1),
        "loop_1000_quantize_x_w_gemm_us": round(loop_all * 1e3, 2),
        "graph_loop_1000_gemm_us": round(graph_gemm * 1e3, 2),
        "graph_loop_1000_quantize_x_w_gemm_us": round(graph_all * 1e3, 2),
        "graph_replay_matches_eager": graph_ok,
    }
    del x1, w1, xq1, wq1, y1

    # ---- 8192 x 8192 quantize-only
    shp = synth.QUANT_ONLY["x"]
    xq_in = to_dev(synth.with_outliers_bf16(2, shp))
    nel = shp[0] * shp[1]
    q8 = torch.empty(shp, dtype=torch.uint8, device=dev)
    s_t = torch.empty(1, dtype=torch.float32, device=dev)
    s_r = torch.empty((shp[0], shp[1] // 128), dtype=torch.float32, device=dev)
    amax_out = torch.empty(1, dtype=torch.float32, device=dev)
    ws_a = torch.empty(fm.lib().fp8_amax_workspace_size(shp[0], shp[1], fm.TENSOR), dtype=torch.uint8, device=dev)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        # read 1 GiB (no dirty lines left behind to be written back while the
        # timed kernel runs)
        flush_buf.sum()

    cases = [("amax", 2 * nel, None, lambda: fm.check(fm.fp8_amax(
        xq_in.data_ptr(), fm.BF16, shp[0], shp[1], shp[1], fm.TENSOR, amax_out.data_ptr(), ws_a.data_ptr(),
        ws_a.numel(), torch.cuda.current_stream().cuda_stream)))]
    for fmt, fname in ((fm.E4M3, "e4m3"), (fm.E5M2, "e5m2")):
        cases += [
            (f"quantize_tensor_{fname}", 3 * nel, 5 * nel,
             lambda fmt=fmt: fm.quantize(xq_in, fmt, fm.TENSOR, scale=s_t, out=q8)),
            (f"cast_given_scale_{fname}", 3 * nel, None,
             lambda fmt=fmt: fm.quantize(xq_in, fmt, fm.TENSOR, fm.GIVEN, scale=s_t, out=q8)),
            (f"quantize_1x128_{fname}", 3 * nel + 4 * nel // 128, None,
             lambda fmt=fmt: fm.quantize(xq_in, fmt, fm.ROW_1x128, scale=s_r, out=q8)),
        ]
    qo = {}
    for name, useful, moved, fn in cases:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ms = _median(time_calls(fn, 15, flush))
        d = _rate(useful, ms)
        if moved:
            d["gbs_moved"] = round(moved / ms / 1e6, 1)
            d["frac_hbm_moved"] = round(moved / ms / 1e6 / PEAK_HBM_GBS, 4)
        qo[name] = d
    res["quantize_only_8192x8192"] = qo
    del xq_in, q8, s_r, flush_buf

    # ---- 12-layer weight-cache refresh
    wl = [to_dev(synth.normal_bf16(70 + l, 1, (3072, 768), 0.02)) for l in range(12)]
    caches = [fm.WeightCache(3072, 768, with_t=True, device=dev) for _ in wl]
    plan = fm.RequantPlan(caches, wl)     # prepared once, as a training loop would
    batched = plan

    def singles():
        for c, w in zip(caches, wl):
            fm.requant_weights([c], [w])
    for _ in range(3):
        batched(), singles()
    torch.cuda.synchronize()
    nbytes = 12 * 3072 * 768 * 6
    res["requant_12_layers_3072x768"] = {
        "batched": _rate(nbytes, _median(time_calls(batched, 30))),
        "twelve_single_calls": _rate(nbytes, _median(time_calls(singles, 30))),
    }
    return res


# Sources each GEMM kernel is compiled from; a stored traffic figure is used
# only while their hash matches the one it was taken with.
KERNEL_SOURCES = {
    "gemm_block_16384x2048x7168": ["gemm.hip", "gemm_common.h", "device_common.h", "fp8mi_internal.h"],
    "gemm_fwd_65536x3072x768": ["gemm_astat.hip", "gemm_common.h", "device_common.h", "fp8mi_internal.h"],
    "gemm_dx_65536x768x3072": ["gemm.hip", "gemm_common.h", "device_common.h", "fp8mi_internal.h"],
}


def sources_hash(stage: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "fp8_scaled_matmul_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(stage: str):
    """HBM bytes per launch of the stage's kernel from the committed counter
    summary profiles/<stage>_traffic.md: FETCH_SIZE + WRITE_SIZE per dispatch
    (KiB), each scaled by the ratio of the calibration copy's known bytes to
    what the same counter read for it.  None when no summary exists or the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_traffic.md")
    if not os.path.exists(path) or stage not in KERNEL_SOURCES:
        return None
    rec = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
    if rec is None or rec.get("sources_sha256") != sources_hash(stage):
        return None
    fetch = rec["fetch_kib"] * 1024.0 * COPY_BYTES / (rec["copy_fetch_kib"] * 1024.0)
    write = rec["write_kib"] * 1024.0 * COPY_BYTES / (rec["copy_write_kib"] * 1024.0)
    return round(fetch + write)


def bf16_matched(torch, x, w, dy, stage_ms: dict, reps: int):
    """The per-tensor GEMMs of the step in bf16 on the same inputs, through
    torch's bf16 matmul (hipBLASLt on the MFMA units), timed after the timed
    region: the FP8 / bf16 speed ratio the pages put at about 2x ("#84 FP8
    Precision", section "Hardware precision").  Transposed operands are made
    contiguous beforehand."""
    wt = w.t().contiguous()          # [768, 3072]
    dyt = dy.t().contiguous()        # [3072, 65536]
    cases = [("gemm_fwd_65536x3072x768", lambda: torch.matmul(x, wt)),
             ("gemm_dx_65536x768x3072", lambda: torch.matmul(dy, w)),
             ("gemm_dw_3072x768x65536", lambda: torch.matmul(dyt, x))]
    out = {}
    for name, fn in cases:
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        out[name] = {"bf16_ms": round(ms, 4), "fp8_ms": round(stage_ms[name], 4),
                     "fp8_speedup": round(ms / stage_ms[name], 2)}
    del wt, dyt
    return out


def cpu_baseline(sample_rows: int, stage_ms: dict):
    """The oracle, as it stands, on a bounded sample of the same work: the
    per-tensor part of the step (oracle quantization of X, W and dY with their
    transposed copies, then its fp64 GEMMs forward, dX and dW) on the first
    `sample_rows` token rows (all 65536 by default).  Reported in the
    metric's unit (GEMM TFLOP/s)."""
    import numpy as np

    import oracle
    import synth

    rows = min(sample_rows, TOK)
    x = synth.normal_bf16(3, 0, (TOK, D), 1.0)[:rows]
    w = synth.normal_bf16(3, 1, (F, D), 0.02)
    dy = synth.normal_bf16(5, 0, (TOK, F), 1e-3)[:rows]
    t0 = time.time()
    xq, xqt, xs, _ = oracle.quantize(x, oracle.E4M3, want_t=True)
    wq, wqt, ws, _ = oracle.quantize(w, oracle.E4M3, want_t=True)
    dyq, dyqt, dys, _ = oracle.quantize(dy, oracle.E5M2, want_t=True)
    y = oracle.gemm(xq, oracle.E4M3, xs, oracle.TENSOR, wq, oracle.E4M3, ws, oracle.TENSOR)
    del y
    dx = oracle.gemm(dyq, oracle.E5M2, dys, oracle.TENSOR, wqt, oracle.E4M3, ws, oracle.TENSOR)
    del dx
    dw = oracle.gemm(dyqt, oracle.E5M2, dys, oracle.TENSOR, xqt, oracle.E4M3, xs, oracle.TENSOR)
    del dw
    dt = time.time() - t0
    flops = 3 * 2.0 * rows * F * D
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"per-tensor up-projection step on {rows} of {TOK} token rows: oracle quantization of X, W, "
                      f"dY (+ transposed copies), fp64 GEMMs fwd {rows}x{F}x{D}, dX {rows}x{D}x{F}, "
                      f"dW {F}x{D}x{rows}; {dt:.1f} s",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
