"""The library under HIP graph capture: a small training step (per-tensor
quantize with transposed copies, forward / dX / split-K dW GEMMs, weight-cache
refresh, 1x128 and 128x128 quantize, block-scaled and E8M0 GEMMs) captured
once with torch.cuda.CUDAGraph and replayed several times, with eager work
between the replays; every replay must reproduce the eager outputs bit for
bit (every kernel here is deterministic).  Nothing in the library allocates,
synchronizes or enqueues a memset, so the capture holds only its kernels."""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import synth
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    T, D, F = 2048, 256, 512
    M, N, K = 512, 256, 1024
    x = dev_bf16(synth.small_shape_bf16(60, (T, D)))
    w = dev_bf16(synth.small_shape_bf16(61, (F, D), 0.02))
    dy = dev_bf16(synth.small_shape_bf16(62, (T, F), 1e-3))
    a = dev_bf16(synth.channel_scaled_bf16(63, 0, 3, (M, K)))
    b = dev_bf16(synth.channel_scaled_bf16(63, 1, 4, (N, K)))
    dev = "cuda"
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    xq, xqt, xs = torch.empty((T, D), **u8), torch.empty((D, T), **u8), torch.empty(1, **f32)
    dq, dqt, ds = torch.empty((T, F), **u8), torch.empty((F, T), **u8), torch.empty(1, **f32)
    y, dx, dw = torch.empty((T, F), **bf), torch.empty((T, D), **bf), torch.empty((F, D), **bf)
    aq, sa = torch.empty((M, K), **u8), torch.empty((M, K // 128), **f32)
    bq, sb = torch.empty((N, K), **u8), torch.empty((N // 128, K // 128), **f32)
    a2, sa2 = torch.empty((M, K), **u8), torch.empty((M, K // 128), **f32)
    b2, sb2 = torch.empty((N, K), **u8), torch.empty((N // 128, K // 128), **f32)
    yb, y2 = torch.empty((M, N), **bf), torch.empty((M, N), **bf)
    cache = fm.WeightCache(F, D, fm.E4M3, fm.TENSOR, with_t=True, device=dev)
    ws = torch.empty(max(fm.lib().fp8_scaled_mm_workspace_size(F, D, T, 0, 0), 1), **u8)
    assert fm.lib().fp8_scaled_mm_workspace_size(F, D, T, 0, 0) > 0   # dW takes the split-K path

    def step():
        fm.requant_weights([cache], [w])
        fm.quantize(x, fm.E4M3, want_t=True, scale=xs, out=xq, out_t=xqt)
        fm.scaled_mm(xq, fm.E4M3, xs, fm.TENSOR, cache.q, fm.E4M3, cache.scale, fm.TENSOR, out=y)
        fm.quantize(dy, fm.E5M2, want_t=True, scale=ds, out=dq, out_t=dqt)
        fm.scaled_mm(dq, fm.E5M2, ds, fm.TENSOR, cache.q_t, fm.E4M3, cache.scale, fm.TENSOR, out=dx)
        fm.scaled_mm(dqt, fm.E5M2, ds, fm.TENSOR, xqt, fm.E4M3, xs, fm.TENSOR, out=dw, workspace=ws)
        fm.quantize(a, fm.E4M3, fm.ROW_1x128, scale=sa, out=aq)
        fm.quantize(b, fm.E4M3, fm.BLOCK_128x128, scale=sb, out=bq)
        fm.scaled_mm(aq, fm.E4M3, sa, fm.ROW_1x128, bq, fm.E4M3, sb, fm.BLOCK_128x128, out=yb)
        fm.quantize(a, fm.E4M3, fm.ROW_1x128, fm.FROM_AMAX_POW2, scale=sa2, out=a2)
        fm.quantize(b, fm.E4M3, fm.BLOCK_128x128, fm.FROM_AMAX_POW2, scale=sb2, out=b2)
        fm.scaled_mm(a2, fm.E4M3, sa2, fm.ROW_1x128_POW2, b2, fm.E4M3, sb2, fm.BLOCK_128x128_POW2, out=y2)

    outs = (xq, xqt, xs, dq, dqt, ds, y, dx, dw, aq, sa, bq, sb, yb, a2, sa2, b2, sb2, y2, cache.q, cache.q_t,
            cache.scale)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                              # warm the capture stream's allocations
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()                       # the replay must rewrite every output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bad = [i for i, (r, t) in enumerate(zip(ref, outs)) if not torch.equal(r, t)]
        assert not bad, f"replay {rep}: outputs {bad} differ from eager"
        step()                              # eager work between the replays
        torch.cuda.synchronize()
        assert all(torch.equal(r, t) for r, t in zip(ref, outs))
