"""fp8_quantize_noalloc, called through the C ABI, against fp8_quantize with
a caller's workspace on the same inputs: codes, transposed copy, scale and
counters identical.  Two calls in a row on one stream, the second on a
smaller tensor (the library-owned scratch keeps the first call's partials,
which the second must not see), for every per-tensor amax mode and a
granularity that needs no scratch."""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import synth
from gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def _run(x, fmt, gran, mode, want_t, noalloc):
    rows, cols = x.shape
    q = torch.full((rows, cols), 0x11, dtype=torch.uint8, device="cuda")
    qt = torch.full((cols, rows), 0x22, dtype=torch.uint8, device="cuda") if want_t else None
    scale = torch.full(fm.scale_shape(gran, rows, cols), -1.0, dtype=torch.float32, device="cuda")
    ctr = fm.Counters()
    stream = torch.cuda.current_stream().cuda_stream
    qt_ptr, ldqt = (qt.data_ptr(), qt.stride(0)) if qt is not None else (None, 0)
    dt = fm.BF16 if x.dtype == torch.bfloat16 else fm.FP32
    if noalloc:
        st = fm.fp8_quantize_noalloc(x.data_ptr(), dt, rows, cols, x.stride(0), fmt, gran, mode,
                                     scale.data_ptr(), q.data_ptr(), q.stride(0), qt_ptr, ldqt, ctr.ptr(), stream)
    else:
        wsb = fm.lib().fp8_quantize_workspace_size(rows, cols, gran, mode)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        st = fm.fp8_quantize(x.data_ptr(), dt, rows, cols, x.stride(0), fmt, gran, mode,
                             scale.data_ptr(), q.data_ptr(), q.stride(0), qt_ptr, ldqt, ctr.ptr(),
                             ws.data_ptr(), wsb, stream)
    fm.check(st)
    return q, qt, scale, ctr


def _inputs():
    big = synth.with_outliers_bf16(2, (2048, 4096))          # 0.1% outliers up to 5000
    small = synth.small_shape_bf16(900, (300, 260), 0.01)   # a much smaller amax
    return dev_bf16(big), dev_bf16(small)


@pytest.mark.parametrize("fmt", [fm.E4M3, fm.E5M2])
@pytest.mark.parametrize("gran,mode,want_t", [(fm.TENSOR, fm.FROM_AMAX, True), (fm.TENSOR, fm.FROM_AMAX, False),
                                              (fm.TENSOR, fm.FROM_AMAX_POW2, False),
                                              (fm.ROW_1x128, fm.FROM_AMAX, False),
                                              (fm.BLOCK_128x128, fm.FROM_AMAX, True)])
def test_noalloc_matches_quantize_twice(fmt, gran, mode, want_t):
    big, small = _inputs()
    # both no-alloc calls are enqueued before either result is read
    n1 = _run(big, fmt, gran, mode, want_t, True)
    n2 = _run(small, fmt, gran, mode, want_t, True)
    r1 = _run(big, fmt, gran, mode, want_t, False)
    r2 = _run(small, fmt, gran, mode, want_t, False)
    torch.cuda.synchronize()
    for (qa, qta, sa, ca), (qb, qtb, sb, cb), what in ((n1, r1, "first"), (n2, r2, "second")):
        assert torch.equal(qa, qb), f"{what} call: codes"
        if want_t:
            assert torch.equal(qta, qtb), f"{what} call: transposed codes"
        assert torch.equal(sa.view(torch.int32), sb.view(torch.int32)), f"{what} call: scales"
        assert ca.read() == cb.read(), f"{what} call: counters"
    # the two tensors have different scales, so a stale partial would show
    assert not torch.equal(n1[2].reshape(-1)[:1], n2[2].reshape(-1)[:1]) or gran != fm.TENSOR


def test_noalloc_fp32_input_and_empty():
    x = torch.from_numpy((np.random.default_rng(3).standard_normal((257, 129)) * 3).astype(np.float32)).cuda()
    a = _run(x, fm.E4M3, fm.TENSOR, fm.FROM_AMAX, True, True)
    b = _run(x, fm.E4M3, fm.TENSOR, fm.FROM_AMAX, True, False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, _, s, _ = _run(e, fm.E4M3, fm.TENSOR, fm.FROM_AMAX, False, True)
    torch.cuda.synchronize()
    assert s.item() == 1.0


def test_noalloc_rejects_bad_arguments_before_launch():
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((64, 64), dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = fm.fp8_quantize_noalloc(x.data_ptr(), fm.BF16, 64, 64, 32, fm.E4M3, fm.TENSOR, fm.FROM_AMAX,
                                 s.data_ptr(), q.data_ptr(), 64, None, 0, None, stream)
    assert st == fm.FP8_ERR_INVALID_ARG
    st = fm.fp8_quantize_noalloc(x.data_ptr(), fm.BF16, 64, 64, 64, fm.E4M3, fm.ROW_1x128, fm.FROM_AMAX,
                                 s.data_ptr(), q.data_ptr(), 64, q.data_ptr(), 64, None, stream)
    assert st == fm.FP8_ERR_UNSUPPORTED_SHAPE
