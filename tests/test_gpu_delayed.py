"""GPU parity of delayed scaling (amax history) against the oracle: bytes,
transposed bytes, scale, counters, the recorded history and its position,
bit-exact, over several consecutive steps, on the one-pass layout (bf16,
whole 128x128 tiles, transposed copy) and on the two-pass layouts, with
growth past the recorded amax (saturation), Inf/NaN inputs, a history value
that is not a bf16 number, and the full 65536 x 3072 dY shape."""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host, same_counters

pytestmark = pytest.mark.gpu
FMTS = [fm.E4M3, fm.E5M2]


def _run_steps(xs, fmt, length, want_t, fp32=False, init=None):
    hist = fm.AmaxHistory(length)
    h_orc = np.zeros(length, np.float32) if init is None else np.asarray(init, np.float32).copy()
    if init is not None:
        hist.values.copy_(torch.from_numpy(h_orc))
    pos_orc = 0
    for step, xb in enumerate(xs):
        ctr = fm.Counters()
        xd = dev_f32(synth.bf16_bits_to_f32(xb)) if fp32 else dev_bf16(xb)
        q, qt, s = fm.quantize_delayed(xd, fmt, hist, want_t=want_t, counters=ctr)
        torch.cuda.synchronize()
        x_orc = synth.bf16_bits_to_f32(xb) if fp32 else xb
        oq, oqt, os_, oc, h_orc, pos_orc = oracle.quantize_delayed(x_orc, fmt, h_orc, pos_orc, want_t)
        what = f"step {step}"
        assert host(s)[0] == os_[0], f"{what}: scale gpu {host(s)[0]} oracle {os_[0]}"
        bad = np.nonzero(host(q) != oq)
        assert bad[0].size == 0, f"{what}: {bad[0].size} codes differ"
        if want_t:
            assert np.array_equal(host(qt), oqt), f"{what}: transposed codes differ"
        c = ctr.read()
        assert same_counters(c, oc), f"{what}: counters gpu {c} oracle {oc}"
        assert np.array_equal(host(hist.values), h_orc), f"{what}: history gpu {host(hist.values)} oracle {h_orc}"
        assert int(host(hist.pos)[0]) == pos_orc, f"{what}: position"
    return h_orc


def _steps(seed, shape, gains):
    """A tensor per step whose magnitude changes by the given factors, so the
    recorded amax lags behind (growth saturates, shrinkage underflows)."""
    base = synth.small_shape_bf16(seed, shape)
    f = synth.bf16_bits_to_f32(base)
    return [synth.f32_to_bf16_bits(f * np.float32(g)) for g in gains]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(256, 384), (128, 128), (512, 256)])
def test_one_pass_layout(fmt, shape):
    _run_steps(_steps(21, shape, [1.0, 3.0, 0.25, 0.25, 8.0]), fmt, 3, want_t=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape,want_t", [((300, 200), True), ((256, 384), False), ((1, 1000), False),
                                          ((129, 257), True)])
def test_two_pass_layouts(fmt, shape, want_t):
    _run_steps(_steps(22, shape, [1.0, 2.0, 0.5, 4.0]), fmt, 2, want_t=want_t)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp32_input(fmt):
    _run_steps(_steps(23, (256, 256), [1.0, 5.0, 0.1]), fmt, 2, want_t=True, fp32=True)


@pytest.mark.parametrize("fmt", FMTS)
def test_nonfinite_inputs(fmt):
    xs = _steps(24, (256, 256), [1.0, 1.0, 2.0])
    xs[1] = xs[1].copy()
    xs[1][3, 7] = 0x7F80      # +Inf
    xs[1][100, 200] = 0xFFC3  # NaN
    xs[2] = xs[2].copy()
    xs[2][0, 0] = 0xFF80      # -Inf
    _run_steps(xs, fmt, 2, want_t=True)


@pytest.mark.parametrize("fmt", FMTS)
def test_history_not_bf16_and_long(fmt):
    # 0.3 is not a bf16 number: the cast takes the IEEE-division path
    _run_steps(_steps(25, (256, 256), [1.0, 1.0]), fmt, 5, want_t=True, init=[0.3, 0.0, 1e-3, 0.0, 0.0])
    _run_steps(_steps(26, (128, 256), [1.0] * 3), fmt, 1000, want_t=True)


def test_every_bf16_pattern():
    x = synth.all_bf16_patterns()
    _run_steps([x, x], fm.E4M3, 1, want_t=True, init=[2.0])


def test_dy_workload_size():
    """dY [65536, 3072] E5M2 with a transposed copy, one pass, after a step
    with half its magnitude (so the largest elements saturate)."""
    dy = synth.normal_bf16(5, 0, (65536, 3072), 1e-3)
    half = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(dy) * np.float32(0.5))
    _run_steps([half, dy], fm.E5M2, 4, want_t=True)


def test_rejects_bad_history():
    x = dev_bf16(synth.small_shape_bf16(27, (16, 16)))
    hist = fm.AmaxHistory(4)
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    q = torch.empty((16, 16), dtype=torch.uint8, device="cuda")
    ws = torch.empty(fm.lib().fp8_quantize_delayed_workspace_size(16, 16), dtype=torch.uint8, device="cuda")
    for length in (0, 4097):
        rc = fm.fp8_quantize_delayed(x.data_ptr(), 0, 16, 16, 16, 0, hist.values.data_ptr(), hist.pos.data_ptr(),
                                     length, s.data_ptr(), q.data_ptr(), 16, None, 0, None, ws.data_ptr(),
                                     ws.numel(), torch.cuda.current_stream().cuda_stream)
        assert rc == 1, length
    rc = fm.fp8_quantize_delayed(x.data_ptr(), 0, 16, 16, 16, 0, None, hist.pos.data_ptr(), 4, s.data_ptr(),
                                 q.data_ptr(), 16, None, 0, None, ws.data_ptr(), ws.numel(),
                                 torch.cuda.current_stream().cuda_stream)
    assert rc == 1
