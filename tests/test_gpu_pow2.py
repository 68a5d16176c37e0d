"""GPU parity of power-of-two (E8M0) scaling against the oracle: quantizer
scales, bytes, transposed bytes and counters bit-exact for every granularity
(fast bf16 kernels and the general ones), on every bf16 pattern, ragged,
fp32 and full-size inputs."""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host, same_counters

pytestmark = pytest.mark.gpu
FMTS = [fm.E4M3, fm.E5M2]
GRANS = [fm.TENSOR, fm.ROW_1x128, fm.BLOCK_128x128]


def _cmp_pow2(x_bits, fmt, gran, want_t=False, fp32=False):
    xd = dev_f32(synth.bf16_bits_to_f32(x_bits)) if fp32 else dev_bf16(x_bits)
    ctr = fm.Counters()
    q, qt, s = fm.quantize(xd, fmt, gran, fm.FROM_AMAX_POW2, want_t=want_t, counters=ctr)
    torch.cuda.synchronize()
    x_orc = synth.bf16_bits_to_f32(x_bits) if fp32 else x_bits
    oq, oqt, os_, oc = oracle.quantize_pow2(x_orc, fmt, gran, want_t)
    assert np.array_equal(host(s).reshape(os_.shape), os_), "scales differ"
    bad = np.nonzero(host(q) != oq)
    assert bad[0].size == 0, f"{bad[0].size} codes differ"
    if want_t:
        assert np.array_equal(host(qt), oqt), "transposed codes differ"
    c = ctr.read()
    assert same_counters(c, oc), f"counters gpu {c} oracle {oc}"
    assert c["saturated"] == 0 or np.isinf(synth.bf16_bits_to_f32(x_bits)).any()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", GRANS)
@pytest.mark.parametrize("shape", [(256, 384), (300, 200), (128, 1024), (1, 130)])
def test_shapes(fmt, gran, shape):
    x = synth.with_outliers_bf16(41, shape)
    _cmp_pow2(x, fmt, gran, want_t=gran != fm.ROW_1x128)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", GRANS)
def test_fp32_input(fmt, gran):
    _cmp_pow2(synth.with_outliers_bf16(42, (256, 256)), fmt, gran, want_t=gran != fm.ROW_1x128, fp32=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", GRANS)
def test_every_bf16_pattern(fmt, gran):
    _cmp_pow2(synth.all_bf16_patterns(), fmt, gran, want_t=gran != fm.ROW_1x128)


@pytest.mark.parametrize("sigma", [1.0, 1e-30, 3e30, 2.0 ** -120])
def test_scale_extremes(sigma):
    x = synth.small_shape_bf16(43, (256, 256), sigma)
    for gran in GRANS:
        _cmp_pow2(x, fm.E4M3, gran)


def test_block_scaled_workload_full_size():
    """A [16384, 7168] 1x128 and B [2048, 7168] 128x128 with power-of-two scales."""
    a = synth.channel_scaled_bf16(4, 0, 3, synth.BLOCK_SCALED["a"])
    b = synth.channel_scaled_bf16(4, 1, 4, synth.BLOCK_SCALED["b"])
    _cmp_pow2(a, fm.E4M3, fm.ROW_1x128)
    _cmp_pow2(b, fm.E4M3, fm.BLOCK_128x128, want_t=True)
    _cmp_pow2(b, fm.E4M3, fm.BLOCK_128x128)


# ------------------------------------------------------------------ GEMM with E8M0 scales in the MFMA
from gpu_util import assert_gemm_close, dev_u8  # noqa: E402


def _gemm_pow2(a, fa, sa, b, fb, sb, workspace=True):
    A, B = dev_u8(a), dev_u8(b)
    SA, SB = dev_f32(np.asarray(sa, np.float32)), dev_f32(np.asarray(sb, np.float32))
    ws = None if workspace else torch.empty(0, dtype=torch.uint8, device="cuda")
    ctr = fm.Counters()
    y = fm.scaled_mm(A, fa, SA, fm.ROW_1x128_POW2, B, fb, SB, fm.BLOCK_128x128_POW2, counters=ctr, workspace=ws)
    return host(y), ctr.read()


@pytest.mark.parametrize("fa,fb", [(fm.E4M3, fm.E4M3), (fm.E5M2, fm.E4M3), (fm.E4M3, fm.E5M2)])
@pytest.mark.parametrize("m,n,k", [(256, 256, 512), (300, 384, 640), (17, 130, 128), (512, 512, 1024),
                                   (64, 256, 256), (130, 260, 384)])
def test_gemm_pow2_small(fa, fb, m, n, k):
    av = synth.channel_scaled_bf16(300, 0, 3, (m, k))
    bv = synth.channel_scaled_bf16(300, 1, 4, (n, k))
    a, _, sa, _ = oracle.quantize_pow2(av, fa, oracle.ROW_1x128)
    b, _, sb, _ = oracle.quantize_pow2(bv, fb, oracle.BLOCK_128x128)
    y, c = _gemm_pow2(a, fa, sa, b, fb, sb)
    assert_gemm_close(y, oracle.gemm(a, fa, sa, 1, b, fb, sb, 2), f"pow2 {m}x{n}x{k}")
    assert c["nonfinite_out"] == 0


def test_gemm_pow2_split_k_and_no_workspace():
    m, n, k = 512, 256, 8192
    av = synth.channel_scaled_bf16(301, 0, 3, (m, k))
    bv = synth.channel_scaled_bf16(301, 1, 4, (n, k))
    a, _, sa, _ = oracle.quantize_pow2(av, fm.E5M2, oracle.ROW_1x128)
    b, _, sb, _ = oracle.quantize_pow2(bv, fm.E4M3, oracle.BLOCK_128x128)
    ref = oracle.gemm(a, 1, sa, 1, b, 0, sb, 2)
    y1, _ = _gemm_pow2(a, 1, sa, b, 0, sb)
    y2, _ = _gemm_pow2(a, 1, sa, b, 0, sb)
    assert np.array_equal(y1, y2), "not deterministic"
    assert_gemm_close(y1, ref, "pow2 split-K")
    y3, _ = _gemm_pow2(a, 1, sa, b, 0, sb, workspace=False)
    assert_gemm_close(y3, ref, "pow2 no workspace")


def test_gemm_pow2_extreme_scales():
    """Scales far from 1 in both directions (E8M0 codes near both ends)."""
    m, n, k = 256, 256, 512
    for sigma in (2.0 ** -100, 2.0 ** 90):
        av = synth.small_shape_bf16(302, (m, k), sigma)
        bv = synth.small_shape_bf16(303, (n, k), 1.0 / sigma if sigma < 1 else 2.0 ** -100)
        a, _, sa, _ = oracle.quantize_pow2(av, fm.E4M3, oracle.ROW_1x128)
        b, _, sb, _ = oracle.quantize_pow2(bv, fm.E4M3, oracle.BLOCK_128x128)
        y, _ = _gemm_pow2(a, 0, sa, b, 0, sb)
        assert_gemm_close(y, oracle.gemm(a, 0, sa, 1, b, 0, sb, 2), f"pow2 sigma {sigma}")
