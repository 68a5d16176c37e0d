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
