"""Seeded random-shape parity sweep of the scaled GEMM against the fp64
oracle, to the same tolerance as the fixed-shape tests (max|y - y_ref| <=
1e-2 max|y_ref|, relative Frobenius <= 5e-3).  The shapes are drawn once from
a fixed seed: m and n anywhere from 1 to a few tiles (ragged in both), k any
multiple of 16 (per-tensor) or of 128 (block-scaled), and short outputs over
deep K so that the split-K forms and both per-tensor kernels are reached.
The quantizers get the same treatment, bit-exact.  Each case prints its
shape in the assertion message."""
import numpy as np
import pytest

import fp8_scaled_matmul_amd as fm
import oracle
import synth
from gpu_util import assert_gemm_close, dev_bf16, dev_f32, dev_u8, host

pytestmark = pytest.mark.gpu
PAIRS = [(fm.E4M3, fm.E4M3), (fm.E5M2, fm.E4M3), (fm.E4M3, fm.E5M2), (fm.E5M2, fm.E5M2)]


def _tensor_cases():
    g = np.random.default_rng(20240611)
    out = []
    for i in range(24):
        if i % 3 == 2:     # short output, deep K
            m, n, k = int(g.integers(1, 300)), int(g.integers(1, 300)), 16 * int(g.integers(128, 384))
        else:
            m, n, k = int(g.integers(1, 700)), int(g.integers(1, 700)), 16 * int(g.integers(1, 96))
        out.append((i, m, n, k))
    return out


def _block_cases():
    g = np.random.default_rng(20240612)
    out = []
    for i in range(12):
        if i % 3 == 2:
            m, n, k = int(g.integers(1, 260)), int(g.integers(1, 260)), 128 * int(g.integers(16, 40))
        else:
            m, n, k = int(g.integers(1, 700)), int(g.integers(1, 700)), 128 * int(g.integers(1, 10))
        out.append((i, m, n, k))
    return out


def _codes(fmt, seed, shape, sigma):
    v = synth.normal_bf16(seed, 0, shape, sigma)
    q, _, s, _ = oracle.quantize(v, fmt)
    return q, s


def _k768_cases():
    g = np.random.default_rng(20240613)
    return [(i, int(g.integers(1, 3000)), 4 * int(g.integers(1, 700))) for i in range(12)]


@pytest.mark.parametrize("i,m,n", _k768_cases())
def test_k768_random_shapes(i, m, n):
    """K = 768 (the A-stationary kernel): the per-tensor GEMM on FP8 codes,
    and the forward with X quantized inside it (codes, transposed codes and
    scale bit-exact, y within tolerance), ragged panels and column units."""
    fa, fb = PAIRS[i % 4]
    k = 768
    x = synth.normal_bf16(3000 + i, 0, (m, k), 1.0)
    a, at, sa, _ = oracle.quantize(x, fa, want_t=True)
    b, sb = _codes(fb, 4000 + i, (n, k), 0.02)
    ref = oracle.gemm(a, fa, sa, oracle.TENSOR, b, fb, sb, oracle.TENSOR)
    what = f"k768 case {i}: {m}x{n} formats {fa},{fb}"
    y = fm.scaled_mm(dev_u8(a), fa, dev_f32(np.float32(sa).reshape(1)), fm.TENSOR,
                     dev_u8(b), fb, dev_f32(np.float32(sb).reshape(1)), fm.TENSOR)
    assert_gemm_close(host(y), ref, what)
    y2, s2, q2, qt2 = fm.quantize_scaled_mm(dev_bf16(x), fa, dev_u8(b), fb, dev_f32(np.float32(sb).reshape(1)),
                                            want_q=True, want_t=True)
    assert_gemm_close(host(y2), ref, what + " fused")
    assert host(s2)[0] == np.float32(sa).reshape(-1)[0], what + " fused scale"
    assert np.array_equal(host(q2), a) and np.array_equal(host(qt2), at), what + " fused codes"


@pytest.mark.parametrize("i,m,n,k", _tensor_cases())
def test_tensor_scaled_random_shapes(i, m, n, k):
    fa, fb = PAIRS[i % 4]
    a, sa = _codes(fa, 1000 + i, (m, k), 1.0)
    b, sb = _codes(fb, 2000 + i, (n, k), 0.02)
    y = fm.scaled_mm(dev_u8(a), fa, dev_f32(np.float32(sa).reshape(1)), fm.TENSOR,
                     dev_u8(b), fb, dev_f32(np.float32(sb).reshape(1)), fm.TENSOR)
    ref = oracle.gemm(a, fa, sa, oracle.TENSOR, b, fb, sb, oracle.TENSOR)
    assert_gemm_close(host(y), ref, f"tensor case {i}: {m}x{n}x{k} formats {fa},{fb}")


@pytest.mark.parametrize("i,m,n,k", _block_cases())
def test_block_scaled_random_shapes(i, m, n, k):
    fa, fb = PAIRS[i % 2]
    pow2 = i % 4 == 3
    quant = oracle.quantize_pow2 if pow2 else oracle.quantize
    av = synth.channel_scaled_bf16(300 + i, 0, 3, (m, k))
    bv = synth.channel_scaled_bf16(300 + i, 1, 4, (n, k))
    a, _, sa, _ = quant(av, fa, oracle.ROW_1x128)
    b, _, sb, _ = quant(bv, fb, oracle.BLOCK_128x128)
    ga, gb = (fm.ROW_1x128_POW2, fm.BLOCK_128x128_POW2) if pow2 else (fm.ROW_1x128, fm.BLOCK_128x128)
    y = fm.scaled_mm(dev_u8(a), fa, dev_f32(sa.reshape(-1)), ga, dev_u8(b), fb, dev_f32(sb.reshape(-1)), gb)
    ref = oracle.gemm(a, fa, sa, oracle.ROW_1x128, b, fb, sb, oracle.BLOCK_128x128)
    assert_gemm_close(host(y), ref, f"block case {i}: {m}x{n}x{k} formats {fa},{fb} pow2={pow2}")


# ------------------------------------------------------------------ quantizers
from gpu_util import gpu_quantize, same_counters  # noqa: E402


def _quant_cases():
    g = np.random.default_rng(20240613)
    out = [(i, int(g.integers(1, 700)), int(g.integers(1, 1100))) for i in range(14)]
    # two larger ones: whole tiles over more than one round of workgroups, plus edges
    return out + [(14, 4100, 3000), (15, 5000, 4500)]


@pytest.mark.parametrize("i,rows,cols", _quant_cases())
def test_quantize_random_shapes(i, rows, cols):
    """Bytes, transposed bytes, scales and counters bit-exact for per-tensor
    (with and without the transposed copy), 1x128 and 128x128 scales."""
    fmt = (fm.E4M3, fm.E5M2)[i % 2]
    x = synth.channel_scaled_bf16(400 + i, 0, 5, (rows, cols))
    xd = dev_bf16(x)
    for gran, want_t in ((fm.TENSOR, False), (fm.TENSOR, True), (fm.ROW_1x128, False), (fm.BLOCK_128x128, True),
                         (fm.BLOCK_128x128, False)):
        q, qt, s, c = gpu_quantize(xd, fmt, gran, fm.FROM_AMAX, None, want_t)
        oq, oqt, os_, oc = oracle.quantize(x, fmt, gran, oracle.FROM_AMAX, None, want_t)
        what = f"case {i}: {rows}x{cols} format {fmt} granularity {gran} transposed {want_t}"
        assert np.array_equal(s.reshape(os_.shape), os_), f"{what}: scales differ"
        assert np.array_equal(q, oq), f"{what}: {int((q != oq).sum())} codes differ"
        if want_t:
            assert np.array_equal(qt, oqt), f"{what}: transposed codes differ"
        assert same_counters(c, oc), f"{what}: counters gpu {c} oracle {oc}"


@pytest.mark.parametrize("i,rows,cols", _quant_cases())
def test_quantize_random_shapes_given_scales(i, rows, cols):
    """Given scales (per tensor, per 1x128 tile, per 128x128 block) between a
    third and three times amax / fmax, so that some elements saturate and
    the rest take the corrected quotient below the scale's limit: bytes,
    transposed bytes and counters bit-exact, ragged edges included."""
    fmt = (fm.E4M3, fm.E5M2)[(i + 1) % 2]
    fmax = 448.0 if fmt == fm.E4M3 else 57344.0
    x = synth.channel_scaled_bf16(450 + i, 0, 5, (rows, cols))
    amax = float(np.abs(synth.bf16_bits_to_f32(x)).max())
    g = np.random.default_rng(460 + i)
    xd = dev_bf16(x)
    for gran, want_t in ((fm.TENSOR, False), (fm.TENSOR, True), (fm.ROW_1x128, False), (fm.BLOCK_128x128, True)):
        shape = oracle.scale_shape(gran, rows, cols)
        sc = (amax / fmax * g.uniform(1 / 3, 3, size=shape)).astype(np.float32)
        q, qt, _, c = gpu_quantize(xd, fmt, gran, fm.GIVEN, sc, want_t)
        oq, oqt, _, oc = oracle.quantize(x, fmt, gran, oracle.GIVEN, sc, want_t)
        what = f"case {i}: {rows}x{cols} format {fmt} granularity {gran} transposed {want_t}, given scales"
        assert np.array_equal(q, oq), f"{what}: {int((q != oq).sum())} codes differ"
        if want_t:
            assert np.array_equal(qt, oqt), f"{what}: transposed codes differ"
        assert same_counters(c, oc), f"{what}: counters gpu {c} oracle {oc}"
