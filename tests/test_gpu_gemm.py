"""GPU parity of the scaled GEMM against the fp64 oracle, to the tolerance
max|y - y_ref| <= 1e-2 max|y_ref| and relative Frobenius <= 5e-3, every
output element: small and ragged shapes, every format pair, both scale
pairs, split K, the persistent kernels over several rounds of tiles, and the
leading-dimension limits.  The full-size workloads are in
test_gpu_workloads.py."""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import oracle
import synth
from gpu_util import assert_gemm_close, dev_bf16, dev_f32, dev_u8, host

pytestmark = pytest.mark.gpu
PAIRS = [(fm.E4M3, fm.E4M3), (fm.E5M2, fm.E4M3), (fm.E4M3, fm.E5M2), (fm.E5M2, fm.E5M2)]


def _codes(fmt, g, shape, sigma=1.0):
    """Codes of N(0, sigma) values quantized by the oracle (finite, realistic)."""
    v = synth.f32_to_bf16_bits((g.standard_normal(shape) * sigma).astype(np.float32))
    q, _, s, _ = oracle.quantize(v, fmt)
    return q, s


def _run(a, fa, sa, ga, b, fb, sb, gb, workspace=True, ctr=None):
    A, B = dev_u8(a), dev_u8(b)
    SA, SB = dev_f32(np.asarray(sa, np.float32).reshape(-1)), dev_f32(np.asarray(sb, np.float32).reshape(-1))
    m, k = a.shape
    n = b.shape[0]
    ws = None
    if not workspace:
        ws = torch.empty(0, dtype=torch.uint8, device="cuda")
    y = fm.scaled_mm(A, fa, SA, ga, B, fb, SB, gb, counters=ctr, workspace=ws if not workspace else None)
    return host(y)


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (16, 16, 128), (33, 17, 256), (256, 256, 128),
                                   (300, 280, 384), (257, 513, 784), (512, 256, 1024), (64, 1000, 48)])
def test_tensor_scaled_small(fa, fb, m, n, k):
    g = np.random.default_rng(m * 7 + n * 3 + k)
    a, sa = _codes(fa, g, (m, k))
    b, sb = _codes(fb, g, (n, k), 0.02)
    y = _run(a, fa, sa, 0, b, fb, sb, 0)
    ref = oracle.gemm(a, fa, sa, 0, b, fb, sb, 0)
    assert_gemm_close(y, ref, f"{m}x{n}x{k}")


@pytest.mark.parametrize("fa,fb", PAIRS[:2])
@pytest.mark.parametrize("m,n,k", [(256, 256, 512), (300, 384, 640), (17, 130, 128), (512, 512, 1024),
                                   (64, 256, 256), (130, 260, 384)])
def test_block_scaled_small(fa, fb, m, n, k):
    g = np.random.default_rng(m + n + k)
    av = synth.channel_scaled_bf16(200, 0, 3, (m, k))
    bv = synth.channel_scaled_bf16(200, 1, 4, (n, k))
    a, _, sa, _ = oracle.quantize(av, fa, oracle.ROW_1x128)
    b, _, sb, _ = oracle.quantize(bv, fb, oracle.BLOCK_128x128)
    y = _run(a, fa, sa, 1, b, fb, sb, 2)
    ref = oracle.gemm(a, fa, sa, 1, b, fb, sb, 2)
    assert_gemm_close(y, ref, f"block {m}x{n}x{k}")
    del g


def test_split_k_and_determinism():
    g = np.random.default_rng(9)
    m, n, k = 512, 256, 8192
    a, sa = _codes(fm.E5M2, g, (m, k), 1e-3)
    b, sb = _codes(fm.E4M3, g, (n, k))
    ref = oracle.gemm(a, fm.E5M2, sa, 0, b, fm.E4M3, sb, 0)
    assert fm.lib().fp8_scaled_mm_workspace_size(m, n, k, 0, 0) > 0
    y1 = _run(a, fm.E5M2, sa, 0, b, fm.E4M3, sb, 0)
    y2 = _run(a, fm.E5M2, sa, 0, b, fm.E4M3, sb, 0)
    assert np.array_equal(y1, y2), "split-K result not deterministic"
    assert_gemm_close(y1, ref, "split-K")
    y3 = _run(a, fm.E5M2, sa, 0, b, fm.E4M3, sb, 0, workspace=False)
    assert_gemm_close(y3, ref, "no workspace")
    # block-scaled with split K
    av = synth.channel_scaled_bf16(201, 0, 3, (m, k))
    bv = synth.channel_scaled_bf16(201, 1, 4, (n, k))
    a, _, sa, _ = oracle.quantize(av, fm.E4M3, oracle.ROW_1x128)
    b, _, sb, _ = oracle.quantize(bv, fm.E4M3, oracle.BLOCK_128x128)
    y = _run(a, 0, sa, 1, b, 0, sb, 2)
    assert_gemm_close(y, oracle.gemm(a, 0, sa, 1, b, 0, sb, 2), "block split-K")


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("m,n,k", [(300, 256, 4096), (257, 130, 4160), (64, 384, 8192)])
def test_tensor_scaled_split_k_formats(fa, fb, m, n, k):
    """Per-tensor GEMMs that split K, every format pair: K a multiple of 128
    runs the 8-wave block kernel with per-tensor scales, K = 4160 the
    persistent kernel's own split; both against the oracle, and a second call
    bit-identical."""
    g = np.random.default_rng(m + 3 * n + 7 * k + 11 * fa + 13 * fb)
    a, sa = _codes(fa, g, (m, k), 0.05)
    b, sb = _codes(fb, g, (n, k), 0.05)
    assert fm.lib().fp8_scaled_mm_workspace_size(m, n, k, 0, 0) > 0
    y1 = _run(a, fa, sa, 0, b, fb, sb, 0)
    y2 = _run(a, fa, sa, 0, b, fb, sb, 0)
    assert np.array_equal(y1, y2), "split-K result not deterministic"
    assert_gemm_close(y1, oracle.gemm(a, fa, sa, 0, b, fb, sb, 0), f"split-K {fa}x{fb} {m}x{n}x{k}")


def test_tensor_scaled_persistent_block_kernel():
    """A per-tensor GEMM with K = 2048 (16 blocks) and 288 output tiles: the
    8-wave kernel runs persistent, some workgroups take two tiles, the second
    one's first K blocks fetched during the first one's last blocks.  Every
    output against the oracle."""
    g = np.random.default_rng(77)
    m, n, k = 4608, 4096, 2048
    a, sa = _codes(fm.E5M2, g, (m, k), 0.05)
    b, sb = _codes(fm.E4M3, g, (n, k), 0.05)
    assert fm.lib().fp8_scaled_mm_workspace_size(m, n, k, 0, 0) == 0
    y = host(fm.scaled_mm(dev_u8(a), fm.E5M2, dev_f32(sa), 0, dev_u8(b), fm.E4M3, dev_f32(sb), 0))
    _check_points(y, a, fm.E5M2, sa, 0, b, fm.E4M3, sb, 0, g, "persistent 4608x4096x2048")


@pytest.mark.parametrize("fa,fb,m,n", [(fm.E4M3, fm.E4M3, 4500, 4100), (fm.E4M3, fm.E5M2, 4500, 4100),
                                         (fm.E5M2, fm.E4M3, 4400, 4098)])
def test_tensor_scaled_deep_k_ragged(fa, fb, m, n):
    """K = 2048 with ragged M and N and more than 256 tiles: the persistent
    8-wave kernel (N % 4 == 0, partial edge tiles on both sides) and the
    single-tile kernel's element stores (N = 4098).  Every output against the
    oracle."""
    g = np.random.default_rng(m + n + fa + 3 * fb)
    k = 2048
    a, sa = _codes(fa, g, (m, k), 0.05)
    b, sb = _codes(fb, g, (n, k), 0.05)
    y = host(fm.scaled_mm(dev_u8(a), fa, dev_f32(sa), 0, dev_u8(b), fb, dev_f32(sb), 0))
    _check_points(y, a, fa, sa, 0, b, fb, sb, 0, g, f"deep K {m}x{n}x{k}")


@pytest.mark.parametrize("n,ld_out", [(250, 250), (252, 260), (252, 254)])
def test_split_k_reduction_layouts(n, ld_out):
    """Split-K outputs through both reductions: four outputs per thread
    (n % 4 == 0, output rows 8-byte aligned) and one per thread (ragged n, or
    an output stride that breaks the 8-byte alignment), into a strided output
    whose padding columns must stay untouched."""
    g = np.random.default_rng(n + ld_out)
    m, k = 300, 4096
    a, sa = _codes(fm.E5M2, g, (m, k), 1e-3)
    b, sb = _codes(fm.E4M3, g, (n, k))
    assert fm.lib().fp8_scaled_mm_workspace_size(m, n, k, 0, 0) > 0
    full = torch.full((m, ld_out), 3.0, dtype=torch.bfloat16, device="cuda")
    out = full[:, :n]
    SA, SB = dev_f32(np.asarray(sa, np.float32).reshape(-1)), dev_f32(np.asarray(sb, np.float32).reshape(-1))
    fm.scaled_mm(dev_u8(a), fm.E5M2, SA, 0, dev_u8(b), fm.E4M3, SB, 0, out=out)
    y = host(out.contiguous())
    assert_gemm_close(y, oracle.gemm(a, fm.E5M2, sa, 0, b, fm.E4M3, sb, 0), f"split-K n={n} ldc={ld_out}")
    if ld_out > n:
        assert torch.all(full[:, n:] == 3.0), "split-K reduction wrote past the output columns"


def test_k_zero_and_empty():
    A = torch.zeros((8, 0), dtype=torch.uint8, device="cuda")
    B = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    y = torch.full((8, 5), 7.0, dtype=torch.bfloat16, device="cuda")
    fm.scaled_mm(A, 0, one, 0, B, 0, one, 0, out=y)
    assert torch.all(y == 0)
    A = torch.zeros((0, 32), dtype=torch.uint8, device="cuda")
    B = torch.zeros((5, 32), dtype=torch.uint8, device="cuda")
    y = fm.scaled_mm(A, 0, one, 0, B, 0, one, 0)
    assert y.shape == (0, 5)


def test_strided_operands_and_output():
    g = np.random.default_rng(10)
    m, n, k = 100, 70, 256
    a, sa = _codes(0, g, (m, k + 64))
    b, sb = _codes(0, g, (n, k + 32))
    A, B = dev_u8(a)[:, :k], dev_u8(b)[:, 16:16 + k]
    out = torch.full((m, n + 10), 1.0, dtype=torch.bfloat16, device="cuda")
    fm.scaled_mm(A, 0, dev_f32(sa), 0, B, 0, dev_f32(sb), 0, out=out[:, :n])
    y = host(out)
    ref = oracle.gemm(np.ascontiguousarray(a[:, :k]), 0, sa, 0, np.ascontiguousarray(b[:, 16:16 + k]), 0, sb, 0)
    assert_gemm_close(y[:, :n], ref, "strided")
    assert np.all(y[:, n:] == 0x3F80), "wrote past n"


def test_nonfinite_output_counter():
    a = np.full((32, 128), 0x7E, np.uint8)          # 448
    b = np.full((32, 128), 0x7E, np.uint8)
    ctr = fm.Counters()
    y = _run(a, 0, [1e30], 0, b, 0, [1e3], 0, ctr=ctr)
    assert ctr.read()["nonfinite_out"] == 32 * 32
    assert np.all((y & 0x7FFF) == 0x7F80)


@pytest.mark.parametrize("kind", ["block_fp32", "block_pow2", "tensor_persistent"])
def test_nonfinite_output_counter_block_kernels(kind):
    """The block kernels keep a running maximum of the stored bf16 words and,
    only when it reaches the all-ones exponent, read their outputs back to
    count the Inf/NaN ones.  A few A rows of 448s times B of 448s overflow
    with the chosen scales, one A row holds a NaN code, the other rows are
    small and finite: the counter equals the Inf/NaN words in y, which are
    exactly those rows.  Shapes: the block-scaled kernel (fp32 and
    power-of-two scales, 4 tiles) and the persistent per-tensor kernel (272
    tiles on 256 CUs, K = 2048)."""
    g = np.random.default_rng(31)
    if kind == "tensor_persistent":
        m, n, k = 4352, 4096, 2048
    else:
        m, n, k = 512, 512, 1024
    small = np.concatenate([np.arange(0x00, 0x39), np.arange(0x80, 0xB9)]).astype(np.uint8)   # |v| <= 1
    a = small[g.integers(0, small.size, size=(m, k))]
    big_rows = [3, 200, m - 1]
    a[big_rows, :] = 0x7E                      # 448
    a[7, k // 2] = 0x7F                        # NaN code
    b = np.full((n, k), 0x7E, np.uint8)
    if kind == "tensor_persistent":
        ga, gb = fm.TENSOR, fm.TENSOR
        sa = np.float32([1e30]).reshape(1)
        sb = np.float32([10.0]).reshape(1)
    else:
        ga = fm.ROW_1x128 if kind == "block_fp32" else fm.ROW_1x128_POW2
        gb = fm.BLOCK_128x128 if kind == "block_fp32" else fm.BLOCK_128x128_POW2
        va, vb = (1e30, 10.0) if kind == "block_fp32" else (2.0 ** 100, 8.0)
        sa = np.full((m, k // 128), va, np.float32)
        sb = np.full((n // 128, k // 128), vb, np.float32)
    ctr = fm.Counters()
    y = host(fm.scaled_mm(dev_u8(a), fm.E4M3, dev_f32(sa), ga, dev_u8(b), fm.E4M3, dev_f32(sb), gb, counters=ctr))
    bad = (y & 0x7F80) == 0x7F80
    rows = np.nonzero(bad.any(axis=1))[0]
    assert sorted(rows.tolist()) == sorted(big_rows + [7]), rows[:10]
    assert bad[rows].all()
    assert ctr.read()["nonfinite_out"] == int(bad.sum()) == (len(big_rows) + 1) * n


def _check_points(y, a, fa, sa, ga, b, fb, sb, gb, g, what):
    """Every output element against the oracle GEMM on the same codes."""
    del g
    return assert_gemm_close(y, oracle.gemm(a, fa, sa, ga, b, fb, sb, gb), what)


@pytest.mark.parametrize("block,k", [(False, 256), (True, 256), (False, 2048)])
def test_largest_leading_dimensions(block, k):
    """lda, ldb just below 2^22 and ldc just below 2^21 (the limits the C ABI
    accepts): the 32-bit offsets inside a tile reach their largest values.
    Per-tensor scales with K = 256 run the 4-wave kernel, with K = 2048 the
    8-wave kernel with per-tensor scales."""
    m, n = 256, 384
    lda = ldb = (1 << 22) - 16
    ldc = (1 << 21) - 8
    g = np.random.default_rng(71)
    if block:
        av = synth.channel_scaled_bf16(310, 0, 3, (m, k))
        bv = synth.channel_scaled_bf16(310, 1, 4, (n, k))
        a, _, sa, _ = oracle.quantize(av, 0, oracle.ROW_1x128)
        b, _, sb, _ = oracle.quantize(bv, 0, oracle.BLOCK_128x128)
        ga, gb = fm.ROW_1x128, fm.BLOCK_128x128
        ref = oracle.gemm(a, 0, sa, 1, b, 0, sb, 2)
    else:
        a, sa = _codes(fm.E4M3, g, (m, k))
        b, sb = _codes(fm.E4M3, g, (n, k), 0.02)
        ga = gb = fm.TENSOR
        ref = oracle.gemm(a, 0, sa, 0, b, 0, sb, 0)
    A = torch.zeros((m, lda), dtype=torch.uint8, device="cuda")
    B = torch.zeros((n, ldb), dtype=torch.uint8, device="cuda")
    A[:, :k].copy_(torch.from_numpy(a))
    B[:, :k].copy_(torch.from_numpy(b))
    C = torch.full((m, ldc), 7.0, dtype=torch.bfloat16, device="cuda")
    y = fm.scaled_mm(A[:, :k], 0, dev_f32(np.asarray(sa, np.float32)), ga, B[:, :k], 0,
                     dev_f32(np.asarray(sb, np.float32)), gb, out=C[:, :n])
    assert_gemm_close(host(y), ref, f"ld limits block={block}")
    # nothing beyond the n output columns of each row was written
    assert bool((C[:, n:n + 64] == 7.0).all())
    del A, B, C
    torch.cuda.empty_cache()
