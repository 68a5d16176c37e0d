"""Pins for the oracle's scaled GEMM (CPU only).

Independent facts used: an exact integer dot product on tiny shapes (codes
turned into integers straight from their bit fields, scaled by 2^9 for E4M3
and 2^16 for E5M2), numpy's fp64 matmul of decoded values (a library
routine), closed forms (all-max inputs, one-hot selection, scale doubling),
and the reduction of the block-scaled form with uniform scales to the
per-tensor form.
"""
import numpy as np
import pytest

import oracle
import synth


def _int_value(fmt, codes):
    """code -> integer value * 2^(9 or 16), from the bit fields alone."""
    codes = np.asarray(codes, dtype=np.int64)
    sign = np.where(codes & 0x80, -1, 1)
    if fmt == oracle.E4M3:
        e, m = (codes >> 3) & 0xF, codes & 7
        mag = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    else:
        e, m = (codes >> 2) & 0x1F, codes & 3
        mag = np.where(e == 0, m, (4 + m) << np.maximum(e - 1, 0))
    return sign * mag


def _finite_codes(fmt, rng, shape):
    bad = {0x7F, 0xFF} if fmt == oracle.E4M3 else set(range(0x7C, 0x80)) | set(range(0xFC, 0x100))
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    mask = np.isin(c, list(bad))
    c[mask] = 0x38
    return c


@pytest.mark.parametrize("fa,fb", [(oracle.E4M3, oracle.E4M3), (oracle.E5M2, oracle.E4M3),
                                   (oracle.E4M3, oracle.E5M2)])
@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (7, 5, 33), (16, 16, 128), (33, 17, 256)])
def test_exact_integer_dot(fa, fb, m, n, k):
    rng = np.random.default_rng(m * 1000 + n * 10 + k)
    a = _finite_codes(fa, rng, (m, k))
    b = _finite_codes(fb, rng, (n, k))
    ia = _int_value(fa, a)
    ib = _int_value(fb, b)
    exact = ia @ ib.T                          # int64: no overflow at these K
    shift = (9 if fa == oracle.E4M3 else 16) + (9 if fb == oracle.E4M3 else 16)
    y = oracle.gemm(a, fa, 1.0, oracle.TENSOR, b, fb, 1.0, oracle.TENSOR)
    want = exact.astype(np.float64) * 2.0 ** -shift
    if fa == oracle.E4M3 and fb == oracle.E4M3:
        assert np.array_equal(y, want)         # fp64 sum is exact for E4M3 x E4M3
    else:
        np.testing.assert_allclose(y, want, rtol=1e-14, atol=2.0 ** -shift)


def test_vs_numpy_matmul_with_scales():
    rng = np.random.default_rng(1)
    a = _finite_codes(oracle.E4M3, rng, (40, 384))
    b = _finite_codes(oracle.E4M3, rng, (24, 384))
    sa, sb = np.float32(0.0123), np.float32(3.7)
    y = oracle.gemm(a, oracle.E4M3, sa, oracle.TENSOR, b, oracle.E4M3, sb, oracle.TENSOR)
    da = oracle.decode(oracle.E4M3, a)
    db = oracle.decode(oracle.E4M3, b)
    ref = (float(sa) * float(sb)) * (da @ db.T)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("fa,fb", [(oracle.E4M3, oracle.E4M3), (oracle.E5M2, oracle.E4M3)])
def test_closed_forms(fa, fb):
    k = 256
    maxa = 0x7E if fa == oracle.E4M3 else 0x7B
    maxb = 0x7E if fb == oracle.E4M3 else 0x7B
    a = np.full((3, k), maxa, dtype=np.uint8)
    b = np.full((2, k), maxb, dtype=np.uint8)
    sa, sb = np.float32(0.5), np.float32(0.25)
    y = oracle.gemm(a, fa, sa, oracle.TENSOR, b, fb, sb, oracle.TENSOR)
    assert np.all(y == k * oracle.fmax(fa) * oracle.fmax(fb) * 0.5 * 0.25)
    # one-hot B row with the code of 1.0 selects a column of s_a s_b A
    one = 0x38 if fb == oracle.E4M3 else 0x3C
    rng = np.random.default_rng(2)
    a = _finite_codes(fa, rng, (5, k))
    b = np.zeros((k, k), dtype=np.uint8)
    b[np.arange(k), np.arange(k)] = one
    y = oracle.gemm(a, fa, 2.0, oracle.TENSOR, b, fb, 0.5, oracle.TENSOR)
    assert np.array_equal(y, oracle.decode(fa, a))
    # doubling s_a doubles y exactly
    b2 = _finite_codes(fb, rng, (6, k))
    y1 = oracle.gemm(a, fa, 0.3, oracle.TENSOR, b2, fb, 1.7, oracle.TENSOR)
    y2 = oracle.gemm(a, fa, np.float32(0.3) * 2, oracle.TENSOR, b2, fb, 1.7, oracle.TENSOR)
    assert np.array_equal(y2, 2 * y1)


def test_block_uniform_equals_tensor():
    rng = np.random.default_rng(3)
    m, n, k = 20, 260, 384
    a = _finite_codes(oracle.E4M3, rng, (m, k))
    b = _finite_codes(oracle.E4M3, rng, (n, k))
    sa, sb = np.float32(0.25), np.float32(4.0)       # powers of two: exact in every order
    y_t = oracle.gemm(a, oracle.E4M3, sa, oracle.TENSOR, b, oracle.E4M3, sb, oracle.TENSOR)
    sa_r = np.full((m, k // 128), sa, dtype=np.float32)
    sb_b = np.full((-(-n // 128), k // 128), sb, dtype=np.float32)
    y_b = oracle.gemm(a, oracle.E4M3, sa_r, oracle.ROW_1x128, b, oracle.E4M3, sb_b, oracle.BLOCK_128x128)
    assert np.array_equal(y_t, y_b)


def test_block_scales_index_the_right_blocks():
    """Each (row, k-block) scale of A and (n-block, k-block) scale of B must
    multiply exactly its own partial sum: perturb one scale at a time and
    check that only the matching outputs move, by the matching amount."""
    rng = np.random.default_rng(4)
    m, n, k = 3, 256, 256
    a = _finite_codes(oracle.E4M3, rng, (m, k))
    b = _finite_codes(oracle.E4M3, rng, (n, k))
    sa = np.ones((m, 2), dtype=np.float32)
    sb = np.ones((2, 2), dtype=np.float32)
    base = oracle.gemm(a, 0, sa, 1, b, 0, sb, 2)
    da, db = oracle.decode(0, a), oracle.decode(0, b)
    part = lambda kb: da[:, kb * 128:(kb + 1) * 128] @ db[:, kb * 128:(kb + 1) * 128].T
    sa2 = sa.copy(); sa2[1, 1] = 2.0
    y = oracle.gemm(a, 0, sa2, 1, b, 0, sb, 2)
    delta = y - base
    assert np.all(delta[[0, 2]] == 0)
    np.testing.assert_allclose(delta[1], part(1)[1], rtol=1e-15)
    sb2 = sb.copy(); sb2[1, 0] = 3.0
    y = oracle.gemm(a, 0, sa, 1, b, 0, sb2, 2)
    delta = y - base
    assert np.all(delta[:, :128] == 0)
    np.testing.assert_allclose(delta[:, 128:], 2 * part(0)[:, 128:], rtol=1e-15)


def test_points_match_full():
    rng = np.random.default_rng(5)
    a = _finite_codes(oracle.E5M2, rng, (50, 256))
    b = _finite_codes(oracle.E4M3, rng, (30, 256))
    y = oracle.gemm(a, oracle.E5M2, 0.1, 0, b, oracle.E4M3, 0.2, 0)
    pm = rng.integers(0, 50, 100)
    pn = rng.integers(0, 30, 100)
    yp = oracle.gemm_points(a, oracle.E5M2, 0.1, 0, b, oracle.E4M3, 0.2, 0, pm, pn)
    assert np.array_equal(yp, y[pm, pn])


def test_k_zero_and_rejects():
    a = np.zeros((4, 0), dtype=np.uint8)
    b = np.zeros((3, 0), dtype=np.uint8)
    y = oracle.gemm(a, 0, 1.0, 0, b, 0, 1.0, 0)
    assert y.shape == (4, 3) and np.all(y == 0)
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((2, 100), np.uint8), 0, np.ones((2, 1), np.float32), 1,
                    np.zeros((2, 100), np.uint8), 0, np.ones((1, 1), np.float32), 2)


def test_bf16_rne_vs_torch():
    import torch
    from fractions import Fraction
    rng = np.random.default_rng(6)
    y = rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)
    y = np.concatenate([y, [0.0, -0.0, 3.4e38, -3.4e38, 1e-45, np.inf]])
    # fp32-representable inputs: torch's fp32 -> bf16 cast is a single rounding
    y32 = y.astype(np.float32)
    ours = oracle.bf16_rne(y32.astype(np.float64))
    theirs = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    # a real value just above a bf16 midpoint whose fp32 rounding lands on the
    # midpoint: the single rounding of the real value must go up
    v = 1.4348188684738241e-08
    lo = synth.bf16_bits_to_f32(np.array([0x3276], np.uint16))[0]
    hi = synth.bf16_bits_to_f32(np.array([0x3277], np.uint16))[0]
    mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
    assert Fraction(v) > mid
    assert int(oracle.bf16_rne(np.array([v]))[0]) == 0x3277
    assert oracle.count_nonfinite_bf16(np.array([3.4e38, 3.39e38, -np.inf, 1.0])) == 2
