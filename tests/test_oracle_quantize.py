"""Pins for the oracle's amax, scale, fine-grained quantizers and the weight
cache refresh (CPU only).

Independent facts used: numpy's max over |x| (a library routine), order
independence, the scale invariant of amax scaling (the largest element lands
exactly on the format maximum, so nothing finite saturates), the reduction of
a 1x128 tile / 128x128 block quantize to a per-tensor quantize of that tile
alone, byte transposition, and requant == quantize by definition.
"""
import numpy as np
import pytest

import oracle
import synth


def _np_amax(xbits):
    f = synth.bf16_bits_to_f32(xbits)
    f = np.abs(f[np.isfinite(f)])
    return np.float32(f.max()) if f.size else np.float32(0)


def test_amax_vs_numpy_and_shuffle():
    x = synth.with_outliers_bf16(2, (512, 384))
    a = oracle.amax(x)[0]
    assert a == _np_amax(x)
    perm = np.random.default_rng(7).permutation(x.size)
    assert oracle.amax(x.reshape(-1)[perm].reshape(x.shape))[0] == a


def test_amax_ignores_nonfinite():
    x = synth.small_shape_bf16(1, (8, 128))
    x[0, 0] = 0x7F80          # +Inf
    x[1, 1] = 0xFF80          # -Inf
    x[2, 2] = 0x7FC0          # NaN
    assert oracle.amax(x)[0] == _np_amax(x)
    allbad = np.full((2, 3), 0x7FC0, dtype=np.uint16)
    assert oracle.amax(allbad)[0] == 0
    q, _, s, ctr = oracle.quantize(allbad, oracle.E4M3)
    assert s[0] == 1.0 and ctr["nan"] == 6


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_scale_invariant(fmt):
    """Under amax scaling every element with |x| = amax encodes to +-fmax,
    no finite element saturates, and codes never exceed the max code."""
    x = synth.with_outliers_bf16(2, (1024, 512))
    q, _, s, ctr = oracle.quantize(x, fmt)
    assert ctr["saturated"] == 0 and ctr["nan"] == 0
    f = synth.bf16_bits_to_f32(x)
    at_max = np.abs(f) == oracle.amax(x)[0]
    maxcode = 0x7E if fmt == oracle.E4M3 else 0x7B
    assert at_max.sum() >= 1
    assert np.all((q[at_max] & 0x7F) == maxcode)
    assert np.all((q & 0x7F) <= maxcode)
    assert s[0] == np.float32(oracle.amax(x)[0]) / np.float32(oracle.fmax(fmt))


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("shape", [(3, 128), (5, 300), (1, 1), (2, 127)])
def test_tile_quantize_is_per_tensor_per_tile(fmt, shape):
    x = synth.with_outliers_bf16(2, shape, frac=0.05)
    q, qt, s, ctr = oracle.quantize(x, fmt, oracle.ROW_1x128)
    assert qt is None
    rows, cols = shape
    nt = -(-cols // 128)
    assert s.shape == (rows, nt)
    tot = {"saturated": 0, "underflow": 0, "nan": 0}
    for r in range(rows):
        for t in range(nt):
            tile = np.ascontiguousarray(x[r:r + 1, t * 128:(t + 1) * 128])
            q1, _, s1, c1 = oracle.quantize(tile, fmt)
            assert s[r, t] == s1[0]
            assert np.array_equal(q[r:r + 1, t * 128:(t + 1) * 128], q1)
            for kk in tot:
                tot[kk] += c1[kk]
    for kk in tot:
        assert ctr[kk] == tot[kk]


@pytest.mark.parametrize("shape", [(128, 128), (200, 300), (256, 128), (7, 5)])
def test_block_quantize_is_per_tensor_per_block(shape):
    fmt = oracle.E4M3
    x = synth.with_outliers_bf16(2, shape, frac=0.01)
    q, qt, s, _ = oracle.quantize(x, fmt, oracle.BLOCK_128x128, want_t=True)
    rows, cols = shape
    assert s.shape == (-(-rows // 128), -(-cols // 128))
    assert np.array_equal(qt, q.T)
    for br in range(s.shape[0]):
        for bc in range(s.shape[1]):
            blk = np.ascontiguousarray(x[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128])
            q1, _, s1, _ = oracle.quantize(blk, fmt)
            assert s[br, bc] == s1[0]
            assert np.array_equal(q[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128], q1)


def test_given_scale_mode():
    x = synth.small_shape_bf16(3, (64, 256))
    q0, _, s0, _ = oracle.quantize(x, oracle.E4M3)
    q1, _, s1, _ = oracle.quantize(x, oracle.E4M3, oracle.TENSOR, oracle.GIVEN, scale=s0)
    assert np.array_equal(q0, q1) and s1[0] == s0[0]
    # tile-granular given scales
    st = np.full((64, 2), 0.01, dtype=np.float32)
    q2, _, _, _ = oracle.quantize(x, oracle.E4M3, oracle.ROW_1x128, oracle.GIVEN, scale=st)
    q3, _, _, _ = oracle.quantize(x, oracle.E4M3, oracle.TENSOR, oracle.GIVEN, scale=np.float32([0.01]))
    assert np.array_equal(q2, q3)


def test_transpose_is_byte_transpose():
    x = synth.small_shape_bf16(4, (33, 70))
    q, qt, _, _ = oracle.quantize(x, oracle.E5M2, want_t=True)
    assert np.array_equal(qt, q.T)


def test_fp32_master_input():
    """An fp32 master holding bf16-representable values quantizes exactly like
    the bf16 tensor."""
    xb = synth.small_shape_bf16(5, (40, 256), sigma=0.02)
    xf = synth.bf16_bits_to_f32(xb).copy()
    a = oracle.quantize(xb, oracle.E4M3, want_t=True)
    b = oracle.quantize(xf, oracle.E4M3, want_t=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2][0] == b[2][0]


def test_empty():
    x = np.zeros((0, 16), dtype=np.uint16)
    q, _, s, ctr = oracle.quantize(x, oracle.E4M3)
    assert q.shape == (0, 16) and s[0] == 1.0 and ctr["underflow"] == 0


def test_requant_cache_refresh():
    """Weight-copy cache: requant(master) is a fresh quantize; repeated refresh
    is idempotent; after an optimizer update the cache changes."""
    w = synth.normal_bf16(3, 1, (3072, 768), 0.02)
    c0 = oracle.requant(w, oracle.E4M3)
    q, qt, s, _ = oracle.quantize(w, oracle.E4M3, want_t=True)
    assert np.array_equal(c0[0], q) and np.array_equal(c0[1], qt) and c0[2][0] == s[0]
    c1 = oracle.requant(w, oracle.E4M3)
    assert np.array_equal(c0[0], c1[0]) and c0[2][0] == c1[2][0]
    w2 = synth.apply_update_bf16(w, synth.update_noise_f32(3, w.shape))
    changed_master = int((w2 != w).sum())
    assert changed_master > 0.1 * w.size
    c2 = oracle.requant(w2, oracle.E4M3)
    assert int((c2[0] != c0[0]).sum()) > 0


def test_synth_bf16_rounding_vs_torch():
    """The shared input generator's fp32->bf16 rounding equals torch's."""
    import torch
    v = (np.random.default_rng(0).standard_normal(100000) * 3).astype(np.float32)
    v[:4] = [np.inf, -np.inf, 3.3895314e38, -0.0]
    ours = synth.f32_to_bf16_bits(v)
    theirs = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
