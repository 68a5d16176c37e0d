"""GPU parity of the FP8 weight-copy cache refresh: after every optimizer
step the cache equals a fresh quantize of the master, byte for byte, and the
oracle's requant of the same master."""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu


def test_speedrun_weight_cache_refresh():
    """W [3072,768] bf16 master, E4M3 per-tensor cache with transposed copy;
    refresh, apply W <- bf16(fp32(W) + N(0,1e-4)), refresh again."""
    w = synth.normal_bf16(3, 1, synth.SPEEDRUN_UP_PROJ["w"], 0.02)
    cache = fm.WeightCache(*w.shape, fmt=fm.E4M3, gran=fm.TENSOR, with_t=True)
    master = dev_bf16(w)
    fm.requant_weights([cache], [master])
    oq, oqt, os_, _ = oracle.requant(w, fm.E4M3)
    assert np.array_equal(host(cache.q), oq) and np.array_equal(host(cache.q_t), oqt)
    assert host(cache.scale)[0] == os_[0]
    before = host(cache.q).copy()
    w2 = synth.apply_update_bf16(w, synth.update_noise_f32(3, w.shape))
    master.copy_(dev_bf16(w2))
    fm.requant_weights([cache], [master])
    oq2, oqt2, os2, _ = oracle.requant(w2, fm.E4M3)
    assert np.array_equal(host(cache.q), oq2) and np.array_equal(host(cache.q_t), oqt2)
    assert host(cache.scale)[0] == os2[0]
    assert int((host(cache.q) != before).sum()) > 0
    # refreshing again without an update changes nothing
    fm.requant_weights([cache], [master])
    assert np.array_equal(host(cache.q), oq2)


def test_many_caches_mixed():
    """Several caches in one call: bf16 and fp32 masters, TENSOR and
    BLOCK_128x128, with and without the transposed copy."""
    g = np.random.default_rng(1)
    shapes = [(3072, 768), (768, 3072), (200, 130), (128, 256)]
    caches, masters, expect = [], [], []
    for i, shp in enumerate(shapes):
        gran = fm.TENSOR if i % 2 == 0 else fm.BLOCK_128x128
        fmt = fm.E4M3 if i < 2 else fm.E5M2
        if i == 2:
            mval = (g.standard_normal(shp) * 0.05).astype(np.float32)
            masters.append(dev_f32(mval))
        else:
            mval = synth.normal_bf16(50 + i, 1, shp, 0.02)
            masters.append(dev_bf16(mval))
        caches.append(fm.WeightCache(*shp, fmt=fmt, gran=gran, with_t=(i != 3)))
        expect.append(oracle.quantize(mval, fmt, gran, oracle.FROM_AMAX, None, i != 3))
    fm.requant_weights(caches, masters)
    for c, (oq, oqt, os_, _) in zip(caches, expect):
        assert np.array_equal(host(c.q), oq)
        if c.q_t is not None:
            assert np.array_equal(host(c.q_t), oqt)
        assert np.array_equal(host(c.scale).reshape(os_.shape), os_)


def test_cache_equals_quantize():
    w = synth.normal_bf16(9, 1, (1024, 512), 0.02)
    master = dev_bf16(w)
    cache = fm.WeightCache(1024, 512, with_t=True)
    fm.requant_weights([cache], [master])
    q, qt, s = fm.quantize(master, fm.E4M3, want_t=True)
    assert torch.equal(q, cache.q) and torch.equal(qt, cache.q_t) and torch.equal(s, cache.scale)
