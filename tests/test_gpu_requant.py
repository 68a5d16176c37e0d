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


def _mixed_cache_set(count, seed):
    """`count` caches of mixed shape (whole and ragged 128x128 tiles, columns
    not a multiple of 8), format, granularity, master dtype and transposed
    copy, each with its own counters; an outlier in some masters so that
    per-block scales differ from the per-tensor one."""
    g = np.random.default_rng(seed)
    base = [(3072, 768), (768, 3072), (200, 130), (128, 256), (257, 129), (64, 100), (1, 1), (130, 7),
            (512, 640), (384, 128), (100, 300), (2304, 768)]
    specs = []
    for i in range(count):
        shp = base[i % len(base)]
        gran = fm.TENSOR if (i * 7) % 3 != 0 else fm.BLOCK_128x128
        fmt = fm.E4M3 if i % 2 == 0 else fm.E5M2
        fp32 = i % 5 == 3
        with_t = i % 4 != 1
        if fp32:
            mval = (g.standard_normal(shp) * 0.05).astype(np.float32)
            if i % 3 == 0 and mval.size > 1:
                mval.reshape(-1)[g.integers(mval.size)] = 37.5
        else:
            mval = synth.normal_bf16(400 + seed * 64 + i, 1, shp, 0.02)
            if i % 3 == 1 and mval.size > 1:
                mval.reshape(-1)[g.integers(mval.size)] = 0x4300   # 128.0
        specs.append((shp, gran, fmt, fp32, with_t, mval))
    return specs


@pytest.mark.parametrize("count", [17, 40])
def test_batched_refresh_matches_oracle(count):
    """One fp8_requant_weights call over many caches (17 fits one launch
    group, 40 spans two): every cache's codes, transposed copy, scale(s) and
    counters equal the oracle's requant of its master, bit for bit."""
    specs = _mixed_cache_set(count, count)
    caches, masters, ctrs, expect = [], [], [], []
    for shp, gran, fmt, fp32, with_t, mval in specs:
        ctr = fm.Counters()
        masters.append(dev_f32(mval) if fp32 else dev_bf16(mval))
        caches.append(fm.WeightCache(*shp, fmt=fmt, gran=gran, with_t=with_t, counters=ctr))
        ctrs.append(ctr)
        expect.append(oracle.requant(mval, fmt, gran, want_t=with_t))
    fm.requant_weights(caches, masters)
    for i, (c, ctr, (oq, oqt, os_, oc)) in enumerate(zip(caches, ctrs, expect)):
        assert np.array_equal(host(c.q), oq), f"cache {i}: codes"
        if c.q_t is not None:
            assert np.array_equal(host(c.q_t), oqt), f"cache {i}: transposed codes"
        assert np.array_equal(host(c.scale).reshape(os_.shape).view(np.uint32), os_.view(np.uint32)), \
            f"cache {i}: scales"
        got = ctr.read()
        for f in ("saturated", "underflow", "nan"):
            assert got[f] == oc[f], f"cache {i}: counter {f}"
    # a second refresh of the same masters is idempotent
    fm.requant_weights(caches, masters)
    for i, (c, (oq, _, _, _)) in enumerate(zip(caches, expect)):
        assert np.array_equal(host(c.q), oq), f"cache {i}: second refresh"


def test_batched_refresh_empty_cache():
    """An empty per-tensor cache among others reports scale 1 and leaves the
    others intact."""
    w = synth.normal_bf16(60, 1, (256, 384), 0.02)
    empty = fm.WeightCache(0, 384, with_t=True)
    empty.scale.fill_(7.0)
    full = fm.WeightCache(256, 384, fmt=fm.E5M2, with_t=True)
    fm.requant_weights([empty, full], [torch.empty((0, 384), dtype=torch.bfloat16, device="cuda"), dev_bf16(w)])
    oq, oqt, os_, _ = oracle.requant(w, fm.E5M2)
    assert host(empty.scale)[0] == 1.0
    assert np.array_equal(host(full.q), oq) and np.array_equal(host(full.q_t), oqt) and host(full.scale)[0] == os_[0]


def test_twelve_layer_refresh():
    """The up-projection caches of a 12-layer model ([3072,768] E4M3, per
    tensor, with transposed copies) refreshed in one call after an update of
    every master."""
    ws = [synth.normal_bf16(70 + l, 1, (3072, 768), 0.02) for l in range(12)]
    caches = [fm.WeightCache(3072, 768, with_t=True) for _ in ws]
    masters = [dev_bf16(w) for w in ws]
    # a prepared plan, called after each update of the masters in place
    plan = fm.RequantPlan(caches, masters)
    plan()
    for l, (c, w) in enumerate(zip(caches, ws)):
        oq, _, os_, _ = oracle.requant(w, fm.E4M3)
        assert np.array_equal(host(c.q), oq) and host(c.scale)[0] == os_[0], f"layer {l}, first refresh"
    ws2 = [synth.apply_update_bf16(w, synth.update_noise_f32(70 + l, w.shape)) for l, w in enumerate(ws)]
    for m, w2 in zip(masters, ws2):
        m.copy_(dev_bf16(w2))
    plan()
    for l, (c, w2) in enumerate(zip(caches, ws2)):
        oq, oqt, os_, _ = oracle.requant(w2, fm.E4M3)
        assert np.array_equal(host(c.q), oq) and np.array_equal(host(c.q_t), oqt), f"layer {l}"
        assert host(c.scale)[0] == os_[0], f"layer {l}"
