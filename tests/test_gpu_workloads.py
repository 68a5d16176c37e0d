"""Full-size parity of the training-step workloads against the oracle, in the
buffer layout the benchmark times.

Every FP8 operand the HIP path produces (codes, transposed copies, scales,
counters) is compared byte for byte with the oracle's quantization of the
same bf16 input, and every output element of every full-size GEMM is
compared with the oracle's fp64 GEMM computed from the ORACLE's codes and
scales, to max|y - y_ref| <= 1e-2 max|y_ref| and relative Frobenius error
<= 5e-3.  No value on the reference side comes from the GPU.

Layouts (as in bench.py): the transposed copies of X and dY have 65536-byte
rows padded to a leading dimension of 65536 + 256 (the padding must stay
untouched); W lives in a weight cache refreshed by fp8_requant_weights (its
transposed copy is the dX operand); dW runs with its split-K workspace.
"""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import oracle
import synth
from gpu_util import assert_gemm_close, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu

TOK, D, F = synth.SPEEDRUN_UP_PROJ["x"][0], synth.SPEEDRUN_UP_PROJ["x"][1], synth.SPEEDRUN_UP_PROJ["w"][0]
LD_PAD = 256
SENTINEL = 0xA5


def _padded_t(cols, rows):
    """[cols, rows] uint8 view of a [cols, rows + LD_PAD] buffer whose padding
    holds SENTINEL."""
    full = torch.full((cols, rows + LD_PAD), SENTINEL, dtype=torch.uint8, device="cuda")
    return full, full[:, :rows]


def _same_quant(gq, gqt, gs, gc, oq, oqt, os_, oc, what):
    assert np.array_equal(gq, oq), f"{what}: codes differ from the oracle"
    if oqt is not None:
        assert np.array_equal(gqt, oqt), f"{what}: transposed codes differ from the oracle"
    assert np.array_equal(np.asarray(gs, np.float32).view(np.uint32),
                          np.asarray(os_, np.float32).reshape(np.shape(gs)).view(np.uint32)), \
        f"{what}: scales differ from the oracle"
    for f in ("saturated", "underflow", "nan"):
        assert gc[f] == oc[f], f"{what}: counter {f} {gc[f]} != oracle {oc[f]}"


@pytest.fixture(scope="module")
def up_proj():
    """X [65536,768] and W [3072,768] of the speedrun up-projection, their
    oracle quantization (E4M3, per-tensor amax scale, transposed copies), and
    the GPU's quantization in the benchmark's layout."""
    x = synth.normal_bf16(3, 0, (TOK, D), 1.0)
    w = synth.normal_bf16(3, 1, (F, D), 0.02)
    o = {}
    o["xq"], o["xqt"], o["xs"], o["xc"] = oracle.quantize(x, oracle.E4M3, want_t=True)
    o["wq"], o["wqt"], o["ws"], o["wc"] = oracle.quantize(w, oracle.E4M3, want_t=True)

    g = {}
    ctr = fm.Counters()
    xfull, xqt = _padded_t(D, TOK)
    xq, _, xs = fm.quantize(dev_bf16(x), fm.E4M3, fm.TENSOR, want_t=True, counters=ctr, out_t=xqt)
    torch.cuda.synchronize()
    g["x_ctr"] = ctr.read()
    g["xq"], g["xqt"], g["xs"], g["xfull"] = xq, xqt, xs, xfull
    wctr = fm.Counters()
    cache = fm.WeightCache(F, D, fm.E4M3, fm.TENSOR, with_t=True, counters=wctr)
    w_dev = dev_bf16(w)
    fm.requant_weights([cache], [w_dev])
    torch.cuda.synchronize()
    g["w_ctr"] = wctr.read()
    g["cache"] = cache
    yield o, g
    del g
    torch.cuda.empty_cache()


def test_x_quantize_full(up_proj):
    """X E4M3 per-tensor with its transposed copy at ld 65536 + 256."""
    o, g = up_proj
    _same_quant(host(g["xq"]), host(g["xqt"].contiguous()), host(g["xs"]), g["x_ctr"],
                o["xq"], o["xqt"], o["xs"], o["xc"], "X [65536,768]")
    assert bool((g["xfull"][:, TOK:] == SENTINEL).all()), "X^T padding was written"


def test_w_cache_full(up_proj):
    """The weight cache (codes, transposed copy, scale) equals the oracle's
    quantization of the master."""
    o, g = up_proj
    c = g["cache"]
    _same_quant(host(c.q), host(c.q_t), host(c.scale), g["w_ctr"], o["wq"], o["wqt"], o["ws"], o["wc"],
                "W cache [3072,768]")


def test_forward_gemm_full(up_proj):
    """y = X W^T [65536,3072]: every output element against the oracle."""
    o, g = up_proj
    ctr = fm.Counters()
    c = g["cache"]
    y = host(fm.scaled_mm(g["xq"], fm.E4M3, g["xs"], fm.TENSOR, c.q, fm.E4M3, c.scale, fm.TENSOR, counters=ctr))
    assert ctr.read()["nonfinite_out"] == 0
    ref = oracle.gemm(o["xq"], 0, o["xs"], 0, o["wq"], 0, o["ws"], 0)
    assert_gemm_close(y, ref, "forward 65536x3072x768")


@pytest.fixture(scope="module")
def backward(up_proj):
    """dY [65536,3072] ~N(0,1e-3): the oracle's E5M2 quantization with its
    transposed copy, and the GPU's in the benchmark's layout."""
    dy = synth.normal_bf16(5, 0, synth.UP_PROJ_BACKWARD["dy"], 1e-3)
    o = {}
    o["q"], o["qt"], o["s"], o["c"] = oracle.quantize(dy, oracle.E5M2, want_t=True)
    ctr = fm.Counters()
    full, qt = _padded_t(F, TOK)
    q, _, s = fm.quantize(dev_bf16(dy), fm.E5M2, fm.TENSOR, want_t=True, counters=ctr, out_t=qt)
    torch.cuda.synchronize()
    g = {"q": q, "qt": qt, "s": s, "full": full, "ctr": ctr.read()}
    del dy
    yield o, g
    del g
    torch.cuda.empty_cache()


def test_dy_quantize_full(backward):
    """dY E5M2 per-tensor with its transposed copy [3072,65536] at ld 65536 + 256."""
    o, g = backward
    _same_quant(host(g["q"]), host(g["qt"].contiguous()), host(g["s"]), g["ctr"], o["q"], o["qt"], o["s"], o["c"],
                "dY [65536,3072]")
    assert bool((g["full"][:, TOK:] == SENTINEL).all()), "dY^T padding was written"


def test_dx_gemm_full(up_proj, backward):
    """dX = dY W [65536,768] (E5M2 x E4M3, B = the cache's transposed copy)."""
    ou, gu = up_proj
    ob, gb = backward
    c = gu["cache"]
    ctr = fm.Counters()
    dx = host(fm.scaled_mm(gb["q"], fm.E5M2, gb["s"], fm.TENSOR, c.q_t, fm.E4M3, c.scale, fm.TENSOR, counters=ctr))
    assert ctr.read()["nonfinite_out"] == 0
    ref = oracle.gemm(ob["q"], 1, ob["s"], 0, ou["wqt"], 0, ou["ws"], 0)
    assert_gemm_close(dx, ref, "dX 65536x768x3072")


def test_dw_gemm_full(up_proj, backward):
    """dW = dY^T X [3072,768] with K = 65536 split over the workspace; both
    operands are the padded transposed copies."""
    ou, gu = up_proj
    ob, gb = backward
    assert fm.lib().fp8_scaled_mm_workspace_size(F, D, TOK, 0, 0) > 0
    ctr = fm.Counters()
    dw = host(fm.scaled_mm(gb["qt"], fm.E5M2, gb["s"], fm.TENSOR, gu["xqt"], fm.E4M3, gu["xs"], fm.TENSOR,
                           counters=ctr))
    assert ctr.read()["nonfinite_out"] == 0
    ref = oracle.gemm(ob["qt"], 1, ob["s"], 0, ou["xqt"], 0, ou["xs"], 0)
    assert_gemm_close(dw, ref, "dW 3072x768x65536")


@pytest.fixture(scope="module")
def fine():
    """A [16384,7168] and B [2048,7168], N(0,1) with 1% of K channels x100:
    the oracle's 1x128 / 128x128 quantization with fp32 scales, and the GPU's."""
    a = synth.channel_scaled_bf16(4, 0, 3, synth.BLOCK_SCALED["a"])
    b = synth.channel_scaled_bf16(4, 1, 4, synth.BLOCK_SCALED["b"])
    o = {}
    o["aq"], _, o["sa"], o["ac"] = oracle.quantize(a, oracle.E4M3, oracle.ROW_1x128)
    o["bq"], _, o["sb"], o["bc"] = oracle.quantize(b, oracle.E4M3, oracle.BLOCK_128x128)
    actr, bctr = fm.Counters(), fm.Counters()
    aq, _, sa = fm.quantize(dev_bf16(a), fm.E4M3, fm.ROW_1x128, counters=actr)
    bq, _, sb = fm.quantize(dev_bf16(b), fm.E4M3, fm.BLOCK_128x128, counters=bctr)
    torch.cuda.synchronize()
    g = {"aq": aq, "sa": sa, "bq": bq, "sb": sb, "ac": actr.read(), "bc": bctr.read()}
    yield o, g
    del g
    torch.cuda.empty_cache()


def test_fine_quantize_full(fine):
    """A 1x128 tiles (917,504 fp32 scales) and B 128x128 blocks (896 fp32
    scales): codes, scales and counters."""
    o, g = fine
    _same_quant(host(g["aq"]), None, host(g["sa"]), g["ac"], o["aq"], None, o["sa"], o["ac"], "A 1x128")
    _same_quant(host(g["bq"]), None, host(g["sb"]), g["bc"], o["bq"], None, o["sb"], o["bc"], "B 128x128")


def test_block_scaled_gemm_full(fine):
    """y = sum_kb s_a s_b (A B^T)_kb [16384,2048], K = 7168: every element."""
    o, g = fine
    ctr = fm.Counters()
    y = host(fm.scaled_mm(g["aq"], fm.E4M3, g["sa"], fm.ROW_1x128, g["bq"], fm.E4M3, g["sb"], fm.BLOCK_128x128,
                          counters=ctr))
    assert ctr.read()["nonfinite_out"] == 0
    ref = oracle.gemm(o["aq"], 0, o["sa"], 1, o["bq"], 0, o["sb"], 2)
    assert_gemm_close(y, ref, "block-scaled 16384x2048x7168")


def test_block_scaled_pow2_gemm_full():
    """The same workload with power-of-two scales (the MFMA applies them as
    E8M0 exponents): GPU codes and scales equal the oracle's power-of-two
    quantization, and every output element is within tolerance of the oracle
    GEMM on those codes."""
    a = synth.channel_scaled_bf16(4, 0, 3, synth.BLOCK_SCALED["a"])
    b = synth.channel_scaled_bf16(4, 1, 4, synth.BLOCK_SCALED["b"])
    oaq, _, osa, _ = oracle.quantize_pow2(a, oracle.E4M3, oracle.ROW_1x128)
    obq, _, osb, _ = oracle.quantize_pow2(b, oracle.E4M3, oracle.BLOCK_128x128)
    aq, _, sa = fm.quantize(dev_bf16(a), fm.E4M3, fm.ROW_1x128, fm.FROM_AMAX_POW2)
    bq, _, sb = fm.quantize(dev_bf16(b), fm.E4M3, fm.BLOCK_128x128, fm.FROM_AMAX_POW2)
    del a, b
    assert np.array_equal(host(aq), oaq) and np.array_equal(host(sa), osa)
    assert np.array_equal(host(bq), obq) and np.array_equal(host(sb), osb)
    y = host(fm.scaled_mm(aq, fm.E4M3, sa, fm.ROW_1x128_POW2, bq, fm.E4M3, sb, fm.BLOCK_128x128_POW2))
    ref = oracle.gemm(oaq, 0, osa, 1, obq, 0, osb, 2)
    assert_gemm_close(y, ref, "block-scaled pow2 16384x2048x7168")


def test_small_up_projection_full():
    """X [256,768], W [3072,768]: GPU codes equal the oracle's, every output
    element against the oracle GEMM on the oracle's codes."""
    x = synth.normal_bf16(1, 0, synth.SMALL_UP_PROJ["x"], 1.0)
    w = synth.normal_bf16(1, 1, synth.SMALL_UP_PROJ["w"], 0.02)
    oxq, _, oxs, _ = oracle.quantize(x, 0)
    owq, _, ows, _ = oracle.quantize(w, 0)
    xq, _, xs = fm.quantize(dev_bf16(x), fm.E4M3)
    wq, _, ws = fm.quantize(dev_bf16(w), fm.E4M3)
    assert np.array_equal(host(xq), oxq) and np.array_equal(host(wq), owq)
    assert host(xs)[0] == oxs[0] and host(ws)[0] == ows[0]
    y = host(fm.scaled_mm(xq, 0, xs, 0, wq, 0, ws, 0))
    assert_gemm_close(y, oracle.gemm(oxq, 0, oxs, 0, owq, 0, ows, 0), "up-proj 256")
    # the same GEMM from the oracle's codes uploaded directly
    y2 = host(fm.scaled_mm(torch.from_numpy(oxq).cuda(), 0, dev_f32(oxs), 0, torch.from_numpy(owq).cuda(), 0,
                           dev_f32(ows), 0))
    assert np.array_equal(y, y2)
