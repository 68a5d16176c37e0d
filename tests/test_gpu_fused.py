"""GPU parity of the A-stationary GEMM (per-tensor, K = 768): plain FP8
operands through fp8_scaled_mm, and fp8_quantize_scaled_mm, which quantizes
its bf16 activation on the way in.  Codes, transposed codes, scale and
counters of the fused call are compared byte for byte with the oracle's
quantization of x; every output element with the oracle GEMM on the
oracle's codes (max|y - y_ref| <= 1e-2 max|y_ref|, relative Frobenius
<= 5e-3)."""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import oracle
import synth
from gpu_util import assert_gemm_close, dev_bf16, dev_f32, dev_u8, host

pytestmark = pytest.mark.gpu
K = 768
PAIRS = [(fm.E4M3, fm.E4M3), (fm.E5M2, fm.E4M3), (fm.E4M3, fm.E5M2), (fm.E5M2, fm.E5M2)]


def _fused(x_bits, fa, bq, fb, sb, want_q=True, want_t=True, ld_pad=0):
    m = x_bits.shape[0]
    ctr = fm.Counters()
    full_t = None
    out_t = None
    if want_t:
        full_t = torch.full((K, m + ld_pad), 0xA5, dtype=torch.uint8, device="cuda")
        out_t = full_t[:, :m]
    y, sa, xq, xqt = fm.quantize_scaled_mm(dev_bf16(x_bits), fa, dev_u8(bq), fb, dev_f32(np.asarray(sb, np.float32)),
                                           want_q=want_q, counters=ctr, out_t=out_t)
    torch.cuda.synchronize()
    return host(y), host(sa), (host(xq) if xq is not None else None), \
        (host(xqt.contiguous()) if xqt is not None else None), ctr.read(), full_t


def _check_fused(x_bits, fa, bq, fb, sb, what, ld_pad=0):
    oq, oqt, os_, oc = oracle.quantize(x_bits, fa, want_t=True)
    y, sa, xq, xqt, c, full_t = _fused(x_bits, fa, bq, fb, sb, ld_pad=ld_pad)
    assert np.array_equal(sa.view(np.uint32), os_.view(np.uint32)), f"{what}: scale"
    assert np.array_equal(xq, oq), f"{what}: codes"
    assert np.array_equal(xqt, oqt), f"{what}: transposed codes"
    for f in ("saturated", "underflow", "nan"):
        assert c[f] == oc[f], f"{what}: counter {f} {c[f]} != {oc[f]}"
    if ld_pad:
        assert bool((full_t[:, x_bits.shape[0]:] == 0xA5).all()), f"{what}: transposed padding written"
    ref = oracle.gemm(oq, fa, os_, 0, bq, fb, sb, 0)
    if np.isfinite(ref).all():
        assert_gemm_close(y, ref, what)
    return y, c


def _wcodes(fb, n, seed, sigma=0.02):
    w = synth.normal_bf16(500 + seed, 1, (n, K), sigma)
    q, _, s, _ = oracle.quantize(w, fb)
    return q, s


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("m,n", [(1, 8), (191, 136), (192, 256), (193, 264), (500, 3072), (1000, 16)])
def test_fused_shapes(fa, fb, m, n):
    """Ragged panels (m not a multiple of 192) and column units (n not a
    multiple of 128), every format pair."""
    x = synth.normal_bf16(600 + m, 0, (m, K), 1.0)
    bq, sb = _wcodes(fb, n, m + n)
    _check_fused(x, fa, bq, fb, sb, f"fused {fa}x{fb} {m}x{n}")


def test_fused_outliers_and_units_spanning_panels():
    """More panels than workgroups hold whole (units of one panel split
    between two workgroups): X [4000, 768] with 0.1% outliers; the codes of
    every panel are written once and counted once."""
    x = synth.with_outliers_bf16(601, (4000, K))
    bq, sb = _wcodes(fm.E4M3, 3072, 7)
    _check_fused(x, fm.E4M3, bq, fm.E4M3, sb, "fused outliers 4000")


@pytest.mark.parametrize("fa", [fm.E4M3, fm.E5M2])
def test_fused_nonfinite_inputs(fa):
    """NaN and +-Inf elements take the IEEE-division cast with every counter
    (NaN codes, saturation of Inf), exactly as fp8_quantize."""
    x = synth.normal_bf16(602, 0, (300, K), 1.0).copy()
    x[3, 5] = 0x7FC0          # NaN
    x[100, 700] = 0xFF80      # -Inf
    x[299, 0] = 0x7F80        # +Inf
    x[150, 17] = 0x0001       # a bf16 subnormal
    bq, sb = _wcodes(fm.E4M3, 256, 8)
    oq, oqt, os_, oc = oracle.quantize(x, fa, want_t=True)
    assert oc["nan"] == 1 and oc["saturated"] == 2
    y, sa, xq, xqt, c, _ = _fused(x, fa, bq, fm.E4M3, sb)
    assert np.array_equal(sa.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(xq, oq) and np.array_equal(xqt, oqt)
    for f in ("saturated", "underflow", "nan"):
        assert c[f] == oc[f], f
    # rows without a non-finite code: the GEMM on the oracle's codes
    ref = oracle.gemm(oq, fa, os_, 0, bq, fm.E4M3, sb, 0)
    ok = np.isfinite(ref).all(axis=1)
    assert_gemm_close(y[ok], ref[ok], "fused non-finite rows excluded")


def test_fused_outputs_optional_and_degenerate():
    """No codes requested (the product alone); n == 0 (codes only); m == 0
    (scale 1)."""
    x = synth.normal_bf16(603, 0, (400, K), 1.0)
    bq, sb = _wcodes(fm.E4M3, 256, 9)
    oq, oqt, os_, _ = oracle.quantize(x, fm.E4M3, want_t=True)
    y, sa, xq, xqt, _, _ = _fused(x, fm.E4M3, bq, fm.E4M3, sb, want_q=False, want_t=False)
    assert xq is None and xqt is None and sa[0] == os_[0]
    assert_gemm_close(y, oracle.gemm(oq, 0, os_, 0, bq, 0, sb, 0), "fused, no codes out")
    b0 = np.zeros((0, K), np.uint8)
    y, sa, xq, xqt, c, _ = _fused(x, fm.E4M3, b0, fm.E4M3, [1.0])
    assert y.shape == (400, 0) and sa[0] == os_[0]
    assert np.array_equal(xq, oq) and np.array_equal(xqt, oqt)
    x0 = np.zeros((0, K), np.uint16)
    ctr = fm.Counters()
    y, sa, _, _ = fm.quantize_scaled_mm(dev_bf16(x0), fm.E4M3, dev_u8(bq), fm.E4M3, dev_f32(np.asarray(sb)),
                                        counters=ctr)
    torch.cuda.synchronize()
    assert y.shape == (0, 256) and host(sa)[0] == 1.0


def test_fused_rejects_unsupported():
    x = torch.zeros((64, 512), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((64, 512), dtype=torch.uint8, device="cuda")
    one = torch.ones(1, dtype=torch.float32, device="cuda")
    with pytest.raises(fm.Fp8Error, match="768"):
        fm.quantize_scaled_mm(x, fm.E4M3, b, fm.E4M3, one)
    x = torch.zeros((64, K), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((63, K), dtype=torch.uint8, device="cuda")
    with pytest.raises(fm.Fp8Error, match="multiples of 4"):
        fm.quantize_scaled_mm(x, fm.E4M3, b, fm.E4M3, one)


def test_fused_speedrun_forward_full():
    """X [65536, 768] ~N(0,1), W [3072, 768] ~N(0,0.02) (the weight cache's
    codes), E4M3: scale, codes, transposed codes (ld 65536 + 256, padding
    untouched), counters and every output element against the oracle."""
    x = synth.normal_bf16(3, 0, synth.SPEEDRUN_UP_PROJ["x"], 1.0)
    w = synth.normal_bf16(3, 1, synth.SPEEDRUN_UP_PROJ["w"], 0.02)
    wq, _, ws, _ = oracle.quantize(w, fm.E4M3)
    y, c = _check_fused(x, fm.E4M3, wq, fm.E4M3, ws, "fused forward 65536x3072x768", ld_pad=256)
    assert c["nonfinite_out"] == 0


@pytest.mark.parametrize("fa,fb", PAIRS)
@pytest.mark.parametrize("m,n", [(1, 8), (191, 16), (193, 136), (207, 24), (208, 256), (209, 260), (417, 132),
                                 (1000, 264), (2500, 1024), (300, 260), (64, 258), (256, 3072), (500, 3072), (700, 3072)])
def test_scaled_mm_k768_shapes(fa, fb, m, n):
    """fp8_scaled_mm with per-tensor scales and K = 768 (the A-stationary
    kernel): ragged panels and column units, every format pair.  Short A
    (every unit of 32 rows x 128 columns in one round: 500 x 3072 is 384
    units, 256 x 3072 192) takes that form, longer A 208-row panels and
    256-column units (500 x 3072, 700 x 3072, 2500 x 1024)."""
    g = np.random.default_rng(m * 3 + n)
    a = synth.f32_to_bf16_bits((g.standard_normal((m, K))).astype(np.float32))
    aq, _, sa, _ = oracle.quantize(a, fa)
    bq, sb = _wcodes(fb, n, 2 * m + n)
    y = host(fm.scaled_mm(dev_u8(aq), fa, dev_f32(sa), fm.TENSOR, dev_u8(bq), fb, dev_f32(sb), fm.TENSOR))
    assert_gemm_close(y, oracle.gemm(aq, fa, sa, 0, bq, fb, sb, 0), f"k768 {fa}x{fb} {m}x{n}")


def test_scaled_mm_k768_units_spanning_panels():
    """More column units than workgroups (units of one panel split between
    two workgroups, which both load it): A [8000, 768] with 0.1% outliers,
    E4M3 x E4M3, every output element against the oracle."""
    x = synth.with_outliers_bf16(604, (8000, K))
    aq, _, sa, _ = oracle.quantize(x, fm.E4M3)
    bq, sb = _wcodes(fm.E4M3, 3072, 13)
    y = host(fm.scaled_mm(dev_u8(aq), 0, dev_f32(sa), 0, dev_u8(bq), 0, dev_f32(sb), 0))
    assert_gemm_close(y, oracle.gemm(aq, 0, sa, 0, bq, 0, sb, 0), "k768 8000x3072")


def test_scaled_mm_k768_strided_and_odd_n():
    """Strided operands and output (padding untouched), and an odd n, which
    the A-stationary kernel does not take (it falls back)."""
    g = np.random.default_rng(11)
    m, n = 400, 300
    a = synth.f32_to_bf16_bits(g.standard_normal((m, K + 64)).astype(np.float32))
    aq, _, sa, _ = oracle.quantize(a, fm.E4M3)
    bq, sb = _wcodes(fm.E4M3, n, 12)
    bpad = np.zeros((n, K + 32), np.uint8)
    bpad[:, :K] = bq
    out = torch.full((m, n + 10), 1.0, dtype=torch.bfloat16, device="cuda")
    fm.scaled_mm(dev_u8(aq)[:, :K], 0, dev_f32(sa), 0, dev_u8(bpad)[:, :K], 0, dev_f32(sb), 0, out=out[:, :n])
    yy = host(out)
    ref = oracle.gemm(np.ascontiguousarray(aq[:, :K]), 0, sa, 0, bq, 0, sb, 0)
    assert_gemm_close(yy[:, :n], ref, "k768 strided")
    assert np.all(yy[:, n:] == 0x3F80), "wrote past n"
    y = host(fm.scaled_mm(dev_u8(np.ascontiguousarray(aq[:, :K])), 0, dev_f32(sa), 0, dev_u8(bq[:299]), 0,
                          dev_f32(sb), 0))
    assert_gemm_close(y, ref[:, :299], "k768 odd n")


def test_scaled_mm_k768_nonfinite_output_counter():
    """Outputs that overflow bf16 are counted exactly (read back)."""
    a = np.full((200, K), 0x7E, np.uint8)
    b = np.full((132, K), 0x7E, np.uint8)
    ctr = fm.Counters()
    y = host(fm.scaled_mm(dev_u8(a), 0, dev_f32(np.array([1e30], np.float32)), 0, dev_u8(b), 0,
                          dev_f32(np.array([1e3], np.float32)), 0, counters=ctr))
    assert ctr.read()["nonfinite_out"] == 200 * 132
    assert np.all((y & 0x7FFF) == 0x7F80)


def test_scaled_mm_k768_nonfinite_rows_at_panel_edges():
    """208-row panels, 480 units of 256 columns (about two per workgroup, so a
    unit's last fragment is stored both inside a panel and at a panel switch):
    rows that overflow bf16 at the panel edges are counted exactly, and the
    other rows stay zero."""
    m, n = 208 * 40, 3072
    a = np.zeros((m, K), np.uint8)
    bad = [0, 191, 192, 207, 208, 415, 416, 4159, 4160, m - 1]
    a[bad] = 0x7E
    b = np.full((n, K), 0x7E, np.uint8)
    ctr = fm.Counters()
    y = host(fm.scaled_mm(dev_u8(a), 0, dev_f32(np.array([1e30], np.float32)), 0, dev_u8(b), 0,
                          dev_f32(np.array([1e3], np.float32)), 0, counters=ctr))
    assert ctr.read()["nonfinite_out"] == len(bad) * n
    assert np.all((y[bad] & 0x7FFF) == 0x7F80)
    good = np.ones(m, bool)
    good[bad] = False
    assert np.all(y[good] == 0)
