"""GPU parity of the quantizers against the oracle: bytes, scales and counters
bit-exact, on every bf16 bit pattern, on many amax-derived scales, on ragged,
strided and empty shapes, and on the full 8192 x 8192 quantize workload."""
import numpy as np
import pytest
import torch

import fp8_scaled_matmul_amd as fm
import oracle
import synth
from gpu_util import dev_bf16, dev_f32, gpu_quantize, host, same_counters

pytestmark = pytest.mark.gpu
FMTS = [fm.E4M3, fm.E5M2]
SCALES = [1.0, 2.0 ** -10, 0.5, 3.0, 1.0 / 448.0, 1.0 / 57344.0, 4.5 / 448.0, 5000.0 / 448.0,
          5000.0 / 57344.0, 0.0213 / 448.0, 1.1920929e-7, 7.3e-3, 1e-30, 3e30,
          # arbitrary significands, and the ends of the corrected quotient's range
          # for a given scale ([2^-64, 2^64]) with a step beyond each
          0.7853982, 1.9999999, 2.0 ** -64, 2.0 ** -64 * 0.99999994, 2.0 ** 64, 2.0 ** 64 * 1.0000001]


def _cmp(x_bits, fmt, gran, mode=fm.FROM_AMAX, scale=None, want_t=False, x_dev=None, x_orc=None):
    xd = x_dev if x_dev is not None else dev_bf16(x_bits)
    q, qt, s, c = gpu_quantize(xd, fmt, gran, mode, scale, want_t)
    oq, oqt, os_, oc = oracle.quantize(x_orc if x_orc is not None else x_bits, fmt, gran, mode, scale, want_t)
    assert np.array_equal(s.reshape(os_.shape), os_), "scales differ"
    bad = np.nonzero(q != oq)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}: gpu {q[bad][0]:#x} oracle {oq[bad][0]:#x}"
    if want_t:
        assert np.array_equal(qt, oqt), "transposed codes differ"
    assert same_counters(c, oc), f"counters gpu {c} oracle {oc}"
    return c


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("s", SCALES)
def test_every_bf16_pattern_given_scale(fmt, s):
    x = synth.all_bf16_patterns()
    _cmp(x, fmt, fm.TENSOR, fm.GIVEN, np.float32([s]))
    _cmp(x, fmt, fm.TENSOR, fm.GIVEN, np.float32([s]), want_t=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", [fm.TENSOR, fm.BLOCK_128x128])
def test_given_scale_saturating_outliers(fmt, gran):
    """A given scale (or per-block scales) below amax / fmax on a tensor
    with 1% outliers of 500-5000: elements past the scale's limit saturate
    and are counted, the rest take the corrected quotient; codes, transposed
    codes and counters bit-exact.  Whole tiles and ragged edges."""
    x = synth.with_outliers_bf16(7, (1000, 1408), frac=0.01)
    g = np.random.default_rng(8)
    if gran == fm.TENSOR:
        sc = np.float32([(200.0 if fmt == fm.E4M3 else 0.05) * g.uniform(0.5, 2.0)]) / np.float32(448.0)
    else:
        sc = (g.uniform(0.2, 2.0, size=oracle.scale_shape(2, *x.shape)) *
              (1.0 if fmt == fm.E4M3 else 0.001)).astype(np.float32)
    c = _cmp(x, fmt, gran, fm.GIVEN, sc)
    _cmp(x, fmt, gran, fm.GIVEN, sc, want_t=True)
    assert c["saturated"] > 0


@pytest.mark.parametrize("fmt", FMTS)
def test_every_bf16_pattern_from_amax(fmt):
    """With Inf/NaN present the kernels take the general branch."""
    _cmp(synth.all_bf16_patterns(), fmt, fm.TENSOR)


AMAXES = [0x7F7F, 0x7F00, 0x4700, 0x43E0, 0x3F80, 0x3C00, 0x2000, 0x1F80, 0x0100, 0x0080, 0x0040, 0x0001]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("amax_bits", AMAXES)
def test_from_amax_every_finite_pattern_below_amax(fmt, amax_bits):
    """Fast branch (finite inputs): every bf16 pattern with |x| <= amax."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mag = pats & 0x7FFF
    x = pats[mag <= amax_bits]
    pad = (-x.size) % 256
    x = np.concatenate([x, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 256)
    _cmp(x, fmt, fm.TENSOR)
    _cmp(x, fmt, fm.TENSOR, want_t=True)


@pytest.mark.parametrize("fmt", FMTS)
def test_row_tiles_thousands_of_scales(fmt):
    """Each 1x128 tile has its own amax, spread over the whole bf16 range, so
    one call exercises thousands of scales."""
    g = np.random.default_rng(11)
    rows, tiles = 512, 12
    x = g.integers(0, 65536, size=(rows, tiles * 128)).astype(np.uint16)
    exp = g.integers(1, 0xFF, size=(rows, tiles, 1)).astype(np.uint16)
    xs = x.reshape(rows, tiles, 128)
    xs = (xs & 0x807F) | (np.minimum(exp, ((xs >> 7) & 0xFF)) << 7).astype(np.uint16)
    x = xs.reshape(rows, tiles * 128)
    _cmp(x, fmt, fm.ROW_1x128)
    # with a few non-finite values sprinkled in (general branch for those tiles)
    x2 = x.copy()
    x2[g.integers(0, rows, 40), g.integers(0, tiles * 128, 40)] = 0x7F80
    x2[g.integers(0, rows, 40), g.integers(0, tiles * 128, 40)] = 0xFFC1
    _cmp(x2, fmt, fm.ROW_1x128)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols", [(1024 + 40, 1536 + 72), (4224 + 40, 4160 + 72)])
def test_block_tiles_thousands_of_scales(fmt, rows, cols):
    """Each 128x128 block has its own amax over the whole bf16 range (full
    blocks plus a ragged edge, with and without the transposed copy), then
    Inf and NaN in a few blocks: scales, codes and counters exact.  96 full
    blocks take one workgroup each; 1056 (more than four per CU) are walked
    by fewer workgroups, each loading its next block ahead."""
    g = np.random.default_rng(12)
    x = g.integers(0, 65536, size=(rows, cols)).astype(np.uint16)
    br, bc = np.arange(rows)[:, None] // 128, np.arange(cols)[None, :] // 128
    cap = g.integers(1, 0xFF, size=(rows // 128 + 1, cols // 128 + 1)).astype(np.uint16)[br, bc]
    x = (x & 0x807F) | (np.minimum(cap, (x >> 7) & 0xFF) << 7).astype(np.uint16)
    _cmp(x, fmt, fm.BLOCK_128x128)
    _cmp(x, fmt, fm.BLOCK_128x128, want_t=True)
    x2 = x.copy()
    x2[g.integers(0, rows, 30), g.integers(0, cols, 30)] = 0x7F80
    x2[g.integers(0, rows, 30), g.integers(0, cols, 30)] = 0xFFC1
    x2[5, 7] = 0xFF80
    _cmp(x2, fmt, fm.BLOCK_128x128)
    _cmp(x2, fmt, fm.BLOCK_128x128, want_t=True)


def test_block_strided_full_tiles():
    """Full 128x128 blocks of a strided input into a strided output: the
    padding of the output is never written."""
    x_full = synth.with_outliers_bf16(13, (300, 600), frac=0.01)
    x = dev_bf16(x_full)[:, 8:520]            # ld 600, cols 512
    xo = np.ascontiguousarray(x_full[:, 8:520])
    out = torch.full((300, 544), 0xAA, dtype=torch.uint8, device="cuda")
    ctr = fm.Counters()
    _, _, s = fm.quantize(x, fm.E5M2, fm.BLOCK_128x128, fm.FROM_AMAX, out=out[:, :512], counters=ctr)
    oq, _, os_, oc = oracle.quantize(xo, fm.E5M2, fm.BLOCK_128x128)
    got = host(out)
    assert np.array_equal(got[:, :512], oq)
    assert np.all(got[:, 512:] == 0xAA), "wrote past cols"
    assert np.array_equal(host(s).reshape(os_.shape), os_)
    assert same_counters(ctr.read(), oc)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(128, 128), (256, 384), (200, 300), (1, 5), (129, 127), (7, 1000)])
def test_block_128_and_transpose(fmt, shape):
    x = synth.with_outliers_bf16(2, shape, frac=0.01)
    _cmp(x, fmt, fm.BLOCK_128x128)
    _cmp(x, fmt, fm.BLOCK_128x128, want_t=True)
    sc = np.random.default_rng(3).uniform(0.001, 10, size=oracle.scale_shape(2, *shape)).astype(np.float32)
    _cmp(x, fmt, fm.BLOCK_128x128, fm.GIVEN, sc, want_t=True)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 1), (3, 17), (64, 128), (100, 1000), (257, 130), (1024, 768)])
def test_ragged_shapes_all_granularities(fmt, shape):
    x = synth.with_outliers_bf16(5, shape, frac=0.02)
    _cmp(x, fmt, fm.TENSOR)
    _cmp(x, fmt, fm.TENSOR, want_t=True)
    _cmp(x, fmt, fm.ROW_1x128)
    sc = np.random.default_rng(4).uniform(0.001, 10, size=oracle.scale_shape(1, *shape)).astype(np.float32)
    _cmp(x, fmt, fm.ROW_1x128, fm.GIVEN, sc)


@pytest.mark.parametrize("fmt", FMTS)
def test_fp32_master_input(fmt):
    g = np.random.default_rng(5)
    x = (g.standard_normal((300, 520)) * 0.02).astype(np.float32)
    x[0, 0] = 3e-41                  # fp32 subnormal
    x[1, 1] = -0.0
    for gran, want_t in [(fm.TENSOR, False), (fm.TENSOR, True), (fm.BLOCK_128x128, True), (fm.ROW_1x128, False)]:
        _cmp(None, fmt, gran, want_t=want_t, x_dev=dev_f32(x), x_orc=x)


def test_strided_inputs_and_outputs():
    x_full = synth.with_outliers_bf16(6, (96, 400), frac=0.02)
    x = dev_bf16(x_full)[:, 16:336]           # ld 400 > cols 320
    xo = np.ascontiguousarray(x_full[:, 16:336])
    for gran in (fm.TENSOR, fm.ROW_1x128, fm.BLOCK_128x128):
        out = torch.full((96, 352), 0xAA, dtype=torch.uint8, device="cuda")
        ctr = fm.Counters()
        q, _, s = fm.quantize(x, fm.E4M3, gran, fm.FROM_AMAX, out=out[:, :320], counters=ctr)
        oq, _, os_, oc = oracle.quantize(xo, fm.E4M3, gran)
        got = host(out)
        assert np.array_equal(got[:, :320], oq)
        assert np.all(got[:, 320:] == 0xAA), "wrote past cols"
        assert np.array_equal(host(s).reshape(os_.shape), os_)


def test_empty_and_degenerate():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    q, _, s = fm.quantize(x, fm.E4M3)
    assert q.shape == (0, 64) and host(s)[0] == 1.0
    z = synth.f32_to_bf16_bits(np.zeros((16, 256), np.float32))
    _cmp(z, fm.E4M3, fm.TENSOR)                      # amax 0 -> scale 1
    _cmp(z, fm.E5M2, fm.ROW_1x128)
    nan = np.full((4, 128), 0x7FC0, dtype=np.uint16)
    _cmp(nan, fm.E4M3, fm.TENSOR)                    # all NaN
    _cmp(nan, fm.E4M3, fm.BLOCK_128x128)


@pytest.mark.parametrize("fmt", FMTS)
def test_amax_entry_point(fmt):
    x = synth.with_outliers_bf16(7, (300, 700), frac=0.01)
    xd = dev_bf16(x)
    for gran in (fm.TENSOR, fm.ROW_1x128, fm.BLOCK_128x128):
        got = host(fm.amax(xd, gran))
        assert np.array_equal(got.reshape(-1), oracle.amax(x, gran).reshape(-1)), gran


def _amax_cases():
    """(host array, device tensor, what) for the per-tensor amax: bf16 and
    fp32, contiguous (one long row), strided rows (ld > cols), rows that are
    not 16-byte aligned, Inf and NaN present, all NaN, one element, and a
    tensor that takes the full 512 workgroups."""
    g = np.random.default_rng(21)
    out = []
    a = synth.with_outliers_bf16(22, (300, 700), frac=0.01)
    out.append((a, dev_bf16(a), "bf16 300x700"))
    b = synth.with_outliers_bf16(23, (2048, 4096), frac=0.001)
    out.append((b, dev_bf16(b), "bf16 2048x4096"))
    f = g.normal(size=(513, 1000)).astype(np.float32)
    f[7, 9], f[300, 2] = np.inf, np.nan
    out.append((f, dev_f32(f), "fp32 513x1000 with Inf and NaN"))
    wide = synth.with_outliers_bf16(24, (257, 1024), frac=0.01)
    out.append((np.ascontiguousarray(wide[:, :1000]), dev_bf16(wide)[:, :1000], "bf16 257x1000, ld 1024"))
    odd = synth.with_outliers_bf16(25, (129, 333), frac=0.01)
    out.append((np.ascontiguousarray(odd[:, :331]), dev_bf16(odd)[:, :331], "bf16 129x331, ld 333"))
    nan = np.full((3, 64), 0x7FC0, dtype=np.uint16)
    out.append((nan, dev_bf16(nan), "bf16 all NaN"))
    one = np.array([[0xC2F7]], dtype=np.uint16)
    out.append((one, dev_bf16(one), "bf16 one element"))
    return out


def test_amax_layouts_and_caller_workspace():
    """The per-tensor amax on the cases above, through a workspace the caller
    holds: random bytes at first, then each call's leftovers, then the keys
    of a large tensor's quantize; and one that is not 8-byte aligned.
    Bit-exact every time."""
    cases = _amax_cases()
    wsb = fm.lib().fp8_amax_workspace_size(1, 1, fm.TENSOR)
    raw = torch.from_numpy(np.random.default_rng(26).integers(0, 256, wsb + 8, dtype=np.uint8)).cuda()

    def run(ws, what):
        for x, xd, name in cases:
            got = host(fm.amax(xd, fm.TENSOR, workspace=ws)).reshape(-1)
            assert np.array_equal(got, oracle.amax(x, fm.TENSOR).reshape(-1)), f"{what}: {name}"

    ws = raw[:wsb]
    run(ws, "random workspace")
    run(ws, "the previous calls' leftovers")
    big = synth.with_outliers_bf16(27, (4096, 4096))
    q, _, s = fm.quantize(dev_bf16(big), fm.E4M3, workspace=ws)
    assert np.array_equal(host(s).reshape(-1), oracle.quantize(big, fm.E4M3)[2].reshape(-1))
    run(ws, "after a quantize on the same workspace")
    run(raw[1:wsb + 1], "unaligned workspace")
    with pytest.raises(ValueError, match="workspace needs"):
        fm.amax(cases[0][1], fm.TENSOR, workspace=ws[: wsb - 1])


def test_hardware_conversion_sweep():
    """fp32 inputs with scale 1 (the quotient is the input): every combination
    of sign, exponent 2^-20 .. 2^16, top 12 mantissa bits and a set of low
    (sticky) bit patterns, so every rounding decision of both formats is met."""
    lows = np.array([0, 1, 2, 0x3FF, 0x400, 0x401, 0x7FE, 0x7FF, 0x155, 0x6AA], dtype=np.uint32)
    exps = np.arange(127 - 20, 127 + 17, dtype=np.uint32)
    top = np.arange(4096, dtype=np.uint32)
    bits = (exps[:, None, None] << 23) | (top[None, :, None] << 11) | lows[None, None, :]
    bits = np.concatenate([bits.reshape(-1), bits.reshape(-1) | 0x80000000]).astype(np.uint32)
    pad = (-bits.size) % 1024
    bits = np.concatenate([bits, np.zeros(pad, np.uint32)])
    x = bits.view(np.float32).reshape(-1, 1024)
    for fmt in FMTS:
        _cmp(None, fmt, fm.TENSOR, fm.GIVEN, np.float32([1.0]), x_dev=dev_f32(x), x_orc=x)


def test_deterministic_repeat():
    x = synth.with_outliers_bf16(8, (1024, 1024))
    xd = dev_bf16(x)
    a = gpu_quantize(xd, fm.E5M2, fm.TENSOR, want_t=True)
    b = gpu_quantize(xd, fm.E5M2, fm.TENSOR, want_t=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[3] == b[3]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", [fm.TENSOR, fm.ROW_1x128])
def test_quantize_only_workload_full_size(fmt, gran):
    """8192 x 8192 bf16, N(0,1) with 0.1% +-U(500,5000) outliers: bytes,
    scales and saturation/underflow counts bit-exact."""
    x = synth.with_outliers_bf16(2, synth.QUANT_ONLY["x"])
    c = _cmp(x, fmt, gran)
    assert c["saturated"] == 0 and c["nan"] == 0
    if gran == fm.TENSOR and fmt == fm.E4M3:
        assert c["underflow"] > 100000      # scale ~11: many N(0,1) values underflow


def _amaxes_over_fmax(fmax, n):
    """bf16 amaxes whose quotient fl32(amax / s), s = fl32(amax / fmax) raised
    to FLT_MIN, lands above fmax (IEEE fp32 arithmetic on the host)."""
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint32)
    a = (bits << 16).view(np.float32)
    s = np.maximum((a / np.float32(fmax)).astype(np.float32), np.float32(np.finfo(np.float32).tiny))
    v = (a / s).astype(np.float32)
    sel = bits[(v > np.float32(fmax)) & (s >= np.float32(2.0 ** -64))]
    assert sel.size > 1000
    return sel[np.linspace(0, sel.size - 1, n).astype(int)].astype(np.uint16)


@pytest.mark.parametrize("fmt", FMTS)
def test_amax_quotient_just_above_fmax(fmt):
    """Groups whose amax element divides to one fp32 ulp above fmax: that
    element still encodes to +-fmax and nothing counts as saturated (the fast
    cast leaves this to the conversion's rounding, with no clamp).  Block
    column j (128 x 128) has amax_j, and every 1x128 row tile in it holds
    +amax_j or -amax_j, so the 1x128, 128x128 and per-tensor paths all see it."""
    fmax = 448.0 if fmt == fm.E4M3 else 57344.0
    top = 0x7E if fmt == fm.E4M3 else 0x7B
    amaxes = _amaxes_over_fmax(fmax, 16)
    g = np.random.default_rng(17)
    rows, nb = 128, amaxes.size
    x = np.zeros((rows, 128 * nb), dtype=np.uint16)
    where = g.integers(0, 128, size=(rows, nb))
    for j, ab in enumerate(amaxes):
        blk = g.integers(1, int(ab), size=(rows, 128)).astype(np.uint16)
        blk |= (g.integers(0, 2, size=(rows, 128)) << 15).astype(np.uint16)
        blk[np.arange(rows), where[:, j]] = ab | ((np.arange(rows) & 1) << 15).astype(np.uint16)
        x[:, 128 * j:128 * (j + 1)] = blk
    for gran, want_t in ((fm.ROW_1x128, False), (fm.BLOCK_128x128, True), (fm.BLOCK_128x128, False)):
        c = _cmp(x, fmt, gran, want_t=want_t)
        assert c["saturated"] == 0
        q, _, _, _ = gpu_quantize(dev_bf16(x), fmt, gran, want_t=want_t)
        codes = q[np.repeat(np.arange(rows), nb), (where + 128 * np.arange(nb)).ravel()]
        assert np.all((codes & 0x7F) == top), "an amax element did not encode to fmax"
    for j in range(4):
        blk = np.ascontiguousarray(x[:, 128 * j:128 * (j + 1)])
        c = _cmp(blk, fmt, fm.TENSOR, want_t=True)
        assert c["saturated"] == 0


def test_caller_workspace():
    """A workspace held by the caller gives the same bytes as a per-call one;
    one that is too small is rejected before any launch."""
    x = synth.with_outliers_bf16(14, (300, 520), frac=0.01)
    xd = dev_bf16(x)
    q1, _, s1 = fm.quantize(xd, fm.E4M3)
    wsb = fm.lib().fp8_quantize_workspace_size(300, 520, fm.TENSOR, fm.FROM_AMAX)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    q2, _, s2 = fm.quantize(xd, fm.E4M3, workspace=ws)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)
    with pytest.raises(ValueError, match="workspace needs"):
        fm.quantize(xd, fm.E4M3, workspace=ws[: wsb - 1])


ONE_LAUNCH_SHAPES = [(128, 128), (256, 768), (3072, 768), (128, 32768), (2048, 2048)]


def _one_launch_cases(fmt, mode, ws, what):
    """Per-tensor quantize of tensors the one-launch kernel takes (bf16,
    whole 128x128 tiles, at most 256 tiles and one per CU), with and without
    the transposed copy, on the caller's workspace ws, against the oracle."""
    for i, shape in enumerate(ONE_LAUNCH_SHAPES):
        x = synth.with_outliers_bf16(30 + i, shape, frac=0.01).copy()
        if i == 2:
            x[5, 7] = 0x7FC0      # NaN: the scale ignores it, the code is 0x7F | sign
            x[100, 1] = 0xFF80    # -Inf: saturates
        xd = dev_bf16(x)
        for want_t in (False, True):
            ctr = fm.Counters()
            q, qt, s = fm.quantize(xd, fmt, fm.TENSOR, mode, want_t=want_t, counters=ctr, workspace=ws)
            torch.cuda.synchronize()
            if mode == fm.FROM_AMAX_POW2:
                oq, oqt, os_, oc = oracle.quantize_pow2(x, fmt, oracle.TENSOR, want_t=want_t)
            else:
                oq, oqt, os_, oc = oracle.quantize(x, fmt, want_t=want_t)
            w = f"{what} {shape} fmt {fmt} mode {mode} transposed {want_t}"
            assert np.array_equal(host(s).reshape(-1), os_.reshape(-1)), f"{w}: scale"
            assert np.array_equal(host(q), oq), f"{w}: codes"
            if want_t:
                assert np.array_equal(host(qt), oqt), f"{w}: transposed codes"
            assert same_counters(ctr.read(), oc), f"{w}: counters"


@pytest.mark.parametrize("fmt", FMTS)
def test_one_launch_small_tensors(fmt):
    """Small per-tensor calls run as one launch whose workgroups exchange
    their tile maxima through the workspace.  The workspace arrives holding
    arbitrary bytes (random, then each call's own leftovers, with calls of
    different tile counts in turn), and with the wait bound set to zero every
    workgroup reads the whole tensor itself: bit-exact either way.  Between
    rounds a large tensor's two-launch quantize writes its amax keys over the
    same workspace."""
    wsb = fm.lib().fp8_quantize_workspace_size(128, 128, fm.TENSOR, fm.FROM_AMAX)
    ws = torch.from_numpy(np.random.default_rng(9).integers(0, 256, wsb, dtype=np.uint8)).cuda()
    _one_launch_cases(fmt, fm.FROM_AMAX, ws, "one launch")
    # a large tensor's amax pass writes its partial keys over the same workspace
    big = synth.with_outliers_bf16(40, (4096, 4096))
    q, _, s = fm.quantize(dev_bf16(big), fmt, workspace=ws)
    oq, _, os_, _ = oracle.quantize(big, fmt)
    assert np.array_equal(host(q), oq) and np.array_equal(host(s).reshape(-1), os_.reshape(-1))
    _one_launch_cases(fmt, fm.FROM_AMAX, ws, "one launch after a two-launch call")
    _one_launch_cases(fmt, fm.FROM_AMAX_POW2, ws, "one launch, power-of-two")
    prev = fm.lib().fp8_debug_set_wait_limit(0)
    try:
        _one_launch_cases(fmt, fm.FROM_AMAX, ws, "every workgroup reads the tensor")
    finally:
        fm.lib().fp8_debug_set_wait_limit(prev)
    assert fm.lib().fp8_debug_set_wait_limit(prev) == prev
