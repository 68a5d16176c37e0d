"""Pins for the oracle's scaled cast and its counters (CPU only).

Pinned against torch's CPU float8 cast (round to nearest even, no saturation:
values past the range become NaN/Inf there) and against hand-derived special
cases at ties, subnormals and the overflow threshold.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

TORCH_DT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}
# scales: unity, powers of two, the amax-derived scales of the workloads'
# magnitudes, and awkward values near 1/448 and 1/57344
SCALES = [1.0, 2.0 ** -10, 0.5, 3.0, 1.0 / 448.0, 1.0 / 57344.0,
          4.5 / 448.0, 5000.0 / 448.0, 5000.0 / 57344.0, 0.0213 / 448.0, 1.1920929e-7, 7.3e-3]


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("s", SCALES)
def test_all_bf16_patterns_vs_torch(fmt, s):
    x = synth.all_bf16_patterns()
    s32 = np.float32(s)
    q, _, _, ctr = oracle.quantize(x, fmt, oracle.TENSOR, oracle.GIVEN, scale=np.array([s32]))
    xf = torch.from_numpy(synth.bf16_bits_to_f32(x))
    v = xf / torch.tensor(s32)                          # IEEE fp32 division on the CPU
    tq = v.to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    tval = v.to(TORCH_DT[fmt]).to(torch.float32).numpy()
    xn = np.isnan(xf.numpy())
    fmax = oracle.fmax(fmt)
    in_range = ~xn & np.isfinite(tval) & (np.abs(tval) <= fmax)
    # in range: identical bytes
    assert np.array_equal(q[in_range], tq[in_range])
    # torch's overflow (NaN/Inf for a non-NaN input) marks exactly the saturated set
    over = ~xn & ~(np.isfinite(tval) & (np.abs(tval) <= fmax))
    assert ctr["saturated"] == int(over.sum())
    sgn = np.where(np.signbit(synth.bf16_bits_to_f32(x)), 0x80, 0)
    assert np.array_equal(q[over], (sgn[over] | (0x7E if fmt == oracle.E4M3 else 0x7B)))
    # NaN inputs: 0x7F | sign, counted
    assert ctr["nan"] == int(xn.sum())
    assert np.array_equal(q[xn], sgn[xn] | 0x7F)
    # underflow: non-zero inputs whose code is +-0
    xnz = (synth.bf16_bits_to_f32(x) != 0) & ~xn
    zero_code = (q & 0x7F) == 0
    assert ctr["underflow"] == int((xnz & zero_code).sum())


def _enc(fmt, v):
    return oracle.encode(fmt, v, src_nonzero=True)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_ties_go_to_even(fmt):
    vals = oracle.decode(fmt, np.arange(0x7F if fmt == oracle.E4M3 else 0x7C))
    for c in range(len(vals) - 1):
        mid = np.float32((vals[c] + vals[c + 1]) / 2)
        assert float(mid) == (vals[c] + vals[c + 1]) / 2     # midpoints are fp32-exact
        code, _ = _enc(fmt, mid)
        assert code == (c if c % 2 == 0 else c + 1), (c, mid)
        lo = np.nextafter(mid, np.float32(0))
        hi = np.nextafter(mid, np.float32(np.inf))
        assert _enc(fmt, lo)[0] == c
        assert _enc(fmt, hi)[0] == c + 1


@pytest.mark.parametrize("fmt,minsub", [(oracle.E4M3, 2.0 ** -9), (oracle.E5M2, 2.0 ** -16)])
def test_underflow_rules(fmt, minsub):
    assert _enc(fmt, minsub / 2) == (0x00, 2)                         # tie at half -> 0 (even), counted
    assert _enc(fmt, -minsub / 2) == (0x80, 2)                        # sign kept
    assert _enc(fmt, np.nextafter(np.float32(minsub / 2), np.float32(1)))[0] == 0x01
    assert _enc(fmt, 1.5 * minsub)[0] == 0x02                         # tie 1 vs 2 -> 2 (even)
    assert _enc(fmt, 2.5 * minsub)[0] == 0x02                         # tie 2 vs 3 -> 2
    assert _enc(fmt, -1e-30) == (0x80, 2)
    assert oracle.encode(fmt, 0.0, src_nonzero=False) == (0x00, 0)
    assert oracle.encode(fmt, -0.0, src_nonzero=False) == (0x80, 0)
    # the division itself can underflow to zero: x != 0, v == 0 -> counted
    code, ctr = oracle.cast_one(fmt, 1e-38, 1e30)
    assert code == 0 and ctr["underflow"] == 1


def test_overflow_threshold():
    # E4M3: 464 is the tie between 448 (even) and the virtual 480 -> 448, not counted
    assert _enc(oracle.E4M3, 464.0) == (0x7E, 0)
    assert _enc(oracle.E4M3, np.nextafter(np.float32(464), np.float32(1e9))) == (0x7E, 1)
    assert _enc(oracle.E4M3, 465.0) == (0x7E, 1)
    assert _enc(oracle.E4M3, -1e6) == (0xFE, 1)
    # E5M2: 61440 ties 57344 (odd mantissa) vs 65536 (even) -> up -> saturated
    assert _enc(oracle.E5M2, 61439.0) == (0x7B, 0)
    assert _enc(oracle.E5M2, 61440.0) == (0x7B, 1)
    assert _enc(oracle.E5M2, -np.inf) == (0xFB, 1)
    assert _enc(oracle.E4M3, np.inf) == (0x7E, 1)
    # NaN keeps its sign bit
    assert _enc(oracle.E4M3, np.float32(np.nan)) == (0x7F, 3)
    assert _enc(oracle.E5M2, -np.float32(np.nan)) == (0xFF, 3)


def test_max_subnormal_to_min_normal_boundary():
    # E4M3: largest subnormal 7*2^-9, smallest normal 2^-6 = 8*2^-9; spacing equal
    assert _enc(oracle.E4M3, 7 * 2.0 ** -9)[0] == 0x07
    assert _enc(oracle.E4M3, 7.5 * 2.0 ** -9)[0] == 0x08       # tie 7 (odd) vs 8 (even)
    assert _enc(oracle.E5M2, 3 * 2.0 ** -16)[0] == 0x03
    assert _enc(oracle.E5M2, 3.5 * 2.0 ** -16)[0] == 0x04


def test_scale_from_amax():
    assert oracle.scale_from_amax(oracle.E4M3, 0.0) == 1.0
    assert oracle.scale_from_amax(oracle.E4M3, 448.0) == 1.0
    assert oracle.scale_from_amax(oracle.E5M2, 57344.0) == 1.0
    assert oracle.scale_from_amax(oracle.E4M3, 4480.0) == np.float32(4480.0) / np.float32(448.0)
    tiny = synth.bf16_bits_to_f32(np.array([0x0001], dtype=np.uint16))[0]   # bf16 subnormal
    assert oracle.scale_from_amax(oracle.E4M3, tiny) == np.finfo(np.float32).tiny
