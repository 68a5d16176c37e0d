"""Pins for the oracle's power-of-two (E8M0) scale rule and quantizer (CPU
only).

Independent facts used: the rule's two defining inequalities (amax / s <=
fmax, and halving s breaks it) checked with exact fp64 arithmetic on every
positive finite bf16 amax; closed forms at amax = fmax * 2^k and at the
bottom clamp; that s is an exact power of two whose exponent field is its
E8M0 code; and, for the quantizer, that nothing saturates (the scale leaves
headroom), that a power-of-two division is exact so the codes equal those of
the plain RNE cast of x * 2^-e, and the reduction of a tile/block quantize to
per-group calls.
"""
import math

import numpy as np
import pytest

import oracle
import synth

FMTS = [(oracle.E4M3, 448.0), (oracle.E5M2, 57344.0)]


@pytest.mark.parametrize("fmt,fm", FMTS)
def test_rule_on_every_bf16_amax(fmt, fm):
    pats = np.arange(1, 0x7F80, dtype=np.uint32)
    amaxes = synth.bf16_bits_to_f32(pats.astype(np.uint16)).astype(np.float64)
    for a in amaxes.tolist():
        s = float(oracle.scale_pow2(fmt, a))
        m, e = math.frexp(s)
        assert m == 0.5, "not a power of two"
        if s > 2.0 ** -126:
            assert a / s <= fm and a / (s / 2) > fm
        else:
            assert a / s <= fm


@pytest.mark.parametrize("fmt,fm", FMTS)
def test_closed_forms(fmt, fm):
    for k in (-20, -3, 0, 1, 7, 60):
        assert oracle.scale_pow2(fmt, fm * 2.0 ** k) == np.float32(2.0 ** k)
        # one fp32 ulp above needs the next power
        above = np.nextafter(np.float32(fm * 2.0 ** k), np.float32(np.inf))
        assert oracle.scale_pow2(fmt, above) == np.float32(2.0 ** (k + 1))
    assert oracle.scale_pow2(fmt, 0.0) == 1.0
    assert oracle.scale_pow2(fmt, 1e-40) == np.float32(2.0 ** -126)
    # E8M0 code = the fp32 exponent field
    s = oracle.scale_pow2(fmt, 3.0)
    assert (int(np.float32(s).view(np.uint32)) >> 23) - 127 == int(math.log2(float(s)))


@pytest.mark.parametrize("fmt,fm", FMTS)
@pytest.mark.parametrize("gran", [oracle.TENSOR, oracle.ROW_1x128, oracle.BLOCK_128x128])
def test_quantize_no_saturation_and_exact_division(fmt, fm, gran):
    x = synth.with_outliers_bf16(31, (256, 384))
    q, _, s, ctr = oracle.quantize_pow2(x, fmt, gran)
    assert ctr["saturated"] == 0
    assert np.all(s > 0) and np.all(np.frexp(s)[0] == 0.5)
    # dividing by 2^e is exact, so the codes are the encodes of x * 2^-e
    xf = synth.bf16_bits_to_f32(x)
    sf = s.reshape(-1)[0] if gran == oracle.TENSOR else None
    if gran == oracle.TENSOR:
        for idx in [(0, 0), (10, 17), (255, 383)]:
            v = np.float32(xf[idx] / sf)
            code, _ = oracle.encode(fmt, float(v), xf[idx] != 0)
            assert q[idx] == code


def test_group_decomposition():
    x = synth.with_outliers_bf16(32, (256, 256))
    q, _, s, _ = oracle.quantize_pow2(x, oracle.E4M3, oracle.BLOCK_128x128)
    for br in range(2):
        for bc in range(2):
            sub = np.ascontiguousarray(x[128 * br:128 * br + 128, 128 * bc:128 * bc + 128])
            qs, _, ss, _ = oracle.quantize_pow2(sub, oracle.E4M3, oracle.TENSOR)
            assert ss[0] == s[br, bc]
            assert np.array_equal(qs, q[128 * br:128 * br + 128, 128 * bc:128 * bc + 128])
