"""Pins for the oracle's FP8 decode/encode (CPU only).

What fixes the answer here is not the oracle itself:
  * the bit splits and maxima printed on the pages (tests/golden/format_facts.json);
  * closed forms of the formats (min subnormal, min normal, counts of codes);
  * an independent construction of the value grid;
  * torch's own CPU float8 casts (a library routine) for in-range values;
  * an exhaustive brute-force comparison over all 2^32 fp32 inputs (C program).
"""
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "format_facts.json")))
FMTS = {"e4m3": oracle.E4M3, "e5m2": oracle.E5M2}
TORCH_DT = {oracle.E4M3: torch.float8_e4m3fn, oracle.E5M2: torch.float8_e5m2}


@pytest.mark.parametrize("name", ["e4m3", "e5m2"])
def test_page_facts(name):
    fmt = FMTS[name]
    f = FACTS[name]
    L = oracle.lib()
    assert L.orc_exp_bits(fmt) == f["exp_bits"]
    assert L.orc_mant_bits(fmt) == f["mant_bits"]
    assert 1 + f["exp_bits"] + f["mant_bits"] == 8
    assert oracle.fmax(fmt) == f["max"]
    # closed forms: 1.75 * 2^8 and 1.75 * 2^15
    assert oracle.fmax(oracle.E4M3) == 1.75 * 2 ** 8
    assert oracle.fmax(oracle.E5M2) == 1.75 * 2 ** 15
    assert FACTS["bf16"]["mant_bits"] == 7 > f["mant_bits"]


def test_code_census():
    v = oracle.decode(oracle.E4M3, np.arange(256))
    assert np.isnan(v).sum() == 2 and np.isinf(v).sum() == 0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    w = oracle.decode(oracle.E5M2, np.arange(256))
    assert np.isnan(w).sum() == 6 and np.isinf(w).sum() == 2
    assert w[0x7C] == np.inf and w[0xFC] == -np.inf
    assert np.isfinite(w).sum() == 248
    for t in (v, w):
        assert t[0x00] == 0.0 and not np.signbit(t[0x00])
        assert t[0x80] == 0.0 and np.signbit(t[0x80])


@pytest.mark.parametrize("fmt,maxcode,minsub,minnorm", [
    (oracle.E4M3, 0x7E, 2.0 ** -9, 2.0 ** -6),
    (oracle.E5M2, 0x7B, 2.0 ** -16, 2.0 ** -14),
])
def test_extremes_and_monotonic(fmt, maxcode, minsub, minnorm):
    v = oracle.decode(fmt, np.arange(256))
    assert v[maxcode] == oracle.fmax(fmt)
    assert v[0x01] == minsub
    mb = oracle.lib().orc_mant_bits(fmt)
    assert v[1 << mb] == minnorm                      # exponent field 1, mantissa 0
    assert v[(1 << mb) - 1] < minnorm                 # largest subnormal below it
    pos = v[: maxcode + 1]
    assert np.all(np.diff(pos) > 0)                   # strictly increasing
    assert np.array_equal(v[0x80: 0x80 + maxcode + 1], -pos)   # sign symmetry


def _grid_by_construction(fmt):
    """Non-negative finite values built from the bit split alone."""
    mb, eb = (3, 4) if fmt == oracle.E4M3 else (2, 5)
    bias = 2 ** (eb - 1) - 1
    vals = [j * 2.0 ** (1 - bias - mb) for j in range(2 ** mb)]
    top = 2 ** eb - 1 - bias if fmt == oracle.E4M3 else 2 ** eb - 2 - bias
    for E in range(1 - bias, top + 1):
        vals += [(2 ** mb + j) * 2.0 ** (E - mb) for j in range(2 ** mb)]
    if fmt == oracle.E4M3:
        vals = vals[:-1]
    return np.array(vals)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_matches_independent_grid(fmt):
    g = _grid_by_construction(fmt)
    v = oracle.decode(fmt, np.arange(len(g)))
    assert np.array_equal(v, g)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_roundtrip(fmt):
    v = oracle.decode(fmt, np.arange(256))
    for c in range(256):
        if not np.isfinite(v[c]):
            continue
        code, ev = oracle.encode(fmt, v[c], src_nonzero=v[c] != 0)
        assert code == c and ev == 0, hex(c)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_decode_vs_torch(fmt):
    """torch's float8 dtypes are the OCP encodings; decode every code there too."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()
    ov = oracle.decode(fmt, np.arange(256))
    same = (tv == ov) | (np.isnan(tv) & np.isnan(ov))
    assert same.all()


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_exhaustive_encode_vs_bruteforce(fmt, tmp_path):
    """All 2^32 fp32 inputs: orc_encode == nearest grid value, ties to even code,
    saturate above the max, count underflow/NaN (C program, OpenMP)."""
    oracle.build(force=False)
    exe = tmp_path / "exh"
    src = os.path.join(HERE, "pins", "exhaustive_encode.c")
    osrc = os.path.join(os.path.dirname(HERE), "oracle", "fp8_oracle.c")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
                           src, osrc, "-o", str(exe), "-lm"])
    stride = os.environ.get("FP8_PIN_STRIDE", "1")
    out = subprocess.run([str(exe), str(fmt), stride], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout[-2000:]
    assert out.stdout.startswith("OK")
