"""C-ABI boundary checks that need no GPU: the library loads, exports every
symbol include/fp8mi.h declares, and rejects bad arguments on the host before
touching the device.  Also the host side of the integer fast division."""
import ctypes
import os
import re
import subprocess

import pytest

import fp8_scaled_matmul_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mi.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fm.LIB_PATH):
        from fp8_scaled_matmul_amd import build
        build.build()
    return fm.lib()


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert len(declared) >= 12
    assert sorted(declared) == sorted(fm.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fm.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fp8_\w+)", out))
    assert set(declared) <= exported


def test_abi_version_and_strings(L):
    assert fm.fp8_abi_version() == 1
    names = [L.fp8_status_string(i).decode() for i in range(5)]
    assert names == ["FP8_OK", "FP8_ERR_INVALID_ARG", "FP8_ERR_UNSUPPORTED_SHAPE",
                     "FP8_ERR_UNSUPPORTED_DEVICE", "FP8_ERR_HIP"]


def test_workspace_sizes(L):
    assert L.fp8_quantize_workspace_size(10, 10, fm.TENSOR, fm.FROM_AMAX) == 8192
    assert L.fp8_quantize_workspace_size(10, 10, fm.TENSOR, fm.GIVEN) == 0
    assert L.fp8_quantize_workspace_size(10, 10, fm.ROW_1x128, fm.FROM_AMAX) == 0
    assert L.fp8_amax_workspace_size(10, 10, fm.TENSOR) == 8192
    # dW of the speedrun backward: few output tiles, long K -> split-K workspace
    assert L.fp8_scaled_mm_workspace_size(3072, 768, 65536, 0, 0) > 0
    assert L.fp8_scaled_mm_workspace_size(65536, 3072, 768, 0, 0) == 0
    assert L.fp8_scaled_mm_workspace_size(0, 3072, 768, 0, 0) == 0


BAD = 0x1000  # a non-null address never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,code", [
    # bad dtype / format / granularity / mode
    (dict(dtype=7), fm.FP8_ERR_INVALID_ARG),
    (dict(fmt=9), fm.FP8_ERR_INVALID_ARG),
    (dict(gran=5), fm.FP8_ERR_INVALID_ARG),
    (dict(mode=3), fm.FP8_ERR_INVALID_ARG),
    # shapes and leading dimensions
    (dict(rows=-1), fm.FP8_ERR_INVALID_ARG),
    (dict(ld=10), fm.FP8_ERR_INVALID_ARG),
    (dict(ldq=10), fm.FP8_ERR_INVALID_ARG),
    (dict(x=None), fm.FP8_ERR_INVALID_ARG),
    (dict(q=None), fm.FP8_ERR_INVALID_ARG),
    (dict(scale=None), fm.FP8_ERR_INVALID_ARG),
    # transposed copy with 1x128 tiles
    (dict(gran=fm.ROW_1x128, mode=fm.FROM_AMAX, q_t=BAD, ldq_t=64), fm.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(q_t=BAD, ldq_t=8), fm.FP8_ERR_INVALID_ARG),
    # per-tensor amax scaling without workspace
    (dict(ws=None, wsb=0), fm.FP8_ERR_INVALID_ARG),
    (dict(wsb=100), fm.FP8_ERR_INVALID_ARG),
])
def test_quantize_rejects_before_device(L, args, code):
    a = dict(x=BAD, dtype=fm.BF16, rows=64, cols=32, ld=32, fmt=fm.E4M3, gran=fm.TENSOR,
             mode=fm.FROM_AMAX, scale=BAD, q=BAD, ldq=32, q_t=None, ldq_t=0, ctr=None,
             ws=BAD, wsb=8192)
    a.update(args)
    rc = fm.fp8_quantize(a["x"], a["dtype"], a["rows"], a["cols"], a["ld"], a["fmt"], a["gran"],
                         a["mode"], a["scale"], a["q"], a["ldq"], a["q_t"], a["ldq_t"], a["ctr"],
                         a["ws"], a["wsb"], None)
    assert rc == code, L.fp8_last_error()
    assert L.fp8_last_error().decode() != ""


@pytest.mark.parametrize("args,code", [
    (dict(fa=3), fm.FP8_ERR_INVALID_ARG),
    (dict(ga=fm.ROW_1x128), fm.FP8_ERR_UNSUPPORTED_SHAPE),                      # (ROW, TENSOR)
    (dict(ga=fm.BLOCK_128x128, gb=fm.BLOCK_128x128), fm.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(ga=fm.ROW_1x128, gb=fm.BLOCK_128x128, k=144, lda=144, ldb=144), fm.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(k=40, lda=48, ldb=48), fm.FP8_ERR_UNSUPPORTED_SHAPE),                  # k % 16
    (dict(lda=136), fm.FP8_ERR_UNSUPPORTED_SHAPE),                              # lda % 16
    (dict(a=BAD + 8), fm.FP8_ERR_UNSUPPORTED_SHAPE),                            # alignment
    (dict(lda=1 << 22), fm.FP8_ERR_UNSUPPORTED_SHAPE),                          # 32-bit tile offsets
    (dict(ldb=1 << 22), fm.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(ldc=1 << 21), fm.FP8_ERR_UNSUPPORTED_SHAPE),
    (dict(lda=64), fm.FP8_ERR_INVALID_ARG),                                     # lda < k
    (dict(ldc=10), fm.FP8_ERR_INVALID_ARG),
    (dict(m=-3), fm.FP8_ERR_INVALID_ARG),
    (dict(sa=None), fm.FP8_ERR_INVALID_ARG),
    (dict(c=BAD + 1), fm.FP8_ERR_INVALID_ARG),
])
def test_scaled_mm_rejects_before_device(L, args, code):
    a = dict(a=BAD, fa=fm.E4M3, lda=128, sa=BAD, ga=fm.TENSOR, b=BAD, fb=fm.E4M3, ldb=128, sb=BAD,
             gb=fm.TENSOR, m=32, n=32, k=128, c=BAD, ldc=32, ws=None, wsb=0, ctr=None)
    a.update(args)
    rc = fm.fp8_scaled_mm(a["a"], a["fa"], a["lda"], a["sa"], a["ga"], a["b"], a["fb"], a["ldb"], a["sb"],
                          a["gb"], a["m"], a["n"], a["k"], a["c"], a["ldc"], a["ws"], a["wsb"], a["ctr"], None)
    assert rc == code, L.fp8_last_error()


def test_amax_and_requant_reject(L):
    assert fm.fp8_amax(BAD, 5, 4, 4, 4, 0, BAD, BAD, 4096, None) == fm.FP8_ERR_INVALID_ARG
    assert fm.fp8_amax(BAD, 0, 4, 4, 4, 0, BAD, None, 0, None) == fm.FP8_ERR_INVALID_ARG
    assert fm.fp8_amax(BAD, 0, 4, 4, 4, 0, None, BAD, 4096, None) == fm.FP8_ERR_INVALID_ARG
    d = fm.WeightCacheDesc(64, 64, fm.E4M3, fm.ROW_1x128, BAD, None, BAD, None)
    assert fm.fp8_requant_weights([d], [BAD], [fm.BF16], BAD, 4096, None) == fm.FP8_ERR_UNSUPPORTED_SHAPE
    d = fm.WeightCacheDesc(64, 64, fm.E4M3, fm.TENSOR, BAD, None, BAD, None)
    assert fm.fp8_requant_weights([d], [BAD], [fm.BF16], None, 0, None) == fm.FP8_ERR_INVALID_ARG
    assert fm.fp8_requant_weights([], [], [], None, 0, None) == fm.FP8_OK
    assert fm.fp8_counters_reset(None, None) == fm.FP8_ERR_INVALID_ARG


@pytest.mark.parametrize("over,code", [
    (dict(length=0), fm.FP8_ERR_INVALID_ARG),
    (dict(length=4097), fm.FP8_ERR_INVALID_ARG),
    (dict(hist=None), fm.FP8_ERR_INVALID_ARG),
    (dict(pos=None), fm.FP8_ERR_INVALID_ARG),
    (dict(ws=None), fm.FP8_ERR_INVALID_ARG),
    (dict(fmt=4), fm.FP8_ERR_INVALID_ARG),
    (dict(ld=10), fm.FP8_ERR_INVALID_ARG),
])
def test_quantize_delayed_rejects_before_device(L, over, code):
    a = dict(x=BAD, dtype=0, rows=16, cols=64, ld=64, fmt=0, hist=BAD, pos=BAD, length=16, scale=BAD,
             q=BAD, ldq=64, q_t=None, ldq_t=0, ctr=None, ws=BAD, wsb=8192)
    a.update(over)
    assert L.fp8_quantize_delayed_workspace_size(16, 64) == 8192
    rc = fm.fp8_quantize_delayed(a["x"], a["dtype"], a["rows"], a["cols"], a["ld"], a["fmt"], a["hist"], a["pos"],
                                 a["length"], a["scale"], a["q"], a["ldq"], a["q_t"], a["ldq_t"], a["ctr"], a["ws"],
                                 a["wsb"], None)
    assert rc == code


def test_fastdiv_host(tmp_path):
    """The magic-number division used to map 1x128 tiles to rows."""
    src = tmp_path / "fd.cpp"
    src.write_text(r'''
#include "fastdiv.h"
#include <cstdio>
#include <random>
int main() {
  std::mt19937 g(1);
  unsigned divs[] = {1,2,3,5,6,7,24,56,64,96,127,128,129,1000,65535,65536,1000003,(1u<<30)+3};
  for (unsigned d : divs) {
    fp8mi::FastDiv f(d);
    for (unsigned n = 0; n < 200000; ++n) if (f.div(n) != n / d) { printf("bad %u %u\n", n, d); return 1; }
    for (int i = 0; i < 200000; ++i) { unsigned n = g() & 0x7fffffffu; if (f.div(n) != n / d) { printf("bad %u %u\n", n, d); return 1; } }
    unsigned n = 0x7fffffffu; if (f.div(n) != n / d) { printf("bad max %u\n", d); return 1; }
  }
  printf("OK\n");
  return 0;
}''')
    exe = tmp_path / "fd"
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "fp8_scaled_matmul_amd", "csrc"),
                           str(src), "-o", str(exe)])
    assert subprocess.run([str(exe)], capture_output=True, text=True).stdout.strip() == "OK"


def test_markstein_quotient_design_check(tmp_path):
    """The cast kernels' multiply-and-correct quotient gives the same FP8 code
    as the IEEE quotient on every input it is used for (C program)."""
    exe = tmp_path / "mk"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
                           os.path.join(ROOT, "tests", "pins", "markstein_div.c"), "-o", str(exe), "-lm"])
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.startswith("OK"), out.stdout[-1000:]
