// C ABI of the FP8 scaled-matmul library (declared in include/fp8mi.h).
//
// Every entry point validates its arguments on the host before enqueuing
// anything, checks once per device that the device is gfx950, enqueues its
// kernels on the caller's stream and returns.  No device memory is allocated
// here; workspaces come from the caller.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fp8mi.h"
#include "fp8mi_internal.h"

using namespace fp8mi;

namespace {

thread_local std::string g_last_error;

fp8_status fail(fp8_status s, const char* what)
{
    g_last_error = what;
    return s;
}

fp8_status hip_fail(hipError_t e, const char* where)
{
    g_last_error = std::string(where) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return FP8_ERR_HIP;
}

// Per-device architecture probe, cached.  FP8MI_FORCE_ARCH overrides the
// reported name (used by tests to exercise the rejection path).
constexpr int kMaxDevices = 64;
int g_arch_ok[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other
std::mutex g_arch_mu;

fp8_status check_device()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(FP8_ERR_UNSUPPORTED_DEVICE, "device index out of range");
    {
        std::lock_guard<std::mutex> lk(g_arch_mu);
        if (g_arch_ok[dev] == 0) {
            hipDeviceProp_t prop;
            e = hipGetDeviceProperties(&prop, dev);
            if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
            const char* forced = std::getenv("FP8MI_FORCE_ARCH");
            const char* arch = forced ? forced : prop.gcnArchName;
            g_arch_ok[dev] = std::strncmp(arch, "gfx950", 6) == 0 ? 1 : 2;
            if (forced) g_arch_ok[dev] = std::strncmp(forced, "gfx950", 6) == 0 ? 1 : 2;
        }
        if (g_arch_ok[dev] != 1) return fail(FP8_ERR_UNSUPPORTED_DEVICE, "this library runs on gfx950 (MI355X) only");
    }
    return FP8_OK;
}

bool valid_fmt(int f) { return f == FP8_E4M3 || f == FP8_E5M2; }
bool valid_dtype(int d) { return d == FP8_IN_BF16 || d == FP8_IN_FP32; }
bool valid_gran(int g) { return g == FP8_TENSOR || g == FP8_ROW_1x128 || g == FP8_BLOCK_128x128; }
bool valid_mode(int m) { return m == FP8_SCALE_FROM_AMAX || m == FP8_SCALE_GIVEN || m == FP8_SCALE_FROM_AMAX_POW2; }
bool amax_mode(int m) { return m == FP8_SCALE_FROM_AMAX || m == FP8_SCALE_FROM_AMAX_POW2; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

fp8_status check_2d(const void* p, int64_t rows, int64_t cols, int64_t ld, const char* name)
{
    static thread_local char buf[160];
    if (rows < 0 || cols < 0) {
        std::snprintf(buf, sizeof buf, "%s: negative size", name);
        return fail(FP8_ERR_INVALID_ARG, buf);
    }
    if (ld < cols || ld < 1) {
        std::snprintf(buf, sizeof buf, "%s: leading dimension %lld < cols %lld", name, (long long)ld, (long long)cols);
        return fail(FP8_ERR_INVALID_ARG, buf);
    }
    if (!p && rows > 0 && cols > 0) {
        std::snprintf(buf, sizeof buf, "%s: null pointer", name);
        return fail(FP8_ERR_INVALID_ARG, buf);
    }
    return FP8_OK;
}

fp8_status check_quantize_args(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                               fp8_format fmt, fp8_granularity gran, fp8_scale_mode mode, float* scale,
                               uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t, void* workspace,
                               size_t workspace_bytes)
{
    if (!valid_dtype(dtype)) return fail(FP8_ERR_INVALID_ARG, "unknown input dtype");
    if (!valid_fmt(fmt)) return fail(FP8_ERR_INVALID_ARG, "unknown FP8 format");
    if (!valid_gran(gran)) return fail(FP8_ERR_INVALID_ARG, "unknown granularity");
    if (!valid_mode(mode)) return fail(FP8_ERR_INVALID_ARG, "unknown scale mode");
    fp8_status s;
    if ((s = check_2d(x, rows, cols, ld, "x")) != FP8_OK) return s;
    if ((s = check_2d(q, rows, cols, ldq, "q")) != FP8_OK) return s;
    if (!scale) return fail(FP8_ERR_INVALID_ARG, "scale: null pointer");
    if (q_t) {
        if (gran == FP8_ROW_1x128)
            return fail(FP8_ERR_UNSUPPORTED_SHAPE, "a transposed copy is not available with 1x128 row tiles");
        if ((s = check_2d(q_t, cols, rows, ldq_t, "q_t")) != FP8_OK) return s;
    }
    const int64_t n = rows * cols;
    if (rows > 0 && cols > 0 && (n / rows != cols || n >= (int64_t)1 << 40))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "tensor too large");
    if (gran == FP8_ROW_1x128 && rows * cdiv(cols, 128) >= ((int64_t)1 << 31))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "too many 1x128 tiles");
    if (gran == FP8_TENSOR && amax_mode(mode) &&
        (!workspace || workspace_bytes < kAmaxWorkspaceBytes))
        return fail(FP8_ERR_INVALID_ARG, "workspace smaller than fp8_quantize_workspace_size()");
    return FP8_OK;
}

}  // namespace

extern "C" {

int32_t fp8_abi_version(void) { return FP8MI_ABI_VERSION; }

const char* fp8_status_string(fp8_status s)
{
    switch (s) {
        case FP8_OK: return "FP8_OK";
        case FP8_ERR_INVALID_ARG: return "FP8_ERR_INVALID_ARG";
        case FP8_ERR_UNSUPPORTED_SHAPE: return "FP8_ERR_UNSUPPORTED_SHAPE";
        case FP8_ERR_UNSUPPORTED_DEVICE: return "FP8_ERR_UNSUPPORTED_DEVICE";
        case FP8_ERR_HIP: return "FP8_ERR_HIP";
    }
    return "FP8_ERR_UNKNOWN";
}

const char* fp8_last_error(void) { return g_last_error.c_str(); }

size_t fp8_amax_workspace_size(int64_t rows, int64_t cols, fp8_granularity gran)
{
    (void)rows;
    (void)cols;
    return gran == FP8_TENSOR ? kAmaxWorkspaceBytes : 0;
}

fp8_status fp8_amax(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                    fp8_granularity gran, float* amax, void* workspace, size_t workspace_bytes,
                    hipStream_t stream)
{
    if (!valid_dtype(dtype)) return fail(FP8_ERR_INVALID_ARG, "unknown input dtype");
    if (!valid_gran(gran)) return fail(FP8_ERR_INVALID_ARG, "unknown granularity");
    fp8_status s = check_2d(x, rows, cols, ld, "x");
    if (s != FP8_OK) return s;
    if (!amax) return fail(FP8_ERR_INVALID_ARG, "amax: null pointer");
    if (gran == FP8_TENSOR && (!workspace || workspace_bytes < kAmaxWorkspaceBytes))
        return fail(FP8_ERR_INVALID_ARG, "workspace smaller than fp8_amax_workspace_size()");
    if (gran == FP8_ROW_1x128 && rows * cdiv(cols, 128) >= ((int64_t)1 << 31))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "too many 1x128 tiles");
    if ((s = check_device()) != FP8_OK) return s;
    hipError_t e = gran == FP8_TENSOR
                       ? launch_amax_tensor(x, dtype, rows, cols, ld, amax, static_cast<uint32_t*>(workspace), stream)
                       : launch_amax_grouped(x, dtype, rows, cols, ld, gran, amax, stream);
    return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_amax launch");
}

size_t fp8_quantize_workspace_size(int64_t rows, int64_t cols, fp8_granularity gran, fp8_scale_mode mode)
{
    (void)rows;
    (void)cols;
    return gran == FP8_TENSOR && amax_mode(mode) ? kAmaxWorkspaceBytes : 0;
}

fp8_status fp8_quantize(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                        fp8_format fmt, fp8_granularity gran, fp8_scale_mode mode, float* scale,
                        uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t, fp8_counters* ctr,
                        void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    fp8_status s = check_quantize_args(x, dtype, rows, cols, ld, fmt, gran, mode, scale, q, ldq, q_t, ldq_t,
                                       workspace, workspace_bytes);
    if (s != FP8_OK) return s;
    if ((s = check_device()) != FP8_OK) return s;
    QuantArgs a;
    a.x = x;
    a.dtype = dtype;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld;
    a.fmt = fmt;
    a.gran = gran;
    a.mode = amax_mode(mode) ? FP8_SCALE_FROM_AMAX : mode;
    a.pow2 = mode == FP8_SCALE_FROM_AMAX_POW2;
    a.scale = scale;
    a.q = q;
    a.ldq = ldq;
    a.qt = q_t;
    a.ldqt = ldq_t;
    a.ctr = ctr;
    a.partials = static_cast<uint32_t*>(workspace);
    hipError_t e = launch_quantize(a, stream);
    return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_quantize launch");
}

fp8_status fp8_quantize_noalloc(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                                fp8_format fmt, fp8_granularity gran, fp8_scale_mode mode, float* scale,
                                uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t, fp8_counters* ctr,
                                hipStream_t stream)
{
    // the scratch must hold every partial the call's workspace would: the
    // per-tensor amax pass writes at most kAmaxPartials keys for any size
    const size_t need = fp8_quantize_workspace_size(rows, cols, gran, mode);
    if (need > kNoAllocScratchWords * sizeof(uint32_t))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "call needs more scratch than fp8_quantize_noalloc holds (8 KiB)");
    // the library's scratch stands in for the workspace argument: checked as
    // present and large enough (its address is resolved after the checks)
    void* const scratch_stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
    fp8_status s = check_quantize_args(x, dtype, rows, cols, ld, fmt, gran, mode, scale, q, ldq, q_t, ldq_t,
                                       scratch_stand_in, kNoAllocScratchWords * sizeof(uint32_t));
    if (s != FP8_OK) return s;
    if ((s = check_device()) != FP8_OK) return s;
    uint32_t* scratch = nullptr;
    hipError_t e = noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e, "fp8_quantize_noalloc scratch address");
    QuantArgs a;
    a.x = x;
    a.dtype = dtype;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld;
    a.fmt = fmt;
    a.gran = gran;
    a.mode = amax_mode(mode) ? FP8_SCALE_FROM_AMAX : mode;
    a.pow2 = mode == FP8_SCALE_FROM_AMAX_POW2;
    a.scale = scale;
    a.q = q;
    a.ldq = ldq;
    a.qt = q_t;
    a.ldqt = ldq_t;
    a.ctr = ctr;
    a.partials = scratch;
    e = launch_quantize(a, stream);
    return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_quantize_noalloc launch");
}

size_t fp8_quantize_delayed_workspace_size(int64_t rows, int64_t cols)
{
    (void)rows;
    (void)cols;
    return kAmaxWorkspaceBytes;
}

fp8_status fp8_quantize_delayed(const void* x, fp8_dtype dtype, int64_t rows, int64_t cols, int64_t ld,
                                fp8_format fmt, float* amax_history, int32_t* history_pos, int32_t history_len,
                                float* scale, uint8_t* q, int64_t ldq, uint8_t* q_t, int64_t ldq_t,
                                fp8_counters* ctr, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    fp8_status s = check_quantize_args(x, dtype, rows, cols, ld, fmt, FP8_TENSOR, FP8_SCALE_FROM_AMAX, scale, q, ldq,
                                       q_t, ldq_t, workspace, workspace_bytes);
    if (s != FP8_OK) return s;
    if (!amax_history || !history_pos) return fail(FP8_ERR_INVALID_ARG, "amax_history / history_pos: null pointer");
    if (history_len < 1 || history_len > 4096) return fail(FP8_ERR_INVALID_ARG, "history_len must be in [1, 4096]");
    if ((s = check_device()) != FP8_OK) return s;
    QuantArgs a;
    a.x = x;
    a.dtype = dtype;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld;
    a.fmt = fmt;
    a.gran = FP8_TENSOR;
    a.mode = FP8_SCALE_GIVEN;
    a.scale = scale;
    a.q = q;
    a.ldq = ldq;
    a.qt = q_t;
    a.ldqt = ldq_t;
    a.ctr = ctr;
    a.partials = static_cast<uint32_t*>(workspace);
    hipError_t e = launch_quantize_delayed(a, amax_history, history_pos, history_len, stream);
    return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_quantize_delayed launch");
}

size_t fp8_scaled_mm_workspace_size(int64_t m, int64_t n, int64_t k, fp8_granularity ga, fp8_granularity gb)
{
    (void)ga;
    (void)gb;
    if (m <= 0 || n <= 0 || k <= 0) return 0;
    const int s = gemm_choose_splits(m, n, k);
    return s > 1 ? (size_t)s * (size_t)m * (size_t)n * sizeof(float) : 0;
}

fp8_status fp8_scaled_mm(const uint8_t* a, fp8_format fa, int64_t lda, const float* scale_a, fp8_granularity ga,
                         const uint8_t* b, fp8_format fb, int64_t ldb, const float* scale_b, fp8_granularity gb,
                         int64_t m, int64_t n, int64_t k, void* c_bf16, int64_t ldc, void* workspace,
                         size_t workspace_bytes, fp8_counters* ctr, hipStream_t stream)
{
    if (!valid_fmt(fa) || !valid_fmt(fb)) return fail(FP8_ERR_INVALID_ARG, "unknown FP8 format");
    const bool pow2 = ga == FP8_ROW_1x128_POW2 && gb == FP8_BLOCK_128x128_POW2;
    if (!pow2 && (!valid_gran(ga) || !valid_gran(gb))) return fail(FP8_ERR_INVALID_ARG, "unknown granularity");
    fp8_status s;
    if ((s = check_2d(a, m, k, lda, "a")) != FP8_OK) return s;
    if ((s = check_2d(b, n, k, ldb, "b")) != FP8_OK) return s;
    if ((s = check_2d(c_bf16, m, n, ldc, "c")) != FP8_OK) return s;
    const bool block = (ga == FP8_ROW_1x128 && gb == FP8_BLOCK_128x128) || pow2;
    if (!block && !(ga == FP8_TENSOR && gb == FP8_TENSOR))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "scale pairs: (TENSOR, TENSOR), (ROW_1x128, BLOCK_128x128) or "
                                               "(ROW_1x128_POW2, BLOCK_128x128_POW2)");
    if (block && k % 128 != 0) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "block scaling needs k % 128 == 0");
    // the operand layout rules matter only when operand bytes are read
    const bool reads = m > 0 && n > 0 && k > 0;
    if (k % 16 != 0 || (reads && (lda % 16 != 0 || ldb % 16 != 0)))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "k, lda and ldb must be multiples of 16");
    if (reads && ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "a and b must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(c_bf16)) & 1u) return fail(FP8_ERR_INVALID_ARG, "c must be 2-byte aligned");
    if (m > 0 && n > 0 && !c_bf16) return fail(FP8_ERR_INVALID_ARG, "c: null pointer");
    if (m >= ((int64_t)1 << 31) || n >= ((int64_t)1 << 31) || k >= ((int64_t)1 << 31))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "dimensions must be below 2^31");
    // byte offsets inside one 256-row operand or output tile are 32-bit
    if (reads && (lda >= ((int64_t)1 << 22) || ldb >= ((int64_t)1 << 22) || ldc >= ((int64_t)1 << 21)))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "lda, ldb must be below 2^22 and ldc below 2^21");
    if (m > 0 && n > 0 && k > 0 && (!scale_a || !scale_b)) return fail(FP8_ERR_INVALID_ARG, "scale: null pointer");
    if ((s = check_device()) != FP8_OK) return s;
    GemmArgs g;
    g.a = a;
    g.b = b;
    g.lda = lda;
    g.ldb = ldb;
    g.sa = scale_a;
    g.sb = scale_b;
    g.fa = fa;
    g.fb = fb;
    g.block_scaled = block;
    g.pow2_scales = pow2;
    g.m = m;
    g.n = n;
    g.k = k;
    g.c = c_bf16;
    g.ldc = ldc;
    g.ctr = ctr;
    g.splits = 1;
    g.ws = nullptr;
    const size_t need = fp8_scaled_mm_workspace_size(m, n, k, ga, gb);
    if (need > 0 && workspace && workspace_bytes >= need) {
        g.splits = gemm_choose_splits(m, n, k);
        g.ws = static_cast<float*>(workspace);
    }
    hipError_t e = launch_gemm(g, stream);
    return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_scaled_mm launch");
}

size_t fp8_quantize_scaled_mm_workspace_size(int64_t m, int64_t n, int64_t k)
{
    (void)m;
    (void)n;
    (void)k;
    return kAmaxWorkspaceBytes;
}

fp8_status fp8_quantize_scaled_mm(const void* x, int64_t ldx, fp8_format fa, float* scale_a, uint8_t* xq, int64_t ldxq,
                                  uint8_t* xq_t, int64_t ldxq_t, const uint8_t* b, fp8_format fb, int64_t ldb,
                                  const float* scale_b, int64_t m, int64_t n, int64_t k, void* c_bf16, int64_t ldc,
                                  fp8_counters* ctr, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!valid_fmt(fa) || !valid_fmt(fb)) return fail(FP8_ERR_INVALID_ARG, "unknown FP8 format");
    fp8_status s;
    if ((s = check_2d(x, m, k, ldx, "x")) != FP8_OK) return s;
    if ((s = check_2d(b, n, k, ldb, "b")) != FP8_OK) return s;
    if ((s = check_2d(c_bf16, m, n, ldc, "c")) != FP8_OK) return s;
    if (xq && (s = check_2d(xq, m, k, ldxq, "xq")) != FP8_OK) return s;
    if (xq_t && (s = check_2d(xq_t, k, m, ldxq_t, "xq_t")) != FP8_OK) return s;
    if (!scale_a || !scale_b) return fail(FP8_ERR_INVALID_ARG, "scale: null pointer");
    if (!workspace || workspace_bytes < kAmaxWorkspaceBytes)
        return fail(FP8_ERR_INVALID_ARG, "workspace smaller than fp8_quantize_scaled_mm_workspace_size()");
    if (k != kAstatK) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "fp8_quantize_scaled_mm takes k == 768");
    const auto mis = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; };
    if (mis(x, 16) || ldx % 8 != 0) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "x: rows must start on 16-byte boundaries");
    if (mis(b, 16) || ldb % 16 != 0) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "b: rows must start on 16-byte boundaries");
    if (xq && (mis(xq, 16) || ldxq % 16 != 0))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "xq: rows must start on 16-byte boundaries");
    if (n > 0 && (n % 4 != 0 || ldc % 4 != 0 || mis(c_bf16, 8)))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "n and ldc must be multiples of 4 and c 8-byte aligned");
    if (ldx >= ((int64_t)1 << 22) || ldb >= ((int64_t)1 << 22) || ldc >= ((int64_t)1 << 21) || m >= ((int64_t)1 << 31) ||
        n >= ((int64_t)1 << 31))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "ldx, ldb below 2^22, ldc below 2^21, m and n below 2^31");
    if ((s = check_device()) != FP8_OK) return s;
    hipError_t e;
    if (m == 0) {
        // an empty activation: scale 1, nothing else to write
        QuantArgs a;
        a.x = x;
        a.dtype = FP8_IN_BF16;
        a.rows = 0;
        a.cols = k;
        a.ld = ldx;
        a.fmt = fa;
        a.gran = FP8_TENSOR;
        a.mode = FP8_SCALE_FROM_AMAX;
        a.scale = scale_a;
        a.q = xq;
        a.ldq = ldxq;
        a.qt = nullptr;
        a.ldqt = 0;
        a.ctr = ctr;
        a.partials = static_cast<uint32_t*>(workspace);
        e = launch_quantize(a, stream);
        return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_quantize_scaled_mm launch");
    }
    int np = 0;
    e = launch_amax_partials(x, FP8_IN_BF16, m, k, ldx, static_cast<uint32_t*>(workspace), &np, stream);
    if (e != hipSuccess) return hip_fail(e, "fp8_quantize_scaled_mm amax launch");
    AstatArgs g;
    g.a = x;
    g.lda = ldx;
    g.bf16_a = true;
    g.fa = fa;
    g.b = b;
    g.ldb = ldb;
    g.fb = fb;
    g.sa = nullptr;
    g.sa_out = scale_a;
    g.sb = scale_b;
    g.partials = static_cast<const uint32_t*>(workspace);
    g.np = np;
    g.xq = xq;
    g.ldxq = ldxq;
    g.xqt = xq_t;
    g.ldxqt = ldxq_t;
    g.m = m;
    g.n = n;
    g.c = c_bf16;
    g.ldc = ldc;
    g.ctr = ctr;
    e = launch_gemm_astat(g, gemm_num_cus(), stream);
    return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_quantize_scaled_mm launch");
}

size_t fp8_requant_workspace_size(const fp8_weight_cache* caches, int32_t count)
{
    if (!caches || count <= 0) return 0;
    size_t n = 0;
    for (int32_t i = 0; i < count; ++i)
        if (caches[i].gran == FP8_TENSOR) n += kAmaxWorkspaceBytes;
    return n;
}

fp8_status fp8_requant_weights(const fp8_weight_cache* caches, const void* const* masters,
                               const fp8_dtype* master_dtypes, int32_t count, void* workspace,
                               size_t workspace_bytes, hipStream_t stream)
{
    if (count < 0) return fail(FP8_ERR_INVALID_ARG, "negative count");
    if (count == 0) return FP8_OK;
    if (!caches || !masters || !master_dtypes) return fail(FP8_ERR_INVALID_ARG, "null descriptor array");
    if (workspace_bytes < fp8_requant_workspace_size(caches, count) ||
        (fp8_requant_workspace_size(caches, count) > 0 && !workspace))
        return fail(FP8_ERR_INVALID_ARG, "workspace smaller than fp8_requant_workspace_size()");
    for (int32_t i = 0; i < count; ++i) {
        const fp8_weight_cache& c = caches[i];
        if (c.gran != FP8_TENSOR && c.gran != FP8_BLOCK_128x128)
            return fail(FP8_ERR_UNSUPPORTED_SHAPE, "weight caches use TENSOR or BLOCK_128x128 scaling");
        if (c.rows >= ((int64_t)1 << 31) || c.cols >= ((int64_t)1 << 31))
            return fail(FP8_ERR_UNSUPPORTED_SHAPE, "weight cache rows and cols must be below 2^31");
        fp8_status s = check_quantize_args(masters[i], master_dtypes[i], c.rows, c.cols, c.cols, c.fmt, c.gran,
                                           FP8_SCALE_FROM_AMAX, c.scale, c.q, c.cols, c.q_t, c.rows,
                                           c.gran == FP8_TENSOR ? workspace : nullptr,
                                           c.gran == FP8_TENSOR ? kAmaxWorkspaceBytes : 0);
        if (s != FP8_OK) return s;
    }
    fp8_status s = check_device();
    if (s != FP8_OK) return s;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    std::vector<QuantArgs> args((size_t)count);
    for (int32_t i = 0; i < count; ++i) {
        const fp8_weight_cache& c = caches[i];
        QuantArgs& a = args[(size_t)i];
        a.x = masters[i];
        a.dtype = master_dtypes[i];
        a.rows = c.rows;
        a.cols = c.cols;
        a.ld = c.cols;
        a.fmt = c.fmt;
        a.gran = c.gran;
        a.mode = FP8_SCALE_FROM_AMAX;
        a.scale = c.scale;
        a.q = c.q;
        a.ldq = c.cols;
        a.qt = c.q_t;
        a.ldqt = c.rows;
        a.ctr = c.ctr;
        a.partials = nullptr;
        if (c.gran == FP8_TENSOR) {
            a.partials = reinterpret_cast<uint32_t*>(ws);
            ws += kAmaxWorkspaceBytes;
        }
    }
    hipError_t e = launch_requant(args.data(), count, stream);
    return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_requant_weights launch");
}

fp8_status fp8_counters_reset(fp8_counters* ctr, hipStream_t stream)
{
    if (!ctr) return fail(FP8_ERR_INVALID_ARG, "counters: null pointer");
    fp8_status s = check_device();
    if (s != FP8_OK) return s;
    hipError_t e = launch_counters_reset(ctr, stream);
    return e == hipSuccess ? FP8_OK : hip_fail(e, "fp8_counters_reset launch");
}

int32_t fp8_debug_set_wait_limit(int32_t polls) { return fp8mi::set_once_wait_limit(polls); }

}  // extern "C"
