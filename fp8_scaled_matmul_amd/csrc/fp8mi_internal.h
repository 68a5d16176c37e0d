// Internal declarations shared by the C-ABI layer and the HIP kernel files.
// Not installed; the public interface is include/fp8mi.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fp8mi.h"

namespace fp8mi {

// Room for the per-workgroup partial maxima of a per-tensor amax pass (the
// workspace size), and the workgroups the pass runs on at most.  Measured on
// 8192 x 8192 with the last-level cache flushed, per-tensor quantize from
// amax: 512 workgroups 64.9 us, 1024 66.0 us, 2048 67.8 us; the step's X and
// dY quantizations were the same with all three.
constexpr int kAmaxPartials = 2048;
constexpr int kAmaxGrid = 512;
static_assert(kAmaxGrid <= kAmaxPartials, "amax grid");
constexpr size_t kAmaxWorkspaceBytes = kAmaxPartials * sizeof(uint32_t);

// Library-owned scratch of fp8_quantize_noalloc: room for the amax partials
// of one call (the largest count any tensor size produces), per device.
constexpr int kNoAllocScratchWords = kAmaxPartials;
constexpr int kMaxScratchDevices = 64;
// The calling thread's current device's scratch address (resolved once per
// device with hipGetSymbolAddress).
hipError_t noalloc_scratch(uint32_t** out);

// Quantizer launch description (all pointers device pointers).
struct QuantArgs {
    const void* x;
    int dtype;          // FP8_IN_BF16 / FP8_IN_FP32
    int64_t rows, cols, ld;
    int fmt;            // FP8_E4M3 / FP8_E5M2
    int gran;           // FP8_TENSOR / FP8_ROW_1x128 / FP8_BLOCK_128x128
    int mode;           // FP8_SCALE_FROM_AMAX / FP8_SCALE_GIVEN
    float* scale;
    uint8_t* q;
    int64_t ldq;
    uint8_t* qt;        // nullable
    int64_t ldqt;
    fp8_counters* ctr;  // nullable
    uint32_t* partials; // per-tensor FROM_AMAX workspace
    int pow2 = 0;       // FROM_AMAX with the power-of-two scale rule
};

// One weight cache of a batched refresh, as the kernels see it (kernel
// argument; all pointers device pointers).
struct RequantItem {
    const void* x;          // master [rows, cols], contiguous
    uint8_t* q;             // [rows, cols]
    uint8_t* qt;            // [cols, rows] or null
    float* scale;
    fp8_counters* ctr;      // nullable
    uint32_t* parts;        // per-tensor: this cache's partial keys
    int64_t tile0;          // first 128x128 tile of this cache in the batch's tile list
    int32_t rows, cols;
    int32_t wg0, nwg;       // per-tensor: its amax workgroups (one partial key each)
    int8_t dtype, fmt, gran;
    int8_t vec_amax, vec_tile;
    int8_t lean;            // bf16 with 16-byte rows: whole tiles go to the 512-thread tile kernel
};
constexpr int kRequantMaxCaches = 24;    // caches per launch (kernel-argument size)
constexpr int kRequantAmaxParts = 256;   // at most this many partial keys per cache
struct RequantBatch {
    int32_t count;
    int64_t total_tiles;
    RequantItem item[kRequantMaxCaches];
};

// Each launcher enqueues on `stream` and returns the hipError_t of the launch.
hipError_t launch_amax_tensor(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                              float* out, uint32_t* partials, hipStream_t stream);
hipError_t launch_amax_grouped(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                               int gran, float* out, hipStream_t stream);
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
// The bounded wait of the one-launch small-tensor quantize: polls before a
// workgroup reads the whole tensor itself; returns the previous value.
int set_once_wait_limit(int polls);
hipError_t launch_quantize_delayed(const QuantArgs& a, float* hist, int32_t* pos, int len, hipStream_t stream);
hipError_t launch_counters_reset(fp8_counters* ctr, hipStream_t stream);
// Every cache's QuantArgs (FROM_AMAX; per-tensor ones with their partials).
hipError_t launch_requant(const QuantArgs* caches, int count, hipStream_t stream);

struct GemmArgs {
    const uint8_t* a;
    const uint8_t* b;
    int64_t lda, ldb;
    const float* sa;
    const float* sb;
    int fa, fb;
    bool block_scaled;
    bool pow2_scales = false;   // block-scaled with power-of-two scales (E8M0 in the MFMA)
    int64_t m, n, k;
    void* c;
    int64_t ldc;
    float* ws;          // split-K partials, or nullptr
    int splits;
    fp8_counters* ctr;
};

// A-stationary per-tensor GEMM (gemm_astat.hip): K is one model width, a
// whole panel of A codes ([208, K], or [192, K] when cast from bf16) stays
// in LDS.  A is FP8 codes, or bf16 quantized on the way in with the amax
// scale of `partials`.
constexpr int kAstatK = 768;
struct AstatArgs {
    const void* a;
    int64_t lda;        // elements of A's dtype
    bool bf16_a;
    int fa;
    const uint8_t* b;
    int64_t ldb;
    int fb;
    const float* sa;    // FP8 A: its scale
    float* sa_out;      // bf16 A: the scale written
    const float* sb;
    const uint32_t* partials;   // bf16 A: amax partial keys
    int np;
    uint8_t* xq;        // bf16 A, optional outputs: codes [m, k] and transposed [k, m]
    int64_t ldxq;
    uint8_t* xqt;
    int64_t ldxqt;
    int64_t m, n;
    void* c;
    int64_t ldc;
    fp8_counters* ctr;
};
bool astat_supported(int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb, int64_t ldc, const void* c);
hipError_t launch_gemm_astat(const AstatArgs& g, int num_cus, hipStream_t stream);
// The first pass of per-tensor quantization: amax partial keys of x; *np
// receives their count (at most kAmaxPartials).
hipError_t launch_amax_partials(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                                uint32_t* partials, int* np, hipStream_t stream);

int gemm_choose_splits(int64_t m, int64_t n, int64_t k);
int gemm_num_cus();
hipError_t launch_gemm_persistent(const GemmArgs& g, int num_cus, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);

}  // namespace fp8mi
