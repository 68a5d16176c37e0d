// FP8 quantizer kernels for gfx950: amax, per-tensor cast (streaming and
// 128x128 tiled with transposed output), 1x128 row-tile and 128x128 block
// quantization.
//
// What they compute (scale, then cast; saturate above the format maximum;
// underflow to signed zero) is the quantization of "#84 FP8 Precision"
// (section "Explanation": divide by the scale before the cast) with the range
// rules of "FP8 stability guardrails" (section "Why FP8 is tempting and why it
// is fragile") and its fine-grained tile / block scaling ("Real products").
//
// Memory-bound design: every thread moves 16-byte vectors; per-tensor scaling
// is two passes (amax partials, then cast) with the scale kept on the device;
// fine-grained scaling is one fused pass per tile or block.
#include <algorithm>

#include "device_common.h"
#include "fastdiv.h"
#include "fp8mi_internal.h"

namespace fp8mi {

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ loads
// 8 consecutive elements as fp32 plus their amax key.  DT 0 = bf16, 1 = fp32.
template <int DT>
__device__ inline void load8(const void* base, int64_t idx, float v[8], uint32_t& key)
{
    if constexpr (DT == 0) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(ws[i]);
            v[2 * i + 1] = bf16_hi(ws[i]);
            key = key_merge(key, absbits_bf16(ws[i] & 0xFFFFu));
            key = key_merge(key, absbits_bf16(ws[i] >> 16));
        }
    } else {
        const float* p = static_cast<const float*>(base) + idx;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
#pragma unroll
        for (int i = 0; i < 8; ++i) key = key_merge(key, absbits_f32(__builtin_bit_cast(uint32_t, v[i])));
    }
}

template <int DT>
__device__ inline float load1(const void* base, int64_t idx, uint32_t& key)
{
    if constexpr (DT == 0) {
        const uint32_t h = static_cast<const uint16_t*>(base)[idx];
        key = key_merge(key, absbits_bf16(h));
        return __builtin_bit_cast(float, h << 16);
    } else {
        const float f = static_cast<const float*>(base)[idx];
        key = key_merge(key, absbits_f32(__builtin_bit_cast(uint32_t, f)));
        return f;
    }
}

// Quotients of 8 values, then 8 codes packed in two words.
template <int FMT, bool FAST>
__device__ inline uint2 cast8(const float x[8], float s, float r, uint32_t& sat, uint32_t& und,
                              uint32_t& nan)
{
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = FAST ? quot_corrected(x[i], s, r) : x[i] / s;
    uint2 o;
    if constexpr (FAST) {
        o.x = encode4_fast<FMT>(v, x, und);
        o.y = encode4_fast<FMT>(v + 4, x + 4, und);
    } else {
        o.x = encode4_general<FMT>(v, x, s, sat, und, nan);
        o.y = encode4_general<FMT>(v + 4, x + 4, s, sat, und, nan);
    }
    return o;
}

template <int FMT, bool FAST>
__device__ inline uint8_t cast1(float x, float s, float r, uint32_t& sat, uint32_t& und, uint32_t& nan)
{
    float xs[4] = {x, 0.0f, 0.0f, 0.0f};
    float v[4] = {FAST ? quot_corrected(x, s, r) : x / s, 0.0f, 0.0f, 0.0f};
    uint32_t w = FAST ? encode4_fast<FMT>(v, xs, und) : encode4_general<FMT>(v, xs, s, sat, und, nan);
    return (uint8_t)(w & 0xFFu);
}

// Reduce the per-tensor amax partials (bit 31 = a non-finite element was
// seen) inside every consuming workgroup; returns the merged key.
__device__ inline uint32_t reduce_partials(const uint32_t* partials, int np)
{
    __shared__ uint32_t sh[kThreads / 64];
    uint32_t k = 0;
    for (int i = threadIdx.x; i < np; i += blockDim.x) k = key_merge(k, partials[i]);
    k = wave_key_merge(k);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = k;
    __syncthreads();
    k = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) k = key_merge(k, sh[w]);
    __syncthreads();
    return k;
}

__device__ inline uint32_t block_key_merge(uint32_t k)
{
    __shared__ uint32_t sh[kThreads / 64];
    k = wave_key_merge(k);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = k;
    __syncthreads();
    k = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) k = key_merge(k, sh[w]);
    __syncthreads();
    return k;
}

// ------------------------------------------------------------------ amax
// Pass 1 of per-tensor scaling: each workgroup reduces a grid-strided share
// of the [rows, cols] tensor (a contiguous tensor arrives as one long row) to
// one key.  vec: rows start 16-byte aligned, so 8-element vectors are used.
template <int DT>
__global__ void __launch_bounds__(kThreads) k_amax_partials(const void* x, int64_t rows, int64_t cols,
                                                            int64_t ld, int vec, uint32_t* partials)
{
    uint32_t key = 0;
    const int64_t nvec = vec ? cols / 8 : 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const int64_t base = r * ld;
        int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        // four vectors in flight per thread
        for (; i + 3 * stride < nvec; i += 4 * stride) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 4; ++u) load8<DT>(x, base + (i + u * stride) * 8, v, key);
        }
        for (; i < nvec; i += stride) {
            float v[8];
            load8<DT>(x, base + i * 8, v, key);
        }
        for (int64_t c = nvec * 8 + (int64_t)blockIdx.x * kThreads + threadIdx.x; c < cols; c += stride)
            (void)load1<DT>(x, base + c, key);
    }
    key = block_key_merge(key);
    if (threadIdx.x == 0) partials[blockIdx.y * gridDim.x + blockIdx.x] = key;
}

__global__ void __launch_bounds__(kThreads) k_amax_finalize(const uint32_t* partials, int np, float* out)
{
    const uint32_t k = reduce_partials(partials, np);
    if (threadIdx.x == 0) out[0] = key_amax(k);
}

// ------------------------------------------------------------------ per-tensor cast
// Pass 2 of per-tensor scaling (or the whole job with a given scale): every
// workgroup rebuilds the amax from the partials, derives s, and streams its
// share of x -> q.  16 elements (32 B of bf16 in, 16 B out) per vector.
template <int FMT, int DT, bool FAST>
__device__ inline void cast_stream(const void* x, int64_t rows, int64_t cols, int64_t ld, int vec,
                                   uint8_t* q, int64_t ldq, float s, float r, uint32_t& sat,
                                   uint32_t& und, uint32_t& nan)
{
    const int64_t nvec = vec ? cols / 16 : 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
        const int64_t xb = row * ld, qb = row * ldq;
        int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        for (; i + stride < nvec; i += 2 * stride) {
            float a[8], b[8], c[8], d[8];
            uint32_t dummy = 0;
            load8<DT>(x, xb + i * 16, a, dummy);
            load8<DT>(x, xb + i * 16 + 8, b, dummy);
            load8<DT>(x, xb + (i + stride) * 16, c, dummy);
            load8<DT>(x, xb + (i + stride) * 16 + 8, d, dummy);
            const uint2 oa = cast8<FMT, FAST>(a, s, r, sat, und, nan);
            const uint2 ob = cast8<FMT, FAST>(b, s, r, sat, und, nan);
            const uint2 oc = cast8<FMT, FAST>(c, s, r, sat, und, nan);
            const uint2 od = cast8<FMT, FAST>(d, s, r, sat, und, nan);
            *reinterpret_cast<uint4*>(q + qb + i * 16) = make_uint4(oa.x, oa.y, ob.x, ob.y);
            *reinterpret_cast<uint4*>(q + qb + (i + stride) * 16) = make_uint4(oc.x, oc.y, od.x, od.y);
        }
        for (; i < nvec; i += stride) {
            float a[8], b[8];
            uint32_t dummy = 0;
            load8<DT>(x, xb + i * 16, a, dummy);
            load8<DT>(x, xb + i * 16 + 8, b, dummy);
            const uint2 oa = cast8<FMT, FAST>(a, s, r, sat, und, nan);
            const uint2 ob = cast8<FMT, FAST>(b, s, r, sat, und, nan);
            *reinterpret_cast<uint4*>(q + qb + i * 16) = make_uint4(oa.x, oa.y, ob.x, ob.y);
        }
        for (int64_t c = nvec * 16 + (int64_t)blockIdx.x * kThreads + threadIdx.x; c < cols; c += stride) {
            uint32_t dummy = 0;
            q[qb + c] = cast1<FMT, FAST>(load1<DT>(x, xb + c, dummy), s, r, sat, und, nan);
        }
    }
}

template <int FMT, int DT>
__global__ void __launch_bounds__(kThreads) k_cast_tensor(const void* x, int64_t rows, int64_t cols,
                                                          int64_t ld, int vec, uint8_t* q, int64_t ldq,
                                                          float* scale, const uint32_t* partials, int np,
                                                          fp8_counters* ctr)
{
    float s;
    bool special = true;
    if (partials) {
        const uint32_t k = reduce_partials(partials, np);
        special = key_special(k);
        s = scale_from_amax<FMT>(key_amax(k));
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) scale[0] = s;
    } else {
        s = scale[0];
    }
    uint32_t sat = 0, und = 0, nan = 0;
    const bool fast = DT == 0 && partials && !special && s >= kCorrectedQuotMinScale;
    if (fast) {
        const float r = 1.0f / s;
        cast_stream<FMT, DT, true>(x, rows, cols, ld, vec, q, ldq, s, r, sat, und, nan);
    } else {
        cast_stream<FMT, DT, false>(x, rows, cols, ld, vec, q, ldq, s, 0.0f, sat, und, nan);
    }
    flush_counters(ctr, sat, und, nan);
}

// ------------------------------------------------------------------ 128x128 tiles
// One workgroup per 128x128 tile (grid-strided).  Thread t owns column chunk
// 8*(t%16) of rows t/16 + 16 i, i = 0..7: 64 elements.  SCALE_MODE:
//   0  one scale for the tensor (from partials, or given in scale[0]);
//   1  one scale per 128x128 block from the block's own amax;
//   2  one given scale per block.
// With qt, the codes go through LDS and leave transposed: thread t writes 64
// consecutive bytes of column (t % 128), rows 64 (t / 128) ...
constexpr int kTile = 128;
constexpr int kTilePitch = kTile + 8;   // bytes per LDS row

template <int FMT, int DT, int SCALE_MODE, bool AMAX_ONLY>
__global__ void __launch_bounds__(kThreads) k_tile128(const void* x, int64_t rows, int64_t cols,
                                                      int64_t ld, int vec, float* scale,
                                                      const uint32_t* partials, int np, uint8_t* q,
                                                      int64_t ldq, uint8_t* qt, int64_t ldqt,
                                                      fp8_counters* ctr)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kTilePitch];
    const int t = threadIdx.x;
    const int cc = (t & 15) * 8;
    const int rr = t >> 4;
    const int64_t tiles_c = (cols + kTile - 1) / kTile;
    const int64_t tiles_r = (rows + kTile - 1) / kTile;
    const int64_t ntiles = tiles_r * tiles_c;

    float s_tensor = 1.0f;
    bool special_tensor = true;
    if constexpr (SCALE_MODE == 0) {
        if (partials) {
            const uint32_t k = reduce_partials(partials, np);
            special_tensor = key_special(k);
            s_tensor = scale_from_amax<FMT>(key_amax(k));
            if (blockIdx.x == 0 && t == 0) scale[0] = s_tensor;
        } else {
            s_tensor = scale[0];
        }
    }
    uint32_t sat = 0, und = 0, nan = 0;

    for (int64_t tid = blockIdx.x; tid < ntiles; tid += gridDim.x) {
        const int64_t r0 = (tid / tiles_c) * kTile;
        const int64_t c0 = (tid % tiles_c) * kTile;
        const bool full = vec && r0 + kTile <= rows && c0 + kTile <= cols;
        float xv[8][8];
        uint32_t key = 0;
        if (full) {
#pragma unroll
            for (int i = 0; i < 8; ++i) load8<DT>(x, (r0 + rr + 16 * i) * ld + c0 + cc, xv[i], key);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int64_t r = r0 + rr + 16 * i, c = c0 + cc + j;
                    xv[i][j] = (r < rows && c < cols) ? load1<DT>(x, r * ld + c, key) : 0.0f;
                }
        }
        float s;
        bool fast;
        if constexpr (SCALE_MODE == 0) {
            s = s_tensor;
            fast = DT == 0 && partials && !special_tensor && s >= kCorrectedQuotMinScale;
        } else if constexpr (SCALE_MODE == 1) {
            key = block_key_merge(key);
            const int64_t sidx = (r0 / kTile) * tiles_c + c0 / kTile;
            if constexpr (AMAX_ONLY) {
                if (t == 0) scale[sidx] = key_amax(key);
                continue;
            }
            s = scale_from_amax<FMT>(key_amax(key));
            if (t == 0) scale[sidx] = s;
            fast = DT == 0 && !key_special(key) && s >= kCorrectedQuotMinScale;
        } else {
            s = scale[(r0 / kTile) * tiles_c + c0 / kTile];
            fast = false;
        }
        uint2 codes[8];
        if (fast) {
            const float r = 1.0f / s;
#pragma unroll
            for (int i = 0; i < 8; ++i) codes[i] = cast8<FMT, true>(xv[i], s, r, sat, und, nan);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (full) {
                    codes[i] = cast8<FMT, false>(xv[i], s, 0.0f, sat, und, nan);
                } else {
                    // count only elements inside the tensor
                    uint32_t w[2] = {0, 0};
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int64_t r = r0 + rr + 16 * i, c = c0 + cc + j;
                        if (r < rows && c < cols)
                            w[j >> 2] |= (uint32_t)cast1<FMT, false>(xv[i][j], s, 0.0f, sat, und, nan) << (8 * (j & 3));
                    }
                    codes[i] = make_uint2(w[0], w[1]);
                }
            }
        }
        // row-major output
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + rr + 16 * i;
            if (full) {
                *reinterpret_cast<uint2*>(q + r * ldq + c0 + cc) = codes[i];
            } else if (r < rows) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (c0 + cc + j < cols)
                        q[r * ldq + c0 + cc + j] = (uint8_t)(((j < 4 ? codes[i].x : codes[i].y) >> (8 * (j & 3))) & 0xFFu);
            }
        }
        if (qt) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<uint2*>(&tile[(rr + 16 * i) * kTilePitch + cc]) = codes[i];
            __syncthreads();
            const int col = t & 127;
            const int rh = (t >> 7) * 64;
            if (c0 + col < cols) {
                uint32_t w[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t b0 = tile[(rh + 4 * j + 0) * kTilePitch + col];
                    const uint32_t b1 = tile[(rh + 4 * j + 1) * kTilePitch + col];
                    const uint32_t b2 = tile[(rh + 4 * j + 2) * kTilePitch + col];
                    const uint32_t b3 = tile[(rh + 4 * j + 3) * kTilePitch + col];
                    w[j] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
                }
                uint8_t* dst = qt + (c0 + col) * ldqt + r0 + rh;
                if (full) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<uint4*>(dst + 16 * j) = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
                } else {
                    for (int j = 0; j < 64 && r0 + rh + j < rows; ++j) dst[j] = (uint8_t)(w[j >> 2] >> (8 * (j & 3)));
                }
            }
            __syncthreads();
        }
    }
    if constexpr (!AMAX_ONLY) flush_counters(ctr, sat, und, nan);
}

// ------------------------------------------------------------------ 1x128 row tiles
// 16 lanes per tile, 8 elements per lane; the 16-lane group reduces its amax
// with lane shuffles, derives its scale and casts.  Scales [rows, ceil(cols/128)].
template <int FMT, int DT, bool GIVEN, bool AMAX_ONLY>
__global__ void __launch_bounds__(kThreads) k_row1x128(const void* x, int64_t rows, int64_t cols,
                                                       int64_t ld, int vec, float* scale, uint8_t* q,
                                                       int64_t ldq, fp8_counters* ctr, uint32_t ntiles,
                                                       FastDiv tiles_per_row)
{
    const int lane = threadIdx.x & 15;
    const uint32_t group = (blockIdx.x * kThreads + threadIdx.x) >> 4;
    const uint32_t ngroups = (gridDim.x * kThreads) >> 4;
    uint32_t sat = 0, und = 0, nan = 0;
    for (uint32_t tile = group; tile < ntiles; tile += ngroups) {
        const uint32_t row = tiles_per_row.div(tile);
        const uint32_t tc = tile - row * tiles_per_row.d;
        const int64_t c = (int64_t)tc * 128 + lane * 8;
        const int64_t base = (int64_t)row * ld;
        const bool full = vec && (int64_t)tc * 128 + 128 <= cols;
        float xv[8];
        uint32_t key = 0;
        if (full) {
            load8<DT>(x, base + c, xv, key);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) xv[j] = c + j < cols ? load1<DT>(x, base + c + j, key) : 0.0f;
        }
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) key = key_merge(key, __shfl_xor(key, off, 16));
        const int64_t sidx = (int64_t)row * tiles_per_row.d + tc;
        if constexpr (AMAX_ONLY) {
            if (lane == 0) scale[sidx] = key_amax(key);
            continue;
        }
        float s;
        bool fast;
        if constexpr (GIVEN) {
            s = scale[sidx];
            fast = false;
        } else {
            s = scale_from_amax<FMT>(key_amax(key));
            if (lane == 0) scale[sidx] = s;
            fast = DT == 0 && !key_special(key) && s >= kCorrectedQuotMinScale;
        }
        uint2 o;
        if (full) {
            o = fast ? cast8<FMT, true>(xv, s, 1.0f / s, sat, und, nan)
                     : cast8<FMT, false>(xv, s, 0.0f, sat, und, nan);
            *reinterpret_cast<uint2*>(q + (int64_t)row * ldq + c) = o;
        } else {
            for (int j = 0; j < 8; ++j)
                if (c + j < cols)
                    q[(int64_t)row * ldq + c + j] = fast ? cast1<FMT, true>(xv[j], s, 1.0f / s, sat, und, nan)
                                                         : cast1<FMT, false>(xv[j], s, 0.0f, sat, und, nan);
        }
    }
    if constexpr (!AMAX_ONLY) flush_counters(ctr, sat, und, nan);
}

__global__ void k_counters_reset(fp8_counters* ctr)
{
    if (threadIdx.x < 4) reinterpret_cast<unsigned long long*>(ctr)[threadIdx.x] = 0ull;
}

__global__ void k_store_one(float* p)
{
    if (threadIdx.x == 0) p[0] = 1.0f;
}

// ------------------------------------------------------------------ host helpers
int g_num_cus = 0;

int num_cus()
{
    if (g_num_cus == 0) {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            g_num_cus = n;
        else
            g_num_cus = 256;
    }
    return g_num_cus;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Flatten a contiguous tensor into one long row.
void flatten(int64_t& rows, int64_t& cols, int64_t& ld, int64_t* ldq = nullptr)
{
    if (rows > 1 && ld == cols && (!ldq || *ldq == cols)) {
        cols = rows * cols;
        ld = cols;
        if (ldq) *ldq = cols;
        rows = 1;
    }
}

dim3 stream_grid(int64_t rows, int64_t cols, int per_thread, int max_wg)
{
    const int64_t work = cdiv(cols, (int64_t)kThreads * per_thread);
    int64_t gx = std::min<int64_t>(std::max<int64_t>(work, 1), max_wg);
    int64_t gy = std::min<int64_t>(std::max<int64_t>(rows, 1), std::max<int64_t>(1, max_wg / gx));
    return dim3((unsigned)gx, (unsigned)gy, 1);
}

template <int FMT, int DT>
hipError_t quantize_typed(const QuantArgs& a, hipStream_t stream)
{
    const int eb = DT == 0 ? 2 : 4;
    const int64_t rows = a.rows, cols = a.cols;
    if (a.gran == FP8_TENSOR) {
        const bool from_amax = a.mode == FP8_SCALE_FROM_AMAX;
        int np = 0;
        if (from_amax) {
            int64_t r = rows, c = cols, ld = a.ld;
            flatten(r, c, ld);
            const int vec = aligned16(a.x) && (r == 1 || (ld * eb) % 16 == 0);
            const dim3 g = stream_grid(r, c, 32, kAmaxPartials);
            np = (int)(g.x * g.y);
            hipLaunchKernelGGL(k_amax_partials<DT>, g, dim3(kThreads), 0, stream, a.x, r, c, ld, vec,
                               a.partials);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const uint32_t* parts = from_amax ? a.partials : nullptr;
        if (a.qt) {
            const int vec = aligned16(a.x) && aligned16(a.q) && aligned16(a.qt) && (a.ld * eb) % 16 == 0 &&
                            a.ldq % 8 == 0 && a.ldqt % 16 == 0;
            const int64_t nt = cdiv(rows, kTile) * cdiv(cols, kTile);
            const int grid = (int)std::min<int64_t>(nt, (int64_t)num_cus() * 8);
            hipLaunchKernelGGL((k_tile128<FMT, DT, 0, false>), dim3(grid), dim3(kThreads), 0, stream, a.x,
                               rows, cols, a.ld, vec, a.scale, parts, np, a.q, a.ldq, a.qt, a.ldqt, a.ctr);
        } else {
            int64_t r = rows, c = cols, ld = a.ld, ldq = a.ldq;
            flatten(r, c, ld, &ldq);
            const int vec = aligned16(a.x) && aligned16(a.q) &&
                            (r == 1 || ((ld * eb) % 16 == 0 && ldq % 16 == 0));
            const dim3 g = stream_grid(r, c, 32, num_cus() * 8);
            hipLaunchKernelGGL((k_cast_tensor<FMT, DT>), g, dim3(kThreads), 0, stream, a.x, r, c, ld, vec,
                               a.q, ldq, a.scale, parts, np, a.ctr);
        }
        return hipGetLastError();
    }
    if (a.gran == FP8_BLOCK_128x128) {
        const int vec = aligned16(a.x) && aligned16(a.q) && (!a.qt || aligned16(a.qt)) && (a.ld * eb) % 16 == 0 &&
                        a.ldq % 8 == 0 && (!a.qt || a.ldqt % 16 == 0);
        const int64_t nt = cdiv(rows, kTile) * cdiv(cols, kTile);
        const int grid = (int)std::min<int64_t>(nt, (int64_t)num_cus() * 8);
        if (a.mode == FP8_SCALE_FROM_AMAX)
            hipLaunchKernelGGL((k_tile128<FMT, DT, 1, false>), dim3(grid), dim3(kThreads), 0, stream, a.x, rows,
                               cols, a.ld, vec, a.scale, nullptr, 0, a.q, a.ldq, a.qt, a.ldqt, a.ctr);
        else
            hipLaunchKernelGGL((k_tile128<FMT, DT, 2, false>), dim3(grid), dim3(kThreads), 0, stream, a.x, rows,
                               cols, a.ld, vec, a.scale, nullptr, 0, a.q, a.ldq, a.qt, a.ldqt, a.ctr);
        return hipGetLastError();
    }
    // ROW_1x128
    const int64_t tpr = cdiv(cols, 128);
    const int64_t ntiles = rows * tpr;
    const int vec = aligned16(a.x) && (a.ld * eb) % 16 == 0 && a.ldq % 8 == 0 && aligned16(a.q);
    const int grid = (int)std::min<int64_t>(cdiv(ntiles, kThreads / 16), (int64_t)num_cus() * 16);
    if (a.mode == FP8_SCALE_FROM_AMAX)
        hipLaunchKernelGGL((k_row1x128<FMT, DT, false, false>), dim3(grid), dim3(kThreads), 0, stream, a.x, rows,
                           cols, a.ld, vec, a.scale, a.q, a.ldq, a.ctr, (uint32_t)ntiles, FastDiv((uint32_t)tpr));
    else
        hipLaunchKernelGGL((k_row1x128<FMT, DT, true, false>), dim3(grid), dim3(kThreads), 0, stream, a.x, rows,
                           cols, a.ld, vec, a.scale, a.q, a.ldq, a.ctr, (uint32_t)ntiles, FastDiv((uint32_t)tpr));
    return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ launchers
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream)
{
    if (a.rows == 0 || a.cols == 0) {
        // nothing to cast; an amax-scaled tensor still reports scale 1
        if (a.gran == FP8_TENSOR && a.mode == FP8_SCALE_FROM_AMAX) {
            hipLaunchKernelGGL(k_store_one, dim3(1), dim3(64), 0, stream, a.scale);
            return hipGetLastError();
        }
        return hipSuccess;
    }
    if (a.fmt == FP8_E4M3)
        return a.dtype == FP8_IN_BF16 ? quantize_typed<0, 0>(a, stream) : quantize_typed<0, 1>(a, stream);
    return a.dtype == FP8_IN_BF16 ? quantize_typed<1, 0>(a, stream) : quantize_typed<1, 1>(a, stream);
}

hipError_t launch_amax_tensor(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, float* out,
                              uint32_t* partials, hipStream_t stream)
{
    const int eb = dtype == FP8_IN_BF16 ? 2 : 4;
    int64_t r = rows, c = cols, l = ld;
    flatten(r, c, l);
    const int vec = aligned16(x) && (r == 1 || (l * eb) % 16 == 0);
    dim3 g = stream_grid(r, c, 32, kAmaxPartials);
    if (rows == 0 || cols == 0) { r = 0; g = dim3(1, 1, 1); }
    if (dtype == FP8_IN_BF16)
        hipLaunchKernelGGL(k_amax_partials<0>, g, dim3(kThreads), 0, stream, x, r, c, l, vec, partials);
    else
        hipLaunchKernelGGL(k_amax_partials<1>, g, dim3(kThreads), 0, stream, x, r, c, l, vec, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(kThreads), 0, stream, partials, (int)(g.x * g.y), out);
    return hipGetLastError();
}

hipError_t launch_amax_grouped(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int gran,
                               float* out, hipStream_t stream)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    const int eb = dtype == FP8_IN_BF16 ? 2 : 4;
    const int vec = aligned16(x) && (ld * eb) % 16 == 0;
    if (gran == FP8_BLOCK_128x128) {
        const int64_t nt = cdiv(rows, kTile) * cdiv(cols, kTile);
        const int grid = (int)std::min<int64_t>(nt, (int64_t)num_cus() * 8);
        if (dtype == FP8_IN_BF16)
            hipLaunchKernelGGL((k_tile128<0, 0, 1, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows, cols, ld,
                               vec, out, nullptr, 0, nullptr, 0, nullptr, 0, nullptr);
        else
            hipLaunchKernelGGL((k_tile128<0, 1, 1, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows, cols, ld,
                               vec, out, nullptr, 0, nullptr, 0, nullptr, 0, nullptr);
        return hipGetLastError();
    }
    const int64_t tpr = cdiv(cols, 128);
    const int64_t ntiles = rows * tpr;
    const int grid = (int)std::min<int64_t>(cdiv(ntiles, kThreads / 16), (int64_t)num_cus() * 16);
    if (dtype == FP8_IN_BF16)
        hipLaunchKernelGGL((k_row1x128<0, 0, false, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows, cols,
                           ld, vec, out, nullptr, 0, nullptr, (uint32_t)ntiles, FastDiv((uint32_t)tpr));
    else
        hipLaunchKernelGGL((k_row1x128<0, 1, false, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows, cols,
                           ld, vec, out, nullptr, 0, nullptr, (uint32_t)ntiles, FastDiv((uint32_t)tpr));
    return hipGetLastError();
}

hipError_t launch_counters_reset(fp8_counters* ctr, hipStream_t stream)
{
    hipLaunchKernelGGL(k_counters_reset, dim3(1), dim3(64), 0, stream, ctr);
    return hipGetLastError();
}

}  // namespace fp8mi
