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
#include <atomic>
#include <mutex>

#include "device_common.h"
#include "fastdiv.h"
#include "fp8mi_internal.h"

namespace fp8mi {

namespace {

constexpr int kThreads = 256;

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Fast amax of bf16 data: the |x| bit patterns of two elements per word,
// maxed two at a time (v_pk_max_u16).  Patterns of finite values order like
// their magnitudes; a result >= 0x7F80 means some element was Inf or NaN, and
// the caller then redoes the exact, flag-carrying merge (key_merge).
__device__ inline us2 pkmax8(us2 m, const uint4& w)
{
    m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w.x & 0x7FFF7FFFu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w.y & 0x7FFF7FFFu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w.z & 0x7FFF7FFFu));
    m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w.w & 0x7FFF7FFFu));
    return m;
}
// The packed max as an fp32 |x| bit pattern (>= 0x7F800000: non-finite seen).
__device__ inline uint32_t pk_raw(us2 m) { return (uint32_t)(m.x > m.y ? m.x : m.y) << 16; }
constexpr uint32_t kRawNonFinite = 0x7F800000u;

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

constexpr int kMaxWaves = 16;

// Reduce the per-tensor amax partials (bit 31 = a non-finite element was
// seen) inside every consuming workgroup; returns the merged key.
__device__ inline uint32_t reduce_partials(const uint32_t* partials, int np)
{
    __shared__ uint32_t sh[kMaxWaves];   // any workgroup size up to 1024
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
    __shared__ uint32_t sh[kMaxWaves];   // any workgroup size up to 1024
    k = wave_key_merge(k);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = k;
    __syncthreads();
    k = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) k = key_merge(k, sh[w]);
    __syncthreads();
    return k;
}

// ------------------------------------------------------------------ amax
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(0) (gfx9 encoding, no LDS or export wait) as a builtin.
constexpr unsigned kWaitVmcnt0 = 0x0F70u;

// 16 bytes read once: a nontemporal load (the data is not reused).
__device__ inline uint4 ld_stream(const void* p)
{
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Each workgroup reads a contiguous range of each row it is given (DRAM
// pages stay open: measured faster than a grid-strided interleave).
template <int DT, bool EXACT>
__device__ inline uint32_t amax_share(const void* x, int64_t rows, int64_t cols, int64_t ld, int vec)
{
    uint32_t key = 0;           // EXACT: merged key; else fp32 |x| bits max (fp32 input)
    us2 pk = us2{0, 0};         // bf16 fast path
    const int64_t nvec = vec ? cols / 8 : 0;
    const int64_t per = (nvec + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = min(nvec, b0 + per);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const int64_t base = r * ld;
        int64_t i = b0 + threadIdx.x;
        if constexpr (DT == 0 && !EXACT) {
            const uint16_t* xb = static_cast<const uint16_t*>(x) + base;
            for (; i + 7 * kThreads < b1; i += 8 * kThreads) {
                uint4 w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) w[u] = ld_stream(xb + (i + u * kThreads) * 8);
#pragma unroll
                for (int u = 0; u < 8; ++u) pk = pkmax8(pk, w[u]);
            }
            for (; i < b1; i += kThreads) pk = pkmax8(pk, ld_stream(xb + i * 8));
            for (int64_t c = nvec * 8 + (int64_t)blockIdx.x * kThreads + threadIdx.x; c < cols; c += stride) {
                const uint32_t h = xb[c] & 0x7FFFu;
                pk.x = pk.x > h ? pk.x : (unsigned short)h;
            }
        } else if constexpr (DT == 1 && !EXACT) {
            const uint32_t* xb = static_cast<const uint32_t*>(x) + base;
            for (; i + 3 * kThreads < b1; i += 4 * kThreads) {
                uint4 w[8];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    w[2 * u] = ld_stream(xb + (i + u * kThreads) * 8);
                    w[2 * u + 1] = ld_stream(xb + (i + u * kThreads) * 8 + 4);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    key = max(max(max(key, w[u].x & 0x7FFFFFFFu), max(w[u].y & 0x7FFFFFFFu, w[u].z & 0x7FFFFFFFu)),
                              w[u].w & 0x7FFFFFFFu);
            }
            for (; i < b1; i += kThreads) {
                const uint4 a = ld_stream(xb + i * 8);
                const uint4 b = ld_stream(xb + i * 8 + 4);
                key = max(max(max(key, a.x & 0x7FFFFFFFu), max(a.y & 0x7FFFFFFFu, a.z & 0x7FFFFFFFu)),
                          a.w & 0x7FFFFFFFu);
                key = max(max(max(key, b.x & 0x7FFFFFFFu), max(b.y & 0x7FFFFFFFu, b.z & 0x7FFFFFFFu)),
                          b.w & 0x7FFFFFFFu);
            }
            for (int64_t c = nvec * 8 + (int64_t)blockIdx.x * kThreads + threadIdx.x; c < cols; c += stride)
                key = max(key, xb[c] & 0x7FFFFFFFu);
        } else {
            for (; i < b1; i += kThreads) {
                float v[8];
                load8<DT>(x, base + i * 8, v, key);
            }
            for (int64_t c = nvec * 8 + (int64_t)blockIdx.x * kThreads + threadIdx.x; c < cols; c += stride)
                (void)load1<DT>(x, base + c, key);
        }
    }
    if constexpr (DT == 0 && !EXACT) key = pk_raw(pk);
    return key;
}

// Pass 1 of per-tensor scaling: each workgroup reduces a grid-strided share
// of the [rows, cols] tensor (a contiguous tensor arrives as one long row) to
// one key.  vec: rows start 16-byte aligned, so 8-element vectors are used.
// A thread whose share holds an Inf or NaN redoes it with the exact merge.
template <int DT>
__global__ void __launch_bounds__(kThreads) k_amax_partials(const void* x, int64_t rows, int64_t cols,
                                                            int64_t ld, int vec, uint32_t* partials)
{
    uint32_t key = amax_share<DT, false>(x, rows, cols, ld, vec);
    if (key >= kRawNonFinite) key = amax_share<DT, true>(x, rows, cols, ld, vec);
    key = block_key_merge(key);
    if (threadIdx.x == 0) partials[blockIdx.y * gridDim.x + blockIdx.x] = key;
}

__global__ void __launch_bounds__(kThreads) k_amax_finalize(const uint32_t* partials, int np, float* out)
{
    const uint32_t k = reduce_partials(partials, np);
    if (threadIdx.x == 0) out[0] = key_amax(k);
}

// Delayed scaling: s from the largest history entry (entries are finite and
// >= 0, so their bit patterns order like their values).
template <int FMT>
__global__ void __launch_bounds__(kThreads) k_delayed_scale(const float* hist, int len, float* scale)
{
    const uint32_t k = reduce_partials(reinterpret_cast<const uint32_t*>(hist), len);
    if (threadIdx.x == 0) scale[0] = scale_from_amax<FMT>(key_amax(k));
}

// Delayed scaling, after the cast: this tensor's amax (finite maximum, from
// the partial keys) replaces the oldest history entry; the position advances.
__global__ void __launch_bounds__(kThreads) k_delayed_record(const uint32_t* partials, int np, float* hist,
                                                             int32_t* pos, int len)
{
    const uint32_t k = reduce_partials(partials, np);
    if (threadIdx.x == 0) {
        int p = pos[0] % len;
        if (p < 0) p += len;
        hist[p] = key_amax(k);
        pos[0] = (p + 1) % len;
    }
}

// ------------------------------------------------------------------ per-tensor cast
// Pass 2 of per-tensor scaling (or the whole job with a given scale): every
// workgroup rebuilds the amax from the partials, derives s, and streams its
// share of x -> q.  16 elements (32 B of bf16 in, 16 B out) per vector.
// This form divides (IEEE) and keeps every counter: fp32 input, non-finite
// tensors, scales outside the corrected quotient's range.
template <int FMT, int DT>
__device__ inline void cast_stream(const void* x, int64_t rows, int64_t cols, int64_t ld, int vec,
                                   uint8_t* q, int64_t ldq, float s, uint32_t& sat, uint32_t& und, uint32_t& nan)
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
            const uint2 oa = cast8<FMT, false>(a, s, 0.0f, sat, und, nan);
            const uint2 ob = cast8<FMT, false>(b, s, 0.0f, sat, und, nan);
            const uint2 oc = cast8<FMT, false>(c, s, 0.0f, sat, und, nan);
            const uint2 od = cast8<FMT, false>(d, s, 0.0f, sat, und, nan);
            *reinterpret_cast<uint4*>(q + qb + i * 16) = make_uint4(oa.x, oa.y, ob.x, ob.y);
            *reinterpret_cast<uint4*>(q + qb + (i + stride) * 16) = make_uint4(oc.x, oc.y, od.x, od.y);
        }
        for (; i < nvec; i += stride) {
            float a[8], b[8];
            uint32_t dummy = 0;
            load8<DT>(x, xb + i * 16, a, dummy);
            load8<DT>(x, xb + i * 16 + 8, b, dummy);
            const uint2 oa = cast8<FMT, false>(a, s, 0.0f, sat, und, nan);
            const uint2 ob = cast8<FMT, false>(b, s, 0.0f, sat, und, nan);
            *reinterpret_cast<uint4*>(q + qb + i * 16) = make_uint4(oa.x, oa.y, ob.x, ob.y);
        }
        for (int64_t c = nvec * 16 + (int64_t)blockIdx.x * kThreads + threadIdx.x; c < cols; c += stride) {
            uint32_t dummy = 0;
            q[qb + c] = cast1<FMT, false>(load1<DT>(x, xb + c, dummy), s, 0.0f, sat, und, nan);
        }
    }
}

// The same stream for bf16 input on the corrected quotient.  PATH 1: the
// scale comes from the tensor's amax (every element qualifies).  PATH 2: a
// given scale; a group of 8 takes the corrected quotient when each |x| is at
// most lim = given_limit(s), else IEEE division and every counter.
template <int FMT, int PATH>
__device__ inline void cast_stream_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int vec,
                                        uint8_t* q, int64_t ldq, float s, float r, uint32_t lim, uint32_t& sat,
                                        uint32_t& und, uint32_t& nan)
{
    auto cast = [&](const uint4& w) -> uint2 {
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        if constexpr (PATH == 2) {
            const us2 m = pkmax8(us2{0, 0}, w);
            if ((uint32_t)(m.x > m.y ? m.x : m.y) > lim) {
                float v[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                              bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
                return cast8<FMT, false>(v, s, 0.0f, sat, und, nan);
            }
        }
        return cast8_bf16_fast<FMT>(ws, s, r, und);
    };
    const int64_t nvec = vec ? cols / 16 : 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
        const uint16_t* xr = x + row * ld;
        uint8_t* qr = q + row * ldq;
        int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
        for (; i + stride < nvec; i += 2 * stride) {
            const uint4 a = ld_stream(xr + i * 16), b = ld_stream(xr + i * 16 + 8);
            const uint4 c = ld_stream(xr + (i + stride) * 16), d = ld_stream(xr + (i + stride) * 16 + 8);
            const uint2 oa = cast(a), ob = cast(b), oc = cast(c), od = cast(d);
            *reinterpret_cast<uint4*>(qr + i * 16) = make_uint4(oa.x, oa.y, ob.x, ob.y);
            *reinterpret_cast<uint4*>(qr + (i + stride) * 16) = make_uint4(oc.x, oc.y, od.x, od.y);
        }
        for (; i < nvec; i += stride) {
            const uint4 a = ld_stream(xr + i * 16), b = ld_stream(xr + i * 16 + 8);
            const uint2 oa = cast(a), ob = cast(b);
            *reinterpret_cast<uint4*>(qr + i * 16) = make_uint4(oa.x, oa.y, ob.x, ob.y);
        }
        for (int64_t c = nvec * 16 + (int64_t)blockIdx.x * kThreads + threadIdx.x; c < cols; c += stride) {
            const uint32_t h = xr[c];
            const float xv = __builtin_bit_cast(float, h << 16);
            qr[c] = (PATH == 1 || (h & 0x7FFFu) <= lim) ? cast1<FMT, true>(xv, s, r, sat, und, nan)
                                                        : cast1<FMT, false>(xv, s, 0.0f, sat, und, nan);
        }
    }
}

template <int FMT, int DT>
__global__ void __launch_bounds__(kThreads) k_cast_tensor(const void* x, int64_t rows, int64_t cols,
                                                          int64_t ld, int vec, uint8_t* q, int64_t ldq,
                                                          float* scale, const uint32_t* partials, int np,
                                                          fp8_counters* ctr, int pow2)
{
    float s;
    bool special = true;
    if (partials) {
        const uint32_t k = reduce_partials(partials, np);
        special = key_special(k);
        s = scale_rule<FMT>(key_amax(k), pow2);
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) scale[0] = s;
    } else {
        s = scale[0];
    }
    uint32_t sat = 0, und = 0, nan = 0;
    bool general = true;
    if constexpr (DT == 0) {
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        if (partials && !special && s >= kCorrectedQuotMinScale) {
            cast_stream_bf16<FMT, 1>(xb, rows, cols, ld, vec, q, ldq, s, 1.0f / s, 0, sat, und, nan);
            general = false;
        } else if (!partials && s >= kCorrectedQuotMinScale && s <= kCorrectedQuotMaxScale) {
            cast_stream_bf16<FMT, 2>(xb, rows, cols, ld, vec, q, ldq, s, 1.0f / s, given_limit<FMT>(s), sat, und,
                                     nan);
            general = false;
        }
    }
    if (general) cast_stream<FMT, DT>(x, rows, cols, ld, vec, q, ldq, s, sat, und, nan);
    flush_counters_block(ctr, sat, und, nan);
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

// One 128x128 tile (tile index tid of the tensor's row-major tile grid).
// s_tensor / special_tensor / from_partials describe the per-tensor scale
// (SCALE_MODE 0); the per-block modes derive or read their own.  `tile` is
// the workgroup's LDS staging area for the transposed copy.
template <int FMT, int DT, int SCALE_MODE, bool AMAX_ONLY>
__device__ inline void tile128_one(const void* x, int64_t rows, int64_t cols, int64_t ld, int vec, float* scale,
                                   float s_tensor, bool special_tensor, bool from_partials, uint8_t* q, int64_t ldq,
                                   uint8_t* qt, int64_t ldqt, int pow2, int64_t tid, uint8_t* tile,
                                   uint32_t& sat, uint32_t& und, uint32_t& nan)
{
    const int t = threadIdx.x;
    const int cc = (t & 15) * 8;
    const int rr = t >> 4;
    const int64_t tiles_c = (cols + kTile - 1) / kTile;
    {
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
            fast = DT == 0 && from_partials && !special_tensor && s >= kCorrectedQuotMinScale;
        } else if constexpr (SCALE_MODE == 1) {
            key = block_key_merge(key);
            const int64_t sidx = (r0 / kTile) * tiles_c + c0 / kTile;
            if constexpr (AMAX_ONLY) {
                if (t == 0) scale[sidx] = key_amax(key);
                return;
            }
            s = scale_rule<FMT>(key_amax(key), pow2);
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
}

// One workgroup per 128x128 tile, grid-strided over the tile grid.
template <int FMT, int DT, int SCALE_MODE, bool AMAX_ONLY>
__global__ void __launch_bounds__(kThreads) k_tile128(const void* x, int64_t rows, int64_t cols,
                                                      int64_t ld, int vec, float* scale,
                                                      const uint32_t* partials, int np, uint8_t* q,
                                                      int64_t ldq, uint8_t* qt, int64_t ldqt,
                                                      fp8_counters* ctr, int only_partial, int pow2)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kTilePitch];
    const int64_t tiles_c = (cols + kTile - 1) / kTile;
    const int64_t tiles_r = (rows + kTile - 1) / kTile;
    const int64_t ntiles = tiles_r * tiles_c;

    float s_tensor = 1.0f;
    bool special_tensor = true;
    if constexpr (SCALE_MODE == 0) {
        if (partials) {
            const uint32_t k = reduce_partials(partials, np);
            special_tensor = key_special(k);
            s_tensor = scale_rule<FMT>(key_amax(k), pow2);
            if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s_tensor;
        } else {
            s_tensor = scale[0];
        }
    }
    uint32_t sat = 0, und = 0, nan = 0;
    for (int64_t tid = blockIdx.x; tid < ntiles; tid += gridDim.x) {
        const int64_t r0 = (tid / tiles_c) * kTile, c0 = (tid % tiles_c) * kTile;
        if (only_partial && r0 + kTile <= rows && c0 + kTile <= cols) continue;   // done by k_tile128_bf16
        tile128_one<FMT, DT, SCALE_MODE, AMAX_ONLY>(x, rows, cols, ld, vec, scale, s_tensor, special_tensor,
                                                    partials != nullptr, q, ldq, qt, ldqt, pow2, tid, tile, sat, und,
                                                    nan);
    }
    if constexpr (!AMAX_ONLY) flush_counters_block(ctr, sat, und, nan);
}

// Workgroup barrier that waits only for this wave's LDS operations, not for
// its outstanding global loads (__syncthreads() also drains vmcnt, which
// would wait for the prefetched next tile).
__device__ inline void barrier_lds_only()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ inline uint32_t block_key_merge_lds(uint32_t k)
{
    __shared__ uint32_t sh[kMaxWaves];   // any workgroup size up to 1024
    k = wave_key_merge(k);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = k;
    barrier_lds_only();
    k = sh[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) k = key_merge(k, sh[w]);
    barrier_lds_only();
    return k;
}

// ------------------------------------------------------------------ 128x128 tiles, bf16 fast path
// Full 128x128 tiles of a 16-byte aligned bf16 tensor.  Thread t owns the
// 8x8 block of rows 8 (t/16) + i, columns 8 (t%16) + j (eight 16-byte row
// loads; 16 lanes cover a 256-byte row segment).  The next tile's loads are
// issued before the current tile is processed.  Codes leave row-major as 8
// bytes per row; for the transposed copy the thread transposes its 8x8 byte
// block in registers (v_perm_b32) and writes 8 bytes per column to an LDS
// tile of 128 output rows x 128 bytes, whose 8-byte chunks are swizzled so
// that both the writes and the 16-byte row reads are free of bank
// conflicts; each thread then stores 64 bytes of one output row.
// SCALE_MODE as in k_tile128.  Edge tiles are left to k_tile128.
__device__ inline int tswz(int c) { return ((c >> 3) & 15) ^ ((c & 7) << 1); }

// Per-tensor scale (SCALE_MODE 0) is held to 3 waves per SIMD (162 VGPRs, no
// scratch) and launched as 3 workgroups per CU, all resident at once; on X
// and dY of the training step that ran 1-3% faster than 2 waves per SIMD with
// 4 workgroups per CU.  The other modes keep their registers: the per-block
// amax and the delayed form would spill under the same cap.
constexpr int kTileWavesPerSimd0 = 3;
template <int FMT, int SCALE_MODE>
__global__ void __launch_bounds__(kThreads)
    __attribute__((amdgpu_waves_per_eu(SCALE_MODE == 0 ? kTileWavesPerSimd0 : 1))) k_tile128_bf16(const uint16_t* x, int64_t rows, int64_t cols,
                                                           int64_t ld, float* scale, const uint32_t* partials,
                                                           int np, uint8_t* q, int64_t ldq, uint8_t* qt,
                                                           int64_t ldqt, fp8_counters* ctr, const float* hist,
                                                           int hist_len, uint32_t* amax_out, int pow2)
{
    __shared__ __attribute__((aligned(16))) uint8_t tt[kTile * kTile];
    const int t = threadIdx.x;
    const int g = t >> 4, k = t & 15;
    const int64_t tiles_c = cols / kTile;       // full tiles only
    const int64_t ntiles = (rows / kTile) * tiles_c;
    const int64_t tiles_c_all = (cols + kTile - 1) / kTile;

    float s_tensor = 1.0f;
    bool special_tensor = true;
    // SCALE_MODE 3 (delayed scaling): the scale comes from the largest amax
    // of the history; an element whose |x| pattern exceeds that amax (or is
    // Inf / NaN) takes the IEEE-division path, the others the corrected
    // quotient, whose proof covers |x| <= amax for a bf16 amax.
    uint32_t hist_bits = 0;
    bool hist_fast = false;
    us2 seen = us2{0, 0};      // packed |x| pattern max of this thread's elements (mode 3)
    if constexpr (SCALE_MODE == 3) {
        const uint32_t hk = reduce_partials(reinterpret_cast<const uint32_t*>(hist), hist_len);
        s_tensor = scale_from_amax<FMT>(key_amax(hk));
        if (blockIdx.x == 0 && t == 0) scale[0] = s_tensor;
        hist_bits = (hk & 0x7FFFFFFFu) >> 16;
        hist_fast = (hk & 0x8000FFFFu) == 0 && hist_bits < 0x7F80u && s_tensor >= kCorrectedQuotMinScale;
    }
    if constexpr (SCALE_MODE == 0) {
        if (partials) {
            const uint32_t kk = reduce_partials(partials, np);
            special_tensor = key_special(kk);
            s_tensor = scale_rule<FMT>(key_amax(kk), pow2);
            if (blockIdx.x == 0 && t == 0) scale[0] = s_tensor;
        } else {
            s_tensor = scale[0];
        }
    }
    // a given per-tensor scale: the corrected quotient for the threads whose
    // elements all have |x| <= given_limit(s) (mode 2 takes it per block)
    const uint32_t lim_tensor = SCALE_MODE == 0 && !partials ? given_limit<FMT>(s_tensor) : 0u;
    uint32_t sat = 0, und = 0, nan = 0;

    auto load = [&](int64_t id, uint4 (&w)[8]) {
        const int64_t r0 = (id / tiles_c) * kTile, c0 = (id % tiles_c) * kTile;
        const uint16_t* src = x + (r0 + 8 * g) * ld + c0 + 8 * k;
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = ld_stream(src + i * ld);
    };

    // a contiguous range of tiles (row-major tile order) per workgroup; the
    // loop is unrolled by two so the prefetch buffers alternate statically
    const int64_t per = (ntiles + gridDim.x - 1) / gridDim.x;
    const int64_t id0 = (int64_t)blockIdx.x * per;
    const int64_t id1 = min(ntiles, id0 + per);

    auto process = [&](const uint4 (&cur)[8], int64_t id) {
        const int64_t r0 = (id / tiles_c) * kTile, c0 = (id % tiles_c) * kTile;

        float s;
        bool fast;
        if constexpr (SCALE_MODE == 0) {
            s = s_tensor;
            if (partials) {
                fast = !special_tensor && s >= kCorrectedQuotMinScale;
            } else {
                us2 m = us2{0, 0};
#pragma unroll
                for (int i = 0; i < 8; ++i) m = pkmax8(m, cur[i]);
                fast = (uint32_t)(m.x > m.y ? m.x : m.y) <= lim_tensor;   // per thread
            }
        } else if constexpr (SCALE_MODE == 1) {
            us2 m = us2{0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) m = pkmax8(m, cur[i]);
            uint32_t key = block_key_merge_lds(pk_raw(m));
            if (key >= kRawNonFinite) {
                // an Inf or NaN in the block: the exact merge (finite amax + flag)
                // (rare: the rows are read again rather than indexed in
                // registers, which would move the tile to scratch memory)
                uint32_t e = 0;
                const uint16_t* src = x + (r0 + 8 * g) * ld + c0 + 8 * k;
#pragma unroll 1
                for (int i = 0; i < 8; ++i) {
                    const uint4 w = *reinterpret_cast<const uint4*>(src + i * ld);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        e = key_merge(e, absbits_bf16(ws[h] & 0xFFFFu));
                        e = key_merge(e, absbits_bf16(ws[h] >> 16));
                    }
                }
                key = block_key_merge_lds(e);
            }
            s = scale_rule<FMT>(key_amax(key), pow2);
            if (t == 0) scale[(r0 / kTile) * tiles_c_all + c0 / kTile] = s;
            fast = !key_special(key) && s >= kCorrectedQuotMinScale;
        } else if constexpr (SCALE_MODE == 3) {
            us2 m = us2{0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) m = pkmax8(m, cur[i]);
            seen = __builtin_elementwise_max(seen, m);
            s = s_tensor;
            fast = hist_fast && (uint32_t)(m.x > m.y ? m.x : m.y) <= hist_bits;   // per thread
        } else {
            s = scale[(r0 / kTile) * tiles_c_all + c0 / kTile];
            us2 m = us2{0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) m = pkmax8(m, cur[i]);
            fast = (uint32_t)(m.x > m.y ? m.x : m.y) <= given_limit<FMT>(s);   // per thread
        }

        uint8_t* qrow = q + (r0 + 8 * g) * ldq + c0 + 8 * k;
        if (fast) {
            const float r = 1.0f / s;
            // rows 4 rb .. 4 rb + 3: cast, store, transpose their 4x8 bytes
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                uint2 code[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint4 w = cur[4 * rb + i];
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
                    code[i] = cast8_bf16_fast<FMT>(ws, s, r, und);
                    *reinterpret_cast<uint2*>(qrow + (4 * rb + i) * ldq) = code[i];
                    // one row at a time: keeps the quotient temporaries of the
                    // other rows from being live at once
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (qt) {
#pragma unroll
                    for (int half = 0; half < 2; ++half) {      // columns 4 half .. +3
                        const uint32_t a = half ? code[0].y : code[0].x;
                        const uint32_t b = half ? code[1].y : code[1].x;
                        const uint32_t c = half ? code[2].y : code[2].x;
                        const uint32_t d = half ? code[3].y : code[3].x;
                        const uint32_t x0 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
                        const uint32_t x1 = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
                        const uint32_t y0 = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
                        const uint32_t y1 = __builtin_amdgcn_perm(d, c, 0x07030602u);   // c2 d2 c3 d3
                        const uint32_t col[4] = {__builtin_amdgcn_perm(y0, x0, 0x05040100u),
                                                 __builtin_amdgcn_perm(y0, x0, 0x07060302u),
                                                 __builtin_amdgcn_perm(y1, x1, 0x05040100u),
                                                 __builtin_amdgcn_perm(y1, x1, 0x07060302u)};
                        // output row cc = 8 k + 4 half + j, logical chunk g, bytes 4 rb .. +3
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int cc = 8 * k + 4 * half + j;
                            *reinterpret_cast<uint32_t*>(&tt[cc * kTile + 8 * (g ^ tswz(cc)) + 4 * rb]) = col[j];
                        }
                    }
                }
            }
        } else {
            // general quotients (IEEE division, all counters), one row at a
            // time; the rows are read again (indexing the registers by a loop
            // variable would move the tile to scratch memory)
            const uint16_t* src = x + (r0 + 8 * g) * ld + c0 + 8 * k;
#pragma unroll 1
            for (int i = 0; i < 8; ++i) {
                const uint4 w = *reinterpret_cast<const uint4*>(src + i * ld);
                float v[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                              bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
                const uint2 code = cast8<FMT, false>(v, s, 0.0f, sat, und, nan);
                *reinterpret_cast<uint2*>(qrow + i * ldq) = code;
                if (qt) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int cc = 8 * k + j;
                        tt[cc * kTile + 8 * (g ^ tswz(cc)) + i] = (uint8_t)((j < 4 ? code.x : code.y) >> (8 * (j & 3)));
                    }
                }
            }
        }

        if (qt) {
            barrier_lds_only();
            const int c = t & 127, hh = t >> 7;
            const int sw = tswz(c);
            uint8_t* dst = qt + (c0 + c) * ldqt + r0 + 64 * hh;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int p0 = (8 * hh + 2 * m) ^ sw;           // physical chunk of logical 8hh+2m
                uint4 v = *reinterpret_cast<const uint4*>(&tt[c * kTile + 8 * (p0 & ~1)]);
                if (p0 & 1) v = make_uint4(v.z, v.w, v.x, v.y);
                *reinterpret_cast<uint4*>(dst + 16 * m) = v;
            }
            barrier_lds_only();
        }
    };

    uint4 bufa[8], bufb[8];
    int64_t id = id0;
    if (id < id1) load(id, bufa);
    while (id < id1) {
        if (id + 1 < id1) load(id + 1, bufb);
        process(bufa, id);
        if (++id >= id1) break;
        if (id + 1 < id1) load(id + 1, bufa);
        process(bufb, id);
        ++id;
    }
    if constexpr (SCALE_MODE == 3) {
        // this workgroup's amax key for the history; an Inf or NaN among its
        // elements (rare) makes it read its tiles again for the exact,
        // flag-carrying merge
        uint32_t key = pk_raw(seen);
        if (key >= kRawNonFinite) {
            key = 0;
#pragma unroll 1
            for (int64_t j = id0; j < id1; ++j) {
                const int64_t r0 = (j / tiles_c) * kTile, c0 = (j % tiles_c) * kTile;
                const uint16_t* src = x + (r0 + 8 * g) * ld + c0 + 8 * k;
#pragma unroll 1
                for (int i = 0; i < 8; ++i) {
                    const uint4 w = *reinterpret_cast<const uint4*>(src + i * ld);
                    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        key = key_merge(key, absbits_bf16(ws[h] & 0xFFFFu));
                        key = key_merge(key, absbits_bf16(ws[h] >> 16));
                    }
                }
            }
        }
        key = block_key_merge(key);
        if (t == 0) amax_out[blockIdx.x] = key;
    }
    flush_counters_block(ctr, sat, und, nan);
}

// ------------------------------------------------------------------ 128x128 blocks, bf16, no transposed copy
// Whole 128 x 128 blocks of a 16-byte aligned bf16 tensor, 512 threads per
// workgroup: thread t holds the 8 columns 8 (t % 16) of rows t / 16 + 32 j
// (j = 0..3, four 16-byte loads).  Workgroup w takes blocks w, w + G, w + 2G
// ... (G workgroups) and loads the next block before it reduces and casts the
// current one, so the loads of later blocks overlap the arithmetic and stores
// of earlier ones (with one block per workgroup every block's loads end
// together, and the arithmetic and stores then run with the memory idle).
// The block's amax is a packed max of |x| patterns; a block holding Inf or NaN
// redoes the exact, flag-carrying merge.  Scale of each block from its own
// amax (pow2: the power-of-two rule).
constexpr int kBlkThreads = 512;
constexpr int kBlkPerCu = 2;       // workgroups per CU (each walks several blocks)
constexpr int kBlkOnePerWgMax = 4; // blocks per CU up to which each workgroup takes one

struct BlockRegs {
    uint4 w[4];
};

__device__ __forceinline__ void block_load(BlockRegs& b, const uint16_t* x, int64_t ld, int64_t blocks_c,
                                           int64_t id)
{
    const int t = threadIdx.x;
    const int64_t br = id / blocks_c, bc = id - br * blocks_c;
    const uint16_t* src = x + (br * kTile + (t >> 4)) * ld + bc * kTile + 8 * (t & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) b.w[j] = ld_stream(src + 32 * j * ld);
}

template <int FMT>
__device__ __forceinline__ void block_cast(const BlockRegs& b, int64_t id, int64_t blocks_c, uint32_t* sh,
                                           float* scale, int64_t scale_ld, uint8_t* q, int64_t ldq, int pow2,
                                           uint32_t& sat, uint32_t& und, uint32_t& nan)
{
    const int t = threadIdx.x;
    us2 pk = us2{0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) pk = pkmax8(pk, b.w[j]);
    uint32_t key = wave_max(pk_raw(pk));
    if ((t & 63) == 0) sh[t >> 6] = key;
    __syncthreads();
    key = sh[0];
#pragma unroll
    for (int i = 1; i < kBlkThreads / 64; ++i) key = max(key, sh[i]);
    if (key >= kRawNonFinite) {
        // an Inf or NaN in the block: the exact merge (finite amax + flag)
        __syncthreads();
        uint32_t e = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t ws[4] = {b.w[j].x, b.w[j].y, b.w[j].z, b.w[j].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                e = key_merge(e, absbits_bf16(ws[h] & 0xFFFFu));
                e = key_merge(e, absbits_bf16(ws[h] >> 16));
            }
        }
        e = wave_key_merge(e);
        if ((t & 63) == 0) sh[t >> 6] = e;
        __syncthreads();
        key = sh[0];
        for (int i = 1; i < kBlkThreads / 64; ++i) key = key_merge(key, sh[i]);
    }
    const int64_t br = id / blocks_c, bc = id - br * blocks_c;
    const float s = scale_rule<FMT>(key_amax(key), pow2);
    if (t == 0) scale[br * scale_ld + bc] = s;
    const bool fast = !key_special(key) && s >= kCorrectedQuotMinScale;
    const float r = 1.0f / s;
    uint8_t* dst = q + (br * kTile + (t >> 4)) * ldq + bc * kTile + 8 * (t & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t ws[4] = {b.w[j].x, b.w[j].y, b.w[j].z, b.w[j].w};
        uint2 o;
        if (fast) {
            o = cast8_bf16_fast<FMT>(ws, s, r, und);
        } else {
            float v[8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[2 * h] = bf16_lo(ws[h]);
                v[2 * h + 1] = bf16_hi(ws[h]);
            }
            o = cast8<FMT, false>(v, s, 0.0f, sat, und, nan);
        }
        *reinterpret_cast<uint2*>(dst + 32 * j * ldq) = o;
    }
}

// PIPE false: one block per workgroup (a tensor of at most 4 blocks per CU:
// at about 60 registers all of them are resident at once, which beats the
// pipelined walk there); PIPE true: the walk above, two workgroups per CU.
template <int FMT, bool PIPE>
__global__ void __launch_bounds__(kBlkThreads) __attribute__((amdgpu_waves_per_eu(PIPE ? 4 : 8))) k_block128_bf16(const uint16_t* x, int64_t ld, int64_t blocks_c,
                                                               int64_t nblocks, float* scale, int64_t scale_ld,
                                                               uint8_t* q, int64_t ldq, fp8_counters* ctr, int pow2)
{
    // two slots: the block after next writes its wave maxima only after every
    // thread has passed the current block's barrier
    __shared__ uint32_t sh[2][kBlkThreads / 64];
    uint32_t sat = 0, und = 0, nan = 0;
    const int64_t G = gridDim.x;
    int64_t id = blockIdx.x;
    BlockRegs b0, b1;
    block_load(b0, x, ld, blocks_c, id);
    // unrolled by two so the register sets alternate statically
    while (PIPE) {
        const int64_t id1 = id + G;
        if (id1 < nblocks) block_load(b1, x, ld, blocks_c, id1);
        block_cast<FMT>(b0, id, blocks_c, sh[0], scale, scale_ld, q, ldq, pow2, sat, und, nan);
        if (id1 >= nblocks) break;
        const int64_t id2 = id1 + G;
        if (id2 < nblocks) block_load(b0, x, ld, blocks_c, id2);
        block_cast<FMT>(b1, id1, blocks_c, sh[1], scale, scale_ld, q, ldq, pow2, sat, und, nan);
        if (id2 >= nblocks) break;
        id = id2;
    }
    if (!PIPE) block_cast<FMT>(b0, id, blocks_c, sh[0], scale, scale_ld, q, ldq, pow2, sat, und, nan);
    flush_counters_block(ctr, sat, und, nan);
}

// ------------------------------------------------------------------ 128x128 tiles, per-tensor scale, with the transposed copy
// Whole 128 x 128 tiles of a 16-byte aligned bf16 tensor with one scale for
// the whole tensor (from the amax partials, or given), codes row-major and
// transposed.  512 threads per tile: thread t holds the 4 x 8 block of rows
// 4 (t / 16) .. +3, columns 8 (t % 16) .. +7 (four 16-byte loads).  Its codes
// leave row-major as 8 bytes per row; two 4 x 4 byte transposes (v_perm_b32)
// turn them into 8 words of 4 transposed bytes, written to an LDS tile of
// 128 output rows x 128 bytes whose words are swizzled by the row (2-way
// bank sharing at most); each thread then stores 32 bytes of one output row.
// One tile per workgroup, for tensors of at most 4 tiles per CU: at about 50
// registers every tile is resident at once, and the weight-sized tensor
// (144 tiles) ran 8% faster than on the 256-thread tile kernel.  Larger
// tensors stay on that kernel: a form of this one that walked the tiles with
// two workgroups per CU and the next tile prefetched was 3.5% slower on the
// 65536 x 3072 gradient (fewer bytes in flight per CU).
// The cast and stores of one tile held as w[4] by thread t of 512 (layout
// above): codes row-major, and transposed through the LDS tile tl when qt is
// not null.
template <int FMT>
__device__ __forceinline__ void tile128t_cast_store(const uint4 (&w)[4], float s, float r, bool fast, int64_t r0,
                                                    int64_t c0, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                                                    uint32_t* tl, uint32_t& sat, uint32_t& und, uint32_t& nan)
{
    const int t = threadIdx.x;
    const int g = t >> 4, k = t & 15;
    uint2 code[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
        if (fast) {
            code[i] = cast8_bf16_fast<FMT>(ws, s, r, und);
        } else {
            float v[8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[2 * h] = bf16_lo(ws[h]);
                v[2 * h + 1] = bf16_hi(ws[h]);
            }
            code[i] = cast8<FMT, false>(v, s, 0.0f, sat, und, nan);
        }
        *reinterpret_cast<uint2*>(q + (r0 + 4 * g + i) * ldq + c0 + 8 * k) = code[i];
    }
    if (!qt) return;
    // column cc = 8 k + 4 half + j of the tile: bytes of rows 4 g .. 4 g + 3,
    // word g of LDS row cc, stored at word g ^ (4 ((cc / 8) % 8))
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint32_t a = half ? code[0].y : code[0].x;
        const uint32_t b = half ? code[1].y : code[1].x;
        const uint32_t c = half ? code[2].y : code[2].x;
        const uint32_t d = half ? code[3].y : code[3].x;
        const uint32_t x0 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
        const uint32_t x1 = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
        const uint32_t y0 = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
        const uint32_t y1 = __builtin_amdgcn_perm(d, c, 0x07030602u);   // c2 d2 c3 d3
        const uint32_t col[4] = {__builtin_amdgcn_perm(y0, x0, 0x05040100u), __builtin_amdgcn_perm(y0, x0, 0x07060302u),
                                 __builtin_amdgcn_perm(y1, x1, 0x05040100u), __builtin_amdgcn_perm(y1, x1, 0x07060302u)};
#pragma unroll
        for (int j = 0; j < 4; ++j) tl[(8 * k + 4 * half + j) * 32 + (g ^ (4 * (k & 7)))] = col[j];
    }
    barrier_lds_only();
    // output row c0 + cc (cc = t % 128), bytes r0 + 32 qq .. +31 (qq = t / 128):
    // logical words 8 qq .. 8 qq + 7 of LDS row cc, two aligned groups of 4
    const int cc = t & 127, qq = t >> 7;
    const int sw = 4 * ((cc >> 3) & 7);
    const uint4 lo = *reinterpret_cast<const uint4*>(&tl[cc * 32 + ((8 * qq) ^ sw)]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&tl[cc * 32 + ((8 * qq + 4) ^ sw)]);
    uint8_t* dst = qt + (c0 + cc) * ldqt + r0 + 32 * qq;
    *reinterpret_cast<uint4*>(dst) = lo;
    *reinterpret_cast<uint4*>(dst + 16) = hi;
}

template <int FMT>
__global__ void __launch_bounds__(kBlkThreads) __attribute__((amdgpu_waves_per_eu(8)))
    k_tile128t_bf16(const uint16_t* x, int64_t ld, int64_t tiles_c, float* scale, const uint32_t* partials, int np,
                    uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, fp8_counters* ctr, int pow2)
{
    __shared__ __attribute__((aligned(16))) uint32_t tl[kTile * kTile / 4];
    const int t = threadIdx.x;
    const int g = t >> 4, k = t & 15;
    float s;
    bool fast = false;
    if (partials) {
        const uint32_t kk = reduce_partials(partials, np);
        s = scale_rule<FMT>(key_amax(kk), pow2);
        fast = !key_special(kk) && s >= kCorrectedQuotMinScale;
        if (blockIdx.x == 0 && t == 0) scale[0] = s;
    } else {
        s = scale[0];
    }
    uint32_t sat = 0, und = 0, nan = 0;
    const int64_t br = blockIdx.x / tiles_c;
    const int64_t r0 = br * kTile, c0 = (blockIdx.x - br * tiles_c) * kTile;
    uint4 w[4];
    const uint16_t* src = x + (r0 + 4 * g) * ld + c0 + 8 * k;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = ld_stream(src + i * ld);
    tile128t_cast_store<FMT>(w, s, 1.0f / s, fast, r0, c0, q, ldq, qt, ldqt, tl, sat, und, nan);
    flush_counters_block(ctr, sat, und, nan);
}

// ------------------------------------------------------------------ per-tensor quantize of a small tensor in one launch
// A bf16 tensor of whole 128 x 128 tiles, at most one tile per CU (and at
// most kOnceMaxTiles), per-tensor scale from its amax: one launch instead of
// the amax pass and the cast.  Each 512-thread workgroup loads its tile,
// reduces the tile's amax key, publishes it in the workspace and waits until
// every tile's key is there, then merges them, derives the scale and casts
// its tile from registers (codes, and the transposed copy when asked).
//
// The keys are matched to the call by a tag: every workgroup reads the
// workspace's call counter before it publishes (so all read the same value
// c: a workgroup only adds its departure to the counter after it has seen
// every tile's key, which each workgroup publishes after its read), writes
// its key and then, with release order, the tag T(c), and waits (acquire)
// for T(c) in every slot.  T is a bijective 64-bit mix, so tags left by an
// earlier call on the same workspace (each call advances the counter by its
// tile count) never match, and words left by other uses of the workspace
// (the amax pass's keys, whose neighbours can differ by one) match only by
// a 64-bit coincidence.  The wait is bounded: a workgroup that
// has not seen every key after `spin_limit` polls (other workgroups not
// resident, or a call on another stream sharing the workspace, which the
// workspace contract excludes) reads the whole tensor for the amax itself:
// slower, the same scale, and every workgroup finishes.
constexpr int kOnceMaxTiles = 256;
// T(c): the finalizer of SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast
// splittable pseudorandom number generators", OOPSLA 2014), a bijection.
__device__ inline uint64_t once_tag(uint64_t c)
{
    uint64_t z = c + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
// Publish a key, then its tag, for a reader elsewhere on the chip that reads
// the tag and then the key with agent-scope atomic loads.  Both stores are
// agent-scope atomics, which the memory system keeps coherent at that scope
// once they complete; waiting for the key's store to complete before the
// tag's store is issued orders them.  (A release store of the tag would
// also write back this XCD's L2 for the sake of ordinary stores, of which
// there are none to publish: with hundreds of workgroups publishing at
// once those write-backs cost several microseconds.)
__device__ inline void publish_key(uint32_t* key_slot, uint32_t key, uint64_t* tag_slot, uint64_t tag)
{
    __hip_atomic_store(key_slot, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // no compiler reordering across
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __hip_atomic_store(tag_slot, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct OnceSlot {
    uint64_t tag;
    uint32_t key;
    uint32_t pad;
};
struct OnceSync {
    uint64_t calls;
    uint64_t pad[7];
    OnceSlot slot[kOnceMaxTiles];
};
static_assert(sizeof(OnceSync) <= kAmaxWorkspaceBytes, "the amax workspace holds the call's slots");

// The amax key of the whole tensor (rows x cols, whole tiles, 16-byte rows)
// read by one workgroup: the fallback of a wait that did not complete.
__device__ inline uint32_t tensor_key_one_workgroup(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld)
{
    const int64_t vpr = cols / 8, nv = rows * vpr;
    us2 m = us2{0, 0};
    for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
        const int64_t r = v / vpr;
        m = pkmax8(m, *reinterpret_cast<const uint4*>(x + r * ld + (v - r * vpr) * 8));
    }
    uint32_t key = pk_raw(m);
    if (block_key_merge(key) >= kRawNonFinite) {
        key = 0;
        for (int64_t v = threadIdx.x; v < nv; v += blockDim.x) {
            const int64_t r = v / vpr;
            const uint4 w = *reinterpret_cast<const uint4*>(x + r * ld + (v - r * vpr) * 8);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                key = key_merge(key, absbits_bf16(ws[h] & 0xFFFFu));
                key = key_merge(key, absbits_bf16(ws[h] >> 16));
            }
        }
    }
    return block_key_merge(key);
}

// At most one workgroup per CU: its 8 waves may take 256 registers each.
template <int FMT>
__global__ void __launch_bounds__(kBlkThreads) __attribute__((amdgpu_waves_per_eu(2)))
    k_tile128t_once(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* scale, OnceSync* sync,
                    uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt, fp8_counters* ctr, int pow2, int spin_limit)
{
    __shared__ __attribute__((aligned(16))) uint32_t tl[kTile * kTile / 4];
    __shared__ uint32_t s_key;
    const int t = threadIdx.x;
    const int g = t >> 4, k = t & 15;
    const int64_t tiles_c = cols / kTile;
    const int ntiles = (int)gridDim.x;
    const int64_t br = blockIdx.x / tiles_c;
    const int64_t r0 = br * kTile, c0 = (blockIdx.x - br * tiles_c) * kTile;
    uint4 w[4];
    const uint16_t* src = x + (r0 + 4 * g) * ld + c0 + 8 * k;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = ld_stream(src + i * ld);

    // this tile's key (the exact merge only for a tile holding Inf or NaN)
    us2 m = us2{0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = pkmax8(m, w[i]);
    uint32_t key = block_key_merge(pk_raw(m));
    if (key >= kRawNonFinite) {
        uint32_t e = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                e = key_merge(e, absbits_bf16(ws[h] & 0xFFFFu));
                e = key_merge(e, absbits_bf16(ws[h] >> 16));
            }
        }
        key = block_key_merge(e);
    }

    // publish, wait for every tile's key, merge (wave 0)
    __shared__ int s_complete;
    if (t < 64) {
        uint64_t c = 0;
        if (t == 0) {
            c = __hip_atomic_load(&sync->calls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            publish_key(&sync->slot[blockIdx.x].key, key, &sync->slot[blockIdx.x].tag, once_tag(c));
        }
        const uint64_t want = once_tag(__shfl(c, 0));
        bool seen = false;
        for (int it = 0; it < spin_limit; ++it) {
            bool mine = true;
            for (int j = t; j < ntiles; j += 64)
                mine &= __hip_atomic_load(&sync->slot[j].tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want;
            if (__all(mine)) {
                seen = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        uint32_t kk = 0;
        if (seen) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the keys after their tags
            for (int j = t; j < ntiles; j += 64)
                kk = key_merge(kk, __hip_atomic_load(&sync->slot[j].key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            kk = wave_key_merge(kk);
        }
        if (t == 0) {
            s_key = kk;
            s_complete = seen;
            __hip_atomic_fetch_add(&sync->calls, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    // the wait did not complete: this workgroup reads the whole tensor
    const uint32_t kk = s_complete ? s_key : tensor_key_one_workgroup(x, rows, cols, ld);

    const float s = scale_rule<FMT>(key_amax(kk), pow2);
    const bool fast = !key_special(kk) && s >= kCorrectedQuotMinScale;
    if (blockIdx.x == 0 && t == 0) scale[0] = s;
    uint32_t sat = 0, und = 0, nan = 0;
    tile128t_cast_store<FMT>(w, s, 1.0f / s, fast, r0, c0, q, ldq, qt, ldqt, tl, sat, und, nan);
    flush_counters_block(ctr, sat, und, nan);
}

// ------------------------------------------------------------------ 1x128 row tiles, bf16 fast path
// Full tiles of a 16-byte aligned bf16 tensor, scale from each tile's amax.
// 16 lanes per tile and 4 tiles per group and iteration, all loads first.
// The 16-lane amax is a packed max of |x| patterns (exact merge only for a
// tile holding Inf or NaN); lane u of each group then divides for tile u and
// the scales and reciprocals are shuffled back, one pair of divisions per
// lane for 4 tiles.
template <int FMT>
__global__ void __launch_bounds__(kThreads) k_row1x128_bf16(const uint16_t* x, int64_t ld, float* scale,
                                                            uint8_t* q, int64_t ldq, fp8_counters* ctr,
                                                            uint32_t ntiles, FastDiv tiles_per_row,
                                                            uint32_t scale_ld, int pow2)
{
    constexpr int U = 4;
    constexpr uint32_t kChunk = (kThreads / 16) * U;     // tiles per workgroup and iteration
    const int lane = threadIdx.x & 15;
    const uint32_t gi = threadIdx.x >> 4;                // group in the workgroup
    uint32_t sat = 0, und = 0, nan = 0;
    // chunks of 64 consecutive tiles (group gi takes tiles 4 gi .. 4 gi + 3 of
    // a chunk; consecutive tiles of a row are consecutive in memory), dealt
    // to the workgroups in turn, so the chip streams through one region of
    // the tensor at a time (measured: 7% faster than a contiguous range of
    // chunks per workgroup)
    const uint32_t g1 = ntiles;
    for (uint32_t t0 = blockIdx.x * kChunk + gi * U; t0 < g1; t0 += kChunk * gridDim.x) {
        uint4 w[U];
        uint32_t row[U], tc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t tile = t0 + u;
            const uint32_t tl = tile < g1 ? tile : g1 - 1;   // clamp: loads stay in range
            row[u] = tiles_per_row.div(tl);
            tc[u] = tl - row[u] * tiles_per_row.d;
            w[u] = ld_stream(x + (int64_t)row[u] * ld + tc[u] * 128 + lane * 8);
        }
        uint32_t key[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            uint32_t k2 = pk_raw(pkmax8(us2{0, 0}, w[u]));
#pragma unroll
            for (int off = 8; off >= 1; off >>= 1) k2 = max(k2, (uint32_t)__shfl_xor(k2, off, 16));
            if (k2 >= kRawNonFinite) {
                const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
                uint32_t e = 0;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    e = key_merge(e, absbits_bf16(ws[h] & 0xFFFFu));
                    e = key_merge(e, absbits_bf16(ws[h] >> 16));
                }
#pragma unroll
                for (int off = 8; off >= 1; off >>= 1) e = key_merge(e, __shfl_xor(e, off, 16));
                k2 = e;
            }
            key[u] = k2;
        }
        // lane u (u < U) of the group derives the scale of tile u
        const uint32_t mykey = lane == 0 ? key[0] : lane == 1 ? key[1] : lane == 2 ? key[2] : key[3];
        const float my_s = scale_rule<FMT>(key_amax(mykey), pow2);
        const float my_r = 1.0f / my_s;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t tile = t0 + u;
            const float s = __shfl(my_s, u, 16);
            const float r = __shfl(my_r, u, 16);
            if (tile >= g1) continue;
            if (lane == 0) scale[(int64_t)row[u] * scale_ld + tc[u]] = s;
            const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
            float v[8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[2 * h] = bf16_lo(ws[h]);
                v[2 * h + 1] = bf16_hi(ws[h]);
            }
            const bool fast = !key_special(key[u]) && s >= kCorrectedQuotMinScale;
            const uint2 o = fast ? cast8_bf16_fast<FMT>(ws, s, r, und) : cast8<FMT, false>(v, s, 0.0f, sat, und, nan);
            *reinterpret_cast<uint2*>(q + (int64_t)row[u] * ldq + tc[u] * 128 + lane * 8) = o;
        }
    }
    flush_counters_block(ctr, sat, und, nan);
}

// ------------------------------------------------------------------ 1x128 row tiles
// 16 lanes per tile, 8 elements per lane; the 16-lane group reduces its amax
// with lane shuffles, derives its scale and casts.  Scales [rows, ceil(cols/128)].
template <int FMT, int DT, bool GIVEN, bool AMAX_ONLY>
__global__ void __launch_bounds__(kThreads) k_row1x128(const void* x, int64_t rows, int64_t cols,
                                                       int64_t ld, int vec, float* scale, uint8_t* q,
                                                       int64_t ldq, fp8_counters* ctr, uint32_t ntiles,
                                                       FastDiv tiles_per_row, int pow2)
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
            s = scale_rule<FMT>(key_amax(key), pow2);
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
    if constexpr (!AMAX_ONLY) flush_counters_block(ctr, sat, und, nan);
}

// ------------------------------------------------------------------ weight-cache refresh, batched
// The refresh of many caches in two launches ("#84 FP8 Precision", section
// "Hardware precision": after each optimizer step the master weights are
// quantized again into their FP8 copies).  k_requant_amax reduces every
// per-tensor cache's master to partial keys (each cache owns a contiguous
// run of workgroups and its own partial array); k_requant_cast then walks the
// 128x128 tiles of all caches, per-tensor ones scaled from their partials,
// per-block ones from each block's own amax, with the same tile code as
// k_tile128.  The caches of one launch travel in the kernel arguments.

// max |x| key over the elements [b, e) of a contiguous tensor (16-byte
// vectors when vec and b is a multiple of 8); the whole workgroup calls it.
template <int DT>
__device__ inline uint32_t amax_range(const void* x, int64_t b, int64_t e, bool vec)
{
    constexpr int per_vec = DT == 0 ? 8 : 4;
    const int64_t nv = vec ? (e - b) / per_vec : 0;
    const int64_t tail0 = b + nv * per_vec;
    uint32_t key = 0;
    if constexpr (DT == 0) {
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        us2 pk = us2{0, 0};
        for (int64_t v = threadIdx.x; v < nv; v += kThreads) pk = pkmax8(pk, ld_stream(xb + b + v * 8));
        for (int64_t c = tail0 + threadIdx.x; c < e; c += kThreads) {
            const uint32_t h = xb[c] & 0x7FFFu;
            pk.x = pk.x > h ? pk.x : (unsigned short)h;
        }
        key = pk_raw(pk);
        if (key >= kRawNonFinite) {
            // an Inf or NaN in this thread's share: the exact, flag-carrying merge
            key = 0;
            for (int64_t v = threadIdx.x; v < nv; v += kThreads) {
                const uint4 w = *reinterpret_cast<const uint4*>(xb + b + v * 8);
                const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    key = key_merge(key, absbits_bf16(ws[h] & 0xFFFFu));
                    key = key_merge(key, absbits_bf16(ws[h] >> 16));
                }
            }
            for (int64_t c = tail0 + threadIdx.x; c < e; c += kThreads) key = key_merge(key, absbits_bf16(xb[c]));
        }
    } else {
        const uint32_t* xb = static_cast<const uint32_t*>(x);
        for (int64_t v = threadIdx.x; v < nv; v += kThreads) {
            const uint4 w = ld_stream(xb + b + v * 4);
            key = key_merge(key, absbits_f32(w.x));
            key = key_merge(key, absbits_f32(w.y));
            key = key_merge(key, absbits_f32(w.z));
            key = key_merge(key, absbits_f32(w.w));
        }
        for (int64_t c = tail0 + threadIdx.x; c < e; c += kThreads) key = key_merge(key, absbits_f32(xb[c]));
    }
    return block_key_merge(key);
}

__global__ void __launch_bounds__(kThreads) k_requant_amax(RequantBatch bt)
{
    const int bid = blockIdx.x;
    int c = 0;
    for (int i = 1; i < bt.count; ++i)
        if (bt.item[i].nwg > 0 && bid >= bt.item[i].wg0) c = i;
    const RequantItem& it = bt.item[c];
    const int local = bid - it.wg0;
    if (it.nwg == 0 || local < 0 || local >= it.nwg) return;   // (never: the grid is the sum of nwg)
    const int64_t n = (int64_t)it.rows * it.cols;
    const int64_t per = ((n + it.nwg - 1) / it.nwg + 7) & ~(int64_t)7;
    const int64_t b = min(n, (int64_t)local * per), e = min(n, b + per);
    const uint32_t key = it.dtype == FP8_IN_BF16 ? amax_range<0>(it.x, b, e, it.vec_amax)
                                                 : amax_range<1>(it.x, b, e, it.vec_amax);
    if (threadIdx.x == 0) it.parts[local] = key;
}

template <int FMT, int DT>
__device__ inline void requant_tile(const RequantItem& it, float s, bool special, int64_t tid, uint8_t* tile,
                                    uint32_t& sat, uint32_t& und, uint32_t& nan)
{
    if (it.gran == FP8_TENSOR)
        tile128_one<FMT, DT, 0, false>(it.x, it.rows, it.cols, it.cols, it.vec_tile, it.scale, s, special, true, it.q,
                                       it.cols, it.qt, it.rows, 0, tid, tile, sat, und, nan);
    else
        tile128_one<FMT, DT, 1, false>(it.x, it.rows, it.cols, it.cols, it.vec_tile, it.scale, 1.0f, true, false,
                                       it.q, it.cols, it.qt, it.rows, 0, tid, tile, sat, und, nan);
}

__global__ void __launch_bounds__(kThreads) k_requant_cast(RequantBatch bt)
{
    __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kTilePitch];
    const int64_t per = (bt.total_tiles + gridDim.x - 1) / gridDim.x;
    const int64_t t0 = (int64_t)blockIdx.x * per, t1 = min(bt.total_tiles, t0 + per);
    int c = -1;
    float s = 1.0f;
    bool special = true;
    uint32_t sat = 0, und = 0, nan = 0;
    for (int64_t f = t0; f < t1; ++f) {
        int cn = 0;
        for (int i = 1; i < bt.count; ++i)
            if (f >= bt.item[i].tile0) cn = i;
        if (cn != c) {
            if (c >= 0) {
                flush_counters_block(bt.item[c].ctr, sat, und, nan);
                __syncthreads();
                sat = und = nan = 0;
            }
            c = cn;
            const RequantItem& it = bt.item[c];
            if (it.gran == FP8_TENSOR) {
                const uint32_t k = reduce_partials(it.parts, it.nwg);
                special = key_special(k);
                s = it.fmt == FP8_E4M3 ? scale_from_amax<0>(key_amax(k)) : scale_from_amax<1>(key_amax(k));
                if (f == it.tile0 && threadIdx.x == 0) it.scale[0] = s;
            }
        }
        const RequantItem& it = bt.item[c];
        const int64_t tid = f - it.tile0;
        if (it.lean) {
            // whole tiles of a lean cache were cast by k_requant_lean
            const int64_t tc = (it.cols + kTile - 1) / kTile, br = tid / tc, bc = tid - br * tc;
            if ((br + 1) * kTile <= it.rows && (bc + 1) * kTile <= it.cols) continue;
        }
        if (it.fmt == FP8_E4M3) {
            if (it.dtype == FP8_IN_BF16) requant_tile<0, 0>(it, s, special, tid, tile, sat, und, nan);
            else requant_tile<0, 1>(it, s, special, tid, tile, sat, und, nan);
        } else {
            if (it.dtype == FP8_IN_BF16) requant_tile<1, 0>(it, s, special, tid, tile, sat, und, nan);
            else requant_tile<1, 1>(it, s, special, tid, tile, sat, und, nan);
        }
        __syncthreads();   // the LDS staging tile and the block amax scratch are reused by the next tile
    }
    if (c >= 0) flush_counters_block(bt.item[c].ctr, sat, und, nan);
}

// Whole bf16 tiles of the batch's lean caches, one tile per 512-thread
// workgroup (the arrangement of k_tile128t_bf16 and k_block128_bf16: 4 x 8
// elements per thread, at most 64 registers, so that a launch of up to 4
// tiles per CU is resident at once; the 12 caches of a 12-layer model's
// up-projection are 1728 tiles).  Per-tensor caches take their scale from
// their amax partials, per-block caches each block's own amax.  Edge tiles,
// and every tile of a cache that is not lean, return at once and are left to
// k_requant_cast.
template <int FMT>
__device__ __forceinline__ void requant_lean_tile(const RequantItem& it, int64_t tid, int64_t tiles_c, uint32_t* tl,
                                                  uint32_t* sh)
{
    const int t = threadIdx.x, g = t >> 4, k = t & 15;
    const int64_t br = tid / tiles_c, bc = tid - br * tiles_c;
    const int64_t r0 = br * kTile, c0 = bc * kTile;
    const int64_t ld = it.cols;
    const uint16_t* x = static_cast<const uint16_t*>(it.x);
    uint4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = ld_stream(x + (r0 + 4 * g + i) * ld + c0 + 8 * k);
    float s;
    bool fast;
    if (it.gran == FP8_TENSOR) {
        const uint32_t kk = reduce_partials(it.parts, it.nwg);
        s = scale_from_amax<FMT>(key_amax(kk));
        fast = !key_special(kk) && s >= kCorrectedQuotMinScale;
        if (tid == 0 && t == 0) it.scale[0] = s;
    } else {
        us2 pk = us2{0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) pk = pkmax8(pk, w[i]);
        uint32_t key = wave_max(pk_raw(pk));
        if ((t & 63) == 0) sh[t >> 6] = key;
        __syncthreads();
        key = sh[0];
#pragma unroll
        for (int i = 1; i < kBlkThreads / 64; ++i) key = max(key, sh[i]);
        if (key >= kRawNonFinite) {
            // an Inf or NaN in the block: the exact merge (finite amax + flag)
            __syncthreads();
            uint32_t e = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    e = key_merge(e, absbits_bf16(ws[h] & 0xFFFFu));
                    e = key_merge(e, absbits_bf16(ws[h] >> 16));
                }
            }
            e = wave_key_merge(e);
            if ((t & 63) == 0) sh[t >> 6] = e;
            __syncthreads();
            key = sh[0];
            for (int i = 1; i < kBlkThreads / 64; ++i) key = key_merge(key, sh[i]);
        }
        s = scale_from_amax<FMT>(key_amax(key));
        fast = !key_special(key) && s >= kCorrectedQuotMinScale;
        if (t == 0) it.scale[br * tiles_c + bc] = s;
    }
    const float r = 1.0f / s;
    uint32_t sat = 0, und = 0, nan = 0;
    uint2 code[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ws[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
        if (fast) {
            code[i] = cast8_bf16_fast<FMT>(ws, s, r, und);
        } else {
            float v[8];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[2 * h] = bf16_lo(ws[h]);
                v[2 * h + 1] = bf16_hi(ws[h]);
            }
            code[i] = cast8<FMT, false>(v, s, 0.0f, sat, und, nan);
        }
        *reinterpret_cast<uint2*>(it.q + (r0 + 4 * g + i) * ld + c0 + 8 * k) = code[i];
    }
    if (it.qt) {
        // the transposed copy through LDS, as in k_tile128t_bf16
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t a = half ? code[0].y : code[0].x;
            const uint32_t b = half ? code[1].y : code[1].x;
            const uint32_t c = half ? code[2].y : code[2].x;
            const uint32_t d = half ? code[3].y : code[3].x;
            const uint32_t x0 = __builtin_amdgcn_perm(b, a, 0x05010400u);
            const uint32_t x1 = __builtin_amdgcn_perm(b, a, 0x07030602u);
            const uint32_t y0 = __builtin_amdgcn_perm(d, c, 0x05010400u);
            const uint32_t y1 = __builtin_amdgcn_perm(d, c, 0x07030602u);
            const uint32_t col[4] = {__builtin_amdgcn_perm(y0, x0, 0x05040100u), __builtin_amdgcn_perm(y0, x0, 0x07060302u),
                                     __builtin_amdgcn_perm(y1, x1, 0x05040100u), __builtin_amdgcn_perm(y1, x1, 0x07060302u)};
#pragma unroll
            for (int j = 0; j < 4; ++j) tl[(8 * k + 4 * half + j) * 32 + (g ^ (4 * (k & 7)))] = col[j];
        }
        barrier_lds_only();
        const int cc = t & 127, qq = t >> 7;
        const int sw = 4 * ((cc >> 3) & 7);
        const uint4 lo = *reinterpret_cast<const uint4*>(&tl[cc * 32 + ((8 * qq) ^ sw)]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&tl[cc * 32 + ((8 * qq + 4) ^ sw)]);
        uint8_t* dst = it.qt + (c0 + cc) * (int64_t)it.rows + r0 + 32 * qq;
        *reinterpret_cast<uint4*>(dst) = lo;
        *reinterpret_cast<uint4*>(dst + 16) = hi;
    }
    flush_counters_block(it.ctr, sat, und, nan);
}

__global__ void __launch_bounds__(kBlkThreads) __attribute__((amdgpu_waves_per_eu(8))) k_requant_lean(RequantBatch bt)
{
    __shared__ __attribute__((aligned(16))) uint32_t tl[kTile * kTile / 4];
    __shared__ uint32_t sh[kBlkThreads / 64];
    const int64_t f = blockIdx.x;
    int c = 0;
    for (int i = 1; i < bt.count; ++i)
        if (f >= bt.item[i].tile0) c = i;
    const RequantItem& it = bt.item[c];
    if (!it.lean) return;
    const int64_t tiles_c = (it.cols + kTile - 1) / kTile;
    const int64_t tid = f - it.tile0;
    const int64_t br = tid / tiles_c, bc = tid - br * tiles_c;
    if ((br + 1) * kTile > it.rows || (bc + 1) * kTile > it.cols) return;   // edge tile
    if (it.fmt == FP8_E4M3)
        requant_lean_tile<0>(it, tid, tiles_c, tl, sh);
    else
        requant_lean_tile<1>(it, tid, tiles_c, tl, sh);
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

// 128x128 tiles: full tiles of an aligned bf16 tensor go to k_tile128_bf16,
// the rest (edge tiles, fp32 input, unaligned layouts) to k_tile128.
template <int FMT, int DT, int SCALE_MODE>
hipError_t launch_tiles(const QuantArgs& a, int vec, const uint32_t* parts, int np, hipStream_t stream)
{
    const int64_t rows = a.rows, cols = a.cols;
    const int64_t nt = cdiv(rows, kTile) * cdiv(cols, kTile);
    const int64_t nfull = (rows / kTile) * (cols / kTile);
    int only_partial = 0;
    if (DT == 0 && vec && nfull > 0 && SCALE_MODE == 1 && !a.qt) {
        // per-block amax and no transposed copy: one block per 512 threads
        const int64_t blocks_c = cols / kTile;
        const uint16_t* xb = static_cast<const uint16_t*>(a.x);
        if (nfull <= (int64_t)num_cus() * kBlkOnePerWgMax)
            hipLaunchKernelGGL((k_block128_bf16<FMT, false>), dim3((unsigned)nfull), dim3(kBlkThreads), 0, stream,
                               xb, a.ld, blocks_c, nfull, a.scale, cdiv(cols, kTile), a.q, a.ldq, a.ctr, a.pow2);
        else
            hipLaunchKernelGGL((k_block128_bf16<FMT, true>), dim3(num_cus() * kBlkPerCu), dim3(kBlkThreads), 0,
                               stream, xb, a.ld, blocks_c, nfull, a.scale, cdiv(cols, kTile), a.q, a.ldq, a.ctr,
                               a.pow2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || nfull == nt) return e;
        only_partial = 1;
    } else if (DT == 0 && vec && nfull > 0 && nfull <= (int64_t)num_cus() * kBlkOnePerWgMax && SCALE_MODE == 0 &&
               a.qt) {
        // per-tensor scale with the transposed copy, a small tensor: one tile
        // per 512-thread workgroup
        hipLaunchKernelGGL((k_tile128t_bf16<FMT>), dim3((unsigned)nfull), dim3(kBlkThreads), 0, stream,
                           static_cast<const uint16_t*>(a.x), a.ld, cols / kTile, a.scale, parts, np, a.q, a.ldq,
                           a.qt, a.ldqt, a.ctr, a.pow2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || nfull == nt) return e;
        only_partial = 1;
    } else if (DT == 0 && vec && nfull > 0) {
        // a workgroup is 4 waves, one per SIMD: per-tensor mode fills each CU once
        const int per_cu = SCALE_MODE == 0 ? kTileWavesPerSimd0 : 4;
        const int grid = (int)std::min<int64_t>(nfull, (int64_t)num_cus() * per_cu);
        hipLaunchKernelGGL((k_tile128_bf16<FMT, SCALE_MODE>), dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(a.x), rows, cols, a.ld, a.scale, parts, np, a.q, a.ldq,
                           a.qt, a.ldqt, a.ctr, nullptr, 0, nullptr, a.pow2);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || nfull == nt) return e;
        only_partial = 1;
    }
    const int grid = (int)std::min<int64_t>(nt, (int64_t)num_cus() * 8);
    hipLaunchKernelGGL((k_tile128<FMT, DT, SCALE_MODE, false>), dim3(grid), dim3(kThreads), 0, stream, a.x, rows,
                       cols, a.ld, vec, a.scale, parts, np, a.q, a.ldq, a.qt, a.ldqt, a.ctr, only_partial,
                       a.pow2);
    return hipGetLastError();
}

// Polls of k_tile128t_once's bounded wait before a workgroup falls back to
// reading the whole tensor (0: always fall back).
std::atomic<int> g_once_wait_limit{1 << 14};

// A per-tensor quantize from amax that k_tile128t_once takes in one launch:
// bf16, whole 128 x 128 tiles, at most one tile per CU, the layouts of its
// vector loads and stores, and an 8-byte aligned workspace for the call's
// slots.
bool once_fits(const QuantArgs& a)
{
    const int64_t nt = (a.rows / kTile) * (a.cols / kTile);
    return a.dtype == FP8_IN_BF16 && a.rows > 0 && a.rows % kTile == 0 && a.cols % kTile == 0 &&
           nt <= std::min<int64_t>(kOnceMaxTiles, num_cus()) && aligned16(a.x) && (a.ld * 2) % 16 == 0 &&
           (reinterpret_cast<uintptr_t>(a.q) & 7u) == 0 && a.ldq % 8 == 0 &&
           (!a.qt || (aligned16(a.qt) && a.ldqt % 16 == 0)) && a.partials &&
           (reinterpret_cast<uintptr_t>(a.partials) & 7u) == 0;
}

template <int FMT, int DT>
hipError_t quantize_typed(const QuantArgs& a, hipStream_t stream)
{
    const int eb = DT == 0 ? 2 : 4;
    const int64_t rows = a.rows, cols = a.cols;
    if (a.gran == FP8_TENSOR) {
        const bool from_amax = a.mode == FP8_SCALE_FROM_AMAX;
        if (DT == 0 && from_amax && once_fits(a)) {
            const unsigned nt = (unsigned)((rows / kTile) * (cols / kTile));
            hipLaunchKernelGGL((k_tile128t_once<FMT>), dim3(nt), dim3(kBlkThreads), 0, stream,
                               static_cast<const uint16_t*>(a.x), rows, cols, a.ld, a.scale,
                               reinterpret_cast<OnceSync*>(a.partials), a.q, a.ldq, a.qt, a.ldqt, a.ctr, a.pow2,
                               g_once_wait_limit.load(std::memory_order_relaxed));
            return hipGetLastError();
        }
        int np = 0;
        if (from_amax) {
            int64_t r = rows, c = cols, ld = a.ld;
            flatten(r, c, ld);
            const int vec = aligned16(a.x) && (r == 1 || (ld * eb) % 16 == 0);
            const dim3 g = stream_grid(r, c, 32, kAmaxGrid);
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
            return launch_tiles<FMT, DT, 0>(a, vec, parts, np, stream);
        } else {
            int64_t r = rows, c = cols, ld = a.ld, ldq = a.ldq;
            flatten(r, c, ld, &ldq);
            const int vec = aligned16(a.x) && aligned16(a.q) &&
                            (r == 1 || ((ld * eb) % 16 == 0 && ldq % 16 == 0));
            const dim3 g = stream_grid(r, c, 32, num_cus() * 8);
            hipLaunchKernelGGL((k_cast_tensor<FMT, DT>), g, dim3(kThreads), 0, stream, a.x, r, c, ld, vec,
                               a.q, ldq, a.scale, parts, np, a.ctr, a.pow2);
        }
        return hipGetLastError();
    }
    if (a.gran == FP8_BLOCK_128x128) {
        const int vec = aligned16(a.x) && aligned16(a.q) && (!a.qt || aligned16(a.qt)) && (a.ld * eb) % 16 == 0 &&
                        a.ldq % 8 == 0 && (!a.qt || a.ldqt % 16 == 0);
        if (a.mode == FP8_SCALE_FROM_AMAX) return launch_tiles<FMT, DT, 1>(a, vec, nullptr, 0, stream);
        return launch_tiles<FMT, DT, 2>(a, vec, nullptr, 0, stream);
    }
    // ROW_1x128
    const int64_t tpr = cdiv(cols, 128);
    const int64_t ntiles = rows * tpr;
    const int vec = aligned16(a.x) && (a.ld * eb) % 16 == 0 && a.ldq % 8 == 0 && aligned16(a.q);
    if (DT == 0 && vec && cols % 128 == 0 && a.mode == FP8_SCALE_FROM_AMAX) {
        const int grid = (int)std::min<int64_t>(cdiv(ntiles, kThreads / 16 * 4), (int64_t)num_cus() * 4);
        hipLaunchKernelGGL(k_row1x128_bf16<FMT>, dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(a.x), a.ld, a.scale, a.q, a.ldq, a.ctr, (uint32_t)ntiles,
                           FastDiv((uint32_t)tpr), (uint32_t)tpr, a.pow2);
        return hipGetLastError();
    }
    const int grid = (int)std::min<int64_t>(cdiv(ntiles, kThreads / 16), (int64_t)num_cus() * 16);
    if (a.mode == FP8_SCALE_FROM_AMAX)
        hipLaunchKernelGGL((k_row1x128<FMT, DT, false, false>), dim3(grid), dim3(kThreads), 0, stream, a.x, rows,
                           cols, a.ld, vec, a.scale, a.q, a.ldq, a.ctr, (uint32_t)ntiles, FastDiv((uint32_t)tpr),
                           a.pow2);
    else
        hipLaunchKernelGGL((k_row1x128<FMT, DT, true, false>), dim3(grid), dim3(kThreads), 0, stream, a.x, rows,
                           cols, a.ld, vec, a.scale, a.q, a.ldq, a.ctr, (uint32_t)ntiles, FastDiv((uint32_t)tpr),
                           a.pow2);
    return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ library-owned scratch
// The per-tensor amax partials of fp8_quantize_noalloc live in this array
// rather than in a caller's workspace: one copy per device, loaded with the
// code object and held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it asks the runtime for the device address once per device and
// passes that.
static __device__ __align__(256) uint32_t scratch[kNoAllocScratchWords];

namespace {
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t noalloc_scratch(uint32_t** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// ------------------------------------------------------------------ launchers
int set_once_wait_limit(int polls) { return g_once_wait_limit.exchange(polls < 0 ? 0 : polls); }

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

// Weight-cache refresh: the caches go in groups of kRequantMaxCaches; per
// group one amax launch over its per-tensor caches (if any), one launch for
// the whole tiles of its bf16 caches (k_requant_lean) and one for every other
// tile (k_requant_cast, left out when there is none).  Empty caches take
// launch_quantize (a per-tensor one still reports scale 1).
hipError_t launch_requant(const QuantArgs* caches, int count, hipStream_t stream)
{
    hipError_t e;
    // one cache: the single-tensor path (its bf16 tile kernel is faster than
    // the batch's general tile code; the launch count is the same)
    if (count == 1) return launch_quantize(caches[0], stream);
    for (int g0 = 0; g0 < count; g0 += kRequantMaxCaches) {
        RequantBatch bt{};
        int wg = 0;
        int64_t tiles = 0, rest = 0;
        bool any_lean = false;
        for (int i = g0; i < std::min(count, g0 + kRequantMaxCaches); ++i) {
            const QuantArgs& a = caches[i];
            if (a.rows == 0 || a.cols == 0) {
                if ((e = launch_quantize(a, stream)) != hipSuccess) return e;
                continue;
            }
            RequantItem& it = bt.item[bt.count++];
            const int eb = a.dtype == FP8_IN_BF16 ? 2 : 4;
            it.x = a.x;
            it.q = a.q;
            it.qt = a.qt;
            it.scale = a.scale;
            it.ctr = a.ctr;
            it.parts = a.partials;
            it.rows = a.rows;
            it.cols = a.cols;
            it.dtype = (int8_t)a.dtype;
            it.fmt = (int8_t)a.fmt;
            it.gran = (int8_t)a.gran;
            it.vec_amax = aligned16(a.x);
            it.vec_tile = aligned16(a.x) && aligned16(a.q) && (!a.qt || aligned16(a.qt)) && (a.cols * eb) % 16 == 0 &&
                          a.cols % 8 == 0 && (!a.qt || a.rows % 16 == 0);
            it.lean = a.dtype == FP8_IN_BF16 && it.vec_tile;
            it.tile0 = tiles;
            tiles += cdiv(a.rows, kTile) * cdiv(a.cols, kTile);
            // tiles left to the general kernel
            rest += it.lean ? cdiv(a.rows, kTile) * cdiv(a.cols, kTile) - (a.rows / kTile) * (a.cols / kTile)
                            : cdiv(a.rows, kTile) * cdiv(a.cols, kTile);
            any_lean |= it.lean && a.rows >= kTile && a.cols >= kTile;
            it.wg0 = wg;
            it.nwg = 0;
            if (a.gran == FP8_TENSOR) {
                const int64_t n = a.rows * a.cols;
                it.nwg = (int)std::min<int64_t>(std::max<int64_t>(cdiv(n, (int64_t)kThreads * 64), 1), kRequantAmaxParts);
                wg += it.nwg;
            }
        }
        if (bt.count == 0) continue;
        bt.total_tiles = tiles;
        if (wg > 0) {
            hipLaunchKernelGGL(k_requant_amax, dim3(wg), dim3(kThreads), 0, stream, bt);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (any_lean && tiles > INT32_MAX) {
            // more tiles than one grid dimension holds: the general kernel takes all
            for (int i = 0; i < bt.count; ++i) bt.item[i].lean = 0;
            any_lean = false;
            rest = tiles;
        }
        if (any_lean) {
            hipLaunchKernelGGL(k_requant_lean, dim3((unsigned)tiles), dim3(kBlkThreads), 0, stream, bt);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (rest > 0) {
            const int grid = (int)std::min<int64_t>(tiles, (int64_t)num_cus() * 4);
            hipLaunchKernelGGL(k_requant_cast, dim3(grid), dim3(kThreads), 0, stream, bt);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Delayed scaling.  A bf16 tensor of whole 128x128 tiles with 16-byte rows
// and a transposed copy takes one pass (cast with the history scale while
// collecting this tensor's amax); any other layout takes the amax pass, the
// history scale and a given-scale cast (same bytes, two reads of x).
hipError_t launch_quantize_delayed(const QuantArgs& a, float* hist, int32_t* pos, int len, hipStream_t stream)
{
    const int64_t rows = a.rows, cols = a.cols;
    const bool one_pass = a.dtype == FP8_IN_BF16 && a.qt && rows % kTile == 0 && cols % kTile == 0 &&
                          aligned16(a.x) && aligned16(a.q) && aligned16(a.qt) && (a.ld * 2) % 16 == 0 &&
                          a.ldq % 8 == 0 && a.ldqt % 16 == 0 && rows > 0 && cols > 0;
    if (one_pass) {
        const int64_t nfull = (rows / kTile) * (cols / kTile);
        const int grid = (int)std::min<int64_t>(nfull, std::min<int64_t>((int64_t)num_cus() * 4, kAmaxPartials));
        if (a.fmt == FP8_E4M3)
            hipLaunchKernelGGL((k_tile128_bf16<0, 3>), dim3(grid), dim3(kThreads), 0, stream,
                               static_cast<const uint16_t*>(a.x), rows, cols, a.ld, a.scale, nullptr, 0, a.q, a.ldq,
                               a.qt, a.ldqt, a.ctr, hist, len, a.partials, 0);
        else
            hipLaunchKernelGGL((k_tile128_bf16<1, 3>), dim3(grid), dim3(kThreads), 0, stream,
                               static_cast<const uint16_t*>(a.x), rows, cols, a.ld, a.scale, nullptr, 0, a.q, a.ldq,
                               a.qt, a.ldqt, a.ctr, hist, len, a.partials, 0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_delayed_record, dim3(1), dim3(kThreads), 0, stream, a.partials, grid, hist, pos, len);
        return hipGetLastError();
    }
    // amax partials of x (its own amax, for the record)
    const int eb = a.dtype == FP8_IN_BF16 ? 2 : 4;
    int64_t r = rows, c = cols, l = a.ld;
    flatten(r, c, l);
    const int vec = aligned16(a.x) && (r == 1 || (l * eb) % 16 == 0);
    dim3 g = stream_grid(r, c, 32, kAmaxGrid);
    if (rows == 0 || cols == 0) { r = 0; g = dim3(1, 1, 1); }
    if (a.dtype == FP8_IN_BF16)
        hipLaunchKernelGGL(k_amax_partials<0>, g, dim3(kThreads), 0, stream, a.x, r, c, l, vec, a.partials);
    else
        hipLaunchKernelGGL(k_amax_partials<1>, g, dim3(kThreads), 0, stream, a.x, r, c, l, vec, a.partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.fmt == FP8_E4M3)
        hipLaunchKernelGGL(k_delayed_scale<0>, dim3(1), dim3(kThreads), 0, stream, hist, len, a.scale);
    else
        hipLaunchKernelGGL(k_delayed_scale<1>, dim3(1), dim3(kThreads), 0, stream, hist, len, a.scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (rows > 0 && cols > 0) {
        QuantArgs b = a;
        b.mode = FP8_SCALE_GIVEN;
        b.partials = nullptr;
        if ((e = launch_quantize(b, stream)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_delayed_record, dim3(1), dim3(kThreads), 0, stream, a.partials, (int)(g.x * g.y), hist, pos,
                       len);
    return hipGetLastError();
}

hipError_t launch_amax_partials(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                                uint32_t* partials, int* np, hipStream_t stream)
{
    const int eb = dtype == FP8_IN_BF16 ? 2 : 4;
    int64_t r = rows, c = cols, l = ld;
    flatten(r, c, l);
    const int vec = aligned16(x) && (r == 1 || (l * eb) % 16 == 0);
    dim3 g = stream_grid(r, c, 32, kAmaxGrid);
    if (rows == 0 || cols == 0) { r = 0; g = dim3(1, 1, 1); }
    if (dtype == FP8_IN_BF16)
        hipLaunchKernelGGL(k_amax_partials<0>, g, dim3(kThreads), 0, stream, x, r, c, l, vec, partials);
    else
        hipLaunchKernelGGL(k_amax_partials<1>, g, dim3(kThreads), 0, stream, x, r, c, l, vec, partials);
    *np = (int)(g.x * g.y);
    return hipGetLastError();
}

hipError_t launch_amax_tensor(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, float* out,
                              uint32_t* partials, hipStream_t stream)
{
    const int eb = dtype == FP8_IN_BF16 ? 2 : 4;
    int64_t r = rows, c = cols, l = ld;
    flatten(r, c, l);
    const int vec = aligned16(x) && (r == 1 || (l * eb) % 16 == 0);
    dim3 g = stream_grid(r, c, 32, kAmaxGrid);
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
                               vec, out, nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0, 0);
        else
            hipLaunchKernelGGL((k_tile128<0, 1, 1, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows, cols, ld,
                               vec, out, nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0, 0);
        return hipGetLastError();
    }
    const int64_t tpr = cdiv(cols, 128);
    const int64_t ntiles = rows * tpr;
    const int grid = (int)std::min<int64_t>(cdiv(ntiles, kThreads / 16), (int64_t)num_cus() * 16);
    if (dtype == FP8_IN_BF16)
        hipLaunchKernelGGL((k_row1x128<0, 0, false, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows, cols,
                           ld, vec, out, nullptr, 0, nullptr, (uint32_t)ntiles, FastDiv((uint32_t)tpr), 0);
    else
        hipLaunchKernelGGL((k_row1x128<0, 1, false, true>), dim3(grid), dim3(kThreads), 0, stream, x, rows, cols,
                           ld, vec, out, nullptr, 0, nullptr, (uint32_t)ntiles, FastDiv((uint32_t)tpr), 0);
    return hipGetLastError();
}

hipError_t launch_counters_reset(fp8_counters* ctr, hipStream_t stream)
{
    hipLaunchKernelGGL(k_counters_reset, dim3(1), dim3(64), 0, stream, ctr);
    return hipGetLastError();
}

}  // namespace fp8mi
