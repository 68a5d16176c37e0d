// Scaled FP8 GEMM for gfx950: y = (s_a A_q)(s_b B_q)^T, A [m,k] and B [n,k]
// both K-contiguous (the TN form _scaled_mm(x, w_fp8, scale_a, scale_b) takes,
// "#84 FP8 Precision", code excerpt), fp32 accumulation on the CDNA4 FP8
// matrix cores, bf16 output.  Block-scaled form: per 128-wide K block, the
// partial product of each 16x16 output tile is promoted into the fp32
// accumulator with s_a[row, kb] * s_b[n/128, kb] ("fine grained tile and block
// scaling", "FP8 stability guardrails", section "Real products").
//
// Design (one workgroup per 256x256 output tile, 4 waves of 128x128):
//   - K steps of 128 bytes; A and B tiles staged in LDS (2 x 64 KB, double
//     buffered) with a 16-byte-chunk XOR swizzle that keeps both the row-wise
//     fills and the fragment reads free of bank conflicts;
//   - v_mfma_scale_f32_16x16x128_f8f6f4 with unit E8M0 scales (exponent 127):
//     every instruction covers exactly one 128-wide K block;
//   - workgroup ids are spread over the 8 XCDs so that each XCD walks a
//     contiguous, M-grouped range of output tiles (A panels stay in its L2);
//   - optional split over K with fp32 partials reduced in a fixed order.
#include <hip/hip_bf16.h>

#include <algorithm>

#include "device_common.h"
#include "fp8mi_internal.h"

namespace fp8mi {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kGemmThreads = 256;
constexpr int kGroupM = 8;
constexpr int kTileBytes = BM * BK;       // 32 KB per operand tile

// 16-byte chunk c (0..7) of row r lives at chunk position swz(r, c).  Any 8
// consecutive rows reading the same logical chunk land in 8 distinct
// positions, and any 16 consecutive rows cover all 16 (row parity x
// position) slots of a 256-byte bank line.
__device__ inline int swz(int r, int c) { return c ^ (((r >> 1) & 7) ^ ((r & 1) << 2)); }

template <int FA, int FB>
__device__ inline v4f mfma(const v8i& a, const v8i& b, const v4f& c)
{
    // unit block scales: E8M0 exponent 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 127, 0, 127);
}

struct KArgs {
    const uint8_t* a;
    const uint8_t* b;
    int64_t lda, ldb;
    const float* sa;
    const float* sb;
    int m, n, k;
    uint16_t* c;
    int64_t ldc;
    float* ws;
    int splits;
    int ktiles;          // ceil(k / BK)
    int tiles_m, tiles_n;
    fp8_counters* ctr;
};

// Operand tiles move from global memory straight into LDS with
// buffer_load_dwordx4 ... lds: one instruction fills 1 KB (8 rows of 128
// bytes) at the wave-uniform LDS address in M0, lane l writing bytes
// 16 l .. 16 l + 15.  Wave w fills rows 64 w .. 64 w + 63 with 8
// instructions; the swizzle is applied on the global side by choosing which
// 16-byte chunk each lane fetches.  Rows past the operand's end fall outside
// the buffer descriptor's range, and K chunks past k are given an offset
// outside it: the range check makes both read as zero, with no branches.
constexpr uint32_t kOutOfRange = 0x80000000u;

struct TileLoader {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t voff[8];   // byte offset of this lane's chunk for instruction j, at k0 = 0
    int ck[2];          // K byte offset of that chunk within a K step (depends on j & 1 only)
};

__device__ inline TileLoader make_loader(const uint8_t* base, int64_t ld, int row0, int rows)
{
    TileLoader L;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t left = (int64_t)rows - row0;
    const int64_t nrec = left <= 0 ? 0 : std::min<int64_t>(left, BM) * ld;
    L.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + (int64_t)row0 * ld), (short)0,
                                               (int)std::min<int64_t>(nrec, 0x7FFFFFF0), 0x00020000);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 64 * w + 8 * j + (l >> 3);
        const int c = swz(r, l & 7);      // the swizzle is its own inverse
        L.voff[j] = (uint32_t)(r * ld + 16 * c);
        if (j < 2) L.ck[j] = 16 * c;
    }
    return L;
}

__device__ inline void issue_tile(const TileLoader& L, uint8_t* lds_tile, int k0, int k)
{
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t off = k0 + L.ck[j & 1] < k ? L.voff[j] + (uint32_t)k0 : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rsrc,
                                                 (__attribute__((address_space(3))) void*)(lds_tile + (w * 8 + j) * 1024),
                                                 16, (int)off, 0, 0, 0);
    }
}

// MFMA operand fragment for rows row0..row0+15 of a staged tile: lane l holds
// row row0 + l%16, K bytes 32*(l/16) .. +32 (the same K assignment is used for
// A and B, so the products pair up element for element).
__device__ inline v8i load_frag(const uint8_t* lds, int row0)
{
    const int l = threadIdx.x & 63;
    const int r = row0 + (l & 15);
    const int c0 = (l >> 4) * 2;
    const uint4 lo = *reinterpret_cast<const uint4*>(lds + r * BK + swz(r, c0) * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(lds + r * BK + swz(r, c0 + 1) * 16);
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
}

__device__ inline uint16_t to_bf16(float v)
{
    return __builtin_bit_cast(uint16_t, __float2bfloat16(v));
}

// Map a linear workgroup id to (split, tile_m, tile_n).  Hardware hands ids
// to XCDs round robin; re-number so that XCD x owns a contiguous block of
// logical ids, then walk tiles M-grouped (kGroupM tile rows at a time).
__device__ inline void tile_of(const KArgs& p, int& split, int& tm, int& tn)
{
    const int total = p.tiles_m * p.tiles_n * p.splits;
    const int bid = blockIdx.x;
    const int xcd = bid & 7, local = bid >> 3;
    const int q = total >> 3, rem = total & 7;
    const int pid = xcd * q + min(xcd, rem) + local;
    const int per_split = p.tiles_m * p.tiles_n;
    split = pid / per_split;
    const int t = pid - split * per_split;
    const int in_group = kGroupM * p.tiles_n;
    const int g = t / in_group;
    const int first_m = g * kGroupM;
    const int gsize = min(p.tiles_m - first_m, kGroupM);
    const int r = t - g * in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

__shared__ __attribute__((aligned(1024))) uint8_t g_lds_a[2 * kTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_lds_b[2 * kTileBytes];
__shared__ __attribute__((aligned(16))) float g_lds_sa[2 * BM];

// Per K step and wave: read all 16 operand fragments of the current stage,
// then start the DMA of the next stage, then run the 64 MFMAs.  Reading
// before the DMA is issued keeps the compiler from making the reads wait for
// the DMA (it cannot tell the two stages apart).
template <int FA, int FB, bool BLOCK>
__global__ void __launch_bounds__(kGemmThreads, 1) k_gemm(KArgs p)
{
    int split, tm, tn;
    tile_of(p, split, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt_per = (p.ktiles + p.splits - 1) / p.splits;
    const int kt0 = split * kt_per;
    const int kt1 = min(p.ktiles, kt0 + kt_per);

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wm = (wave >> 1) * 128;
    const int wn = (wave & 1) * 128;
    const int nkb = p.k / BK;   // block-scale columns (k % 128 == 0 in block mode)
    const int nb = (n0 + wn) / 128;
    const bool wave_has_cols = n0 + wn < p.n;

    v4f acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const TileLoader la_ = make_loader(p.a, p.lda, m0, p.m);
    const TileLoader lb_ = make_loader(p.b, p.ldb, n0, p.n);
    if (kt0 < kt1) {
        issue_tile(la_, g_lds_a, kt0 * BK, p.k);
        issue_tile(lb_, g_lds_b, kt0 * BK, p.k);
        if constexpr (BLOCK)
            g_lds_sa[threadIdx.x] = (m0 + (int)threadIdx.x < p.m) ? p.sa[(int64_t)(m0 + threadIdx.x) * nkb + kt0] : 0.0f;
    }
    for (int kt = kt0; kt < kt1; ++kt) {
        const int buf = (kt - kt0) & 1;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const uint8_t* la = g_lds_a + buf * kTileBytes;
        const uint8_t* lb = g_lds_b + buf * kTileBytes;
        v8i bf[8], af[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bf[j] = load_frag(lb, wn + 16 * j);
#pragma unroll
        for (int i = 0; i < 8; ++i) af[i] = load_frag(la, wm + 16 * i);
        float4 sa4[8];
        float sbv = 0.0f;
        if constexpr (BLOCK) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                sa4[i] = *reinterpret_cast<const float4*>(&g_lds_sa[buf * BM + wm + 16 * i + 4 * (lane >> 4)]);
            sbv = wave_has_cols ? p.sb[(int64_t)nb * nkb + kt] : 0.0f;
        }
        if (kt + 1 < kt1) {
            issue_tile(la_, g_lds_a + (buf ^ 1) * kTileBytes, (kt + 1) * BK, p.k);
            issue_tile(lb_, g_lds_b + (buf ^ 1) * kTileBytes, (kt + 1) * BK, p.k);
            if constexpr (BLOCK)
                g_lds_sa[(buf ^ 1) * BM + threadIdx.x] =
                    (m0 + (int)threadIdx.x < p.m) ? p.sa[(int64_t)(m0 + threadIdx.x) * nkb + kt + 1] : 0.0f;
        }
        if constexpr (!BLOCK) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = mfma<FA, FB>(af[i], bf[j], acc[i][j]);
        } else {
            // Each MFMA covers one 128-deep K block of a 16x16 tile; its 4
            // results are promoted kLag MFMAs later, so the FMAs find them
            // written without the wait states an immediate read would need.
            constexpr int kLag = 3;
            v4f part[kLag + 1];
            v4f cf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                cf[i] = v4f{sa4[i].x * sbv, sa4[i].y * sbv, sa4[i].z * sbv, sa4[i].w * sbv};
#pragma unroll
            for (int s = 0; s < 64 + kLag; ++s) {
                if (s < 64) part[s % (kLag + 1)] = mfma<FA, FB>(af[s >> 3], bf[s & 7], v4f{0.0f, 0.0f, 0.0f, 0.0f});
                if (s >= kLag) {
                    const int q = s - kLag, i = q >> 3, j = q & 7;
                    const v4f pr = part[q % (kLag + 1)];
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(pr[r], cf[i][r], acc[i][j][r]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // epilogue: lane holds column n0+wn+16j+lane%16, rows m0+wm+16i+4(lane/16)+r
    const int col_l = lane & 15;
    const int row_l = 4 * (lane >> 4);
    if (p.ws) {
        float* ws = p.ws + (int64_t)split * p.m * p.n;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = n0 + wn + 16 * j + col_l;
                if (col >= p.n) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + wm + 16 * i + row_l + r;
                    if (row < p.m) ws[(int64_t)row * p.n + col] = acc[i][j][r];
                }
            }
        return;
    }
    const float scale = BLOCK ? 1.0f : p.sa[0] * p.sb[0];
    uint32_t nonfinite = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int col = n0 + wn + 16 * j + col_l;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + wm + 16 * i + row_l + r;
                if (row < p.m && col < p.n) {
                    const uint16_t h = to_bf16(acc[i][j][r] * scale);
                    nonfinite += (h & 0x7F80u) == 0x7F80u;
                    p.c[(int64_t)row * p.ldc + col] = h;
                }
            }
        }
    flush_counters(p.ctr, 0, 0, 0, nonfinite);
}

// Fixed-order reduction of split-K partials: y = bf16(scale * sum_s ws[s]).
__global__ void __launch_bounds__(256) k_splitk_reduce(const float* ws, int splits, int m, int n, float scale_mode_tensor,
                                                       const float* sa, const float* sb, uint16_t* c, int64_t ldc,
                                                       fp8_counters* ctr)
{
    const float scale = scale_mode_tensor != 0.0f ? sa[0] * sb[0] : 1.0f;
    const int64_t total = (int64_t)m * n;
    uint32_t nonfinite = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        float s = 0.0f;
        for (int sp = 0; sp < splits; ++sp) s += ws[(int64_t)sp * total + i];
        const uint16_t h = to_bf16(s * scale);
        nonfinite += (h & 0x7F80u) == 0x7F80u;
        const int64_t row = i / n, col = i - row * n;
        c[row * ldc + col] = h;
    }
    flush_counters(ctr, 0, 0, 0, nonfinite);
}

__global__ void k_zero_bf16(uint16_t* c, int m, int n, int64_t ldc)
{
    const int64_t total = (int64_t)m * n;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / n, col = i - row * n;
        c[row * ldc + col] = 0;
    }
}

template <int FA, int FB>
hipError_t gemm_fmt(const KArgs& p, bool block, int grid, hipStream_t stream)
{
    if (block)
        hipLaunchKernelGGL((k_gemm<FA, FB, true>), dim3(grid), dim3(kGemmThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((k_gemm<FA, FB, false>), dim3(grid), dim3(kGemmThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int gemm_num_cus()
{
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

// Split K when the output has too few 256x256 tiles to fill the 256 CUs and
// each split keeps at least 8 K steps.
int gemm_choose_splits(int64_t m, int64_t n, int64_t k)
{
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    const int64_t ktiles = (k + BK - 1) / BK;
    if (tiles >= 128 || ktiles < 16) return 1;
    int64_t s = 256 / tiles;                 // one wave of workgroups
    s = std::min<int64_t>(s, ktiles / 8);
    return (int)std::max<int64_t>(1, std::min<int64_t>(s, 64));
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream)
{
    if (g.m == 0 || g.n == 0) return hipSuccess;
    if (g.k == 0) {
        const int64_t total = g.m * g.n;
        const int grid = (int)std::min<int64_t>((total + 255) / 256, 4096);
        hipLaunchKernelGGL(k_zero_bf16, dim3(grid), dim3(256), 0, stream, static_cast<uint16_t*>(g.c), (int)g.m,
                           (int)g.n, g.ldc);
        return hipGetLastError();
    }
    KArgs p;
    p.a = g.a;
    p.b = g.b;
    p.lda = g.lda;
    p.ldb = g.ldb;
    p.sa = g.sa;
    p.sb = g.sb;
    p.m = (int)g.m;
    p.n = (int)g.n;
    p.k = (int)g.k;
    p.c = static_cast<uint16_t*>(g.c);
    p.ldc = g.ldc;
    p.ws = g.splits > 1 ? g.ws : nullptr;
    p.splits = g.splits > 1 ? g.splits : 1;
    p.ktiles = (int)((g.k + BK - 1) / BK);
    p.tiles_m = (int)((g.m + BM - 1) / BM);
    p.tiles_n = (int)((g.n + BN - 1) / BN);
    p.ctr = g.ctr;
    // never leave a split without K steps
    if (p.splits > 1) {
        const int kt_per = (p.ktiles + p.splits - 1) / p.splits;
        p.splits = (p.ktiles + kt_per - 1) / kt_per;
        if (p.splits == 1) p.ws = nullptr;
    }
    hipError_t e;
    if (!g.block_scaled) {
        e = launch_gemm_persistent(g, gemm_num_cus(), stream);
        if (e != hipSuccess || !p.ws) return e;
        const int64_t total = g.m * g.n;
        const int rgrid = (int)std::min<int64_t>((total + 255) / 256, 8192);
        hipLaunchKernelGGL(k_splitk_reduce, dim3(rgrid), dim3(256), 0, stream, p.ws, p.splits, p.m, p.n, 1.0f,
                           g.sa, g.sb, p.c, g.ldc, g.ctr);
        return hipGetLastError();
    }
    const int grid = p.tiles_m * p.tiles_n * p.splits;
    if (g.fa == FP8_E4M3)
        e = g.fb == FP8_E4M3 ? gemm_fmt<0, 0>(p, g.block_scaled, grid, stream)
                             : gemm_fmt<0, 1>(p, g.block_scaled, grid, stream);
    else
        e = g.fb == FP8_E4M3 ? gemm_fmt<1, 0>(p, g.block_scaled, grid, stream)
                             : gemm_fmt<1, 1>(p, g.block_scaled, grid, stream);
    if (e != hipSuccess || !p.ws) return e;
    const int64_t total = g.m * g.n;
    const int rgrid = (int)std::min<int64_t>((total + 255) / 256, 8192);
    hipLaunchKernelGGL(k_splitk_reduce, dim3(rgrid), dim3(256), 0, stream, p.ws, p.splits, p.m, p.n,
                       g.block_scaled ? 0.0f : 1.0f, g.sa, g.sb, p.c, g.ldc, g.ctr);
    return hipGetLastError();
}

}  // namespace fp8mi
