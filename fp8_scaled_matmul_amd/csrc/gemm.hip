// Scaled FP8 GEMM for gfx950: y = (s_a A_q)(s_b B_q)^T, A [m,k] and B [n,k]
// both K-contiguous (the TN form _scaled_mm(x, w_fp8, scale_a, scale_b) takes,
// "#84 FP8 Precision", code excerpt), fp32 accumulation on the CDNA4 FP8
// matrix cores, bf16 output.  This file holds the block-scaled form (per
// 128-wide K block, the partial product of each 16x16 output tile is promoted
// into the fp32 accumulator with s_a[row, kb] * s_b[n/128, kb]: "fine grained
// tile and block scaling", "FP8 stability guardrails", section "Real
// products"), the same kernel with per-tensor scales for K splits, the
// split-K reduction and the launch logic; the other per-tensor GEMMs run the
// persistent kernel of gemm_persistent.hip.
//
// Block-scaled design (one workgroup of 8 waves per 256x256 output tile):
//   - each wave owns 128x64 outputs, so its 128 fp32 accumulators stay in
//     VGPRs and the promotion is one v_fmac per output and K block, with no
//     AGPR copies; two waves share each SIMD, so one wave's promotion FMAs
//     run while the other's MFMAs occupy the matrix core;
//   - one v_mfma_f32_16x16x128_f8f6f4 covers exactly one K block of a 16x16
//     tile; its result is promoted three MFMAs later, when it is written (the
//     power-of-two form uses v_mfma_scale_f32_16x16x128_f8f6f4 and needs no
//     promotion);
//   - A and B K blocks (2 x 32 KB) are double buffered in LDS, filled by
//     buffer_load ... lds DMA two K blocks ahead: B early in the block, A in
//     two halves, each as soon as every wave has read the rows it refills,
//     so the requests are spread over the block; s_a arrives by DMA two K
//     blocks ahead and the workgroup turns it into s_a s_b per row and N
//     block once, in LDS;
//   - operand fragments, the next K block's included, are read from LDS
//     while the MFMAs run; three barriers per K block: once every wave holds
//     the block's B fragments, after the read of A fragment group 3, and
//     after the block's last A read;
//   - B rows are permuted in LDS so that each lane ends up with 4 adjacent
//     output columns (8-byte bf16 stores).
#include <hip/hip_bf16.h>

#include <algorithm>

#include "device_common.h"
#include "fp8mi_internal.h"
#include "gemm_common.h"

namespace fp8mi {

namespace {

using gemm::v4f;
using gemm::v4u;
using gemm::v8i;
using gemm::BM;
using gemm::BN;
using gemm::BK;
using gemm::kTileBytes;

constexpr int kBlockThreads = 512;
constexpr int kModeBlock = 0, kModeE8M0 = 1, kModeTensor = 2;   // scales: fp32 blocks, E8M0 blocks, per tensor
// MFMA results are promoted kLag MFMAs after their issue (1..3: at most 4
// partial tiles live), by which time they are written.
#ifndef FP8MI_BLOCK_LAG
#define FP8MI_BLOCK_LAG 3
#endif
constexpr int kLag = FP8MI_BLOCK_LAG;

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
    int fast_store;      // 8-byte bf16 (16-byte fp32) stores are aligned
    int group_m;         // M tiles per group of the tile order
    fp8_counters* ctr;
};

// Map a linear workgroup id to (split, tile_m, tile_n).  Hardware hands ids
// to XCDs round robin; re-number so that XCD x owns a contiguous block of
// logical ids, then walk tiles M-grouped (p.group_m tile rows at a time).
__device__ inline void item_of(const KArgs& p, int bid, int& split, int& tm, int& tn)
{
    const int total = p.tiles_m * p.tiles_n * p.splits;
    const int xcd = bid & 7, local = bid >> 3;
    const int q = total >> 3, rem = total & 7;
    const int pid = xcd * q + min(xcd, rem) + local;
    const int per_split = p.tiles_m * p.tiles_n;
    split = pid / per_split;
    const int t = pid - split * per_split;
    const int in_group = p.group_m * p.tiles_n;
    const int g = t / in_group;
    const int first_m = g * p.group_m;
    const int gsize = min(p.tiles_m - first_m, p.group_m);
    const int r = t - g * in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

__device__ inline void tile_of(const KArgs& p, int& split, int& tm, int& tn) { item_of(p, blockIdx.x, split, tm, tn); }

// Non-finite outputs: the epilogue keeps the running maximum of the stored
// |bf16| patterns (two packed maxima per 8-byte store) and counts exactly,
// by reading its outputs back, only when that maximum reaches the all-ones
// exponent (an Inf or NaN was written).
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void track_max(us2& mx, uint32_t w)
{
    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, w & 0x7FFF7FFFu));
    // pinned here: left alone, the compiler keeps every stored word live to
    // take their maximum after the last store
    uint32_t v = __builtin_bit_cast(uint32_t, mx);
    asm volatile("" : "+v"(v));
    mx = __builtin_bit_cast(us2, v);
}
#pragma clang diagnostic pop
__device__ inline bool saw_nonfinite(us2 mx) { return mx.x >= 0x7F80u || mx.y >= 0x7F80u; }

// Exact count of the Inf/NaN outputs this lane stored for the tile at (m0,
// n0) (wave w's 128 x 64 part, four adjacent columns of each of its rows per
// lane), read back once the stores have completed.
__device__ inline uint32_t recount_tile(const KArgs& p, int m0, int n0)
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = n0 + (wave >> 1) * 64 + 4 * (lane & 15);
    const int row0 = m0 + (wave & 1) * 128 + 4 * (lane >> 4);
    uint32_t n = 0;
    for (int i = 0; i < 8; ++i)
        for (int r = 0; r < 4; ++r) {
            const int row = row0 + 16 * i + r;
            if (row >= p.m) continue;
            for (int j = 0; j < 4; ++j)
                if (col + j < p.n) n += (p.c[(int64_t)row * p.ldc + col + j] & 0x7F80u) == 0x7F80u;
        }
    return n;
}

__shared__ __attribute__((aligned(1024))) uint8_t g_lds_a[2 * kTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_lds_b[2 * kTileBytes];
__shared__ __attribute__((aligned(16))) float g_lds_sa[4 * BM];       // s_a of 4 K blocks (ring)
__shared__ __attribute__((aligned(16))) float g_lds_f[4 * 2 * BM];    // s_a s_b: [K block ring][N block][row]
__shared__ __attribute__((aligned(16))) float g_lds_sb[4 * 64];       // s_b of the tile's 2 N blocks (lanes 0, 1)
// Power-of-two scales: the E8M0 code (fp32 exponent field) of s_a per K block
// ring slot, laid out [slot][row / 128][row % 16][(row % 128) / 16] so that a
// lane reads the codes of its 8 A fragments as one 8-byte word.
__shared__ __attribute__((aligned(16))) uint8_t g_lds_e[4 * 2 * 16 * 8];

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// buffer_load_dwordx4 ... lds with a wave-uniform byte offset in soffset:
// lane l's 16 bytes from voff + soff land at lds + 16 l.
__device__ inline void dma16_so(uint32_t lds, uint32_t voff, const v4u& rsrc, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// DMA geometry of one wave (w = 0..7).  Each instruction fills 8 LDS rows
// (1 KB); lane l writes position l%8 of row R, which receives logical chunk
// swz(R, l%8) of global row g(R).
// A: instruction j fills rows R = 128 (w/4) + 32 j + 8 (w%4) + l/8, so the 8
// waves' instruction j together fill rows 32 j .. 32 j + 31 and 128 + 32 j ..
// 128 + 32 j + 31: the rows of A fragment groups 2 j and 2 j + 1 of both
// wave rows, which the K loop refills once every wave has read them;
// g(R) = R.  B: instruction j fills rows R = 32 w + 8 j + l/8; within each
// 64-row group g(R) = 4 (R%16) + (R%64)/16, so that lane p of the fragment at
// LDS rows 16 j' .. 16 j' + 15 of a group carries output column 4 p + j'.
// The swizzle depends on R%16: one lane offset for A (rows 32 apart), two for
// B (rows R and R + 16 are 1 global row apart), plus a row step.  The row
// step is added to the lane offset, not to the uniform offset (which holds
// only the K offset), so that rows past the operand's end fail the
// descriptor's range check and read as zeros.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// v + u (u uniform) in a fresh register at each use: written as a volatile
// instruction so that the compiler does not keep a register per row step
// alive across the K loop.
__device__ inline uint32_t add_lane_offset(uint32_t v, uint32_t u)
{
    uint32_t r;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(u), "v"(v));
    return r;
}
#pragma clang diagnostic pop

struct BlockDma {
    v4u ra, rb, rs;           // A, B and s_a descriptors of this tile
    uint32_t va, vb[2];       // lane offsets: A instruction 0; B even and odd j
    uint32_t vs;              // lane offset of this wave's 64 s_a rows
    uint32_t step_a, step_b;  // byte step between A instructions j and j + 1, B j and j + 2
    uint32_t lds_a, lds_b, lds_s;   // this wave's LDS targets in stage 0 / ring slot 0 (uniform)
    v4u rsb;                  // s_b descriptor
    uint32_t vsb, lds_sb;     // lanes 0, 1: the tile's two N blocks; others out of range
};

__device__ inline BlockDma block_dma(const KArgs& p, int m0, int n0, int w, bool block_scales)
{
    BlockDma d;
    const int l = threadIdx.x & 63;
    const int q = l >> 3, pos = l & 7;
    const int64_t rows_a = min(p.m - m0, BM), rows_b = min(p.n - n0, BN);
    d.ra = gemm::make_rsrc(p.a + (int64_t)m0 * p.lda, (uint32_t)(rows_a * p.lda));
    d.rb = gemm::make_rsrc(p.b + (int64_t)n0 * p.ldb, (uint32_t)(rows_b * p.ldb));
    const int nkb = p.k / BK;
    // per-tensor scales: no scale blocks to fetch (zero-length descriptors)
    d.rs = gemm::make_rsrc(p.sa + (int64_t)m0 * nkb, block_scales ? (uint32_t)(rows_a * nkb * 4) : 0u);
    {
        const int R = 128 * (w >> 2) + 8 * (w & 3) + q;
        d.va = (uint32_t)(R * p.lda + 16 * gemm::swz(R, pos));
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int R = 32 * w + 8 * e + q;
        const int c = gemm::swz(R, pos);
        const int g = 64 * (w >> 1) + 32 * e + 4 * q + 2 * (w & 1);
        d.vb[e] = (uint32_t)(g * p.ldb + 16 * c);
    }
    d.vs = (uint32_t)((64 * (w & 3) + l) * nkb * 4);
    d.step_a = (uint32_t)(32 * p.lda);
    d.step_b = (uint32_t)p.ldb;
    d.lds_a = gemm::lds_addr(g_lds_a) + 16384u * (w >> 2) + 1024u * (w & 3);
    d.lds_b = gemm::lds_addr(g_lds_b) + 4096u * w;
    d.lds_s = gemm::lds_addr(g_lds_sa) + 256u * (w & 3);
    const int nbs = (p.n + 127) / 128;
    d.rsb = gemm::make_rsrc(p.sb, block_scales ? (uint32_t)(nbs * nkb * 4) : 0u);
    d.vsb = l < 2 ? (uint32_t)(((n0 >> 7) + l) * nkb * 4) : gemm::kOutOfRange;
    d.lds_sb = gemm::lds_addr(g_lds_sb);
    return d;
}

// Instruction j (0..8) of the DMA of K block kb into stage `stage`: 0..3 A,
// 4..7 B, 8 the s_a column and the two s_b values of K block kbs into ring
// slot kbs & 3 (waves w and w + 4 fetch the same 64 rows; every wave the same
// s_b pair).  `live` false turns the instruction into a
// no-op fill (a zero-length descriptor: every lane reads as zero) so that
// the K loop needs no branches past the end of the K range.
__device__ inline void block_dma_one(const BlockDma& d, int j, int stage, int kb, int kbs, bool live, int slot = -1)
{
    if (slot < 0) slot = kbs;
    const uint32_t k0 = (uint32_t)kb * BK;
    if (j < 4) {
        v4u r = d.ra;
        r.z = live ? r.z : 0u;
        const uint32_t va = j ? add_lane_offset(d.va, (uint32_t)j * d.step_a) : d.va;
        dma16_so(d.lds_a + stage * kTileBytes + 4096 * j, va, r, k0);
    } else if (j < 8) {
        const int jb = j - 4;
        v4u r = d.rb;
        r.z = live ? r.z : 0u;
        const uint32_t vb = (jb >> 1) ? add_lane_offset(d.vb[jb & 1], d.step_b) : d.vb[jb & 1];
        dma16_so(d.lds_b + stage * kTileBytes + 1024 * jb, vb, r, k0);
    } else {
        v4u r = d.rs;
        r.z = live ? r.z : 0u;
        gemm::dma4(d.lds_s + (slot & 3) * BM * 4, d.vs + (uint32_t)kbs * 4u, r);
        v4u rb = d.rsb;
        rb.z = live ? rb.z : 0u;
        gemm::dma4(d.lds_sb + (slot & 3) * 256, d.vsb + (uint32_t)kbs * 4u, rb);
    }
}

// s_a s_b of K block kb (ring slot kb & 3) for this tile: wave w handles
// rows 64 (w%4) .. +63 of N block w/4.  s_a and s_b of kb are in their LDS
// rings (zero past the end of the K range, where the slot is never read).
__device__ inline void block_factors(int kb, int w)
{
    const int nbi = w >> 2, row = 64 * (w & 3) + (threadIdx.x & 63);
    const float sbv = g_lds_sb[(kb & 3) * 64 + nbi];
    g_lds_f[(kb & 3) * 2 * BM + nbi * BM + row] = g_lds_sa[(kb & 3) * BM + row] * sbv;
}

// acc + (2^(ea-127) A)(2^(eb-127) B)^T over one 128-deep K block: byte `sel`
// of `ea4` is the E8M0 code of this lane's A row, eb the B code.
template <int FA, int FB>
__device__ inline v4f mfma_e8m0(int sel, const v8i& a, const v8i& b, const v4f& c, uint32_t ea4, uint32_t eb)
{
    switch (sel) {   // the byte select is an immediate of the instruction
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, (int)ea4, 0, (int)eb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 1, (int)ea4, 0, (int)eb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 2, (int)ea4, 0, (int)eb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 3, (int)ea4, 0, (int)eb);
    }
}

// Power-of-two scales: the E8M0 codes of s_a of K block kb into their ring
// slot, one row per lane (waves w and w + 4 write the same row; only the
// exponent field of each scale is used).
__device__ inline void block_codes(int kb, int w)
{
    const int row = 64 * (w & 3) + (threadIdx.x & 63);
    const uint32_t code = (__builtin_bit_cast(uint32_t, g_lds_sa[(kb & 3) * BM + row]) >> 23) & 0xFFu;
    g_lds_e[(kb & 3) * 256 + ((row >> 7) * 16 + (row & 15)) * 8 + ((row & 127) >> 4)] = (uint8_t)code;
}

// One K block per iteration.  Slot s (0..31) of a block issues the MFMA of
// A fragment i = s/4 and B fragment j = s%4, then promotes the result of
// slot s - 3.  Reads run one fragment group ahead.  At slot 1 the waves meet
// once every wave holds this block's B fragments: the B half of this
// block's stage then takes the B DMA of block kb + 2.  The barrier of slot
// 10 releases the rows of A fragment groups 0-3 for their half of A.  After
// the block's last A fragment read (slot 24) every wave waits for its DMA of
// the next block and meets the others at the barrier of slot 26, after which
// groups 4-7 take the other half and the next block's data is visible.
// MODE kModeE8M0: the scales are powers of two; each MFMA applies them
// itself (per-lane E8M0 code of its A row, the N block's code for B) and
// accumulates in place, with no promotion.  MODE kModeTensor: one scale per
// operand; the MFMAs accumulate in place and the epilogue (or the split-K
// reduction) multiplies by s_a s_b.
template <int FA, int FB, int MODE>
__global__ void __launch_bounds__(kBlockThreads, 1) k_gemm_block(KArgs p)
{
    constexpr bool E8M0 = MODE == kModeE8M0;
    constexpr bool TENSOR = MODE == kModeTensor;
    constexpr bool PROMOTE = MODE == kModeBlock;
    // the per-tensor output scale, read before any DMA is in flight
    const float out_scale = (TENSOR && !p.ws) ? p.sa[0] * p.sb[0] : 1.0f;
    int split, tm, tn;
    tile_of(p, split, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kt_per = (p.ktiles + p.splits - 1) / p.splits;
    const int kt0 = split * kt_per;
    const int ntk = min(p.ktiles, kt0 + kt_per) - kt0;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wm = (wave & 1) * 128;
    const int wn = (wave >> 1) * 64;
    const int fcol = (wn >> 7) * BM + wm + 4 * (lane >> 4);   // factor row base of this lane

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const BlockDma d = block_dma(p, m0, n0, wave, !TENSOR);
    // prologue: A/B of blocks 0 and 1, s_a of blocks 0, 1, 2
#pragma unroll
    for (int j = 0; j < 8; ++j) block_dma_one(d, j, 0, kt0, 0, true);
    block_dma_one(d, 8, 0, 0, kt0, true);
    block_dma_one(d, 8, 0, 0, kt0 + 1, ntk > 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) block_dma_one(d, j, 1, kt0 + 1, 0, ntk > 1);
    block_dma_one(d, 8, 0, 0, kt0 + 2, ntk > 2);
    // block 0's A/B and the scales of blocks 0 and 1 (older than the newest
    // 10 instructions: block 1's 8 and the 2 of block 2's scales); block 1
    // arrives while block 0 runs and is waited for at its slot 26
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    gemm::barrier_lds();
    if constexpr (E8M0) {
        block_codes(kt0, wave);
        block_codes(kt0 + 1, wave);
    } else if constexpr (PROMOTE) {
        block_factors(kt0, wave);
        block_factors(kt0 + 1, wave);
    }
    gemm::barrier_lds();

    v8i af[2], bf[4];
    v4f fc[2], part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = gemm::load_frag(g_lds_b, wn + 16 * j);
    af[0] = gemm::load_frag(g_lds_a, wm);
    fc[0] = *reinterpret_cast<const v4f*>(&g_lds_f[(kt0 & 3) * 2 * BM + fcol]);
    fc[1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) part[e] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // E8M0: this lane's 8 A row codes and the wave's B code, for the current
    // block (ec, bc) and read ahead for the next (ecn, bcn)
    const int ecol = (wm >> 7) * 16 + (lane & 15);
    const int nbi_w = wn >> 7;
    uint2 ec = uint2{0, 0}, ecn = uint2{0, 0};
    uint32_t bc = 0, bcn = 0;
    if constexpr (E8M0) {
        ec = *reinterpret_cast<const uint2*>(&g_lds_e[(kt0 & 3) * 256 + ecol * 8]);
        bc = (__builtin_bit_cast(uint32_t, g_lds_sb[(kt0 & 3) * 64 + nbi_w]) >> 23) & 0xFFu;
    }

    // No branches inside: past the last block the reads fetch unused data
    // and the DMA is a no-op fill.
    for (int t = 0; t < ntk; ++t) {
        const int kb = kt0 + t;
        const uint8_t* la = g_lds_a + (t & 1) * kTileBytes;
        const uint8_t* la_next = g_lds_a + ((t + 1) & 1) * kTileBytes;
        const uint8_t* lb_next = g_lds_b + ((t + 1) & 1) * kTileBytes;
        const float* lf = g_lds_f + (kb & 3) * 2 * BM + fcol;
        const float* lf_next = g_lds_f + ((kb + 1) & 3) * 2 * BM + fcol;
        const bool live2 = t + 2 < ntk, live3 = t + 3 < ntk;
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            const int i = s >> 2, j = s & 3;
            if (j == 0) af[(i + 1) & 1] = gemm::load_frag(i < 7 ? la : la_next, i < 7 ? wm + 16 * (i + 1) : wm);
            if constexpr (E8M0) {
                acc[i][j] = mfma_e8m0<FA, FB>(i & 3, af[i & 1], bf[j], acc[i][j], i < 4 ? ec.x : ec.y, bc);
                if (s == 31) {
                    ecn = *reinterpret_cast<const uint2*>(&g_lds_e[((kb + 1) & 3) * 256 + ecol * 8]);
                    bcn = (__builtin_bit_cast(uint32_t, g_lds_sb[((kb + 1) & 3) * 64 + nbi_w]) >> 23) & 0xFFu;
                }
            } else if constexpr (TENSOR) {
                acc[i][j] = gemm::mfma<FA, FB>(af[i & 1], bf[j], acc[i][j]);
            } else {
                part[s & 3] = gemm::mfma<FA, FB>(af[i & 1], bf[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
            }
            if constexpr (PROMOTE) {
                // promote slot s - kLag (the previous block's last slots at s < kLag)
                const int q = (s + 32 - kLag) & 31, iq = q >> 2, jq = q & 3;
                const v4f pr = part[(s + 4 - kLag) & 3];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[iq][jq][r] = __builtin_fmaf(pr[r], fc[iq & 1][r], acc[iq][jq][r]);
            }
            // factors of group i + 1: group i - 1's last promotion (slot 4 i - 1) ran at slot 4 i + 2
            if (PROMOTE && j == 3) fc[(i + 1) & 1] = *reinterpret_cast<const v4f*>(i < 7 ? lf + 16 * (i + 1) : lf_next);
            if (i == 7) bf[j] = gemm::load_frag(lb_next, wn + 16 * j);
            // Block kb + 2 into this block's stage, as its parts are released.
            // B early in the block: this block's B fragments are in registers
            // once every wave has passed the barrier of slot 1, so the stage's
            // B half is free.  A in two halves: the rows of fragment groups
            // 0-3 are free once every wave has read group 3 (slot 8), those of
            // groups 4-7 after the block's last A read (slot 24), so the halves
            // go out after the barriers of slots 10 and 26.  The requests
            // reach the memory system spread over the block (a split into four
            // parts, with a third barrier, measured no faster).
            if (s == 1 || s == 10) gemm::barrier_lds();
            if (s >= 2 && s <= 5) block_dma_one(d, 4 + (s - 2), t & 1, kb + 2, 0, live2);
            if (s == 10) block_dma_one(d, 0, t & 1, kb + 2, 0, live2);
            if (s == 11) block_dma_one(d, 1, t & 1, kb + 2, 0, live2);
            if (s == 26) {
                // all but the 6 instructions of block kb + 2 issued in this block
                // (loads complete in order): block kb + 1 and the scales of kb + 2
                asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
                gemm::barrier_lds();
                block_dma_one(d, 2, t & 1, kb + 2, 0, live2);
                block_dma_one(d, 3, t & 1, kb + 2, 0, live2);
            }
            if (s == 30) block_dma_one(d, 8, 0, 0, kb + 3, live3);   // s_a of block kb + 3
            if (s == 27) {
                if constexpr (E8M0)
                    block_codes(kb + 2, wave);
                else if constexpr (PROMOTE)
                    block_factors(kb + 2, wave);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (E8M0) {
            ec = ecn;
            bc = bcn;
        }
    }
    // promotions of the last block's last kLag slots
#pragma unroll
    for (int s = 0; s < (PROMOTE ? kLag : 0); ++s) {
        const int q = 32 - kLag + s, jq = q & 3;
        const v4f pr = part[(s + 4 - kLag) & 3];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[7][jq][r] = __builtin_fmaf(pr[r], fc[1][r], acc[7][jq][r]);
    }

    // epilogue: lane holds columns n0 + wn + 4 (lane%16) + j (j = 0..3) of rows
    // m0 + wm + 16 i + 4 (lane/16) + r
    const int col = n0 + wn + 4 * (lane & 15);
    const int row_l = m0 + wm + 4 * (lane >> 4);
    if (p.ws && p.fast_store) {
        // fp32 partials: 16-byte stores through a descriptor spanning the
        // tile's valid rows (rows past m dropped by its range check)
        const int64_t rows_c = min(p.m - m0, BM);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            p.ws + ((int64_t)split * p.m + m0) * p.n, (short)0, (int)(rows_c * p.n * 4), 0x00020000);
        const bool col_ok = col < p.n;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lrow = wm + 16 * i + 4 * (lane >> 4) + r;
                const uint32_t off = col_ok ? (uint32_t)((lrow * p.n + col) * 4) : gemm::kOutOfRange;
                const v4f v = v4f{acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rw, (int)off, 0, 0);
            }
        return;
    }
    if (p.ws) {
        float* ws = p.ws + (int64_t)split * p.m * p.n;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row_l + 16 * i + r;
                if (row >= p.m) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (col + j < p.n) ws[(int64_t)row * p.n + col + j] = acc[i][j][r];
            }
        return;
    }
    uint32_t nonfinite = 0;
    if (p.fast_store) {
        const int64_t rows_c = min(p.m - m0, BM);
        const __amdgpu_buffer_rsrc_t rc =
            __builtin_amdgcn_make_buffer_rsrc(p.c + (int64_t)m0 * p.ldc, (short)0,
                                              (int)std::min<int64_t>(rows_c * p.ldc * 2, 0x7FFFFFF0), 0x00020000);
        const bool col_ok = col < p.n;
        us2 mx = us2{0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lrow = wm + 16 * i + 4 * (lane >> 4) + r;
                const uint32_t lo = gemm::pack_bf16(acc[i][0][r] * out_scale, acc[i][1][r] * out_scale);
                const uint32_t hi = gemm::pack_bf16(acc[i][2][r] * out_scale, acc[i][3][r] * out_scale);
                // rows past m: zero accumulators (their operand rows read as zeros), stores dropped
                const uint32_t off = col_ok ? (uint32_t)((lrow * p.ldc + col) * 2) : gemm::kOutOfRange;
                typedef uint32_t v2u __attribute__((ext_vector_type(2)));
                __builtin_amdgcn_raw_buffer_store_b64(v2u{lo, hi}, rc, (int)off, 0, 2);   // nontemporal
                track_max(mx, lo);
                track_max(mx, hi);
            }
        if (saw_nonfinite(mx)) nonfinite = recount_tile(p, m0, n0);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = row_l + 16 * i + r;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (row < p.m && col + j < p.n) {
                        const uint16_t h = gemm::to_bf16(acc[i][j][r] * out_scale);
                        nonfinite += (h & 0x7F80u) == 0x7F80u;
                        p.c[(int64_t)row * p.ldc + col + j] = h;
                    }
            }
    }
    flush_counters(p.ctr, 0, 0, 0, nonfinite);
}

// Position in a workgroup's stream of K blocks: the persistent form walks the
// items (tile, K split) blockIdx.x, blockIdx.x + gridDim.x, ... and the K
// blocks of each.  All fields are uniform over the workgroup.
struct BlockPos {
    int id;         // item id; >= the item count once the stream has ended
    int t;          // K block within the item
    int kt0, ntk;   // the item's first K block and block count
    int m0, n0, split;
};

__device__ inline void pos_load(const KArgs& p, BlockPos& q, int id)
{
    const int total = p.tiles_m * p.tiles_n * p.splits;
    q.id = id;
    q.t = 0;
    if (id < total) {
        int split, tm, tn;
        item_of(p, id, split, tm, tn);
        const int kt_per = (p.ktiles + p.splits - 1) / p.splits;
        q.split = split;
        q.kt0 = split * kt_per;
        q.ntk = min(p.ktiles, q.kt0 + kt_per) - q.kt0;
        q.m0 = tm * BM;
        q.n0 = tn * BN;
    } else {
        q.split = 0;
        q.kt0 = 0;
        q.ntk = 1;
        q.m0 = 0;
        q.n0 = 0;
    }
}

// Next K block; true when the position moved to another item.
__device__ inline bool pos_next(const KArgs& p, BlockPos& q)
{
    if (++q.t < q.ntk) return false;
    pos_load(p, q, q.id + (int)gridDim.x);
    return true;
}

// The DMA descriptors of one item (uniform): A and B panels, and, for block
// scales, s_a's rows and s_b (zero length for per-tensor scales).
struct ItemDesc {
    v4u ra, rb, rs, rsb;
    int n0;
};

__device__ inline ItemDesc item_desc(const KArgs& p, const BlockPos& q, bool block_scales)
{
    ItemDesc e;
    const int64_t rows_a = min(p.m - q.m0, BM), rows_b = min(p.n - q.n0, BN);
    const int nkb = p.k / BK;
    const int nbs = (p.n + 127) / 128;
    e.ra = gemm::make_rsrc(p.a + (int64_t)q.m0 * p.lda, (uint32_t)(rows_a * p.lda));
    e.rb = gemm::make_rsrc(p.b + (int64_t)q.n0 * p.ldb, (uint32_t)(rows_b * p.ldb));
    e.rs = gemm::make_rsrc(p.sa + (int64_t)q.m0 * nkb, block_scales ? (uint32_t)(rows_a * nkb * 4) : 0u);
    e.rsb = gemm::make_rsrc(p.sb, block_scales ? (uint32_t)(nbs * nkb * 4) : 0u);
    e.n0 = q.n0;
    return e;
}

// A/B instruction j (0..7) of K block kb of an item into `stage`; lane
// offsets and LDS targets from the workgroup's BlockDma.
__device__ inline void item_dma_ab(const BlockDma& d, const ItemDesc& e, int j, int stage, int kb, bool live)
{
    const uint32_t k0 = (uint32_t)kb * BK;
    if (j < 4) {
        v4u r = e.ra;
        r.z = live ? r.z : 0u;
        const uint32_t va = j ? add_lane_offset(d.va, (uint32_t)j * d.step_a) : d.va;
        dma16_so(d.lds_a + stage * kTileBytes + 4096 * j, va, r, k0);
    } else {
        const int jb = j - 4;
        v4u r = e.rb;
        r.z = live ? r.z : 0u;
        const uint32_t vb = (jb >> 1) ? add_lane_offset(d.vb[jb & 1], d.step_b) : d.vb[jb & 1];
        dma16_so(d.lds_b + stage * kTileBytes + 1024 * jb, vb, r, k0);
    }
}

// s_a of K block kb and the item's two s_b values into ring slot `slot`.
__device__ inline void item_dma_scales(const KArgs& p, const BlockDma& d, const ItemDesc& e, int slot, int kb, bool live)
{
    const int l = threadIdx.x & 63;
    const int nkb = p.k / BK;
    v4u r = e.rs;
    r.z = live ? r.z : 0u;
    gemm::dma4(d.lds_s + (slot & 3) * BM * 4, d.vs + (uint32_t)kb * 4u, r);
    v4u rb = e.rsb;
    rb.z = live ? rb.z : 0u;
    const uint32_t vsb = l < 2 ? (uint32_t)(((e.n0 >> 7) + l) * nkb * 4 + kb * 4) : gemm::kOutOfRange;
    gemm::dma4(d.lds_sb + (slot & 3) * 256, vsb, rb);
}

// Persistent form of k_gemm_block: the same K-block schedule, but over the
// whole stream of the workgroup's items, so the DMA of the next tile's first
// blocks runs during the current tile's last blocks and its epilogue.  LDS
// stages and rings are indexed by the position u in the stream; one DMA
// cursor runs two positions ahead, fetching each position's scales (slot 2)
// before its B half (slots 2-5) and A in two halves (slots 10-11 and 26).
// Launched only
// when every output row segment can be stored whole (fast_store).
template <int FA, int FB, int MODE>
__global__ void __launch_bounds__(kBlockThreads, 1) k_gemm_block_p(KArgs p)
{
    constexpr bool E8M0 = MODE == kModeE8M0;
    constexpr bool TENSOR = MODE == kModeTensor;
    constexpr bool PROMOTE = MODE == kModeBlock;
    const float out_scale = (TENSOR && !p.ws) ? p.sa[0] * p.sb[0] : 1.0f;
    const int total = p.tiles_m * p.tiles_n * p.splits;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wm = (wave & 1) * 128;
    const int wn = (wave >> 1) * 64;
    const int fcol = (wn >> 7) * BM + wm + 4 * (lane >> 4);

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    BlockPos c;
    pos_load(p, c, blockIdx.x);
    BlockPos da = c;     // DMA position, two blocks ahead of c
    const BlockDma dl = block_dma(p, 0, 0, wave, false);   // lane offsets and LDS targets only
    ItemDesc de = item_desc(p, da, !TENSOR);
    // prologue: scales and A/B of positions 0 and 1
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        item_dma_scales(p, dl, de, u, da.kt0 + da.t, da.id < total);
#pragma unroll
        for (int j = 0; j < 8; ++j) item_dma_ab(dl, de, j, u, da.kt0 + da.t, da.id < total);
        if (pos_next(p, da)) de = item_desc(p, da, !TENSOR);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    gemm::barrier_lds();
    if constexpr (E8M0) {
        block_codes(0, wave);
        block_codes(1, wave);
    } else if constexpr (PROMOTE) {
        block_factors(0, wave);
        block_factors(1, wave);
    }
    gemm::barrier_lds();

    v8i af[2], bf[4];
    v4f fc[2], part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = gemm::load_frag(g_lds_b, wn + 16 * j);
    af[0] = gemm::load_frag(g_lds_a, wm);
    fc[0] = *reinterpret_cast<const v4f*>(&g_lds_f[fcol]);
    fc[1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int e = 0; e < 4; ++e) part[e] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    const int ecol = (wm >> 7) * 16 + (lane & 15);
    const int nbi_w = wn >> 7;
    uint2 ec = uint2{0, 0}, ecn = uint2{0, 0};
    uint32_t bc = 0, bcn = 0;
    if constexpr (E8M0) {
        ec = *reinterpret_cast<const uint2*>(&g_lds_e[ecol * 8]);
        bc = (__builtin_bit_cast(uint32_t, g_lds_sb[nbi_w]) >> 23) & 0xFFu;
    }

    us2 mx = us2{0, 0};   // over every tile's bf16 output
    for (int u = 0; c.id < total; ++u) {
        const uint8_t* la = g_lds_a + (u & 1) * kTileBytes;
        const uint8_t* la_next = g_lds_a + ((u + 1) & 1) * kTileBytes;
        const uint8_t* lb_next = g_lds_b + ((u + 1) & 1) * kTileBytes;
        const float* lf = g_lds_f + (u & 3) * 2 * BM + fcol;
        const float* lf_next = g_lds_f + ((u + 1) & 3) * 2 * BM + fcol;
        const bool live2 = da.id < total;
        const int kb2 = da.kt0 + da.t;
#pragma unroll
        for (int s = 0; s < 32; ++s) {
            const int i = s >> 2, j = s & 3;
            if (j == 0) af[(i + 1) & 1] = gemm::load_frag(i < 7 ? la : la_next, i < 7 ? wm + 16 * (i + 1) : wm);
            if constexpr (E8M0) {
                acc[i][j] = mfma_e8m0<FA, FB>(i & 3, af[i & 1], bf[j], acc[i][j], i < 4 ? ec.x : ec.y, bc);
                if (s == 31) {
                    ecn = *reinterpret_cast<const uint2*>(&g_lds_e[((u + 1) & 3) * 256 + ecol * 8]);
                    bcn = (__builtin_bit_cast(uint32_t, g_lds_sb[((u + 1) & 3) * 64 + nbi_w]) >> 23) & 0xFFu;
                }
            } else if constexpr (TENSOR) {
                acc[i][j] = gemm::mfma<FA, FB>(af[i & 1], bf[j], acc[i][j]);
            } else {
                part[s & 3] = gemm::mfma<FA, FB>(af[i & 1], bf[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
            }
            if constexpr (PROMOTE) {
                const int q = (s + 32 - kLag) & 31, iq = q >> 2, jq = q & 3;
                const v4f pr = part[(s + 4 - kLag) & 3];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[iq][jq][r] = __builtin_fmaf(pr[r], fc[iq & 1][r], acc[iq][jq][r]);
            }
            if (PROMOTE && j == 3) fc[(i + 1) & 1] = *reinterpret_cast<const v4f*>(i < 7 ? lf + 16 * (i + 1) : lf_next);
            if (i == 7) bf[j] = gemm::load_frag(lb_next, wn + 16 * j);
            // the DMA schedule of k_gemm_block (B at slots 2-5, A's halves
            // after the barriers of slots 10 and 26)
            if (s == 1 || s == 10) gemm::barrier_lds();
            if (s == 2) item_dma_scales(p, dl, de, u + 2, kb2, live2);
            if (s >= 2 && s <= 5) item_dma_ab(dl, de, 4 + (s - 2), u & 1, kb2, live2);
            if (s == 10) item_dma_ab(dl, de, 0, u & 1, kb2, live2);
            if (s == 11) item_dma_ab(dl, de, 1, u & 1, kb2, live2);
            if (s == 26) {
                // all but the 6 A/B instructions issued in this block (loads
                // complete in order; an epilogue's stores before them are
                // waited for too)
                asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
                gemm::barrier_lds();
                item_dma_ab(dl, de, 2, u & 1, kb2, live2);
                item_dma_ab(dl, de, 3, u & 1, kb2, live2);
            }
            if (s == 27) {
                if constexpr (E8M0)
                    block_codes(u + 2, wave);
                else if constexpr (PROMOTE)
                    block_factors(u + 2, wave);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (E8M0) {
            ec = ecn;
            bc = bcn;
        }
        if (pos_next(p, da)) de = item_desc(p, da, !TENSOR);
        if (c.t + 1 < c.ntk) {
            ++c.t;
            continue;
        }
        // the item's last block: its last kLag promotions, then the epilogue
#pragma unroll
        for (int s = 0; s < (PROMOTE ? kLag : 0); ++s) {
            const int q = 32 - kLag + s, jq = q & 3;
            const v4f pr = part[(s + 4 - kLag) & 3];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[7][jq][r] = __builtin_fmaf(pr[r], fc[1][r], acc[7][jq][r]);
        }
        // lane holds columns n0 + wn + 4 (lane%16) + j of rows m0 + wm + 16 i + 4 (lane/16) + r
        const int m0 = c.m0, n0 = c.n0;
        const int col = n0 + wn + 4 * (lane & 15);
        const bool col_ok = col < p.n;
        const int64_t rows_c = min(p.m - m0, BM);
        if (p.ws) {
            // fp32 partials: range-checked 16-byte stores
            const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                p.ws + ((int64_t)c.split * p.m + m0) * p.n, (short)0, (int)(rows_c * p.n * 4), 0x00020000);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lrow = wm + 16 * i + 4 * (lane >> 4) + r;
                    const uint32_t off = col_ok ? (uint32_t)((lrow * p.n + col) * 4) : gemm::kOutOfRange;
                    const v4f v = v4f{acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rw, (int)off, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
        } else {
            const __amdgpu_buffer_rsrc_t rc =
                __builtin_amdgcn_make_buffer_rsrc(p.c + (int64_t)m0 * p.ldc, (short)0,
                                                  (int)std::min<int64_t>(rows_c * p.ldc * 2, 0x7FFFFFF0), 0x00020000);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lrow = wm + 16 * i + 4 * (lane >> 4) + r;
                    const uint32_t lo = gemm::pack_bf16(acc[i][0][r] * out_scale, acc[i][1][r] * out_scale);
                    const uint32_t hi = gemm::pack_bf16(acc[i][2][r] * out_scale, acc[i][3][r] * out_scale);
                    track_max(mx, lo);
                    track_max(mx, hi);
                    const uint32_t off = col_ok ? (uint32_t)((lrow * p.ldc + col) * 2) : gemm::kOutOfRange;
                    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
                    __builtin_amdgcn_raw_buffer_store_b64(v2u{lo, hi}, rc, (int)off, 0, 2);   // nontemporal
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        // the next block's first kLag slots promote zeros (finite factors)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[e] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        fc[1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        pos_next(p, c);
    }
    uint32_t nonfinite = 0;
    if (saw_nonfinite(mx))
        for (int id = blockIdx.x; id < total; id += gridDim.x) {
            int split, tm, tn;
            item_of(p, id, split, tm, tn);
            nonfinite += recount_tile(p, tm * BM, tn * BN);
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
        const uint16_t h = gemm::to_bf16(s * scale);
        nonfinite += (h & 0x7F80u) == 0x7F80u;
        const int64_t row = i / n, col = i - row * n;
        c[row * ldc + col] = h;
    }
    flush_counters(ctr, 0, 0, 0, nonfinite);
}

// The same reduction, four consecutive outputs of a row per thread and step
// (16-byte partial loads, one 8-byte bf16 store): n % 4 == 0, the partials
// 16-byte and the output 8-byte aligned, ldc % 4 == 0, m * n < 2^31.  The
// sum of each output runs over the splits in the same order as above.
__global__ void __launch_bounds__(256) k_splitk_reduce4(const float* ws, int splits, int m, int n,
                                                        float scale_mode_tensor, const float* sa, const float* sb,
                                                        uint16_t* c, int64_t ldc, fp8_counters* ctr)
{
    const float scale = scale_mode_tensor != 0.0f ? sa[0] * sb[0] : 1.0f;
    const uint32_t total = (uint32_t)m * (uint32_t)n;
    const uint32_t n4 = (uint32_t)n >> 2;
    uint32_t nonfinite = 0;
    for (uint32_t v = blockIdx.x * blockDim.x + threadIdx.x; v < total / 4; v += gridDim.x * blockDim.x) {
        float4 acc = reinterpret_cast<const float4*>(ws)[v];
        for (int sp = 1; sp < splits; ++sp) {
            const float4 w = reinterpret_cast<const float4*>(ws + (int64_t)sp * total)[v];
            acc.x += w.x;
            acc.y += w.y;
            acc.z += w.z;
            acc.w += w.w;
        }
        const uint32_t lo = gemm::pack_bf16(acc.x * scale, acc.y * scale);
        const uint32_t hi = gemm::pack_bf16(acc.z * scale, acc.w * scale);
        nonfinite += ((lo & 0x7F80u) == 0x7F80u) + ((lo & 0x7F800000u) == 0x7F800000u) +
                     ((hi & 0x7F80u) == 0x7F80u) + ((hi & 0x7F800000u) == 0x7F800000u);
        const uint32_t row = v / n4, col = 4 * (v - row * n4);
        *reinterpret_cast<uint2*>(c + (int64_t)row * ldc + col) = make_uint2(lo, hi);
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

hipError_t launch_reduce(const KArgs& p, const GemmArgs& g, float scale_mode_tensor, hipStream_t stream)
{
    const int64_t total = g.m * g.n;
    const bool vec = g.n % 4 == 0 && g.ldc % 4 == 0 && total < ((int64_t)1 << 31) &&
                     (reinterpret_cast<uintptr_t>(p.ws) & 15u) == 0 && (reinterpret_cast<uintptr_t>(g.c) & 7u) == 0;
    if (vec) {
        const int rgrid = (int)std::min<int64_t>((total / 4 + 255) / 256, 8192);
        hipLaunchKernelGGL(k_splitk_reduce4, dim3(rgrid), dim3(256), 0, stream, p.ws, p.splits, p.m, p.n,
                           scale_mode_tensor, g.sa, g.sb, p.c, g.ldc, g.ctr);
    } else {
        const int rgrid = (int)std::min<int64_t>((total + 255) / 256, 8192);
        hipLaunchKernelGGL(k_splitk_reduce, dim3(rgrid), dim3(256), 0, stream, p.ws, p.splits, p.m, p.n,
                           scale_mode_tensor, g.sa, g.sb, p.c, g.ldc, g.ctr);
    }
    return hipGetLastError();
}

template <int FA, int FB>
hipError_t gemm_fmt(const KArgs& p, int grid, int mode, hipStream_t stream)
{
    // per-tensor scales with whole row segments and more tiles than CUs: the
    // persistent form (its epilogue stays within the register budget only in
    // this mode; with one tile per workgroup it only adds cursor work: 2%
    // slower on 3072x768x65536 split 7 ways)
    if (p.fast_store && mode == kModeTensor && grid > gemm_num_cus()) {
        const int g = std::min(grid, gemm_num_cus());
        hipLaunchKernelGGL((k_gemm_block_p<FA, FB, kModeTensor>), dim3(g), dim3(kBlockThreads), 0, stream, p);
        return hipGetLastError();
    }
    if (mode == kModeE8M0)
        hipLaunchKernelGGL((k_gemm_block<FA, FB, kModeE8M0>), dim3(grid), dim3(kBlockThreads), 0, stream, p);
    else if (mode == kModeTensor)
        hipLaunchKernelGGL((k_gemm_block<FA, FB, kModeTensor>), dim3(grid), dim3(kBlockThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((k_gemm_block<FA, FB, kModeBlock>), dim3(grid), dim3(kBlockThreads), 0, stream, p);
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
    // Per-tensor scales: the 8-wave kernel of the block-scaled form (with
    // per-tensor scales, persistent over tiles) when K is a multiple of 128 and
    // either split or at least 16 blocks deep; else the 4-wave persistent
    // kernel.  Measured in the step: 3072x768x65536 (split) 14% and
    // 65536x768x3072 3% faster on the 8-wave kernel, 65536x3072x768 (6 blocks
    // per tile) 2% slower.
    // Per-tensor GEMMs whose K is one model width (768) and that do not split
    // K: the A-stationary kernel (the whole [192, 768] A panel in LDS, only B
    // streams).
    if (!g.block_scaled && !p.ws && astat_supported(g.m, g.n, g.k, g.lda, g.ldb, g.ldc, g.c)) {
        AstatArgs a;
        a.a = g.a;
        a.lda = g.lda;
        a.bf16_a = false;
        a.fa = g.fa;
        a.b = g.b;
        a.ldb = g.ldb;
        a.fb = g.fb;
        a.sa = g.sa;
        a.sa_out = nullptr;
        a.sb = g.sb;
        a.partials = nullptr;
        a.np = 0;
        a.xq = nullptr;
        a.ldxq = 0;
        a.xqt = nullptr;
        a.ldxqt = 0;
        a.m = g.m;
        a.n = g.n;
        a.c = g.c;
        a.ldc = g.ldc;
        a.ctr = g.ctr;
        return launch_gemm_astat(a, gemm_num_cus(), stream);
    }
    const bool tensor_via_block = !g.block_scaled && g.k % BK == 0 && (p.ws || g.k >= 16 * BK);
    if (!g.block_scaled && !tensor_via_block) {
        e = launch_gemm_persistent(g, gemm_num_cus(), stream);
        if (e != hipSuccess || !p.ws) return e;
        return launch_reduce(p, g, 1.0f, stream);
    }
    const int grid = p.tiles_m * p.tiles_n * p.splits;
    // M tiles per group of the tile order, measured per kernel form in the
    // step: 4 for the single-tile form (block-scaled 16384x2048x7168 1.3%
    // faster than 8), 8 for the persistent per-tensor form (65536x768x3072 3%
    // faster than 4); 2 and 16 were no better
    p.group_m = (tensor_via_block && grid > gemm_num_cus()) ? 8 : 4;
    if (p.ws)
        p.fast_store = (g.n % 4 == 0) && ((reinterpret_cast<uintptr_t>(g.ws) & 15u) == 0) &&
                       (int64_t)BM * g.n * 4 < 0x7FFFFFF0;   // a tile's rows of partials fit one descriptor
    else
        p.fast_store = (g.n % 4 == 0) && (g.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(g.c) & 7u) == 0);
    const int mode = !g.block_scaled ? kModeTensor : g.pow2_scales ? kModeE8M0 : kModeBlock;
    if (g.fa == FP8_E4M3)
        e = g.fb == FP8_E4M3 ? gemm_fmt<0, 0>(p, grid, mode, stream) : gemm_fmt<0, 1>(p, grid, mode, stream);
    else
        e = g.fb == FP8_E4M3 ? gemm_fmt<1, 0>(p, grid, mode, stream) : gemm_fmt<1, 1>(p, grid, mode, stream);
    if (e != hipSuccess || !p.ws) return e;
    return launch_reduce(p, g, g.block_scaled ? 0.0f : 1.0f, stream);
}

}  // namespace fp8mi
