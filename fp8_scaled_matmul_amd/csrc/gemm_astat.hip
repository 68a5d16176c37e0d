// A-stationary per-tensor FP8 GEMM for projections whose K is one model
// width (768): y = bf16(s_a s_b sum_k A[m,k] B[n,k]) in the TN form of
// _scaled_mm(x, w_fp8, scale_a, scale_b) ("#84 FP8 Precision", code excerpt
// and "Explanation").  Optionally the A operand arrives as bf16 and is
// quantized on its way into the matrix cores, with the per-tensor amax scale
// and the exact cast of fp8_quantize ("FP8 stability guardrails", section
// "Why FP8 is tempting and why it is fragile": the activation's memory
// traffic is what FP8 halves).
//
// Design (gfx950: 160 KB of LDS per CU, 256 CUs, L2-to-CU delivery about
// 21 bytes per clock per CU):
//   - a workgroup of 4 waves keeps a whole 208 x 768 panel of A codes
//     (156 KB; 192 rows when it casts bf16 A) in LDS and walks the output
//     columns in units of 256; only B
//     streams from L2, straight into each wave's registers (each wave owns
//     64 columns, so no B byte is fetched twice per CU).  Per 128-deep K step
//     a CU moves 32 KB of B for 13.6 MFLOP: 416 flops per byte (384 with
//     192 rows), against 256 for a 256 x 256 tile that stages both operands;
//   - every unit is 6 K steps of 52 v_mfma_f32_16x16x128_f8f6f4 per wave
//     (13 A fragments from LDS x 4 B fragments); B is fetched two K steps
//     ahead, across unit boundaries;
//   - one accumulator set (208 AGPRs); the epilogue (scale, bf16, 8-byte
//     stores of four adjacent columns) trails the last K step's MFMAs by one
//     fragment, so the matrix pipe does not wait for it;
//   - workgroups are persistent over contiguous unit ranges (units in panel
//     order, ranges of one XCD adjacent), so a panel is loaded by at most two
//     workgroups; with bf16 A, the workgroup whose range holds the panel's
//     first unit also writes its codes (row-major and transposed) and counts
//     its quantization events.
#include "device_common.h"
#include "fp8mi_internal.h"
#include "gemm_common.h"

#include <algorithm>

namespace fp8mi {

namespace {

using gemm::v4f;
using gemm::v4u;
using gemm::v8i;

// A unit is 64 BF output columns: each wave takes 16 BF of them as BF B
// fragments per K step (BF = 4, 256 columns; short A: BF = 2, 128 columns).
template <int BF>
constexpr int unit_cols() { return 64 * BF; }
constexpr int kAsKB = kAstatK / 128;         // 128-deep MFMA steps per unit
constexpr int kAsChunks = kAstatK / 16;      // 16-byte chunks per panel row
constexpr int kAsThreads = 256;
// B fragments are requested kBAhead K steps before use, into a ring of
// kBRing steps (a unit's K steps are a multiple of it, so ring slots are
// fixed at compile time): 64 KB of B in flight per CU.
constexpr int kBRing = 3, kBAhead = 2;
static_assert(kAstatK / 128 % kBRing == 0 && kBAhead < kBRing, "B ring");

// The A panel held in LDS: 208 rows (13 fragments, 156 KB) of FP8 codes, or
// 192 rows (12 fragments) when it is cast from bf16 A.  Measured on the
// 65536 x 3072 forward: 208 rows run 6-8% faster than 192 (8% fewer B bytes
// per flop, and 3792 units spread over 256 CUs as 14-15 each instead of 4104
// as 16-17); the cast form ran 2% slower with them.  Short A (every unit of
// 32-row panels fits in one round of workgroups) takes 32-row panels: one
// unit per workgroup, whose time is then its B stream rather than the load
// of a 156 KB panel; its units are 128 columns wide, so twice as many CUs
// share the B stream.  A fragments are read from LDS `ahead` steps before
// use, into a ring of `ring` slots (a unit's 6 x frags steps are a multiple
// of it).
constexpr int kAsRowsCodes = 208, kAsRowsCast = 192, kAsRowsShort = 32;
template <int ROWS>
struct Panel {
    static constexpr int rows = ROWS;
    static constexpr int frags = rows / 16;
    static constexpr int bytes = rows * kAstatK;
    static constexpr int ahead = 3, ring = kAsKB * frags % 4 == 0 ? 4 : 6;
    static_assert(rows % 16 == 0 && kAsKB * frags % ring == 0 && ahead < ring, "A ring");
    // the next unit's first MFMAs (fragment 0) run before the previous
    // unit's last fragment is stored
    static_assert(frags >= 2, "panel of at least two fragments");
};
constexpr int kAsMinRows = kAsRowsShort, kAsMaxBytes = Panel<kAsRowsCodes>::bytes;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding, with no LDS or export wait.
constexpr unsigned waitcnt_vm(int n) { return (((unsigned)n >> 4) & 3u) << 14 | ((unsigned)n & 15u) | 7u << 4 | 15u << 8; }
static_assert(waitcnt_vm(63) == 0xCF7Fu && waitcnt_vm(0) == 0x0F70u, "s_waitcnt encoding");

struct AsArgs {
    const void* a;          // FP8 codes [m, k] (lda bytes) or bf16 [m, k] (lda elements)
    int64_t lda;
    const uint8_t* b;       // [n, k] FP8 codes
    int64_t ldb;
    const float* sa;        // given s_a (FP8 A)
    float* sa_out;          // bf16 A: the amax scale, written by workgroup 0
    const float* sb;
    const uint32_t* partials;   // bf16 A: amax partial keys of A
    int np;
    uint8_t* xq;            // bf16 A, optional: the codes [m, k]
    int64_t ldxq;
    uint8_t* xqt;           // bf16 A, optional: the transposed codes [k, m]
    int64_t ldxqt;
    int xqt_words;          // xqt and ldxqt allow 4-byte stores
    int m, n;
    uint16_t* c;
    int64_t ldc;
    int ntn, units;         // units = panels * ntn
    fp8_counters* ctr;
};

__shared__ __attribute__((aligned(1024))) uint8_t s_panel[kAsMaxBytes];
__shared__ uint32_t s_red[kAsThreads / 64];

// 16-byte chunk lc of panel row r sits at chunk lc ^ (r % 16) of the row
// (the XOR stays inside the row's 16-chunk group).  Rows are 768 bytes, a
// multiple of 256, so the 16 rows of a fragment read (lanes 0..15, one chunk
// each) land in 16 distinct 16-byte slots of the 256-byte bank window.
__device__ inline uint32_t panel_off(int r, int lc) { return (uint32_t)(r * kAstatK + ((lc ^ (r & 15)) << 4)); }

// A fragment i of K step kb: lane l reads row 16 i + l % 16, K bytes
// 128 kb + 32 (l / 16) .. +32 (the B fragment uses the same K assignment).
// With p = l % 16 and q = l / 16, chunk 8 kb + 2 q + h of row 16 i + p sits
// at byte (16 i + p) 768 + 256 (kb / 2) + 16 (((8 (kb % 2)) | (2 q + h)) ^ p):
// four per-lane bases (kb % 2, h) plus offsets that are immediates.
struct AFragBase {
    uint32_t base[2][2];
};

__device__ inline AFragBase a_frag_base()
{
    const int l = threadIdx.x & 63, p = l & 15, q = l >> 4;
    AFragBase a;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            a.base[e][h] = (uint32_t)(p * kAstatK + 16 * (((8 * e) | (2 * q + h)) ^ p));
    return a;
}

__device__ inline v8i a_frag(const AFragBase& ab, int i, int kb)
{
    const uint32_t imm = (uint32_t)(16 * i * kAstatK + 256 * (kb >> 1));
    const uint4 lo = *reinterpret_cast<const uint4*>(s_panel + ab.base[kb & 1][0] + imm);
    const uint4 hi = *reinterpret_cast<const uint4*>(s_panel + ab.base[kb & 1][1] + imm);
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
}

// B fragment f (0 .. BF - 1) of K step kb for this wave: lane l (slot
// p = l % 16) reads B row 16 BF w + BF p + f of the unit, so lane p ends up
// holding output columns BF p .. BF p + BF - 1 of the wave's 16 BF.  Rows
// past n read as zeros (range check).  boff[f] is the lane's byte offset at
// K step 0; the K step goes in soffset (every row in range stays in range
// with it: k <= ldb).
template <int BF>
__device__ inline v8i b_frag(__amdgpu_buffer_rsrc_t rs, const uint32_t (&boff)[BF], int f, int kb)
{
    const v4u lo = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)boff[f], 128 * kb, 0);
    const v4u hi = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)boff[f], 128 * kb + 16, 0);
    v8i v;
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    return v;
}

template <int BF>
__device__ inline __amdgpu_buffer_rsrc_t b_rsrc(const AsArgs& p, int u, int u1)
{
    const int nt = u < u1 ? u % p.ntn : 0;
    const int n0 = nt * unit_cols<BF>();
    const int rows = u < u1 ? min(unit_cols<BF>(), p.n - n0) : 0;
    return gemm::make_store_rsrc(const_cast<uint8_t*>(p.b) + (int64_t)n0 * p.ldb, (uint32_t)(rows * p.ldb));
}

__device__ inline uint32_t block_reduce_key(uint32_t k)
{
    k = wave_key_merge(k);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = k;
    __syncthreads();
    k = s_red[0];
    for (int w = 1; w < kAsThreads / 64; ++w) k = key_merge(k, s_red[w]);
    __syncthreads();
    return k;
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Stores of rows 16 i .. 16 i + 15 (fragment i) of a finished unit: lane l
// holds columns n0 + 16 BF w + BF (l % 16) + 0 .. BF - 1 of rows
// 16 i + 4 (l / 16) + r (one 2 BF-byte store per row).  voff is the lane's
// byte offset (its columns
// and row group, or out of range), the row 16 i + r goes in soffset; a row
// at or past `rows` (the rows of the panel inside the matrix) is dropped
// through voff, so no store depends on whether the range check counts
// soffset.  mx keeps the running maximum of the stored |bf16| patterns
// (>= 0x7F80: an Inf or NaN was written; counted exactly at the end, see
// recount()).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// The running maximum as it stands here, in a register: without this the
// compiler keeps every stored word live to the end of the unit and takes
// their maximum there, in one stretch of VALU work with the matrix pipe
// idle.
__device__ inline void settle(us2& m)
{
    uint32_t w = __builtin_bit_cast(uint32_t, m);
    asm volatile("" : "+v"(w));
    m = __builtin_bit_cast(us2, w);
}
#pragma clang diagnostic pop

// The row offset goes in the lane offset, which the descriptor's range check
// covers (the uniform offset is not range checked): rc spans the unit's
// valid rows, so the stores of rows past the matrix are dropped, and so are
// those of a lane whose columns are past it (voff out of range).
template <int NF, int BF>
__device__ inline void store_row(const v4f (&acc)[NF][BF], int i, int r, __amdgpu_buffer_rsrc_t rc, uint32_t voff,
                                 uint32_t row_bytes, float scale, us2& mx)
{
    static_assert(BF == 2 || BF == 4, "unit width");
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    const uint32_t vo = voff + (uint32_t)(16 * i + r) * row_bytes;
    const uint32_t lo = gemm::pack_bf16(acc[i][0][r] * scale, acc[i][1][r] * scale);
    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, lo & 0x7FFF7FFFu));
    if constexpr (BF == 2) {
        __builtin_amdgcn_raw_buffer_store_b32(lo, rc, (int)vo, 0, 2);   // nontemporal
    } else {
        const uint32_t hi = gemm::pack_bf16(acc[i][2][r] * scale, acc[i][3][r] * scale);
        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, hi & 0x7FFF7FFFu));
        __builtin_amdgcn_raw_buffer_store_b64(v2u{lo, hi}, rc, (int)vo, 0, 2);   // nontemporal
    }
    settle(mx);
}

template <int NF, int BF>
__device__ inline void store_frag(const v4f (&acc)[NF][BF], int i, __amdgpu_buffer_rsrc_t rc, uint32_t voff,
                                  uint32_t row_bytes, float scale, us2& mx)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) store_row(acc, i, r, rc, voff, row_bytes, scale, mx);
}

// The panel of rows m0 .. m0 + Panel::rows - 1 into LDS.  FP8 A: the codes are copied.
// bf16 A: each 16-element chunk is cast with the scale (the corrected
// quotient when `fast`, IEEE division otherwise, exactly as fp8_quantize
// does), and, when `own`, its codes go to xq and its events are counted.
template <int FA, int ASRC, int ROWS>
__device__ __attribute__((always_inline)) inline void load_panel(const AsArgs& p, int m0, bool own, float s, float rcp, bool fast, uint32_t& sat,
                                  uint32_t& und, uint32_t& nan)
{
    using P = Panel<ROWS>;
    const int rows = min(P::rows, p.m - m0);
    const int t = threadIdx.x;
    constexpr int per = P::rows * kAsChunks / kAsThreads;   // chunks per thread
    constexpr int batch = 4;
    if constexpr (ASRC == 0) {
        // LDS DMA: instruction j of wave w fills panel bytes
        // [1024 (per_wave w + j), +1024); lane l's 16 bytes land at offset 16 l,
        // which is chunk pc = (P % 768) / 16 of row r = P / 768 (P the byte
        // position), so the lane fetches logical chunk pc ^ (r % 16).  All
        // requests of a wave are in flight at once; rows past m read as
        // zeros (range-checked descriptor).
        const v4u ra = gemm::make_rsrc(static_cast<const uint8_t*>(p.a) + (int64_t)m0 * p.lda, (uint32_t)(rows * p.lda));
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), l = threadIdx.x & 63;
        const uint32_t lds0 = gemm::lds_addr(s_panel);
        constexpr int per_wave = P::bytes / 1024 / (kAsThreads / 64);
        static_assert(P::bytes % (1024 * (kAsThreads / 64)) == 0, "panel DMA");
#pragma unroll 4
        for (int j = 0; j < per_wave; ++j) {
            const int slot = per_wave * w + j;
            const int P = 1024 * slot + 16 * l;
            const int r = P / kAstatK, pc = (P - r * kAstatK) >> 4;
            const int lc = pc ^ (r & 15);
            gemm::dma16(__builtin_amdgcn_readfirstlane(lds0 + 1024u * (uint32_t)slot), (uint32_t)(r * p.lda + 16 * lc),
                        ra);
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // a wait the compiler sees: the B ring is complete too
    } else {
        const __amdgpu_buffer_rsrc_t rx = gemm::make_store_rsrc(
            const_cast<uint16_t*>(static_cast<const uint16_t*>(p.a)) + (int64_t)m0 * p.lda,
            (uint32_t)(rows * p.lda * 2));
        // rows past m read as zeros: their codes are zeros and count nothing
        uint8_t* const xq = own ? p.xq : nullptr;
        const int64_t ldxq = p.ldxq;
        const uint32_t row_x = (uint32_t)(p.lda * 2);
        if (fast) {
            // the corrected quotient (bf16 input, finite tensor, s >= 2^-64)
            static_assert(per % batch == 0, "cast batches");
            uint32_t u_loc = 0;
#pragma unroll 1
            for (int j0 = 0; j0 < per; j0 += batch) {
                v4u v[batch][2];
#pragma unroll
                for (int j = 0; j < batch; ++j) {
                    const int ch = t + kAsThreads * (j0 + j);
                    const int r = ch / kAsChunks, lc = ch - r * kAsChunks;
                    const uint32_t off = (uint32_t)r * row_x + 32u * lc;
                    v[j][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
                    v[j][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16), 0, 0);
                }
#pragma unroll
                for (int j = 0; j < batch; ++j) {
                    const uint32_t w0[4] = {v[j][0].x, v[j][0].y, v[j][0].z, v[j][0].w};
                    const uint32_t w1[4] = {v[j][1].x, v[j][1].y, v[j][1].z, v[j][1].w};
                    const uint2 c0 = cast8_bf16_fast<FA>(w0, s, rcp, u_loc);
                    const uint2 c1 = cast8_bf16_fast<FA>(w1, s, rcp, u_loc);
                    const int ch = t + kAsThreads * (j0 + j);
                    const int r = ch / kAsChunks, lc = ch - r * kAsChunks;
                    const v4u code = v4u{c0.x, c0.y, c1.x, c1.y};
                    *reinterpret_cast<v4u*>(s_panel + panel_off(r, lc)) = code;
                    if (xq && r < rows) *reinterpret_cast<v4u*>(xq + (int64_t)(m0 + r) * ldxq + 16 * lc) = code;
                }
            }
            if (own) und += u_loc;
        } else {
            // IEEE division and every counter (non-finite elements, tiny scales)
            uint32_t s_loc = 0, u_loc = 0, n_loc = 0;
#pragma unroll 1
            for (int j = 0; j < per; ++j) {
                const int ch = t + kAsThreads * j;
                const int r = ch / kAsChunks, lc = ch - r * kAsChunks;
                const uint32_t off = (uint32_t)r * row_x + 32u * lc;
                const v4u v0 = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
                const v4u v1 = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16), 0, 0);
                const uint32_t ws[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                uint32_t code[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    float x[4], q[4];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        x[2 * e] = bf16_lo(ws[2 * h + e]);
                        x[2 * e + 1] = bf16_hi(ws[2 * h + e]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) q[e] = x[e] / s;
                    code[h] = encode4_general<FA>(q, x, s, s_loc, u_loc, n_loc);
                }
                const v4u cv = v4u{code[0], code[1], code[2], code[3]};
                *reinterpret_cast<v4u*>(s_panel + panel_off(r, lc)) = cv;
                if (xq && r < rows) *reinterpret_cast<v4u*>(xq + (int64_t)(m0 + r) * ldxq + 16 * lc) = cv;
            }
            if (own) {
                sat += s_loc;
                und += u_loc;
                nan += n_loc;
            }
        }
    }
}

// The transposed codes of the panel (rows m0 .. m0 + rows - 1, all K) from
// LDS: thread blocks of 4 rows x 4 K bytes, transposed in registers; lanes
// with consecutive row quads write consecutive 4-byte words of a q_t row.
__device__ __attribute__((always_inline)) inline void store_panel_t(const AsArgs& p, int m0)
{
    using P = Panel<kAsRowsCast>;
    const int rows = min(P::rows, p.m - m0);
    constexpr int rq_n = P::rows / 4, kq_n = kAstatK / 4;
#pragma unroll 1
    for (int b = threadIdx.x; b < rq_n * kq_n; b += kAsThreads) {
        const int rq = b % rq_n, kq = b / rq_n;
        const int r0 = 4 * rq;
        if (r0 >= rows) continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = r0 + e;
            w[e] = *reinterpret_cast<const uint32_t*>(s_panel + panel_off(r, kq >> 2) + 4 * (kq & 3));
        }
        // 4x4 byte transpose: out[j] = byte j of w[0..3]
        const uint32_t x0 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);   // w0b0 w1b0 w0b1 w1b1
        const uint32_t x1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);   // w0b2 w1b2 w0b3 w1b3
        const uint32_t y0 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
        const uint32_t y1 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
        const uint32_t o[4] = {__builtin_amdgcn_perm(y0, x0, 0x05040100u), __builtin_amdgcn_perm(y0, x0, 0x07060302u),
                               __builtin_amdgcn_perm(y1, x1, 0x05040100u), __builtin_amdgcn_perm(y1, x1, 0x07060302u)};
        uint8_t* dst = p.xqt + (int64_t)(4 * kq) * p.ldxqt + m0 + r0;
        if (p.xqt_words && r0 + 4 <= rows) {
#pragma unroll
            for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t*>(dst + (int64_t)j * p.ldxqt) = o[j];
        } else {
            for (int j = 0; j < 4; ++j)
                for (int e = 0; e < 4 && r0 + e < rows; ++e) dst[(int64_t)j * p.ldxqt + e] = (uint8_t)(o[j] >> (8 * e));
        }
    }
}

// Exact count of the non-finite outputs this lane stored for units
// u0 .. u1 - 1 (only run when one was seen: reads the outputs back).
template <int ROWS, int BF>
__device__ __attribute__((always_inline)) inline uint32_t recount(const AsArgs& p, int u0, int u1)
{
    using P = Panel<ROWS>;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t n = 0;
    for (int u = u0; u < u1; ++u) {
        const int m0 = (u / p.ntn) * P::rows, n0 = (u % p.ntn) * unit_cols<BF>();
        const int col = n0 + 16 * BF * w + BF * (l & 15);
        if (col >= p.n) continue;
        for (int i = 0; i < P::frags; ++i)
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + 16 * i + 4 * (l >> 4) + r;
                if (row >= p.m) continue;
                for (int j = 0; j < BF; ++j)
                    n += (p.c[(int64_t)row * p.ldc + col + j] & 0x7F80u) == 0x7F80u;
            }
    }
    return n;
}

// One unit is 6 F fragment steps, F = Panel::frags (K step kb = s / F, A
// fragment i = s % F): four MFMAs on A fragment i and the K step's four B
// fragments; the A fragment of step s + 3 is read from LDS (into the ring);
// at i == 0 the B fragments of K step kb + 2 are requested (into the next
// unit at the end).  One accumulator set: in the last K step, fragment
// i - 1 (final once its last MFMA, issued one step earlier, has run) is
// scaled, rounded and stored at step i, and fragment F - 1 at the next
// unit's first step (whose MFMAs write fragment 0), one row after each of
// the step's MFMAs; a fragment is overwritten by the next unit only after
// it has been read out.  Scheduling barriers keep each step's MFMAs and
// read-out rows in that order.
template <int FA, int FB, int ASRC, int ROWS, int BF>
__global__ void __launch_bounds__(kAsThreads, 1) k_gemm_astat(AsArgs p)
{
    // unit range of this workgroup: ranges of one XCD (workgroups b = x mod 8)
    // are adjacent, so a panel shared by two workgroups is read through one L2
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int rank = (b & 7) * (G >> 3) + min(b & 7, G & 7) + (b >> 3);
    const int u0 = (int)((int64_t)rank * p.units / G);
    const int u1 = (int)((int64_t)(rank + 1) * p.units / G);
    if (u0 >= u1) return;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;

    float sa, rcp = 1.0f;
    bool fast = false;
    if constexpr (ASRC == 1) {
        uint32_t k = 0;
        for (int i = threadIdx.x; i < p.np; i += kAsThreads) k = key_merge(k, p.partials[i]);
        k = block_reduce_key(k);
        sa = scale_from_amax<FA>(key_amax(k));
        fast = !key_special(k) && sa >= kCorrectedQuotMinScale;
        rcp = 1.0f / sa;
        if (b == 0 && threadIdx.x == 0) p.sa_out[0] = sa;
    } else {
        sa = p.sa[0];
    }
    const float out_scale = sa * p.sb[0];
    uint32_t sat = 0, und = 0, nan = 0;
    us2 mx = us2{0, 0};

    static_assert(ASRC == 0 || ROWS == kAsRowsCast, "panel of the cast form");
    using P = Panel<ROWS>;
    constexpr int kF = P::frags;
    v4f acc[kF][BF];
    v8i bb[kBRing][BF];
    v8i af[P::ring];
    const AFragBase ab = a_frag_base();
    uint32_t boff[BF];
#pragma unroll
    for (int f = 0; f < BF; ++f) boff[f] = (uint32_t)((16 * BF * w + BF * (l & 15) + f) * p.ldb + 32 * (l >> 4));
    const uint32_t row_bytes = (uint32_t)(p.ldc * 2);
    __amdgpu_buffer_rsrc_t rs_cur = b_rsrc<BF>(p, u0, u1), rs_next = b_rsrc<BF>(p, u0 + 1, u1);
    // Codes in A: the B ring is loaded once here and then only by the unit
    // body (the next unit's first steps), live across panel loads, so every
    // unit starts from the same registers.
    if constexpr (ASRC == 0) {
#pragma unroll
        for (int kb = 0; kb < kBAhead; ++kb)
#pragma unroll
            for (int f = 0; f < BF; ++f) bb[kb][f] = b_frag(rs_cur, boff, f, kb);
    }

    bool pending = false;   // fragment kF - 1 of the previous unit not stored yet
    int pm0 = 0, pn0 = 0;

    auto out_rsrc = [&](int m0) {
        return gemm::make_store_rsrc(p.c + (int64_t)m0 * p.ldc, (uint32_t)(min(P::rows, p.m - m0) * p.ldc * 2));
    };
    // the lane's store offset within a unit's rows: its columns and row group
    // (n % 4 == 0: a lane's BF columns are inside the matrix or past it entirely)
    auto col_off = [&](int n0) {
        const int col = n0 + 16 * BF * w + BF * (l & 15);
        return col < p.n ? (uint32_t)(col * 2) + (uint32_t)(4 * (l >> 4)) * row_bytes : gemm::kOutOfRange;
    };

    // Outer loop: the panels of the unit range; inner loop: the units of one
    // panel, a body with no branch around it.  (With the panel load as a
    // branch inside one unit loop, the compiler joined the two paths at every
    // unit start and made the first MFMAs wait for every outstanding memory
    // operation, the previous unit's output stores included.)
    for (int u = u0; u < u1;) {
        const int panel = u / p.ntn;
        const int m0 = panel * P::rows;
        const int u_end = min(u1, (panel + 1) * p.ntn);
        if (pending) {
            store_frag(acc, kF - 1, out_rsrc(pm0), col_off(pn0), row_bytes, out_scale, mx);
            pending = false;
        }
        __syncthreads();   // every wave is done with the previous panel
        const bool own = ASRC == 1 && u == panel * p.ntn;
        load_panel<FA, ASRC, ROWS>(p, m0, own, sa, rcp, fast, sat, und, nan);
        __syncthreads();
        if (ASRC == 1 && own && p.xqt) store_panel_t(p, m0);
        // the first A fragments of the panel (the same for every unit of it);
        // bf16 A: this unit's first B steps again (the B ring is left dead
        // across the cast, whose loads then have its registers)
#pragma unroll
        for (int j = 0; j < P::ahead; ++j) af[j] = a_frag(ab, j % kF, j / kF);
        if constexpr (ASRC == 1) {
#pragma unroll
            for (int kb = 0; kb < kBAhead; ++kb)
#pragma unroll
                for (int f = 0; f < BF; ++f) bb[kb][f] = b_frag(rs_cur, boff, f, kb);
        }
        const __amdgpu_buffer_rsrc_t rc = out_rsrc(m0);
        // what the panel's first unit drains (to an offset past the range)
#pragma unroll
        for (int f = 0; f < BF; ++f) acc[kF - 1][f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        for (; u < u_end; ++u) {
            const int n0 = (u - panel * p.ntn) * unit_cols<BF>();
            const uint32_t co = col_off(n0);
            // fragment kF - 1 of the previous unit of the same panel, stored at
            // step 0; in a panel's first unit there is none, and its step 0
            // stores zeros to an offset past the range (dropped)
            const uint32_t co_drain = pending ? col_off(pn0) : gemm::kOutOfRange;
#pragma unroll
            for (int s = 0; s < kAsKB * kF; ++s) {
                const int kb = s / kF, i = s % kF;
                if (i == 0) {
                    const int kf = kb + kBAhead;
#pragma unroll
                    for (int f = 0; f < BF; ++f)
                        bb[kf % kBRing][f] =
                            kf < kAsKB ? b_frag(rs_cur, boff, f, kf) : b_frag(rs_next, boff, f, kf - kAsKB);
                }
                // A fragment of step s + 3 (wrapping to the next unit's first K step)
                {
                    const int s3 = (s + P::ahead) % (kAsKB * kF);
                    af[(s + P::ahead) % P::ring] = a_frag(ab, s3 % kF, s3 / kF);
                }
                const v8i& a = af[s % P::ring];
                // a fragment's read-out goes out one row at a time between the
                // MFMAs (4 / BF rows after each), so the VALU work runs while
                // the matrix pipe has an MFMA to execute
#pragma unroll
                for (int f = 0; f < BF; ++f) {
                    acc[i][f] =
                        gemm::mfma<FA, FB>(a, bb[kb % kBRing][f], kb == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : acc[i][f]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int r = f * 4 / BF; r < (f + 1) * 4 / BF; ++r) {
                        if (s == 0) store_row(acc, kF - 1, r, rc, co_drain, row_bytes, out_scale, mx);
                        if (kb == kAsKB - 1 && i >= 1) store_row(acc, i - 1, r, rc, co, row_bytes, out_scale, mx);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            pending = true;
            pm0 = m0;
            pn0 = n0;
            rs_cur = rs_next;
            rs_next = b_rsrc<BF>(p, u + 2, u1);
        }
    }
    if (pending)
        store_frag(acc, kF - 1, out_rsrc(pm0), col_off(pn0), row_bytes, out_scale, mx);
    const uint32_t nonfinite = (mx.x >= 0x7F80u || mx.y >= 0x7F80u) ? recount<ROWS, BF>(p, u0, u1) : 0u;
    flush_counters(p.ctr, 0, 0, 0, nonfinite);
    if constexpr (ASRC == 1) flush_counters_block(p.ctr, sat, und, nan);
}

}  // namespace

bool astat_supported(int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb, int64_t ldc, const void* c)
{
    return k == kAstatK && m > 0 && n > 0 && n % 4 == 0 && ldc % 4 == 0 &&
           (reinterpret_cast<uintptr_t>(c) & 7u) == 0 && lda < ((int64_t)1 << 22) && ldb < ((int64_t)1 << 22) &&
           ldc < ((int64_t)1 << 21) &&
           (m + kAsMinRows - 1) / kAsMinRows * ((n + unit_cols<2>() - 1) / unit_cols<2>()) < ((int64_t)1 << 31);
}

hipError_t launch_gemm_astat(const AstatArgs& g, int num_cus, hipStream_t stream)
{
    AsArgs p;
    p.a = g.a;
    p.lda = g.lda;
    p.b = g.b;
    p.ldb = g.ldb;
    p.sa = g.sa;
    p.sa_out = g.sa_out;
    p.sb = g.sb;
    p.partials = g.partials;
    p.np = g.np;
    p.xq = g.xq;
    p.ldxq = g.ldxq;
    p.xqt = g.xqt;
    p.ldxqt = g.ldxqt;
    p.xqt_words = (reinterpret_cast<uintptr_t>(g.xqt) & 3u) == 0 && g.ldxqt % 4 == 0;
    p.m = (int)g.m;
    p.n = (int)g.n;
    p.c = static_cast<uint16_t*>(g.c);
    p.ldc = g.ldc;
    p.ctr = g.ctr;
    // form: 0 codes (208-row panels, 256-column units), 1 cast from bf16
    // (192 rows, 256 columns), 2 short A (32 rows, 128 columns)
    int form = g.bf16_a ? 1 : 0;
    if (!g.bf16_a && (g.m + kAsRowsShort - 1) / kAsRowsShort * ((g.n + unit_cols<2>() - 1) / unit_cols<2>()) <= num_cus)
        form = 2;
    const int rows = form == 1 ? kAsRowsCast : form == 2 ? kAsRowsShort : kAsRowsCodes;
    const int cols = form == 2 ? unit_cols<2>() : unit_cols<4>();
    // n == 0 still walks one (empty) column unit per panel, so that the
    // panel's codes and counters are produced
    p.ntn = std::max(1, (int)((g.n + cols - 1) / cols));
    const int panels = (int)((g.m + rows - 1) / rows);
    p.units = panels * p.ntn;
    const int grid = std::min(p.units, num_cus);
    const int sel = (g.fa * 2 + g.fb) * 3 + form;
    switch (sel) {
#define FP8MI_ASTAT(FA_, FB_, F_, S_, R_, BF_)                                                                \
    case (FA_ * 2 + FB_) * 3 + F_:                                                                            \
        hipLaunchKernelGGL((k_gemm_astat<FA_, FB_, S_, R_, BF_>), dim3(grid), dim3(kAsThreads), 0, stream, p); \
        break;
#define FP8MI_ASTAT3(FA_, FB_)                       \
    FP8MI_ASTAT(FA_, FB_, 0, 0, kAsRowsCodes, 4)     \
    FP8MI_ASTAT(FA_, FB_, 1, 1, kAsRowsCast, 4)      \
    FP8MI_ASTAT(FA_, FB_, 2, 0, kAsRowsShort, 2)
        FP8MI_ASTAT3(0, 0) FP8MI_ASTAT3(0, 1) FP8MI_ASTAT3(1, 0) FP8MI_ASTAT3(1, 1)
#undef FP8MI_ASTAT3
#undef FP8MI_ASTAT
    }
    return hipGetLastError();
}

}  // namespace fp8mi
