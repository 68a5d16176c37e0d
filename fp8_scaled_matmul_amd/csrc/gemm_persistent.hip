// Persistent per-tensor-scaled FP8 GEMM for gfx950:
//   y = bf16(s_a s_b sum_k A[m,k] B[n,k])
// (the scaled product of _scaled_mm(x, w_fp8, scale_a, scale_b), "#84 FP8
// Precision", code excerpt and "Explanation"), or, for a K split, the fp32
// partial sums of one K range.
//
// One workgroup of 4 waves per CU walks a list of 256x256 output tiles (each
// wave owns 128x128).  The list of each XCD is a contiguous, M-grouped range,
// so the A panels and the B operand that the XCD's workgroups share stay in
// its L2.  The K dimension of all the workgroup's tiles forms one stream of
// 64-deep half steps; each half step is 16 v_mfma_f32_32x32x64_f8f6f4
// per wave.
//
// Pipeline (one wave per SIMD, so nothing may stall the MFMA issue):
//   - 4 LDS stages of 32 KB (A and B, 64 K each); the DMA of half step t+4
//     (buffer_load ... lds, waited for with counted vmcnt) refills the stage
//     half step t has just released;
//   - two fragment register sets: while the 16 MFMAs of half step t run, the
//     16 ds_read_b128 of half step t+1 and the 8 DMA instructions of half
//     step t+4 are issued between them (a DMA issue can block while the
//     address unit is busy; spread out, the queued MFMA covers it);
//   - one barrier per half step.
// The next tile's first half steps load while the current tile's epilogue
// writes its output.
//
// Output layout: B rows are placed in LDS so that MFMA lane p of column
// fragment j holds output column 4p + j; each lane owns four consecutive
// columns of every output row it touches (one 8-byte bf16 store, or one
// 16-byte fp32 store, per row).
#include "device_common.h"
#include "fp8mi_internal.h"
#include "gemm_common.h"

#include <type_traits>

namespace fp8mi {

using namespace gemm;

namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

constexpr int KH = 64;                      // K bytes per half step (one stage)
constexpr int kStages = 4;
constexpr int kStageBytes = BM * KH;        // 16 KB per operand per stage
constexpr int kDmaPerHalf = 8;              // DMA instructions per thread per half step
constexpr int kStoresBf16 = 64;             // epilogue stores per thread, bf16 output
constexpr int kStoresF32 = 64;              // fp32 split partials
constexpr int kOutBf16 = 0, kOutF32 = 1, kOutGeneric = 2;

struct PArgs {
    const uint8_t* a;
    const uint8_t* b;
    int64_t lda, ldb;
    const float* sa;
    const float* sb;
    int m, n, k;
    uint16_t* c;
    int64_t ldc;
    float* ws;          // split partials [splits][m][n] fp32, or nullptr
    int splits, h_per, nhalves;
    int tiles_m, tiles_n;
    int items, per_xcd, g8;
    int fast_store;     // row-segment stores are aligned and in range
    int group_m;        // M tiles per group of the tile order
    fp8_counters* ctr;
};

__shared__ __attribute__((aligned(1024))) uint8_t s_lds_a[kStages * kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t s_lds_b[kStages * kStageBytes];

// 16-byte chunk c (0..3) of the 64-byte LDS row r sits at position
// swz4(r, c).  For 8 aligned consecutive rows reading the same chunk the
// (row parity, position) pairs are distinct (no conflict with 32 banks), and
// so are the (row mod 4, position) pairs of 16 aligned rows (64 banks).  An
// involution.
__device__ inline int swz4(int r, int c) { return c ^ (((r >> 1) ^ (r >> 2)) & 3); }

template <int FA, int FB>
__device__ inline v16f mfma32(const v8i& a, const v8i& b, const v16f& c)
{
    // FA / FB: 0 = E4M3, 1 = E5M2.  Zero scale operands select the unscaled
    // v_mfma_f32_32x32x64_f8f6f4 (no v_mfma_ld_scale_b32 prefix).
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// 32x64 operand fragment of one stage: lane l reads row row0 + l%32, K bytes
// 32 (l/32) .. +32 (A and B alike, so the products pair up whatever order the
// instruction gives the 64 K values).
__device__ inline v8i frag32(const uint8_t* stage, int row0)
{
    const int l = threadIdx.x & 63;
    const int r = row0 + (l & 31);
    const int c0 = (l >> 5) * 2;
    const uint4 lo = *reinterpret_cast<const uint4*>(stage + r * KH + swz4(r, c0) * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(stage + r * KH + swz4(r, c0 + 1) * 16);
    v8i f;
    f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
    f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
    return f;
}

// The accumulators live in AGPRs; an arithmetic use needs a copy into a
// VGPR.  Issuing it here keeps the compiler from copying all 256 at once
// (which runs out of VGPRs) at the end of the K loop.
__device__ inline float agpr_read(float a)
{
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

struct Item {
    int m0, n0, h0, h1, split;
};

__device__ inline Item decode_item(const PArgs& p, int item)
{
    const int per_split = p.tiles_m * p.tiles_n;
    Item it;
    it.split = item / per_split;
    const int t = item - it.split * per_split;
    const int in_group = p.group_m * p.tiles_n;
    const int g = t / in_group;
    const int first_m = g * p.group_m;
    const int gsize = min(p.tiles_m - first_m, p.group_m);
    const int r = t - g * in_group;
    // all of it is uniform over the workgroup: keep it in scalar registers
    it.m0 = __builtin_amdgcn_readfirstlane((first_m + r % gsize) * BM);
    it.n0 = __builtin_amdgcn_readfirstlane((r / gsize) * BN);
    it.h0 = __builtin_amdgcn_readfirstlane(it.split * p.h_per);
    it.h1 = __builtin_amdgcn_readfirstlane(min(p.nhalves, it.h0 + p.h_per));
    it.split = __builtin_amdgcn_readfirstlane(it.split);
    return it;
}

// Position of one workgroup in its stream of (item, half step).
struct Cursor {
    int s;          // index in this workgroup's item list
    int item_end;   // end of this XCD's item range
    Item it;
    int h;
    bool valid;
    v4u ra, rb;     // the item's A and B panels (zero length once the stream has ended),
                    // formed once per item rather than for every half step's DMA job
};

__device__ inline void cursor_load(const PArgs& p, Cursor& c, int xcd, int slot)
{
    const int item = __builtin_amdgcn_readfirstlane(xcd * p.per_xcd + slot + p.g8 * c.s);
    c.valid = item < c.item_end;
    if (c.valid) {
        c.it = decode_item(p, item);
        c.h = c.it.h0;
    } else {
        c.it = Item{0, 0, 0, 0, 0};
        c.h = 0;
    }
    c.ra = make_rsrc(p.a + (int64_t)c.it.m0 * p.lda, c.valid ? (uint32_t)(min(BM, p.m - c.it.m0) * p.lda) : 0u);
    c.rb = make_rsrc(p.b + (int64_t)c.it.n0 * p.ldb, c.valid ? (uint32_t)(min(BN, p.n - c.it.n0) * p.ldb) : 0u);
}

__device__ inline void cursor_next(const PArgs& p, Cursor& c, int xcd, int slot)
{
    if (++c.h >= c.it.h1) {
        ++c.s;
        cursor_load(p, c, xcd, slot);
    }
}

// Per-lane byte offsets of the 4 DMA instructions per operand and half step
// of this wave: instruction j fills LDS rows 64 w + 16 j .. +15; lane l
// writes row R = 64 w + 16 j + l/4, position l%4, which receives logical
// chunk swz4(R, l%4) of global row g(R).  A: g(R) = R.  B: within each
// 128-row half, g(R) = 4 (R%32) + R/32, so that fragment j's lane p (LDS row
// 32 j + p) carries output column 4 p + j.  The chunk index does not depend
// on j (16 j and 64 w do not change the swizzle).
struct Offsets {
    uint32_t voff[4];
    int ck;         // K byte offset of this lane's chunk
};

__device__ inline Offsets make_offsets(int64_t ld, bool permute)
{
    Offsets o;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int R = 64 * w + 16 * j + (l >> 2);
        const int c = swz4(R, l & 3);
        const int g = permute ? (R & 128) + 4 * (R & 31) + ((R & 127) >> 5) : R;
        o.voff[j] = (uint32_t)(g * ld + 16 * c);
        if (j == 0) o.ck = 16 * c;
    }
    return o;
}

// The 8 DMA instructions (4 for A, 4 for B) of one half step of one wave.
// Once the stream has ended the descriptors have zero length: the loads
// then write zeros into a stage nothing reads any more, which keeps the
// count of pending operations the same for every half step.
struct DmaJob {
    v4u ra, rb;
    uint32_t lds_a, lds_b;      // this wave's first 1 KB slot of the stage
    int k0;
};

// Instruction j (0..7) of a job.  k is a multiple of 16: a chunk is
// entirely inside K or entirely past it (then its offset is out of range and
// the DMA writes zeros).
__device__ inline void dma_one(const DmaJob& job, const Offsets& oa, const Offsets& ob, int j, int k)
{
    const bool in_k = job.k0 + oa.ck < k;     // (oa.ck == ob.ck)
    if (j < 4)
        dma16(job.lds_a + (uint32_t)j * 1024u, in_k ? oa.voff[j] + (uint32_t)job.k0 : kOutOfRange, job.ra);
    else
        dma16(job.lds_b + (uint32_t)(j - 4) * 1024u, in_k ? ob.voff[j - 4] + (uint32_t)job.k0 : kOutOfRange,
              job.rb);
}

// One half step: 16 MFMAs on the current fragments.  The first kEarly of
// them go out before `sync` (the wait for this half step's DMA and the
// barrier): they use only fragments read during the previous half step, so
// the matrix pipe has work queued while the wave waits (measured 1-3% faster
// than waiting first; 1 and 3 no better, 4 slower).  Between the others go
// the 16 LDS reads of the next half step's fragments and, after every second
// read, one DMA instruction of the job, so that neither the LDS reads nor the
// DMA issue (which can stall while the address FIFO is full) hold up the
// MFMA stream.
constexpr int kEarly = 2;
constexpr int read_slot(int q) { return kEarly + q * (16 - kEarly) / 16; }

template <int FA, int FB, bool FIRST, typename Sync>
__device__ inline void half_step(v16f (&acc)[4][4], const v8i (&ca)[4], const v8i (&cb)[4], v8i (&na)[4],
                                 v8i (&nb)[4], const uint8_t* la, const uint8_t* lb, int wm, int wn,
                                 const DmaJob& job, const Offsets& oa, const Offsets& ob, int k, Sync&& sync)
{
    if constexpr (kEarly == 0) sync();
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int i = s >> 2, j = s & 3;
        if constexpr (FIRST)
            acc[i][j] = mfma32<FA, FB>(ca[i], cb[j], v16f{});
        else
            acc[i][j] = mfma32<FA, FB>(ca[i], cb[j], acc[i][j]);
        if (kEarly > 0 && s == kEarly - 1) {
            __builtin_amdgcn_sched_barrier(0);
            sync();
        }
        // reads: B fragments first (q = 0..7), then A; DMA instruction f after
        // the second half of fragment f
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            if (read_slot(q) != s) continue;
            const int f = q >> 1;
            const int row0 = f < 4 ? wn + 32 * f : wm + 32 * (f - 4);
            const uint8_t* base = f < 4 ? lb : la;
            const int l = threadIdx.x & 63;
            const int r = row0 + (l & 31);
            const int c = (l >> 5) * 2 + (q & 1);
            const uint4 v = *reinterpret_cast<const uint4*>(base + r * KH + swz4(r, c) * 16);
            v8i& dst = f < 4 ? nb[f] : na[f - 4];
            if ((q & 1) == 0) {
                dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
            } else {
                dst[4] = v.x; dst[5] = v.y; dst[6] = v.z; dst[7] = v.w;
                dma_one(job, oa, ob, f, k);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // Pin the MFMAs to this half step: an MFMA touches no memory, so without
    // a use here the compiler may sink it past the next half step's wait and
    // barrier.  (Empty asm: no instruction, no wait for the results.)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
}

template <int FA, int FB, int OUT>
__global__ void __launch_bounds__(256, 1) k_gemm_persistent(PArgs p)
{
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = (wave >> 1) * 128;
    const int wn = (wave & 1) * 128;

    // the per-tensor output scale, loaded before any DMA is in flight so that
    // waiting for it never waits for the DMA
    float out_scale = 1.0f;
    if constexpr (OUT != kOutF32) out_scale = p.ws ? 1.0f : p.sa[0] * p.sb[0];
    asm volatile("" : "+v"(out_scale));

    const Offsets oa = make_offsets(p.lda, false);
    const Offsets ob = make_offsets(p.ldb, true);
    const uint32_t lds_a0 = lds_addr(s_lds_a), lds_b0 = lds_addr(s_lds_b);

    Cursor d;   // DMA cursor, four half steps ahead of the compute cursor
    d.s = 0;
    d.item_end = min((xcd + 1) * p.per_xcd, p.items);
    cursor_load(p, d, xcd, slot);
    Cursor c = d;
    if (!c.valid) return;

    const int wave_slot = wave * 4 * 1024;
    auto make_job = [&](int stage) -> DmaJob {
        DmaJob job;
        const bool v = d.valid;
        job.ra = d.ra;
        job.rb = d.rb;
        job.lds_a = lds_a0 + stage * kStageBytes + wave_slot;
        job.lds_b = lds_b0 + stage * kStageBytes + wave_slot;
        job.k0 = d.h * KH;
        if (v) cursor_next(p, d, xcd, slot);
        return job;
    };

    // prologue: half steps 0..3 into stages 0..3, then the fragments of half 0
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const DmaJob job = make_job(q);
#pragma unroll
        for (int j = 0; j < kDmaPerHalf; ++j) dma_one(job, oa, ob, j, p.k);
    }
    wait_vmcnt(3 * kDmaPerHalf);
    barrier_only();
    v8i ra0[4], rb0[4], ra1[4], rb1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rb0[j] = frag32(s_lds_b, wn + 32 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) ra0[i] = frag32(s_lds_a, wm + 32 * i);

    int s3 = 0, s2 = 0, s1 = 0;    // stores issued in half steps t-3, t-2, t-1
    uint32_t nonfinite = 0;
    v16f acc[4][4];
    int t = 0;                     // half-step index in this workgroup's stream

    // Half step t: MFMAs on (cur_a, cur_b), fragments of half step t+1 read
    // into (nxt_a, nxt_b), DMA of half step t+4 into the stage half step t
    // has released.  Every half step issues its 8 DMA instructions, then
    // (after a tile's last half step) the epilogue's stores, so DMA(t+1),
    // issued in half step t-3, is complete once at most the stores of
    // t-3..t-1 and the 16 DMA instructions of t+2, t+3 are pending.
    auto half = [&](auto first, const v8i (&cur_a)[4], const v8i (&cur_b)[4], v8i (&nxt_a)[4], v8i (&nxt_b)[4]) {
        const DmaJob job = make_job(t & 3);
        const int pending = 2 * kDmaPerHalf + s3 + s2 + s1;
        auto sync = [&]() {
            // pending is 16, or at least 80 while an epilogue's stores are in
            // flight; the counter's field saturates at 63, and waiting until at
            // most 63 operations are pending waits at least as long
            static_assert(2 * kDmaPerHalf == 16 && kStoresBf16 >= 48 && kStoresF32 >= 48,
                          "the two waits below assume 16 DMA operations or more than 63 pending");
            if (pending > 2 * kDmaPerHalf)
                asm volatile("s_waitcnt vmcnt(63)" ::: "memory");
            else
                asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
            // every wave has read its half-t fragments out of stage t%4, and
            // half t+1's data is in stage (t+1)%4
            barrier_lds();
        };
        // (after the stream's last half step this reads a stale stage: harmless)
        const uint8_t* la = s_lds_a + ((t + 1) & 3) * kStageBytes;
        const uint8_t* lb = s_lds_b + ((t + 1) & 3) * kStageBytes;
        half_step<FA, FB, decltype(first)::value>(acc, cur_a, cur_b, nxt_a, nxt_b, la, lb, wm, wn, job, oa, ob,
                                                  p.k, sync);
        s3 = s2;
        s2 = s1;
        s1 = 0;
        ++t;
    };
    using First = std::true_type;
    using Next = std::false_type;

    while (c.valid) {
        // the tile's half steps; its fragments start (and end) in set 0
        const int nh = c.it.h1 - c.it.h0;
        half(First{}, ra0, rb0, ra1, rb1);
        int h = 1;
        for (; h + 2 <= nh; h += 2) {
            half(Next{}, ra1, rb1, ra0, rb0);
            half(Next{}, ra0, rb0, ra1, rb1);
        }
        if (h < nh) {
            half(Next{}, ra1, rb1, ra0, rb0);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ra0[i] = ra1[i];
                rb0[i] = rb1[i];
            }
        }

        // epilogue: lane owns columns n0 + wn + 4 (lane%32) + 0..3 of rows
        // m0 + wm + 32 i + 8 (v/4) + 4 (lane/32) + v%4 (accumulator i, element v)
        const Item& it = c.it;
        // lane constants formed here (pinned by an empty asm) rather than
        // kept live across the K loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int col = it.n0 + ((tid >> 6) & 1) * 128 + 4 * (tid & 31);
        const int rrow = ((tid >> 7) & 1) * 128 + 4 * ((tid & 63) >> 5);
        if constexpr (OUT == kOutBf16) {
            // the reads below are inline asm, which the compiler's hazard
            // checks do not see: give the last MFMA's results the wait
            // states an XDL write needs before an AGPR read (at most 19)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
            const __amdgpu_buffer_rsrc_t rs =
                make_store_rsrc(p.c + (int64_t)it.m0 * p.ldc, (uint32_t)(min(BM, p.m - it.m0) * p.ldc * 2));
            uint32_t base = col < p.n ? (uint32_t)((rrow * p.ldc + col) * 2) : kOutOfRange;
            asm volatile("" : "+v"(base));
            const uint32_t row_bytes = (uint32_t)(p.ldc * 2);
            // running max of |bf16| patterns: >= 0x7F80 marks Inf / NaN
            // (outputs outside the matrix are zeros: their operands read as zero)
            us2 mx = us2{0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rr = 32 * i + 8 * (v >> 2) + (v & 3);
                    const uint32_t off = base == kOutOfRange ? kOutOfRange : base + (uint32_t)rr * row_bytes;
                    const float e0 = agpr_read(acc[i][0][v]), e1 = agpr_read(acc[i][1][v]);
                    const float e2 = agpr_read(acc[i][2][v]), e3 = agpr_read(acc[i][3][v]);
                    v2u w;
                    w.x = pack_bf16(e0 * out_scale, e1 * out_scale);
                    w.y = pack_bf16(e2 * out_scale, e3 * out_scale);
                    // nontemporal (aux bit 1, "nt"): the output streams out (measured:
                    // 4-8% faster on the 65536-row shapes than the default policy)
                    __builtin_amdgcn_raw_buffer_store_b64(w, rs, (int)off, 0, 2);
                    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, w.x & 0x7FFF7FFFu));
                    mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, w.y & 0x7FFF7FFFu));
                    if ((v & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                }
            s1 = kStoresBf16;
            if (mx.x >= 0x7F80u || mx.y >= 0x7F80u) {
                // rare: count exactly, reading back what this lane stored
                // (after its stores have completed; the accumulators are
                // not kept alive for this).  Leaving s1 as it is only
                // overstates the pending operations of DMAs that this drain
                // has already completed.
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                for (int i = 0; i < 4; ++i)
                    for (int v = 0; v < 16; ++v) {
                        const int row = it.m0 + rrow + 32 * i + 8 * (v >> 2) + (v & 3);
                        if (row >= p.m || col >= p.n) continue;
                        const v2u w = *reinterpret_cast<const v2u*>(p.c + (int64_t)row * p.ldc + col);
                        nonfinite += ((w.x & 0x7F80u) == 0x7F80u) + ((w.x & 0x7F800000u) == 0x7F800000u) +
                                     ((w.y & 0x7F80u) == 0x7F80u) + ((w.y & 0x7F800000u) == 0x7F800000u);
                    }
            }
        } else if constexpr (OUT == kOutF32) {
            float* wsb = p.ws + ((int64_t)it.split * p.m + it.m0) * p.n;
            const __amdgpu_buffer_rsrc_t rs = make_store_rsrc(wsb, (uint32_t)(min(BM, p.m - it.m0) * p.n * 4));
            uint32_t base = col < p.n ? (uint32_t)((rrow * p.n + col) * 4) : kOutOfRange;
            asm volatile("" : "+v"(base));
            const uint32_t row_bytes = (uint32_t)(p.n * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rr = 32 * i + 8 * (v >> 2) + (v & 3);
                    const uint32_t off = base == kOutOfRange ? kOutOfRange : base + (uint32_t)rr * row_bytes;
                    // (copy the elements to scalars first: a bit cast of an
                    // ext_vector element expression reads element 0)
                    const float e0 = acc[i][0][v], e1 = acc[i][1][v], e2 = acc[i][2][v], e3 = acc[i][3][v];
                    store16(v4u{__builtin_bit_cast(uint32_t, e0), __builtin_bit_cast(uint32_t, e1),
                                __builtin_bit_cast(uint32_t, e2), __builtin_bit_cast(uint32_t, e3)},
                            off, rs);
                    if ((v & 3) == 3) __builtin_amdgcn_sched_barrier(0);
                }
            s1 = kStoresF32;
        } else {
            // any alignment: element stores, then drain
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = it.m0 + rrow + 32 * i + 8 * (v >> 2) + (v & 3);
                    if (row >= p.m) continue;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (col + j >= p.n) continue;
                        const float e = acc[i][j][v];
                        if (p.ws) {
                            p.ws[((int64_t)it.split * p.m + row) * p.n + col + j] = e;
                        } else {
                            const uint16_t hb = to_bf16(e * out_scale);
                            nonfinite += (hb & 0x7F80u) == 0x7F80u;
                            p.c[(int64_t)row * p.ldc + col + j] = hb;
                        }
                    }
                }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        ++c.s;
        cursor_load(p, c, xcd, slot);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    flush_counters(p.ctr, 0, 0, 0, nonfinite);
}

}  // namespace

// Persistent launch: one workgroup per CU (at most), eight XCD groups.
hipError_t launch_gemm_persistent(const GemmArgs& g, int num_cus, hipStream_t stream)
{
    PArgs p;
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
    p.ctr = g.ctr;
    p.nhalves = (int)((g.k + KH - 1) / KH);
    // split ranges in whole 128-deep steps: the split points the workspace
    // size and the reduce are computed with
    const int ktiles = (int)((g.k + BK - 1) / BK);
    int splits = g.splits > 1 && g.ws ? g.splits : 1;
    const int kt_per = (ktiles + splits - 1) / splits;
    splits = (ktiles + kt_per - 1) / kt_per;      // no empty split
    p.splits = splits;
    p.h_per = 2 * kt_per;
    p.ws = splits > 1 ? g.ws : nullptr;
    p.tiles_m = (int)((g.m + BM - 1) / BM);
    p.tiles_n = (int)((g.n + BN - 1) / BN);
    // M tiles per group of the tile order (65536x3072x768: 4.5% faster with 4
    // than with 8; 2 and 16 no better)
    p.group_m = 4;
    p.items = p.tiles_m * p.tiles_n * p.splits;
    const int max_g8 = std::max(1, num_cus / 8);
    int grid;
    if (p.items < 8) {
        p.per_xcd = 1;
        p.g8 = 1;
        grid = p.items;
    } else {
        p.per_xcd = (p.items + 7) / 8;
        p.g8 = std::min(max_g8, p.per_xcd);
        grid = 8 * p.g8;
    }
    if (p.ws)
        p.fast_store = (g.n % 4 == 0) && ((reinterpret_cast<uintptr_t>(g.ws) & 15u) == 0);
    else
        p.fast_store = (g.n % 4 == 0) && (g.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(g.c) & 7u) == 0);
    const int out = !p.fast_store ? kOutGeneric : (p.ws ? kOutF32 : kOutBf16);
    const int fmt = g.fa * 2 + g.fb;
    switch (fmt * 3 + out) {
#define FP8MI_CASE(FA_, FB_, OUT_)                                                                      \
    case (FA_ * 2 + FB_) * 3 + OUT_:                                                                    \
        hipLaunchKernelGGL((k_gemm_persistent<FA_, FB_, OUT_>), dim3(grid), dim3(256), 0, stream, p); \
        break;
        FP8MI_CASE(0, 0, 0) FP8MI_CASE(0, 0, 1) FP8MI_CASE(0, 0, 2)
        FP8MI_CASE(0, 1, 0) FP8MI_CASE(0, 1, 1) FP8MI_CASE(0, 1, 2)
        FP8MI_CASE(1, 0, 0) FP8MI_CASE(1, 0, 1) FP8MI_CASE(1, 0, 2)
        FP8MI_CASE(1, 1, 0) FP8MI_CASE(1, 1, 1) FP8MI_CASE(1, 1, 2)
#undef FP8MI_CASE
    }
    return hipGetLastError();
}

}  // namespace fp8mi
