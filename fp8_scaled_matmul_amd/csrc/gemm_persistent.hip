// Persistent per-tensor-scaled FP8 GEMM for gfx950:
//   y = bf16(s_a s_b sum_k A[m,k] B[n,k])
// (the scaled product of _scaled_mm(x, w_fp8, scale_a, scale_b), "#84 FP8
// Precision", code excerpt and "Explanation"), or, for a K split, the fp32
// partial sums of one K range.
//
// One workgroup of 4 waves per CU walks a list of 256x256 output tiles.  The
// list of each XCD is a contiguous, M-grouped range, so the A panels and the
// B operand a wave of workgroups shares sit in that XCD's L2.  The K steps
// of all the workgroup's tiles form one stream: step q's operands (two
// 32 KB tiles) arrive in LDS stage q%2 by DMA issued two steps earlier, so
// the first steps of the next tile load while the current tile finishes and
// writes its output.  Per step and wave: read the 16 MFMA fragments of the
// stage into registers, release the stage, start the DMA of step q+2 into
// it, run 64 MFMAs (16x16x128) into 256 fp32 accumulators.
//
// Output layout trick: B rows are placed in LDS so that MFMA lane p of
// column fragment j holds output column 8p + j.  Each lane then owns eight
// consecutive columns of every output row it touches, and the epilogue
// writes a row segment with one 16-byte store.
#include "device_common.h"
#include "fp8mi_internal.h"
#include "gemm_common.h"

namespace fp8mi {

using namespace gemm;

namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

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
    int splits, kt_per, ktiles;
    int tiles_m, tiles_n;
    int items, per_xcd, g8;
    int fast_store;     // 16-byte row-segment stores are aligned and in range
    fp8_counters* ctr;
};

__shared__ __attribute__((aligned(1024))) uint8_t p_lds_a[2 * kTileBytes];
__shared__ __attribute__((aligned(1024))) uint8_t p_lds_b[2 * kTileBytes];

struct Item {
    int m0, n0, kt0, kt1, split;
};

__device__ inline Item decode_item(const PArgs& p, int item)
{
    const int per_split = p.tiles_m * p.tiles_n;
    Item it;
    it.split = item / per_split;
    const int t = item - it.split * per_split;
    const int in_group = kGroupM * p.tiles_n;
    const int g = t / in_group;
    const int first_m = g * kGroupM;
    const int gsize = min(p.tiles_m - first_m, kGroupM);
    const int r = t - g * in_group;
    it.m0 = (first_m + r % gsize) * BM;
    it.n0 = (r / gsize) * BN;
    it.kt0 = it.split * p.kt_per;
    it.kt1 = min(p.ktiles, it.kt0 + p.kt_per);
    // all of it is uniform over the workgroup: keep it in scalar registers
    it.m0 = __builtin_amdgcn_readfirstlane(it.m0);
    it.n0 = __builtin_amdgcn_readfirstlane(it.n0);
    it.kt0 = __builtin_amdgcn_readfirstlane(it.kt0);
    it.kt1 = __builtin_amdgcn_readfirstlane(it.kt1);
    it.split = __builtin_amdgcn_readfirstlane(it.split);
    return it;
}

// Position of one workgroup in its stream of (item, K step).
struct Cursor {
    int s;          // index in this workgroup's item list
    int item_end;   // end of this XCD's item range
    int item;
    Item it;
    int kt;
    bool valid;
};

__device__ inline void cursor_load(const PArgs& p, Cursor& c, int xcd, int slot)
{
    const int item = __builtin_amdgcn_readfirstlane(xcd * p.per_xcd + slot + p.g8 * c.s);
    c.valid = item < c.item_end;
    if (c.valid) {
        c.item = item;
        c.it = decode_item(p, item);
        c.kt = c.it.kt0;
    }
}

__device__ inline void cursor_next(const PArgs& p, Cursor& c, int xcd, int slot)
{
    if (++c.kt >= c.it.kt1) {
        ++c.s;
        cursor_load(p, c, xcd, slot);
    }
}

// Per-lane byte offsets of the 8 DMA chunks of one operand tile (tile base
// and K offset excluded).  Wave w fills LDS rows 64 w .. 64 w + 63; LDS slot
// (row R, position l%8) receives the logical chunk swz(R, l%8) of global
// row g(R).  A: g(R) = R.  B: within each 128-row half, g(R) = 8 (R%16) + R/16,
// so that fragment j's lane p (LDS row 16 j + p) holds column 8 p + j.
struct Offsets {
    uint32_t voff[8];
    int ck[2];      // K byte offset of the chunk, for instruction parity j & 1
};

__device__ inline Offsets make_offsets(int64_t ld, bool permute)
{
    Offsets o;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int R = 64 * w + 8 * j + (l >> 3);
        const int c = swz(R, l & 7);
        const int g = permute ? (R & 128) + 8 * (R & 15) + ((R & 127) >> 4) : R;
        o.voff[j] = (uint32_t)(g * ld + 16 * c);
        if (j < 2) o.ck[j] = 16 * c;
    }
    return o;
}

__device__ inline void dma_tile(const Offsets& o, const v4u& rsrc, uint32_t lds_base, int k0, int k)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t off = k0 + o.ck[j & 1] < k ? o.voff[j] + (uint32_t)k0 : kOutOfRange;
        dma16(lds_base + (uint32_t)(w * 8 + j) * 1024u, off, rsrc);
    }
}

constexpr int kOutBf16 = 0, kOutF32 = 1, kOutGeneric = 2;

constexpr int kDmaPerStep = 16;     // DMA instructions per thread per K step
constexpr int kStoresBf16 = 32;     // epilogue store instructions per thread (bf16 out)
constexpr int kStoresF32 = 64;      // (fp32 split partials)

template <int FA, int FB, int OUT>
__global__ void __launch_bounds__(256, 1) k_gemm_persistent(PArgs p)
{
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int wm = (wave >> 1) * 128;
    const int wn = (wave & 1) * 128;

    // the per-tensor output scale, loaded before any DMA is in flight so that
    // waiting for it never waits for the DMA
    float out_scale = 1.0f;
    if constexpr (OUT != kOutF32) out_scale = p.ws ? 1.0f : p.sa[0] * p.sb[0];
    asm volatile("" : "+v"(out_scale));

    const Offsets oa = make_offsets(p.lda, false);
    const Offsets ob = make_offsets(p.ldb, true);
    const uint32_t lds_a0 = lds_addr(p_lds_a), lds_b0 = lds_addr(p_lds_b);

    const int item_end = min((xcd + 1) * p.per_xcd, p.items);
    Cursor d;   // DMA cursor, two steps ahead of the compute cursor
    d.s = 0;
    d.item_end = item_end;
    cursor_load(p, d, xcd, slot);
    Cursor c = d;

    auto issue = [&](const Cursor& cur, int stage) -> int {
        if (!cur.valid) return 0;
        const Item& it = cur.it;
        const int k0 = cur.kt * BK;
        const uint32_t ra_bytes = (uint32_t)(min(BM, p.m - it.m0) * p.lda);
        const uint32_t rb_bytes = (uint32_t)(min(BN, p.n - it.n0) * p.ldb);
        const v4u ra = make_rsrc(p.a + (int64_t)it.m0 * p.lda, ra_bytes);
        const v4u rb = make_rsrc(p.b + (int64_t)it.n0 * p.ldb, rb_bytes);
        dma_tile(oa, ra, lds_a0 + stage * kTileBytes, k0, p.k);
        dma_tile(ob, rb, lds_b0 + stage * kTileBytes, k0, p.k);
        return kDmaPerStep;
    };

    // prologue: steps 0 and 1 into stages 0 and 1
    int n_dma_next;            // DMA instructions of the step after the current one
    issue(d, 0);
    cursor_next(p, d, xcd, slot);
    n_dma_next = issue(d, 1);
    cursor_next(p, d, xcd, slot);
    int stores_prev2 = 0, stores_prev1 = 0;

    uint32_t nonfinite = 0;
    int q = 0;
    v4f acc[8][8];
    while (c.valid) {
      for (bool first = true; ; first = false) {
        const int stage = q & 1;
        // step q's DMA is complete once at most the operations issued after
        // it are pending: the stores of steps q-2 and q-1 and step q+1's DMA
        wait_vmcnt(stores_prev2 + n_dma_next + stores_prev1);
        barrier_only();
        const uint8_t* la = p_lds_a + stage * kTileBytes;
        const uint8_t* lb = p_lds_b + stage * kTileBytes;
        v8i af[8], bf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) bf[j] = load_frag(lb, wn + 16 * j);
#pragma unroll
        for (int i = 0; i < 8; ++i) af[i] = load_frag(la, wm + 16 * i);
        // every wave has its fragments: the stage is free for step q+2
        barrier_lds();
        const int n_dma_new = issue(d, stage);
        cursor_next(p, d, xcd, slot);
        if (first) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = mfma<FA, FB>(af[i], bf[j], v4f{0.0f, 0.0f, 0.0f, 0.0f});
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = mfma<FA, FB>(af[i], bf[j], acc[i][j]);
        }
        stores_prev2 = stores_prev1;
        stores_prev1 = 0;
        n_dma_next = n_dma_new;
        ++q;
        if (c.kt + 1 >= c.it.kt1) break;
        ++c.kt;
      }
        int stores_now = 0;
        {
            // epilogue of this tile: lane owns columns n0 + wn + 8 (lane%16) + 0..7
            // of rows m0 + wm + 16 i + 4 (lane/16) + r
            const Item& it = c.it;
            // lane constants recomputed here (pinned by an empty asm) rather
            // than kept live across the K loop
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int col = it.n0 + ((tid >> 6) & 1) * 128 + 8 * (tid & 15);
            const int rrow = ((tid >> 7) & 1) * 128 + 4 * ((tid & 63) >> 4);
            if constexpr (OUT == kOutBf16) {
                const float scale = out_scale;
                const __amdgpu_buffer_rsrc_t rs = make_store_rsrc(p.c + (int64_t)it.m0 * p.ldc, (uint32_t)(min(BM, p.m - it.m0) * p.ldc * 2));
                // running max of |bf16| bit patterns: an exponent field of all ones
                // (>= 0x7F80) marks Inf / NaN; outputs outside the matrix hold zeros
                us2 mx = us2{0, 0};
                // offsets are formed here from one base (an empty asm keeps the
                // compiler from hoisting 32 of them out of the loop)
                uint32_t base = col < p.n ? (uint32_t)((rrow * p.ldc + col) * 2) : kOutOfRange;
                asm volatile("" : "+v"(base));
                const uint32_t row_bytes = (uint32_t)(p.ldc * 2);
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t off = base == kOutOfRange ? kOutOfRange : base + (uint32_t)(16 * i + r) * row_bytes;
                        v4u v;
                        v.x = pack_bf16(acc[i][0][r] * scale, acc[i][1][r] * scale);
                        v.y = pack_bf16(acc[i][2][r] * scale, acc[i][3][r] * scale);
                        v.z = pack_bf16(acc[i][4][r] * scale, acc[i][5][r] * scale);
                        v.w = pack_bf16(acc[i][6][r] * scale, acc[i][7][r] * scale);
                        store16(v, off, rs);
                        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, v.x & 0x7FFF7FFFu));
                        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, v.y & 0x7FFF7FFFu));
                        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, v.z & 0x7FFF7FFFu));
                        mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, v.w & 0x7FFF7FFFu));
                        if (r == 3) __builtin_amdgcn_sched_barrier(0);
                    }
                if (mx.x >= 0x7F80u || mx.y >= 0x7F80u) {
                    // rare: count exactly
#pragma unroll
                    for (int i = 0; i < 8; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (it.m0 + rrow + 16 * i + r >= p.m || col >= p.n) continue;
#pragma unroll
                            for (int j = 0; j < 8; ++j)
                                nonfinite += (to_bf16(acc[i][j][r] * scale) & 0x7F80u) == 0x7F80u;
                        }
                }
                stores_now = kStoresBf16;
            } else if constexpr (OUT == kOutF32) {
                float* wsb = p.ws + ((int64_t)it.split * p.m + it.m0) * p.n;
                const __amdgpu_buffer_rsrc_t rs = make_store_rsrc(wsb, (uint32_t)(min(BM, p.m - it.m0) * p.n * 4));
                uint32_t base = col < p.n ? (uint32_t)((rrow * p.n + col) * 4) : kOutOfRange;
                asm volatile("" : "+v"(base));
                const uint32_t row_bytes = (uint32_t)(p.n * 4);
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t off = base == kOutOfRange ? kOutOfRange : base + (uint32_t)(16 * i + r) * row_bytes;
                        // (copy the element to a scalar first: a bit cast of an
                        // ext_vector element expression reads element 0)
                        uint32_t w[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float f = acc[i][j][r];
                            w[j] = __builtin_bit_cast(uint32_t, f);
                        }
                        store16(v4u{w[0], w[1], w[2], w[3]}, off, rs);
                        store16(v4u{w[4], w[5], w[6], w[7]}, off + (off == kOutOfRange ? 0u : 16u), rs);
                        if (r == 3) __builtin_amdgcn_sched_barrier(0);
                    }
                stores_now = kStoresF32;
            } else {
                // any alignment: element stores, then drain
                const float scale = out_scale;
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = it.m0 + rrow + 16 * i + r;
                        if (row >= p.m) continue;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            if (col + j >= p.n) continue;
                            if (p.ws) {
                                p.ws[((int64_t)it.split * p.m + row) * p.n + col + j] = acc[i][j][r];
                            } else {
                                const uint16_t h = to_bf16(acc[i][j][r] * scale);
                                nonfinite += (h & 0x7F80u) == 0x7F80u;
                                p.c[(int64_t)row * p.ldc + col + j] = h;
                            }
                        }
                    }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
        }
        // the epilogue's stores were issued after step q-1's DMA
        stores_prev1 = stores_now;
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
    p.ktiles = (int)((g.k + BK - 1) / BK);
    p.splits = g.splits > 1 && g.ws ? g.splits : 1;
    p.kt_per = (p.ktiles + p.splits - 1) / p.splits;
    p.splits = (p.ktiles + p.kt_per - 1) / p.kt_per;      // no empty split
    p.ws = p.splits > 1 ? g.ws : nullptr;
    p.tiles_m = (int)((g.m + BM - 1) / BM);
    p.tiles_n = (int)((g.n + BN - 1) / BN);
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
        p.fast_store = (g.n % 8 == 0) && ((reinterpret_cast<uintptr_t>(g.ws) & 15u) == 0);
    else
        p.fast_store = (g.n % 8 == 0) && (g.ldc % 8 == 0) && ((reinterpret_cast<uintptr_t>(g.c) & 15u) == 0);
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
