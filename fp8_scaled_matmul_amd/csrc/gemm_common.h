// Pieces shared by the GEMM kernels: operand tile geometry, the LDS swizzle,
// the FP8 MFMA, LDS fragment reads, and the buffer-descriptor based memory
// operations (DMA into LDS, 16-byte stores) issued from inline assembly so
// that the kernels, not the compiler, decide when to wait for them.
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace fp8mi {
namespace gemm {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kTileBytes = BM * BK;     // 32 KB: one operand tile of one K step
constexpr uint32_t kOutOfRange = 0x80000000u;

// 16-byte chunk c (0..7) of the 128-byte LDS row r lives at chunk position
// swz(r, c) = c ^ f(r), f(r) = (r2, r1, r3) as bits 0..2.  A fragment read
// (lanes 0..15 rows 16 i + 0..15 at chunk c, lanes 16..31 at chunk c + 2, and
// so on) then places the 16 lanes of each quarter wave in 16 distinct
// 16-byte slots of a 256-byte line, and the 32 lanes of each half wave in 32
// distinct slots of a 512-byte line.  Measured on gfx950 with ds_read_b128:
// full LDS rate (about 256 bytes per clock per CU), where the earlier
// f(r) = (r1, r2, r3 ^ r0) pattern, distinct only within quarter waves, ran at
// half rate.  The row fills write 1 KB contiguous runs.  An involution.
__device__ inline int swz(int r, int c) { return c ^ (((r >> 2) & 1) | (r & 2) | ((r >> 1) & 4)); }

template <int FA, int FB>
__device__ inline v4f mfma(const v8i& a, const v8i& b, const v4f& c)
{
    // FA / FB: 0 = E4M3, 1 = E5M2.  Zero scale operands select the unscaled
    // v_mfma_f32_16x16x128_f8f6f4 (8 bytes), not the scaled form, which is
    // issued as a v_mfma_ld_scale_b32 prefix plus the MFMA.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

// MFMA operand fragment for LDS rows row0..row0+15 of a staged tile: lane l
// reads row row0 + l%16, K bytes 32 (l/16) .. +32.  A and B use the same K
// assignment, so the products pair up element for element whatever order
// the hardware gives the 128 K values inside one instruction.
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

__device__ inline uint16_t to_bf16(float v) { return __builtin_bit_cast(uint16_t, __float2bfloat16(v)); }

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two fp32 values to a word of two bf16 (round to nearest even), one
// v_cvt_pk_bf16_f32.
__device__ inline uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

// Raw buffer descriptor (stride 0, byte-addressed, range-checked against
// `bytes`): out-of-range loads return zero, out-of-range stores are dropped.
__device__ inline v4u make_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    v4u r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu);
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = 0x00020000u;
    return r;
}

__device__ inline uint32_t lds_addr(const void* p)
{
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p));
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 64 lanes x 16 bytes from the buffer into LDS [lds, lds + 1024): lane l's
// bytes land at lds + 16 l.  Counted by vmcnt only; the caller waits.  A
// write of M0 needs one wait state before an LDS DMA reads it.
__device__ inline void dma16(uint32_t lds, uint32_t voff, const v4u& rsrc)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// 64 lanes x 4 bytes into LDS [lds, lds + 256).
__device__ inline void dma4(uint32_t lds, uint32_t voff, const v4u& rsrc)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Descriptor for the compiler's buffer builtins (same fields as make_rsrc).
__device__ inline __amdgpu_buffer_rsrc_t make_store_rsrc(void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

// 16-byte store through a range-checked descriptor (dropped when out of
// range).  Issued through the compiler so that its hazard checks cover the
// VALU writes of the data registers; exactly one buffer_store_dwordx4.
__device__ inline void store16(const v4u& data, uint32_t voff, __amdgpu_buffer_rsrc_t rsrc)
{
    __builtin_amdgcn_raw_buffer_store_b128(data, rsrc, (int)voff, 0, 0);
}

// Workgroup barrier without the memory fences of __syncthreads() (which
// would also wait for every outstanding vector memory operation, including
// the DMA of later steps and the output stores).  The caller has waited for
// what the other waves must see.
__device__ inline void barrier_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ inline void barrier_only()
{
    asm volatile("s_barrier" ::: "memory");
}

// s_waitcnt vmcnt(n) for a run-time n (the instruction needs an immediate):
// waits until at most n of this wave's vector memory operations are pending.
__device__ inline void wait_vmcnt(int n)
{
    n = __builtin_amdgcn_readfirstlane(n);   // uniform: scalar branches only
    if (n >= 63) {
        asm volatile("s_waitcnt vmcnt(63)" ::: "memory");
        return;
    }
    switch (n >> 3) {   // round down to a multiple of 8 (waits at least as long)
    case 7: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
}

}  // namespace gemm
}  // namespace fp8mi
