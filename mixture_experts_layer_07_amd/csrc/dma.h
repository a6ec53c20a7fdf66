// Device helpers of the direct-to-LDS tile engines (the two-call grouped
// GEMMs and the fused FC1+FC2 kernel): LDS DMA transfers, explicit wait
// counts, LDS-only barriers, swizzled LDS addressing and the MFMA forms.
#pragma once

#include "common.h"

namespace moe {
namespace {

constexpr int kMaxGroups = MOE_MAX_EXPERTS + 64;

// One 16x16 result block from a 16-row fragment pair (K-contiguous rows of
// each operand): lane l gets rows 4*(l/16) + i (i < 4) of column l%16, rows
// indexing the first operand's fragment and columns the second's.
__device__ __forceinline__ f32x4_t mfma_frag(u32x4_t a, u32x4_t b, f32x4_t c, bf16_t)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Byte offset of logical 16-byte chunk kc of a staged 128-byte row: chunk
// kc ^ (row & 7), measured free of bank conflicts on gfx950 for the fragment
// reads (16 rows x 4 chunks per ds_read_b128) and for the 1 KB DMA writes.
__device__ __forceinline__ int dma_off(int row, int kc) { return row * 128 + ((kc ^ (row & 7)) << 4); }

// Same for a 64-byte fp8 weight row: chunk kc ^ ((row >> 2) & 3), so that the
// 8-byte fragment reads of 16 consecutive rows spread over all banks.
__device__ __forceinline__ int dma_off_w8(int row, int kc) { return row * 64 + ((kc ^ ((row >> 2) & 3)) << 4); }

// Eight e4m3 codes -> eight bf16 (exact), two per conversion: the scale
// operand of this conversion acts through its exponent only, so 1.0.
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(uint32_t w0, uint32_t w1)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return u32x4_t{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                   __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
}

// vmcnt <= n for a wave-uniform runtime n in [0, MAX]
template <int MAX>
__device__ __forceinline__ void wait_vmcnt_le(int n);

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MAX>
__device__ __forceinline__ void wait_vmcnt_le(int n)
{
    if constexpr (MAX > 0) {
        if (n < MAX) { wait_vmcnt_le<MAX - 1>(n); return; }
    }
    wait_vmcnt<MAX>();
}

// One 16-byte-per-lane global->LDS transfer into the 1 KB at LDS byte address
// `lds_addr` (wave-uniform), from `base` (wave-uniform, scalar registers) plus
// a 32-bit per-lane byte offset.  Written as inline asm on purpose: the compiler's
// own tracking of LDS DMA inserts a full vmcnt(0) wait before every later LDS
// read, which would drain the ring each slice; the kernel instead waits for
// exactly the stage it needs (wait_vmcnt) before the barrier that publishes it.
// M0 is reserved by the compiler and used by nothing else in this kernel.
__device__ __forceinline__ void dma16(unsigned lds_addr, const char* base, uint32_t off)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_addr), "v"(off), "s"(base) : "memory", "m0");
}

// Same with 4 bytes per lane: lane l lands at byte 4*l of the 256 bytes at
// `lds_addr`.
__device__ __forceinline__ void dma4(unsigned lds_addr, const char* base, uint32_t off)
{
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(lds_addr), "v"(off), "s"(base) : "memory", "m0");
}

// A pointer that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ const char* uniform_ptr(const char* p)
{
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// 16x16x128 MFMA on e4m3 codes (format 0 for both operands); its per-lane
// power-of-two block-scale operands are left at 2^0 (E8M0 code 127).
__device__ __forceinline__ f32x4_t mfma_fp8(const i32x8_t& a, const i32x8_t& b)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                            127, 0, 127);
}

// Lane group g's 32 fp8 codes of one row of a staged 128-byte K block: logical
// chunks g and g+4 (K bytes [16g, 16g+16) and [64+16g, 64+16g+16)).  The MFMA
// sums over the whole block, so any assignment of K positions to lane groups
// is valid when both operands use the same one; with this one every
// ds_read_b128 has the lane groups on four consecutive chunks, the pattern of
// the bf16 fragment reads, which is free of bank conflicts on gfx950.
// (Chunks 2g and 2g+1 measured 1.1e9 conflict cycles in the fp8 x fp8
// DeepSeek-V3 prefill FC1.)
__device__ __forceinline__ i32x8_t lds_row32(const char* base, int row, int g)
{
    const u32x4_t x0 = *reinterpret_cast<const u32x4_t*>(base + dma_off(row, g));
    const u32x4_t x1 = *reinterpret_cast<const u32x4_t*>(base + dma_off(row, g + 4));
    return i32x8_t{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
}

// Barrier that orders LDS only (s_waitcnt lgkmcnt(0) + s_barrier): unlike
// __syncthreads() it does not wait for the DMA loads still in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace
}  // namespace moe
