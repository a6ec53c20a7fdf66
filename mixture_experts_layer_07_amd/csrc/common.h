// Internal helpers shared by the gfx950 kernels of libmoe (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Storage types.  bf16 and fp8 values travel as raw bits.
using bf16_t = uint16_t;
using fp8_t = uint8_t;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// Two fp32 -> two bf16 packed (a in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950 (checked on the part against the rounding
// above for every bf16 value, its midpoints and neighbours, subnormals
// included, and 2^20 random bit patterns).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ float bf16_to_f32(bf16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

template <class T> struct dtype_of;
template <> struct dtype_of<float> { static constexpr int value = MOE_F32; };
template <> struct dtype_of<bf16_t> { static constexpr int value = MOE_BF16; };
template <> struct dtype_of<fp8_t> { static constexpr int value = MOE_FP8_E4M3; };

// Load 8 consecutive elements (bf16 or fp32 storage) as fp32.
__device__ __forceinline__ void load8_f32(const bf16_t* p, float v[8])
{
    uint4 q = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ void load8_f32(const float* p, float v[8])
{
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store8_f32(bf16_t* p, const float v[8])
{
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void store8_f32(float* p, const float v[8])
{
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Four fp32 values -> four OCP e4m3fn codes of v / s (one IEEE division
// each), round to nearest even, packed little-endian; s == 0 gives zeros.
// The conversion instruction turns magnitudes above 464 into NaN, so the
// quotient is clamped to +-448 first, which is exactly saturation (448 is the
// largest finite value and everything in [448, 464) rounds to it anyway).
__device__ __forceinline__ uint32_t fp8x4_code(const float (&v)[4], float s)
{
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (s == 0.0f) ? 0.0f : fminf(fmaxf(v[i] / s, -448.0f), 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
    return (uint32_t)w;
}

// ------------------------------------------------------------ host side
// Brackets one launch with a pair of events while timing is enabled; the
// pair joins the pending list only once both are recorded.
struct TimedLaunch {
    TimedLaunch(int kid, hipStream_t s);
    ~TimedLaunch();
    int kid_;
    hipStream_t s_;
    hipEvent_t a_ = nullptr, b_ = nullptr;
};

int device_cu_count();                        // CUs of the current device
moe_status set_error(moe_status st, const char* fmt, ...);
moe_status launch_status(const char* what);   // checks hipGetLastError()

// Launchers (one per source file).  Arguments are already validated.
moe_status launch_route(const float* logits, int T, int E, int method, int k, int n_group,
                        int topk_group, const float* bias, float scaling, unsigned flags,
                        int32_t* ids, float* scales, hipStream_t s);
size_t permute_scratch_bytes(int T, int k, int E);
moe_status launch_permute(const int32_t* ids, int T, int k, int E, int n_shared,
                          int32_t* offsets, int32_t* permuted_pair, int32_t* unpermute,
                          void* ws, hipStream_t s);
size_t ffn_scratch_bytes(int T, int k, int n_shared, int I, int act);
moe_status launch_ffn(const void* x, int act, int T, int H, int I, int k, int E, int n_shared,
                      const int32_t* offsets, const int32_t* permuted_pair, const void* w13,
                      const void* w2, int wdt, const float* w13_scale, const float* w2_scale,
                      void* fc2_out, void* ws, hipStream_t s);
size_t ffn_fp8_scratch_bytes(int T, int k, int n_shared, int I);
moe_status launch_ffn_fp8(const uint8_t* xq, const float* x_scale, int T, int H, int I, int k, int E,
                          int n_shared, const int32_t* offsets, const int32_t* permuted_pair,
                          const uint8_t* w13, const uint8_t* w2, const float* w13_scale,
                          const float* w2_scale, void* fc2_out, void* ws, hipStream_t s);
moe_status launch_ffn_fused(const void* x, const float* x_scale, int act, int T, int H, int I, int k,
                            int E, int n_shared, const int32_t* offsets, const int32_t* permuted_pair,
                            const void* w13, const void* w2, int wdt, const float* w13_scale,
                            const float* w2_scale, int split, void* fc2_out, hipStream_t s);
// Device address of this GPU's copy of the static scratch behind
// moe_expert_ffn_noalloc (MOE_NOALLOC_SCRATCH_BYTES), resolved once per
// device; null with the error set if the lookup fails.
void* noalloc_scratch();
moe_status launch_quantize_fp8(const void* x, int dt, int rows, int cols, uint8_t* q, float* scale,
                               hipStream_t s);
moe_status launch_finalize(const void* fc2_out, int dt, const int32_t* unpermute,
                           const float* scales, int T, int k, int H, int n_shared, void* y,
                           int ydt, hipStream_t s);

}  // namespace moe
