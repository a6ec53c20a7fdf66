// moe_quantize_fp8: the quantise-input step that runs before the MoE GEMMs
// ("TensorRT-LLM 源码完全拆解(十三)", sections "MoEScheduler:两条执行路径,两套相反
// 的约定" and "“自适应顺序”里的一个细节"), in the block form of the fp8 fused MoE
// on the vLLM page ("量化与 MoE Kernel 选择", after DeepSeek-V3's fp8 scheme):
// each row is cut into blocks of 128 consecutive values, a block's scale is
// s = fl32(amax / 448) and its codes are e4m3fn(fl32(v / s)), rounded to
// nearest even and saturating; a block with s == 0 encodes as zeros.
//
// HBM-bound (2 bytes read, 1 + 1/32 written per bf16 value).  One wave covers
// four consecutive blocks per step: 16 lanes per block, 8 values (16 bytes of
// bf16) per lane, the block maximum by four xor-shuffles inside the 16 lanes,
// then 8 codes (one 8-byte store) per lane and one scale per block.  Blocks of
// a row are consecutive in memory, so block b starts at element 128 b.
#include "common.h"

namespace moe {
namespace {

template <class T>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* __restrict__ x, long nblocks,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ scale)
{
    const int lane = threadIdx.x & 63;
    const long wave = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const long nwaves = ((long)gridDim.x * blockDim.x) >> 6;
    for (long b4 = wave * 4; b4 < nblocks; b4 += nwaves * 4) {
        const long blk = b4 + (lane >> 4);
        const bool ok = blk < nblocks;
        const size_t e0 = (size_t)blk * 128 + (size_t)(lane & 15) * 8;
        float v[8];
        if (ok) {
            load8_f32(x + e0, v);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.0f;
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
        const float s = amax / 448.0f;
        if (ok) {
            const float lo[4] = {v[0], v[1], v[2], v[3]};
            const float hi[4] = {v[4], v[5], v[6], v[7]};
            typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2_t*>(q + e0) = u32x2_t{fp8x4_code(lo, s), fp8x4_code(hi, s)};
            if ((lane & 15) == 0) scale[blk] = s;
        }
    }
}

}  // namespace

moe_status launch_quantize_fp8(const void* x, int dt, int rows, int cols, uint8_t* q, float* scale,
                               hipStream_t s)
{
    const long nblocks = (long)rows * (cols / 128);
    const long waves = (nblocks + 3) / 4;
    long grid = (waves + 3) / 4;
    const long cap = (long)device_cu_count() * 8;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    {
        TimedLaunch tl(MOE_KID_QUANT, s);
        if (dt == MOE_BF16)
            hipLaunchKernelGGL(quantize_fp8_kernel<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                               static_cast<const bf16_t*>(x), nblocks, q, scale);
        else
            hipLaunchKernelGGL(quantize_fp8_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s,
                               static_cast<const float*>(x), nblocks, q, scale);
    }
    return launch_status("quantize_fp8_kernel");
}

}  // namespace moe
