// moe_finalize: y_t = sum_j s_tj * fc2_out[unpermute[t*k + j]] + sum_s fc2_out[P + s*T + t].
//
// The routing weight is applied after FC2 (TensorRT-LLM page "MoE 层前向执行",
// sections "通信与计算融合的方向" and "小结").  One workgroup per token gathers
// its k rows (16-byte vectors, all k loads in flight together), accumulates in
// fp32 in j order and rounds once; no atomics, so the result is deterministic.
#include "common.h"

namespace moe {
namespace {

template <class Tin, class Tout>
__global__ __launch_bounds__(256) void finalize_kernel(const Tin* __restrict__ fc2,
                                                       const int32_t* __restrict__ unpermute,
                                                       const float* __restrict__ scales, int T,
                                                       int k, int H, int n_shared,
                                                       Tout* __restrict__ y)
{
    __shared__ int s_row[MOE_MAX_TOPK];
    __shared__ float s_w[MOE_MAX_TOPK];
    const int t = blockIdx.x;
    const int P = T * k;
    if (threadIdx.x < k) {
        int r = unpermute[(size_t)t * k + threadIdx.x];
        s_row[threadIdx.x] = r < 0 ? 0 : (r >= P ? P - 1 : r);
        s_w[threadIdx.x] = scales[(size_t)t * k + threadIdx.x];
    }
    __syncthreads();
    const int nvec = H / 8;
    for (int c = threadIdx.x; c < nvec; c += blockDim.x) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float v[MOE_MAX_TOPK][8];
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j)
            if (j < k) load8_f32(fc2 + (size_t)s_row[j] * H + c * 8, v[j]);
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j) {
            if (j < k) {
                const float wj = s_w[j];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += wj * v[j][i];
            }
        }
        for (int s = 0; s < n_shared; ++s) {
            float sv[8];
            load8_f32(fc2 + ((size_t)P + (size_t)s * T + t) * H + c * 8, sv);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += sv[i];
        }
        store8_f32(y + (size_t)t * H + c * 8, acc);
    }
}

template <class Tin, class Tout>
void launch_one(const void* fc2, const int32_t* unpermute, const float* scales, int T, int k,
                int H, int n_shared, void* y, hipStream_t s)
{
    TimedLaunch tl(MOE_KID_FINALIZE, s);
    hipLaunchKernelGGL((finalize_kernel<Tin, Tout>), dim3(T), dim3(256), 0, s,
                       static_cast<const Tin*>(fc2), unpermute, scales, T, k, H, n_shared,
                       static_cast<Tout*>(y));
}

}  // namespace

moe_status launch_finalize(const void* fc2_out, int dt, const int32_t* unpermute,
                           const float* scales, int T, int k, int H, int n_shared, void* y,
                           int ydt, hipStream_t s)
{
    if (dt == MOE_BF16 && ydt == MOE_BF16)
        launch_one<bf16_t, bf16_t>(fc2_out, unpermute, scales, T, k, H, n_shared, y, s);
    else if (dt == MOE_BF16 && ydt == MOE_F32)
        launch_one<bf16_t, float>(fc2_out, unpermute, scales, T, k, H, n_shared, y, s);
    else if (dt == MOE_F32 && ydt == MOE_BF16)
        launch_one<float, bf16_t>(fc2_out, unpermute, scales, T, k, H, n_shared, y, s);
    else
        launch_one<float, float>(fc2_out, unpermute, scales, T, k, H, n_shared, y, s);
    return launch_status("finalize_kernel");
}

}  // namespace moe
