// moe_finalize: y_t = sum_j s_tj * fc2_out[unpermute[t*k + j]] + sum_s fc2_out[P + s*T + t].
//
// The routing weight is applied after FC2 (TensorRT-LLM page "MoE 层前向执行",
// sections "通信与计算融合的方向" and "小结").  A workgroup owns TB consecutive
// tokens (TB chosen per call so that the grid still covers every CU several
// times): it stages their k row indices and weights in LDS, then its threads
// walk the flattened (token, 16-byte column chunk) space of those tokens, UNR
// chunks per thread at a time, so every thread has UNR * (k + 1) row loads in
// flight and no thread idles on a partial pass over one row.  Each output
// chunk accumulates in fp32 in j order, then the shared rows in order, and is
// rounded once; no atomics, so the result is deterministic.  HBM-bound: it
// reads R*H and writes T*H activation values.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

constexpr int kFinTokens = 2;    // tokens per workgroup (at most)
constexpr int kFinThreads = 256;
constexpr int kFinUnroll = 2;    // column chunks per thread in flight

// 8 consecutive values of the FC2 output as raw 16-byte words (bf16: one,
// fp32: two), widened to fp32 only where they are used.  Loaded with the
// non-temporal hint: each FC2 row is read once (measured on MI355X at the
// DeepSeek-V3 prefill shape: 0.235 -> 0.210 ms; 2 or 4 tokens and 1-3 chunks
// per thread, 128-512 threads all within 0.209-0.238 ms).
template <class Tin>
struct Chunk {
    static constexpr int W = sizeof(Tin) / 2;
    u32x4_t w[W];
    __device__ __forceinline__ void load(const Tin* p)
    {
#pragma unroll
        for (int i = 0; i < W; ++i)
            w[i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(p) + 16 * i));
    }
    __device__ __forceinline__ float operator[](int i) const
    {
        if constexpr (W == 1) {
            const uint32_t u = w[0][i >> 1];
            return __uint_as_float((i & 1) ? (u & 0xffff0000u) : (u << 16));
        } else {
            return __uint_as_float(w[i >> 2][i & 3]);
        }
    }
};

template <class Tin, class Tout>
__global__ __launch_bounds__(kFinThreads) void finalize_kernel(const Tin* __restrict__ fc2,
                                                               const int32_t* __restrict__ unpermute,
                                                               const float* __restrict__ scales, int T,
                                                               int k, int H, int n_shared, int tb,
                                                               Tout* __restrict__ y)
{
    __shared__ int s_row[kFinTokens][MOE_MAX_TOPK];
    __shared__ float s_w[kFinTokens][MOE_MAX_TOPK];
    const int t0 = blockIdx.x * tb;
    const int nt = min(tb, T - t0);
    const int P = T * k;
    for (int i = threadIdx.x; i < nt * k; i += kFinThreads) {
        const int tl = i / k, j = i - tl * k;
        const int r = unpermute[(size_t)(t0 + tl) * k + j];
        s_row[tl][j] = r < 0 ? 0 : (r >= P ? P - 1 : r);
        s_w[tl][j] = scales[(size_t)(t0 + tl) * k + j];
    }
    __syncthreads();
    const int nvec = H / 8;
    const int items = nt * nvec;
    for (int base = threadIdx.x; base < items; base += kFinThreads * kFinUnroll) {
        Chunk<Tin> v[kFinUnroll][MOE_MAX_TOPK];
        Chunk<Tin> sv[kFinUnroll];
        int tl[kFinUnroll], c[kFinUnroll];
        bool ok[kFinUnroll];
#pragma unroll
        for (int u = 0; u < kFinUnroll; ++u) {
            const int it = base + u * kFinThreads;
            ok[u] = it < items;
            tl[u] = ok[u] ? it / nvec : 0;
            c[u] = ok[u] ? it - tl[u] * nvec : 0;
        }
        // all loads of the UNR chunks first: k routed rows and the first shared row
#pragma unroll
        for (int u = 0; u < kFinUnroll; ++u) {
            if (!ok[u]) continue;
#pragma unroll
            for (int j = 0; j < MOE_MAX_TOPK; ++j)
                if (j < k) v[u][j].load(fc2 + (size_t)s_row[tl[u]][j] * H + c[u] * 8);
            if (n_shared > 0) sv[u].load(fc2 + ((size_t)P + t0 + tl[u]) * H + c[u] * 8);
        }
#pragma unroll
        for (int u = 0; u < kFinUnroll; ++u) {
            if (!ok[u]) continue;
            const int t = t0 + tl[u];
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < MOE_MAX_TOPK; ++j) {
                if (j < k) {
                    const float wj = s_w[tl[u]][j];
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[i] += wj * v[u][j][i];
                }
            }
            if (n_shared > 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += sv[u][i];
            }
            for (int s = 1; s < n_shared; ++s) {
                Chunk<Tin> w8;
                w8.load(fc2 + ((size_t)P + (size_t)s * T + t) * H + c[u] * 8);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] += w8[i];
            }
            store8_f32(y + (size_t)t * H + c[u] * 8, acc);
        }
    }
}

template <class Tin, class Tout>
void launch_one(const void* fc2, const int32_t* unpermute, const float* scales, int T, int k,
                int H, int n_shared, void* y, hipStream_t s)
{
    // up to kFinTokens tokens per workgroup, fewer when T would leave CUs idle
    const int tb = std::max(1, std::min(kFinTokens, T / (4 * device_cu_count())));
    TimedLaunch tl(MOE_KID_FINALIZE, s);
    const unsigned grid = (unsigned)((T + tb - 1) / tb);
    hipLaunchKernelGGL((finalize_kernel<Tin, Tout>), dim3(grid), dim3(kFinThreads), 0, s,
                       static_cast<const Tin*>(fc2), unpermute, scales, T, k, H, n_shared, tb,
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
