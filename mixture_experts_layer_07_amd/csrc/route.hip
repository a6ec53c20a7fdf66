// moe_route kernel: one 64-lane wavefront per token.
//
// Methods (TensorRT-LLM page "MoE 层前向执行", sections "路由方法枚举" and
// "DeepSeek-V3 的 noaux_tc"; vLLM page, section "FusedTopKRouter"):
//   Default            softmax over all E, keep top-k (optionally renormalised)
//   Renormalize        top-k, then softmax over the k kept logits
//   RenormalizeNaive   softmax, top-k, renormalise (same values as above)
//   DeepSeekV3         sigmoid scores; bias added for selection only; group
//                      score = sum of the group's two best biased keys; keep
//                      topk_group groups; top-k experts among them; weights
//                      = unbiased sigmoid / (sum + 1e-20) * scaling.
//   Llama4             top-k logits, each weighted by its own sigmoid
//   MiniMax2           sigmoid + bias for selection, top-k, unbiased sigmoids
//                      renormalised (DeepSeekV3 with one group, no 1e-20)
//   SigmoidRenorm      sigmoid, top-k, renormalise
//
// Layout: lane l owns experts l, l+64, l+128, l+192 (E <= 256).  Each of the
// k selection rounds takes the wave maximum of the order-preserving fp32 key
// bits (DPP steps within the wave, no LDS round trips), then the lowest expert
// index holding that key from four ballots (index = 64 * slot + lane, slots
// checked in order); k rounds give the ids in selection order.  Group scores
// and group ranks go through LDS.
#include <math.h>

#include "common.h"

namespace moe {
namespace {

constexpr int kWaves = 4;  // tokens per 256-thread block

__device__ __forceinline__ uint32_t ordered_bits(float v)
{
    v = v + 0.0f;  // -0 and +0 compare equal: make them the same key
    uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// max(v, v of the lane that DPP control `ctrl` names); rows outside
// `row_mask` and lanes without a source keep v
template <int ctrl, int row_mask>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v)
{
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, ctrl, row_mask, 0xf, false);
    return o > v ? o : v;
}

// Maximum over the 64 lanes (all active), the same in every lane: pairs and
// quads, half-rows and rows of 16 by lane permutations, then rows 0..3
// folded into lane 63 by the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = dpp_max<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
    v = dpp_max<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
    v = dpp_max<0x141, 0xf>(v);  // row_half_mirror
    v = dpp_max<0x140, 0xf>(v);  // row_mirror
    v = dpp_max<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// (a1 >= a2) := the two largest of (a1, a2) and the pair held by the lane
// that DPP control `ctrl` names (all lanes active; no NaN in either pair).
template <int ctrl>
__device__ __forceinline__ void dpp_top2(float& a1, float& a2)
{
    const float c1 = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(a1), __float_as_int(a1),
                                                                ctrl, 0xf, 0xf, false));
    const float c2 = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(a2), __float_as_int(a2),
                                                                ctrl, 0xf, 0xf, false));
    const float lo = c1 > a1 ? a1 : c1;
    const float hi2 = c2 > a2 ? c2 : a2;
    a1 = c1 > a1 ? c1 : a1;
    a2 = lo > hi2 ? lo : hi2;
}

// Running top-2 of a group's keys (selects, not branches, so that the pair
// stays in registers); NaN keys never enter.
__device__ __forceinline__ void top2_add(float v, float& b1, float& b2)
{
    const bool above1 = v > b1, above2 = v > b2;
    b2 = above1 ? b1 : (above2 ? v : b2);
    b1 = above1 ? v : b1;
}

// fl32 of the fp64 sigmoid: the fp32 key both sides of a parity check agree on.
__device__ __forceinline__ float sigmoid_key(float l)
{
#pragma clang fp contract(off)
    double d = 1.0 / (1.0 + exp(-(double)l));
    return (float)d;
}

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int method, int k, int n_group,
                                                    int topk_group,
                                                    const float* __restrict__ bias,
                                                    float scaling, unsigned flags,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ scales)
{
#pragma clang fp contract(off)
    __shared__ float s_sig[kWaves][256];
    __shared__ float s_key[kWaves][256];
    __shared__ float s_gs[kWaves][128];
    __shared__ int s_gsel[kWaves][128];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kWaves + wave;
    const bool active = t < T;
    const bool dsv3 = method == MOE_ROUTE_DEEPSEEKV3;
    // sigmoid-scored methods select on fl32(sigmoid) (+ bias)
    const bool sigm = dsv3 || method == MOE_ROUTE_MINIMAX2 || method == MOE_ROUTE_SIGMOID_RENORM;

    float logit[4], key[4];
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        valid[i] = active && e < E;
        logit[i] = valid[i] ? logits[(size_t)t * E + e] : 0.0f;
        key[i] = logit[i];
    }

    if (sigm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (valid[i]) {
                const float sg = sigmoid_key(logit[i]);
                key[i] = bias ? sg + bias[e] : sg;  // one fp32 add (bias given: DSV3, MiniMax2)
                s_sig[wave][e] = sg;
                s_key[wave][e] = key[i];
            }
        }
        if (!dsv3) {
            // The weights below read s_sig entries that other lanes of this
            // wave stored (DeepSeek-V3 reaches them through __syncthreads).
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        }
    }
    if (dsv3) {
        const int gsz = E / n_group;
        __syncthreads();
        // group score: sum of the two largest biased keys of the group (one
        // fp32 add of the same two values whichever lanes find them).  With
        // n_group a power of two and at most 16 lanes per group, the group's
        // `parts` consecutive lanes each scan a slice and merge their top-2
        // pairs by DPP steps within aligned blocks of 2, 4, 8, 16 lanes;
        // otherwise one lane scans each group.
        const int parts = n_group <= 64 ? 64 / n_group : 0;
        const bool split = parts >= 1 && parts <= 16 && (n_group & (n_group - 1)) == 0 &&
                           gsz % parts == 0;
        if (active && split) {
            const int g = lane / parts, len = gsz / parts;
            const float* src = &s_key[wave][g * gsz + (lane % parts) * len];
            float b1 = -INFINITY, b2 = -INFINITY;
            for (int i = 0; i < len; ++i) top2_add(src[i], b1, b2);
            if (parts >= 2) dpp_top2<0xb1>(b1, b2);   // quad_perm [1,0,3,2]
            if (parts >= 4) dpp_top2<0x4e>(b1, b2);   // quad_perm [2,3,0,1]
            if (parts >= 8) dpp_top2<0x141>(b1, b2);  // row_half_mirror
            if (parts >= 16) dpp_top2<0x140>(b1, b2); // row_mirror
            if (lane % parts == 0) s_gs[wave][g] = b1 + b2;
        } else if (active) {
            for (int g = lane; g < n_group; g += 64) {
                float b1 = -INFINITY, b2 = -INFINITY;
                for (int i = 0; i < gsz; ++i) top2_add(s_key[wave][g * gsz + i], b1, b2);
                s_gs[wave][g] = b1 + b2;
            }
        }
        __syncthreads();
        // a group is kept when fewer than topk_group groups beat it
        if (active) {
            for (int g = lane; g < n_group; g += 64) {
                const float gs = s_gs[wave][g];
                int rank = 0;
                for (int o = 0; o < n_group; ++o) {
                    const float v = s_gs[wave][o];
                    rank += (v > gs) || (v == gs && o < g);
                }
                s_gsel[wave][g] = rank < topk_group;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (valid[i]) valid[i] = s_gsel[wave][e / gsz] != 0;
        }
    }
    if (!active) return;  // no block-wide barrier below this point

    uint32_t kb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kb[i] = ordered_bits(key[i]);

    int sel_id[MOE_MAX_TOPK];
    float sel_key[MOE_MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        sel_id[j] = 0;
        sel_key[j] = 0.0f;
        if (j < k) {
            // invalid candidates enter the maximum as 0, at or below every
            // valid key, and never win a ballot
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) m = (valid[i] && kb[i] > m) ? kb[i] : m;
            m = wave_max_u32(m);
            int e = 0;  // no valid candidate left: expert 0 (cannot happen after validation)
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                const uint64_t b = __ballot(valid[i] && kb[i] == m);
                if (b) e = 64 * i + __ffsll((unsigned long long)b) - 1;
            }
            sel_id[j] = e;
            sel_key[j] = from_ordered_bits(m);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (64 * i + lane == e) valid[i] = false;
        }
    }

    // weights, in fp64, rounded once
    double w[MOE_MAX_TOPK];
    double wsum = 0.0;
    if (sigm) {
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j) {
            w[j] = (j < k) ? (double)s_sig[wave][sel_id[j]] : 0.0;
            wsum += w[j];
        }
        if (dsv3) wsum += 1e-20;
    } else if (method == MOE_ROUTE_LLAMA4) {
        // the kept logits' own sigmoids, not renormalised
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j)
            w[j] = (j < k) ? 1.0 / (1.0 + exp(-(double)sel_key[j])) : 0.0;
        wsum = 1.0;
    } else {
        const double m = (double)sel_key[0];
#pragma unroll
        for (int j = 0; j < MOE_MAX_TOPK; ++j) {
            w[j] = (j < k) ? exp((double)sel_key[j] - m) : 0.0;
            wsum += w[j];
        }
        const bool renorm = method != MOE_ROUTE_DEFAULT || (flags & MOE_ROUTE_FLAG_RENORMALIZE);
        if (!renorm) {
            // plain softmax probability: divide by the sum over all E experts
            double z = 0.0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (lane + 64 * i < E) z += exp((double)logit[i] - m);
            wsum = wave_sum_f64(z);
        }
    }
    const double sc = (double)scaling;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (j < k && lane == j) {
            ids[(size_t)t * k + j] = sel_id[j];
            scales[(size_t)t * k + j] = (float)(w[j] / wsum * sc);
        }
    }
}

}  // namespace

moe_status launch_route(const float* logits, int T, int E, int method, int k, int n_group,
                        int topk_group, const float* bias, float scaling, unsigned flags,
                        int32_t* ids, float* scales, hipStream_t s)
{
    const int blocks = (T + kWaves - 1) / kWaves;
    {
        TimedLaunch tl(MOE_KID_ROUTE, s);
        hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(256), 0, s, logits, T, E, method, k,
                           n_group, topk_group, bias, scaling, flags, ids, scales);
    }
    return launch_status("route_kernel");
}

}  // namespace moe
