/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward.
 *
 * The layer computes, for every token t with activation x_t,
 *     y_t = sum_{i in TopK(x_t)} g_i(x_t) * E_i(x_t)   (+ shared experts)
 * ("TensorRT-LLM 源码完全拆解(十三): MoE 层前向执行", section "MoE 在推理侧到底特殊在
 * 哪里"), as four asynchronous calls on one HIP stream:
 *
 *   moe_route      router logits -> (expert ids int32 [T,k], scales fp32 [T,k])
 *   moe_permute    counting sort of the T*k (token, expert) pairs into
 *                  contiguous per-expert row blocks + offsets
 *   moe_expert_ffn grouped GEMM FC1 with fused SwiGLU, then grouped GEMM FC2
 *   moe_finalize   weighted gather-sum of each token's k FFN rows (+ shared)
 *
 * With fp8 activations the FFN step is moe_quantize_fp8 (of x) followed by
 * moe_expert_ffn_fp8; route, permute and finalize are unchanged.  The FFN step
 * can also run as one kernel that keeps h on chip (moe_expert_ffn_fused,
 * moe_expert_ffn_fp8_fused; same results, no workspace).
 *
 * Conventions shared by every call:
 *  - Pointers named as device buffers are device pointers (hipMalloc'd or
 *    torch CUDA tensors); scalars are passed by value.  All arrays are dense,
 *    row-major, contiguous.
 *  - The caller owns and allocates every buffer, including the workspace
 *    (sized by moe_workspace_size); the library never allocates device
 *    memory on these paths.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    kernels and return; nothing synchronises the device and no value is read
 *    back to the host, so the sequence can be captured into a HIP graph.
 *  - Argument errors are detected on the host before anything is launched and
 *    returned as a status; moe_last_error() then gives the reason.  A failed
 *    kernel launch returns MOE_ERR_DEVICE.  There is no fallback path: shapes
 *    outside the kernels' limits return MOE_ERR_UNSUPPORTED (the pages'
 *    position: a fused kernel has hard shape limits and the caller must be
 *    told, section "融合算子与回退阈值").
 *  - T == 0 is valid: the call returns MOE_OK and launches nothing.
 *  - Not thread-safe per stream: calls that overlap on one stream or share a
 *    workspace race.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* inconsistent sizes, null required pointer, bad enum */
    MOE_ERR_UNSUPPORTED = 2, /* valid request outside the kernels' limits */
    MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than moe_workspace_size */
    MOE_ERR_DEVICE = 4       /* a HIP call or kernel launch failed */
} moe_status;

/* Routing methods, numbered as the RoutingMethodType enum on the TensorRT-LLM
 * page (section "路由方法枚举"). */
typedef enum moe_route_method {
    MOE_ROUTE_DEFAULT = 0,           /* softmax over all E -> top-k          */
    MOE_ROUTE_RENORMALIZE = 1,       /* top-k -> softmax over the k kept     */
    MOE_ROUTE_DEEPSEEKV3 = 2,        /* noaux_tc grouped sigmoid routing     */
    MOE_ROUTE_LLAMA4 = 3,            /* top-k logits -> own sigmoid each     */
    MOE_ROUTE_RENORMALIZE_NAIVE = 4, /* softmax -> top-k -> renormalise      */
    MOE_ROUTE_MINIMAX2 = 5,          /* sigmoid + bias -> top-k -> renormalise
                                        the unbiased sigmoids                 */
    MOE_ROUTE_SIGMOID_RENORM = 6     /* sigmoid -> top-k -> renormalise      */
} moe_route_method;
/* 7 (DeepSeek-V4) and 8 (unspecified) are listed by the enum but not defined
 * on the pages: MOE_ERR_UNSUPPORTED. */

/* Honoured by MOE_ROUTE_DEFAULT only: divide the k kept probabilities by their
 * sum (the renormalize switch of vLLM's FusedTopKRouter). */
#define MOE_ROUTE_FLAG_RENORMALIZE 1u

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Shape limits of the kernels (the expert-count and top-k limits of the fused
 * routing kernel on the TensorRT-LLM page, section "融合算子与回退阈值"; its
 * 32-expert group-size limit does not apply here: groups go through LDS). */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8
/* Largest intermediate size of the fused FC1+FC2 kernels (h of a 16-row tile
 * is kept in LDS). */
#define MOE_FUSED_MAX_I 2048
/* Bytes of the library's static device scratch used by moe_expert_ffn_noalloc
 * (64 MiB per GPU the library runs on, held until the process ends). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * moe_route -- per-token expert selection and weights.
 * TensorRT-LLM page, sections "路由方法枚举" and "DeepSeek-V3 的 noaux_tc";
 * vLLM page ("vLLM 源码完全拆解(八)"), section "FusedTopKRouter".
 *
 *  logits   device fp32 [T, E]   router scores.
 *  method   moe_route_method.
 *  k        experts per token, 1 <= k <= min(E, 8).
 *  n_group, topk_group   DeepSeek-V3 only: E is split into n_group equal
 *           groups of E/n_group >= 2 experts; a group scores the sum of its
 *           two largest biased keys; the topk_group best groups are kept and
 *           the k experts are chosen among them (k <= topk_group * E/n_group).
 *           Ignored by the other methods.
 *  bias     device fp32 [E] or NULL (= zeros); DeepSeek-V3 and MiniMax2 only:
 *           added to the sigmoid scores for selection, never to the weights.
 *  scaling  multiplies every returned scale (routed scaling factor; pass 1.0
 *           when the model has none).
 *  flags    MOE_ROUTE_FLAG_RENORMALIZE (DEFAULT only).
 *  ids      device int32 [T, k] out: chosen experts, ordered by key
 *           descending, ties to the lower expert index (groups likewise).
 *  scales   device fp32 [T, k] out: weights of `ids`, same order.
 * Selection precision: softmax methods and Llama4 select on the fp32 logits
 * (softmax is monotone); DeepSeek-V3, MiniMax2 and SigmoidRenorm select on
 * fl32(sigmoid) (+ bias) with the sigmoid evaluated in fp64 and rounded once
 * to fp32.  Weights are computed in fp64 and rounded once: Llama4 weighs each
 * kept expert by its own sigmoid (the name fixes k = 1; larger k keeps the
 * rule); MiniMax2 and SigmoidRenorm divide the kept sigmoids by their sum
 * (DeepSeek-V3 adds 1e-20 to that sum).  NaN logits give unspecified (but
 * in-bounds) ids.
 */
moe_status moe_route(const float* logits, int T, int E, int method, int k, int n_group,
                     int topk_group, const float* bias, float scaling, unsigned flags,
                     int32_t* ids, float* scales, void* stream);

/*
 * moe_permute -- counting sort of the P = T*k pairs p = t*k + j by expert id,
 * stable in p, giving each expert one contiguous block of rows ("从 Dense GEMM
 * 到 TP MoE 的演进逻辑", section 2.1: one offset array marks where each group
 * starts; section 2.2: permute each expert's tokens into one block).
 *
 *  ids            device int32 [T, k]; values must lie in [0, E) (values
 *                 outside are clamped into range: memory-safe, not meaningful).
 *  n_shared       shared experts (every token, weight 1) appended as groups
 *                 E .. E+n_shared-1; shared group s owns rows P + s*T + t.
 *  expert_offsets device int32 [E + n_shared + 1] out: first row of each group;
 *                 expert_offsets[E] == P, last entry == P + n_shared*T.
 *  permuted_pair  device int32 [P] out: row -> pair index p.
 *  unpermute      device int32 [P] out: pair index p -> row.
 *  ws, ws_bytes   device workspace of at least
 *                 moe_workspace_size(T, k, E, n_shared, H, I, act) bytes (any
 *                 H, I, act: the permute scratch does not depend on them).
 * Integer results are bit-exact and deterministic.
 */
moe_status moe_permute(const int32_t* ids, int T, int k, int E, int n_shared,
                       int32_t* expert_offsets, int32_t* permuted_pair, int32_t* unpermute,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn -- every group's expert FFN on its rows, as two grouped GEMMs
 * over one flattened list of (group, M-tile, N-tile) work items ("从 Dense GEMM
 * 到 TP MoE 的演进逻辑", section 2.2: tile scheduling over all groups):
 *     h_r   = silu(W1_g x_t) * (W3_g x_t)        (FC1 + SwiGLU, kept in ws)
 *     out_r = W2_g h_r                           (FC2)
 * for every row r of group g (token t = permuted_pair[r] / k, or r - offset
 * for shared groups).  Weight layout of the vLLM page, section "专家权重如何存
 * 储"; gated expansion of FC1 to 2*I of the TensorRT-LLM page, section "权重加
 * 载".
 *
 *  x          device [T, H] in `act` (MOE_F32 or MOE_BF16).
 *  H, I       hidden and intermediate sizes, multiples of 128.
 *  expert_offsets, permuted_pair   as produced by moe_permute for the same
 *             T, k, E, n_shared.  Their contents are device data and are not
 *             checked: other values may make the kernels read or write out of
 *             bounds.  The same holds for every FFN entry point below.
 *  w13        device [E + n_shared, 2I, H] in `wdt`: rows [0, I) are the gate
 *             projection W1, rows [I, 2I) the up projection W3.
 *  w2         device [E + n_shared, H, I] in `wdt`.
 *  wdt        MOE_F32 (with act MOE_F32), MOE_BF16 or MOE_FP8_E4M3 (OCP e4m3fn,
 *             with act MOE_BF16).
 *  w13_scale  device fp32 [E + n_shared, 2I/128, H/128] for fp8 (else NULL):
 *             the weight is code * scale of its 128x128 block.
 *  w2_scale   device fp32 [E + n_shared, H/128, I/128] for fp8 (else NULL).
 *  fc2_out    device [T*k + n_shared*T, H] out, in `act`: FFN output per row
 *             (unweighted).
 *  ws         device workspace (moe_workspace_size bytes) holding h.
 * Accumulation is fp32; h and fc2_out are rounded once to `act`.
 * Limits (MOE_ERR_UNSUPPORTED beyond): x, h [T*k + n_shared*T, I] and one
 * expert's w13 each below 4 GiB (the kernels use 32-bit byte offsets).
 */
moe_status moe_expert_ffn(const void* x, int act, int T, int H, int I, int k, int E,
                          int n_shared, const int32_t* expert_offsets,
                          const int32_t* permuted_pair, const void* w13, const void* w2,
                          int wdt, const float* w13_scale, const float* w2_scale,
                          void* fc2_out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_noalloc -- moe_expert_ffn for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): same arguments minus the workspace, same kernels and
 * bit-identical results.  h lives in a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES instead; a shape whose h, (T*k + n_shared*T) * I
 * activation values, does not fit returns MOE_ERR_UNSUPPORTED before anything
 * is launched.  Nothing is allocated: no hipMalloc, no hipFree (the scratch's
 * device address is looked up once per GPU, on the first call there).  h is
 * written before it is read, so nothing is cleared between calls.  Every call
 * on one GPU shares that GPU's scratch, which keeps the last call's contents:
 * calls that overlap on one GPU (two streams, two threads) race.  With
 * moe_timing_enable on, the timing hooks create HIP events; keep timing off
 * where nothing may be allocated.
 */
moe_status moe_expert_ffn_noalloc(const void* x, int act, int T, int H, int I, int k, int E,
                                  int n_shared, const int32_t* expert_offsets,
                                  const int32_t* permuted_pair, const void* w13, const void* w2,
                                  int wdt, const float* w13_scale, const float* w2_scale,
                                  void* fc2_out, void* stream);

/*
 * moe_finalize -- y_t = sum_j scales[t,j] * fc2_out[unpermute[t*k+j]]
 *                       + sum_s fc2_out[T*k + s*T + t]
 * accumulated in fp32 in j order, rounded once to `ydt`; a gather, no atomics,
 * so results are deterministic.  The routing weight is applied here, after
 * FC2 (TensorRT-LLM page, sections "通信与计算融合的方向" and "小结").
 *
 *  fc2_out    device [T*k + n_shared*T, H] in `dt` (MOE_F32 or MOE_BF16).
 *  unpermute, scales   from moe_permute / moe_route for the same T, k, E,
 *             n_shared (unpermute is not checked: other values may make the
 *             gather read out of bounds).
 *  y          device [T, H] out in `ydt` (MOE_F32 or MOE_BF16).
 *  H          multiple of 8.
 */
moe_status moe_finalize(const void* fc2_out, int dt, const int32_t* unpermute,
                        const float* scales, int T, int k, int H, int n_shared, void* y,
                        int ydt, void* stream);

/*
 * moe_quantize_fp8 -- the quantise-input step that precedes the MoE GEMMs
 * (TensorRT-LLM page, sections "MoEScheduler:两条执行路径,两套相反的约定" and
 * "“自适应顺序”里的一个细节"), in the form of the fp8 fused MoE on the vLLM page
 * (section "量化与 MoE Kernel 选择", after DeepSeek-V3's fp8 scheme): every row
 * is cut into blocks of 128 consecutive values;
 *     s = fl32(amax / 448),   code = e4m3fn(fl32(v / s))
 * rounded to nearest even and saturating at +-448 (OCP e4m3fn codes); a block
 * whose scale is 0 encodes as zeros.  Call it on x [T, H] once per layer,
 * before the permute (one GPU has no dispatch, and quantising the T tokens
 * writes k times fewer bytes than quantising the T*k permuted rows).
 *
 *  x        device [rows, cols] in `dt` (MOE_BF16 or MOE_F32).
 *  cols     a multiple of 128.
 *  xq       device uint8 [rows, cols] out: e4m3fn codes.
 *  x_scale  device fp32 [rows, cols / 128] out.
 * Codes and scales are deterministic and bit-exact.  NaN inputs give
 * unspecified codes.
 */
moe_status moe_quantize_fp8(const void* x, int dt, int rows, int cols, uint8_t* xq,
                            float* x_scale, void* stream);

/*
 * moe_expert_ffn_fp8 -- moe_expert_ffn with fp8 activations on fp8 x fp8 MFMA
 * (vLLM page, section "量化与 MoE Kernel 选择"):
 *     h_r   = silu(W1_g xq_t) * (W3_g xq_t),  xq_t = dequantised x_t
 *     hq_r  = h_r rounded to fp32, quantised like moe_quantize_fp8 per row and
 *             128 intermediate channels
 *     out_r = W2_g hq_r
 * Products of e4m3 codes are exact; sums are fp32; each 128-wide K block is
 * added times (activation block scale x weight block scale).
 *
 *  xq, x_scale   moe_quantize_fp8 of x [T, H].
 *  w13, w2, w13_scale, w2_scale   fp8 e4m3fn weights with fp32 128x128 block
 *             scales, laid out as for moe_expert_ffn with wdt MOE_FP8_E4M3.
 *  fc2_out    device bf16 [T*k + n_shared*T, H] out (unweighted FFN rows).
 *  ws         device workspace of moe_workspace_size(T, k, E, n_shared, H, I,
 *             MOE_FP8_E4M3) bytes.  On return it holds hq: e4m3fn codes
 *             [R, I] at byte 0 (R = T*k + n_shared*T, rows in permuted order)
 *             and their fp32 scales [R, I/128] from the next 256-byte
 *             boundary.
 * H and I are multiples of 128; xq, hq and one expert's w13 below 4 GiB;
 * other arguments as for moe_expert_ffn.
 */
moe_status moe_expert_ffn_fp8(const uint8_t* xq, const float* x_scale, int T, int H, int I, int k,
                              int E, int n_shared, const int32_t* expert_offsets,
                              const int32_t* permuted_pair, const uint8_t* w13, const uint8_t* w2,
                              const float* w13_scale, const float* w2_scale, void* fc2_out,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_fused -- moe_expert_ffn as ONE kernel that keeps h on chip:
 * FC1 and FC2 fused, the intermediate never written to memory (the FC12 form
 * of the TensorRT-LLM page, section "后端的三种形态与两个调度器家族").  A
 * workgroup takes 16 rows of one group, computes their h [16, I] into LDS
 * (FC1 + SwiGLU over all I channels), then their FC2 rows from it.
 * Results are bit-identical to moe_expert_ffn for the same arguments.
 *
 *  act        MOE_BF16 (MOE_F32 is MOE_ERR_UNSUPPORTED).
 *  wdt        MOE_BF16 or MOE_FP8_E4M3 (with w13_scale, w2_scale).
 *  I          at most MOE_FUSED_MAX_I (h of 16 rows fills the LDS);
 *             larger I is MOE_ERR_UNSUPPORTED.
 *  split      workgroups that share one 16-row tile: each computes the tile's
 *             h (FC1 repeated) and takes every split-th 128- or 256-column
 *             block of its FC2.  0 = automatic (currently 1: each extra split
 *             re-reads the expert's whole w13).  Values above the number of
 *             FC2 column blocks are clamped to it; negative values and values
 *             above 64 are MOE_ERR_INVALID_ARG.  Results do not depend on it.
 *  other arguments as for moe_expert_ffn; there is no workspace.
 * Limits: x and one expert's w13 below 4 GiB.
 */
moe_status moe_expert_ffn_fused(const void* x, int act, int T, int H, int I, int k, int E,
                                int n_shared, const int32_t* expert_offsets,
                                const int32_t* permuted_pair, const void* w13, const void* w2,
                                int wdt, const float* w13_scale, const float* w2_scale, int split,
                                void* fc2_out, void* stream);

/*
 * moe_expert_ffn_fp8_fused -- moe_expert_ffn_fp8 as one kernel with h on chip:
 * the e4m3 codes of h and their per-row, per-128-channel scales (quantised as
 * moe_expert_ffn_fp8 quantises them) stay in LDS between FC1 and FC2.
 * Results are bit-identical to moe_expert_ffn_fp8.  I <= MOE_FUSED_MAX_I;
 * split as for moe_expert_ffn_fused; no workspace; other arguments as for
 * moe_expert_ffn_fp8.
 */
moe_status moe_expert_ffn_fp8_fused(const uint8_t* xq, const float* x_scale, int T, int H, int I,
                                    int k, int E, int n_shared, const int32_t* expert_offsets,
                                    const int32_t* permuted_pair, const uint8_t* w13,
                                    const uint8_t* w2, const float* w13_scale,
                                    const float* w2_scale, int split, void* fc2_out, void* stream);

/* Bytes of workspace that moe_permute and moe_expert_ffn need for this shape
 * (0 on invalid arguments).  One buffer of this size serves both calls.
 * act = MOE_FP8_E4M3 sizes it for moe_expert_ffn_fp8.  The size depends only
 * on the shape (T*k rows, never on how tokens are routed), so a caller can
 * allocate it once, up front, and reuse it on every call: the gsyq.cn
 * article's remedy for allocator fragmentation in grouped-GEMM MoE layers
 * (section 4.4, "显存碎片导致的 OOM").  Host-only; never fails otherwise. */
size_t moe_workspace_size(int T, int k, int E, int n_shared, int H, int I, int act);

/* Static, never-NULL description of a status code (unknown codes included).
 * Part of reporting unsupported requests loudly instead of degrading
 * silently (TensorRT-LLM page, section "融合算子与回退阈值"). */
const char* moe_status_string(int status);

/* Reason for the last non-OK status returned on the calling thread (a
 * thread-local, NUL-terminated string owned by the library, valid until that
 * thread's next call; "" before any failure): the message that names the
 * limit an unsupported shape exceeds (same section as above). */
const char* moe_last_error(void);

/*
 * Per-kernel timing (measurement support for the benchmark, not a step of the
 * layer; off by default).  When enabled,
 * every launch is bracketed by two HIP events recorded on the launch stream;
 * moe_kernel_times() waits for the recorded events and returns, per kernel
 * id, the summed milliseconds and the launch count since the last reset.
 */
enum {
    MOE_KID_ROUTE = 0,
    MOE_KID_PERMUTE_COUNT = 1,
    MOE_KID_PERMUTE_SCAN = 2,
    MOE_KID_PERMUTE_SCATTER = 3,
    MOE_KID_FC1 = 4,
    MOE_KID_FC2 = 5,
    MOE_KID_FINALIZE = 6,
    MOE_KID_QUANT = 7,
    MOE_KID_FFN_FUSED = 8,
    MOE_KID_PERMUTE_ONE = 9,   /* the one-workgroup permute (inputs of up to 8192 pairs) */
    MOE_NUM_KIDS = 10
};
moe_status moe_timing_enable(int enable);
moe_status moe_kernel_times(double* ms /*[MOE_NUM_KIDS]*/, int64_t* launches /*[MOE_NUM_KIDS]*/,
                            int reset);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
