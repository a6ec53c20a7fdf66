// C ABI of libmoe: argument validation, workspace sizing, error reporting and
// per-kernel timing.  Every check runs on the host before anything is
// launched; the launchers in the kernel sources assume validated arguments.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "common.h"

namespace moe {

static thread_local char g_err[512] = "";

moe_status set_error(moe_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

moe_status launch_status(const char* what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return set_error(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return MOE_OK;
}

int device_cu_count()
{
    static std::atomic<int> cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// ------------------------------------------------------------------ timing
namespace {
struct TimingState {
    std::mutex mu;
    std::atomic<bool> enabled{false};
    struct Rec { int kid; hipEvent_t a, b; };
    std::vector<Rec> pending;
    std::vector<hipEvent_t> free_events;
    double ms[MOE_NUM_KIDS] = {0};
    int64_t n[MOE_NUM_KIDS] = {0};
};
TimingState& timing()
{
    static TimingState t;
    return t;
}
hipEvent_t take_event(TimingState& t)
{
    if (!t.free_events.empty()) {
        hipEvent_t e = t.free_events.back();
        t.free_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

TimedLaunch::TimedLaunch(int kid, hipStream_t s) : kid_(kid), s_(s)
{
    TimingState& t = timing();
    if (!t.enabled.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> g(t.mu);
    hipEvent_t a = take_event(t), b = take_event(t);
    if (!a || !b) {
        if (a) t.free_events.push_back(a);
        if (b) t.free_events.push_back(b);
        return;
    }
    a_ = a;
    b_ = b;
    (void)hipEventRecord(a_, s_);
}

TimedLaunch::~TimedLaunch()
{
    if (!b_) return;
    TimingState& t = timing();
    (void)hipEventRecord(b_, s_);
    std::lock_guard<std::mutex> g(t.mu);
    t.pending.push_back({kid_, a_, b_});
}

}  // namespace moe

using namespace moe;

namespace {

bool valid_act(int d) { return d == MOE_F32 || d == MOE_BF16; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// The GEMM kernels address activation rows, h rows and one group's weights
// with 32-bit byte offsets from a scalar base.
bool gemm_offsets_fit(int T, int k, int n_shared, int H, int I, int asz, int wsz)
{
    const unsigned long long lim = 1ull << 32;
    const unsigned long long R = (unsigned long long)T * k + (unsigned long long)n_shared * T;
    return (unsigned long long)T * H * asz < lim && R * I * asz < lim &&
           2ull * I * H * wsz < lim;
}

moe_status check_common(int T, int k, int E, int n_shared)
{
    if (T < 0) return set_error(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
    if (E < 1) return set_error(MOE_ERR_INVALID_ARG, "E must be >= 1 (got %d)", E);
    if (E > MOE_MAX_EXPERTS)
        return set_error(MOE_ERR_UNSUPPORTED, "E = %d exceeds the kernel limit %d", E, MOE_MAX_EXPERTS);
    if (k < 1 || k > E) return set_error(MOE_ERR_INVALID_ARG, "k must be in [1, E] (k=%d, E=%d)", k, E);
    if (k > MOE_MAX_TOPK)
        return set_error(MOE_ERR_UNSUPPORTED, "k = %d exceeds the kernel limit %d", k, MOE_MAX_TOPK);
    if (n_shared < 0 || n_shared > 64)
        return set_error(MOE_ERR_INVALID_ARG, "n_shared must be in [0, 64] (got %d)", n_shared);
    const long long R = (long long)T * k + (long long)n_shared * T;
    if (R > (1ll << 30))
        return set_error(MOE_ERR_UNSUPPORTED, "T*k + n_shared*T = %lld rows exceeds 2^30", R);
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int st)
{
    switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or type outside the kernels' limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: HIP call or kernel launch failed";
    default: return "unknown moe_status";
    }
}

const char* moe_last_error(void) { return g_err; }

size_t moe_workspace_size(int T, int k, int E, int n_shared, int H, int I, int act)
{
    (void)H;
    if (check_common(T, k, E, n_shared) != MOE_OK || I < 0 || !(valid_act(act) || act == MOE_FP8_E4M3))
        return 0;
    const size_t a = align256(permute_scratch_bytes(T, k, E));
    const size_t b = act == MOE_FP8_E4M3 ? ffn_fp8_scratch_bytes(T, k, n_shared, I)
                                         : ffn_scratch_bytes(T, k, n_shared, I, act);
    return (a > b ? a : b) + 256;
}

moe_status moe_route(const float* logits, int T, int E, int method, int k, int n_group,
                     int topk_group, const float* bias, float scaling, unsigned flags,
                     int32_t* ids, float* scales, void* stream)
{
    moe_status st = check_common(T, k, E, 0);
    if (st != MOE_OK) return st;
    if (method == 7 || method == 8)
        return set_error(MOE_ERR_UNSUPPORTED, "routing method %d is not implemented (supported: 0-6)", method);
    if (method < MOE_ROUTE_DEFAULT || method > MOE_ROUTE_SIGMOID_RENORM)
        return set_error(MOE_ERR_INVALID_ARG, "unknown routing method %d", method);
    if (flags & ~MOE_ROUTE_FLAG_RENORMALIZE)
        return set_error(MOE_ERR_INVALID_ARG, "unknown routing flags 0x%x", flags);
    if (!isfinite(scaling)) return set_error(MOE_ERR_INVALID_ARG, "scaling must be finite");
    if (method == MOE_ROUTE_DEEPSEEKV3) {
        if (n_group < 1 || E % n_group != 0)
            return set_error(MOE_ERR_INVALID_ARG, "n_group=%d must divide E=%d", n_group, E);
        const int gsz = E / n_group;
        if (gsz < 2)
            return set_error(MOE_ERR_INVALID_ARG, "groups need >= 2 experts for the top-2 group score (E/n_group=%d)", gsz);
        if (topk_group < 1 || topk_group > n_group)
            return set_error(MOE_ERR_INVALID_ARG, "topk_group=%d must be in [1, n_group=%d]", topk_group, n_group);
        if (k > topk_group * gsz)
            return set_error(MOE_ERR_INVALID_ARG, "k=%d exceeds the experts of the kept groups (%d)", k, topk_group * gsz);
    }
    if (T == 0) return MOE_OK;
    if (!logits || !ids || !scales)
        return set_error(MOE_ERR_INVALID_ARG, "logits, ids and scales must be non-null");
    return launch_route(logits, T, E, method, k, n_group, topk_group,
                        (method == MOE_ROUTE_DEEPSEEKV3 || method == MOE_ROUTE_MINIMAX2) ? bias : nullptr,
                        scaling, flags, ids,
                        scales, static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const int32_t* ids, int T, int k, int E, int n_shared,
                       int32_t* expert_offsets, int32_t* permuted_pair, int32_t* unpermute,
                       void* ws, size_t ws_bytes, void* stream)
{
    moe_status st = check_common(T, k, E, n_shared);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!ids || !expert_offsets || !permuted_pair || !unpermute)
        return set_error(MOE_ERR_INVALID_ARG,
                         "ids, expert_offsets, permuted_pair and unpermute must be non-null");
    const size_t need = permute_scratch_bytes(T, k, E);
    if (!ws || ws_bytes < need)
        return set_error(MOE_ERR_WORKSPACE, "permute needs %zu workspace bytes (got %zu)", need, ws_bytes);
    return launch_permute(ids, T, k, E, n_shared, expert_offsets, permuted_pair, unpermute, ws,
                          static_cast<hipStream_t>(stream));
}

// Host checks of moe_expert_ffn and moe_expert_ffn_noalloc (everything but
// the workspace).
static moe_status check_ffn(const void* x, int act, int T, int H, int I, int k, int E, int n_shared,
                            const int32_t* expert_offsets, const int32_t* permuted_pair,
                            const void* w13, const void* w2, int wdt, const float* w13_scale,
                            const float* w2_scale, void* fc2_out)
{
    moe_status st = check_common(T, k, E, n_shared);
    if (st != MOE_OK) return st;
    if (!valid_act(act)) return set_error(MOE_ERR_INVALID_ARG, "activation dtype %d must be MOE_F32 or MOE_BF16", act);
    if (wdt != MOE_F32 && wdt != MOE_BF16 && wdt != MOE_FP8_E4M3)
        return set_error(MOE_ERR_INVALID_ARG, "unknown weight dtype %d", wdt);
    if (H < 1 || I < 1) return set_error(MOE_ERR_INVALID_ARG, "H and I must be positive (H=%d, I=%d)", H, I);
    if (H % 128 || I % 128)
        return set_error(MOE_ERR_UNSUPPORTED, "H and I must be multiples of 128 (H=%d, I=%d)", H, I);
    if (act == MOE_F32 && wdt != MOE_F32)
        return set_error(MOE_ERR_UNSUPPORTED, "fp32 activations need fp32 weights");
    if (act == MOE_BF16 && wdt == MOE_F32)
        return set_error(MOE_ERR_UNSUPPORTED, "bf16 activations need bf16 or fp8 weights");
    if (wdt == MOE_FP8_E4M3 && (!w13_scale || !w2_scale))
        return set_error(MOE_ERR_INVALID_ARG, "fp8 weights need w13_scale and w2_scale");
    if (!gemm_offsets_fit(T, k, n_shared, H, I, act == MOE_F32 ? 4 : 2, wdt == MOE_F32 ? 4 : wdt == MOE_BF16 ? 2 : 1))
        return set_error(MOE_ERR_UNSUPPORTED, "x, h or one expert's weights exceed 4 GiB (T=%d, H=%d, I=%d)", T, H, I);
    if (T == 0) return MOE_OK;
    if (!x || !expert_offsets || !w13 || !w2 || !fc2_out || (E > 0 && !permuted_pair))
        return set_error(MOE_ERR_INVALID_ARG, "x, expert_offsets, permuted_pair, w13, w2 and fc2_out must be non-null");
    return MOE_OK;
}

moe_status moe_expert_ffn(const void* x, int act, int T, int H, int I, int k, int E,
                          int n_shared, const int32_t* expert_offsets,
                          const int32_t* permuted_pair, const void* w13, const void* w2,
                          int wdt, const float* w13_scale, const float* w2_scale,
                          void* fc2_out, void* ws, size_t ws_bytes, void* stream)
{
    moe_status st = check_ffn(x, act, T, H, I, k, E, n_shared, expert_offsets, permuted_pair, w13, w2,
                              wdt, w13_scale, w2_scale, fc2_out);
    if (st != MOE_OK || T == 0) return st;
    const size_t need = ffn_scratch_bytes(T, k, n_shared, I, act);
    if (!ws || ws_bytes < need)
        return set_error(MOE_ERR_WORKSPACE, "expert_ffn needs %zu workspace bytes (got %zu)", need, ws_bytes);
    return launch_ffn(x, act, T, H, I, k, E, n_shared, expert_offsets, permuted_pair, w13, w2, wdt,
                      wdt == MOE_FP8_E4M3 ? w13_scale : nullptr,
                      wdt == MOE_FP8_E4M3 ? w2_scale : nullptr, fc2_out, ws,
                      static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_noalloc(const void* x, int act, int T, int H, int I, int k, int E,
                                  int n_shared, const int32_t* expert_offsets,
                                  const int32_t* permuted_pair, const void* w13, const void* w2,
                                  int wdt, const float* w13_scale, const float* w2_scale,
                                  void* fc2_out, void* stream)
{
    moe_status st = check_ffn(x, act, T, H, I, k, E, n_shared, expert_offsets, permuted_pair, w13, w2,
                              wdt, w13_scale, w2_scale, fc2_out);
    if (st != MOE_OK || T == 0) return st;
    const size_t need = ffn_scratch_bytes(T, k, n_shared, I, act);
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return set_error(MOE_ERR_UNSUPPORTED,
                         "expert_ffn_noalloc: h needs %zu bytes, the static scratch holds %zu "
                         "(use moe_expert_ffn with a workspace)", need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
    void* ws = noalloc_scratch();
    if (!ws) return MOE_ERR_DEVICE;
    return launch_ffn(x, act, T, H, I, k, E, n_shared, expert_offsets, permuted_pair, w13, w2, wdt,
                      wdt == MOE_FP8_E4M3 ? w13_scale : nullptr,
                      wdt == MOE_FP8_E4M3 ? w2_scale : nullptr, fc2_out, ws,
                      static_cast<hipStream_t>(stream));
}

moe_status moe_quantize_fp8(const void* x, int dt, int rows, int cols, uint8_t* xq,
                            float* x_scale, void* stream)
{
    if (rows < 0) return set_error(MOE_ERR_INVALID_ARG, "rows must be >= 0 (got %d)", rows);
    if (cols < 1) return set_error(MOE_ERR_INVALID_ARG, "cols must be positive (got %d)", cols);
    if (cols % 128) return set_error(MOE_ERR_UNSUPPORTED, "cols must be a multiple of 128 (got %d)", cols);
    if (!valid_act(dt)) return set_error(MOE_ERR_INVALID_ARG, "x dtype %d must be MOE_F32 or MOE_BF16", dt);
    if (rows == 0) return MOE_OK;
    if (!x || !xq || !x_scale) return set_error(MOE_ERR_INVALID_ARG, "x, xq and x_scale must be non-null");
    return launch_quantize_fp8(x, dt, rows, cols, xq, x_scale, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_fp8(const uint8_t* xq, const float* x_scale, int T, int H, int I, int k,
                              int E, int n_shared, const int32_t* expert_offsets,
                              const int32_t* permuted_pair, const uint8_t* w13, const uint8_t* w2,
                              const float* w13_scale, const float* w2_scale, void* fc2_out,
                              void* ws, size_t ws_bytes, void* stream)
{
    moe_status st = check_common(T, k, E, n_shared);
    if (st != MOE_OK) return st;
    if (H < 1 || I < 1) return set_error(MOE_ERR_INVALID_ARG, "H and I must be positive (H=%d, I=%d)", H, I);
    if (H % 128 || I % 128)
        return set_error(MOE_ERR_UNSUPPORTED, "H and I must be multiples of 128 (H=%d, I=%d)", H, I);
    if (!gemm_offsets_fit(T, k, n_shared, H, I, 1, 1))
        return set_error(MOE_ERR_UNSUPPORTED, "xq, hq or one expert's weights exceed 4 GiB (T=%d, H=%d, I=%d)", T, H, I);
    if (T == 0) return MOE_OK;
    if (!xq || !x_scale || !expert_offsets || !w13 || !w2 || !w13_scale || !w2_scale || !fc2_out ||
        (E > 0 && !permuted_pair))
        return set_error(MOE_ERR_INVALID_ARG,
                         "xq, x_scale, expert_offsets, permuted_pair, w13, w2, their scales and fc2_out "
                         "must be non-null");
    const size_t need = ffn_fp8_scratch_bytes(T, k, n_shared, I);
    if (!ws || ws_bytes < need)
        return set_error(MOE_ERR_WORKSPACE, "expert_ffn_fp8 needs %zu workspace bytes (got %zu)", need, ws_bytes);
    return launch_ffn_fp8(xq, x_scale, T, H, I, k, E, n_shared, expert_offsets, permuted_pair, w13, w2,
                          w13_scale, w2_scale, fc2_out, ws, static_cast<hipStream_t>(stream));
}

// Checks shared by the two fused entry points (act: MOE_BF16 or, for the
// fp8 x fp8 form, MOE_FP8_E4M3).
static moe_status check_fused(int T, int H, int I, int k, int E, int n_shared, int act, int wdt,
                              int split)
{
    moe_status st = check_common(T, k, E, n_shared);
    if (st != MOE_OK) return st;
    if (H < 1 || I < 1) return set_error(MOE_ERR_INVALID_ARG, "H and I must be positive (H=%d, I=%d)", H, I);
    if (H % 128 || I % 128)
        return set_error(MOE_ERR_UNSUPPORTED, "H and I must be multiples of 128 (H=%d, I=%d)", H, I);
    if (I > MOE_FUSED_MAX_I)
        return set_error(MOE_ERR_UNSUPPORTED, "I = %d exceeds the fused kernel's limit %d (h is kept in LDS)",
                         I, MOE_FUSED_MAX_I);
    if (split < 0 || split > 64) return set_error(MOE_ERR_INVALID_ARG, "split must be in [0, 64] (got %d)", split);
    const unsigned long long lim = 1ull << 32;
    const int asz = act == MOE_FP8_E4M3 ? 1 : 2, wsz = wdt == MOE_FP8_E4M3 ? 1 : 2;
    if ((unsigned long long)T * H * asz >= lim || 2ull * I * H * wsz >= lim)
        return set_error(MOE_ERR_UNSUPPORTED, "x or one expert's weights exceed 4 GiB (T=%d, H=%d, I=%d)", T, H, I);
    return MOE_OK;
}

moe_status moe_expert_ffn_fused(const void* x, int act, int T, int H, int I, int k, int E,
                                int n_shared, const int32_t* expert_offsets,
                                const int32_t* permuted_pair, const void* w13, const void* w2,
                                int wdt, const float* w13_scale, const float* w2_scale, int split,
                                void* fc2_out, void* stream)
{
    if (act == MOE_F32) return set_error(MOE_ERR_UNSUPPORTED, "the fused kernel takes bf16 activations");
    if (act != MOE_BF16) return set_error(MOE_ERR_INVALID_ARG, "activation dtype %d must be MOE_BF16", act);
    if (wdt == MOE_F32) return set_error(MOE_ERR_UNSUPPORTED, "bf16 activations need bf16 or fp8 weights");
    if (wdt != MOE_BF16 && wdt != MOE_FP8_E4M3) return set_error(MOE_ERR_INVALID_ARG, "unknown weight dtype %d", wdt);
    moe_status st = check_fused(T, H, I, k, E, n_shared, act, wdt, split);
    if (st != MOE_OK) return st;
    if (wdt == MOE_FP8_E4M3 && (!w13_scale || !w2_scale))
        return set_error(MOE_ERR_INVALID_ARG, "fp8 weights need w13_scale and w2_scale");
    if (T == 0) return MOE_OK;
    if (!x || !expert_offsets || !permuted_pair || !w13 || !w2 || !fc2_out)
        return set_error(MOE_ERR_INVALID_ARG, "x, expert_offsets, permuted_pair, w13, w2 and fc2_out must be non-null");
    return launch_ffn_fused(x, nullptr, act, T, H, I, k, E, n_shared, expert_offsets, permuted_pair, w13, w2,
                            wdt, wdt == MOE_FP8_E4M3 ? w13_scale : nullptr,
                            wdt == MOE_FP8_E4M3 ? w2_scale : nullptr, split, fc2_out,
                            static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_fp8_fused(const uint8_t* xq, const float* x_scale, int T, int H, int I,
                                    int k, int E, int n_shared, const int32_t* expert_offsets,
                                    const int32_t* permuted_pair, const uint8_t* w13,
                                    const uint8_t* w2, const float* w13_scale,
                                    const float* w2_scale, int split, void* fc2_out, void* stream)
{
    moe_status st = check_fused(T, H, I, k, E, n_shared, MOE_FP8_E4M3, MOE_FP8_E4M3, split);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!xq || !x_scale || !expert_offsets || !permuted_pair || !w13 || !w2 || !w13_scale || !w2_scale ||
        !fc2_out)
        return set_error(MOE_ERR_INVALID_ARG,
                         "xq, x_scale, expert_offsets, permuted_pair, w13, w2, their scales and fc2_out "
                         "must be non-null");
    return launch_ffn_fused(xq, x_scale, MOE_FP8_E4M3, T, H, I, k, E, n_shared, expert_offsets, permuted_pair,
                            w13, w2, MOE_FP8_E4M3, w13_scale, w2_scale, split, fc2_out,
                            static_cast<hipStream_t>(stream));
}

moe_status moe_finalize(const void* fc2_out, int dt, const int32_t* unpermute,
                        const float* scales, int T, int k, int H, int n_shared, void* y,
                        int ydt, void* stream)
{
    if (T < 0) return set_error(MOE_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
    if (k < 1) return set_error(MOE_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
    if (k > MOE_MAX_TOPK) return set_error(MOE_ERR_UNSUPPORTED, "k = %d exceeds the kernel limit %d", k, MOE_MAX_TOPK);
    if (n_shared < 0 || n_shared > 64) return set_error(MOE_ERR_INVALID_ARG, "n_shared must be in [0, 64]");
    if (!valid_act(dt) || !valid_act(ydt))
        return set_error(MOE_ERR_INVALID_ARG, "fc2_out and y dtypes must be MOE_F32 or MOE_BF16");
    if (H < 1) return set_error(MOE_ERR_INVALID_ARG, "H must be positive");
    if (H % 8) return set_error(MOE_ERR_UNSUPPORTED, "H must be a multiple of 8 (got %d)", H);
    if ((long long)T * k + (long long)n_shared * T > (1ll << 30))
        return set_error(MOE_ERR_UNSUPPORTED, "too many rows");
    if (T == 0) return MOE_OK;
    if (!fc2_out || !unpermute || !scales || !y)
        return set_error(MOE_ERR_INVALID_ARG, "fc2_out, unpermute, scales and y must be non-null");
    return launch_finalize(fc2_out, dt, unpermute, scales, T, k, H, n_shared, y, ydt,
                           static_cast<hipStream_t>(stream));
}

moe_status moe_timing_enable(int enable)
{
    TimingState& t = timing();
    t.enabled.store(enable != 0, std::memory_order_relaxed);
    return MOE_OK;
}

moe_status moe_kernel_times(double* ms, int64_t* launches, int reset)
{
    TimingState& t = timing();
    std::lock_guard<std::mutex> g(t.mu);
    for (auto& r : t.pending) {
        if (hipEventSynchronize(r.b) != hipSuccess)
            return set_error(MOE_ERR_DEVICE, "hipEventSynchronize failed while reading kernel times");
        float v = 0.f;
        if (hipEventElapsedTime(&v, r.a, r.b) == hipSuccess) {
            t.ms[r.kid] += v;
            t.n[r.kid] += 1;
        }
        t.free_events.push_back(r.a);
        t.free_events.push_back(r.b);
    }
    t.pending.clear();
    for (int i = 0; i < MOE_NUM_KIDS; ++i) {
        if (ms) ms[i] = t.ms[i];
        if (launches) launches[i] = t.n[i];
        if (reset) {
            t.ms[i] = 0;
            t.n[i] = 0;
        }
    }
    return MOE_OK;
}

}  // extern "C"
