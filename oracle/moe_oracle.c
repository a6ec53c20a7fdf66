/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle of the MoE layer
 * forward.  TEST INFRASTRUCTURE ONLY: it exists so tests, the smoke check and
 * the benchmark's CPU baseline can check the HIP path.  The product path never
 * links, loads or calls it, and it shares no code, header or table with it.
 *
 * Sources (the pages this follows):
 *  [TRT]  "TensorRT-LLM 源码完全拆解(十三): MoE 层前向执行——路由、Fused Kernel 与
 *         专家并行的三段拼装", sections "MoE 在推理侧到底特殊在哪里" (the layer
 *         formula y = sum_{i in TopK(x)} g_i(x) E_i(x) and the shared expert),
 *         "路由方法枚举" (RoutingMethodType comments), "DeepSeek-V3 的 noaux_tc"
 *         (sigmoid, bias for selection only, top-2 group sums, group mask,
 *         unbiased renormalisation + 1e-20 + routed scaling factor; the
 *         Llama4 "Top1 -> Sigmoid", MiniMaxM2 "Sigmoid -> RoutingBiasAdd ->
 *         TopK -> Renormalize(without bias)" and SigmoidRenorm "Sigmoid ->
 *         TopK -> Renormalize" comments of the enum),
 *         "权重加载" (fused gate/up projection, gated activation expands FC1
 *         to 2*I), "小结" (FC1 -> act -> FC2 then apply weights / finalize).
 *  [VLLM] "vLLM 源码完全拆解(八): MoE 层的前向执行", sections "FusedTopKRouter"
 *         (softmax -> top-k -> optional renormalise) and "专家权重如何存储"
 *         (w13 [E, 2I, H], w2 [E, H, I]).
 *  [GG]   "从 Dense GEMM 到 TP MoE 的演进逻辑" (gsyq.cn), sections 2.1-2.2
 *         (offset array marking each group's start; permute of each
 *         expert's tokens into one contiguous block).
 *  fp8 activations: [TRT] sections "MoEScheduler:两条执行路径,两套相反的约定"
 *         and "“自适应顺序”里的一个细节" (a quantise-input step of the backend
 *         runs before the MoE GEMMs, before or after dispatch) and [VLLM]
 *         section "量化与 MoE Kernel 选择" (the fp8 fused MoE follows
 *         DeepSeek-V3's fp8 mixed-precision scheme; read here as 1x128
 *         activation blocks and 128x128 weight blocks with fp32 scales).
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes of the repository):
 *  - Softmax methods select on the fp32 logits (softmax is strictly monotone,
 *    so the top-k set is the same in exact arithmetic).
 *  - Ties: lower expert index wins; lower group index wins for groups; the k
 *    ids of a token are listed in selection order (key desc, index asc).
 *  - DeepSeek-V3 sigmoid is the fp64 value 1/(1+exp(-l)) rounded once to
 *    fp32; values within 2^-45 (relative) of an fp32 rounding midpoint are
 *    re-evaluated in long double and counted ("hard cases").
 *  - The biased key and the group score are single fp32 additions.
 *  - Default honours an explicit renormalise flag (vLLM FusedTopKRouter).
 *  - The 1e-20 guard applies to DeepSeek-V3 only; the routed scaling factor
 *    multiplies every method's scales (1.0 unless given).
 *  - Llama4: the k largest logits (the name fixes k = 1; larger k keeps the
 *    same rule), each weighted by its own sigmoid, no renormalisation.
 *  - MiniMax2 / SigmoidRenorm select on the same fp32 keys as DeepSeek-V3
 *    with one group (fl32 sigmoid, plus the bias for MiniMax2 only) and
 *    divide the chosen unbiased sigmoids by their sum.
 *  - w13 rows [0, I) are the gate projection, rows [I, 2I) the up projection;
 *    SwiGLU h = silu(gate) * up with silu(z) = z / (1 + exp(-z)).
 *  - fp8 weights: OCP e4m3fn codes times an fp32 scale per 128x128 block of
 *    each [out, in] matrix.
 *  - The shared expert is group E (+s), weight 1.0, rows P + s*T + t.
 *  - fp8 activations: each row is cut into blocks of 128 consecutive
 *    channels; a block's scale is s = fl32(amax / 448) and its codes are
 *    e4m3(fl32(v / s)), rounded to nearest, ties to even, saturating at
 *    +-448; a block whose scale is 0 encodes as zeros.  The input x is
 *    quantised once per token (before the permute); the FFN intermediate h
 *    is rounded once to fp32 and quantised the same way per row and 128
 *    intermediate channels before FC2.
 *
 * All floating point is fp64 except where the method itself fixes fp32 (the
 * selection keys).  Inputs in bf16/fp8/fp32 are decoded exactly to fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "moe_oracle.h"

/* ---------------------------------------------------------------- formats */

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_decode_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP float8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent 0 is subnormal (m/8 * 2^-6). */
double oracle_decode_e4m3(uint8_t bits)
{
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int m = bits & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

static double load_elem(const void* base, int dtype, size_t i)
{
    switch (dtype) {
    case ORACLE_F32:
        return (double)((const float*)base)[i];
    case ORACLE_BF16:
        return oracle_decode_bf16(((const uint16_t*)base)[i]);
    default:
        return oracle_decode_e4m3(((const uint8_t*)base)[i]);
    }
}

/* fp32 -> OCP e4m3fn code: round to nearest, ties to even; magnitudes past
 * the largest finite value (448) saturate to it; the sign of zero is kept;
 * NaN -> 0x7F.  Normal codes hold (1 + m/8) 2^(e-7), subnormals m/8 2^-6, so
 * the quantum is 2^-9 below 2^-6 and 2^(e-3) in binade [2^e, 2^(e+1)). */
uint8_t oracle_encode_e4m3(float f)
{
    if (isnan(f))
        return 0x7F;
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    double a = fabs((double)f);
    if (a >= 448.0)
        return sign | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* n/8 * 2^-6 for n = 0..8; n = 8 is the smallest normal, code 0x08 */
        double n = rint(a / ldexp(1.0, -9)); /* exact scaling, ties to even */
        return sign | (uint8_t)n;
    }
    int ex;
    frexp(a, &ex); /* a = fr 2^ex, fr in [0.5, 1): binade e = ex - 1 */
    int e = ex - 1;
    double n = rint(a / ldexp(1.0, e - 3)); /* 8..16 */
    if (n == 16.0) {
        e += 1;
        n = 8.0;
    }
    return sign | (uint8_t)(((e + 7) << 3) | ((int)n - 8));
}

/* One block of `n` fp32 values: s = fl32(amax / 448), q = e4m3(fl32(v / s)).
 * Both divisions are single-precision IEEE divisions (correctly rounded). */
static float quantize_block(const float* v, int n, uint8_t* q)
{
    float amax = 0.0f;
    for (int i = 0; i < n; ++i)
        if (fabsf(v[i]) > amax)
            amax = fabsf(v[i]);
    float s = amax / 448.0f;
    for (int i = 0; i < n; ++i)
        q[i] = (s == 0.0f) ? 0 : oracle_encode_e4m3(v[i] / s);
    return s;
}

/* 1x128 block quantisation of x [rows, cols] (fp32 or bf16 values; cols a
 * multiple of 128): q [rows, cols] e4m3 codes, s [rows, cols / 128]. */
int oracle_quantize_fp8(const void* x, int dt, int rows, int cols, uint8_t* q, float* s)
{
    if (cols % 128 != 0 || (dt != ORACLE_F32 && dt != ORACLE_BF16))
        return -1;
    float v[128];
    for (int r = 0; r < rows; ++r)
        for (int b = 0; b < cols / 128; ++b) {
            size_t base = (size_t)r * cols + (size_t)b * 128;
            for (int i = 0; i < 128; ++i)
                v[i] = (float)load_elem(x, dt, base + i); /* exact */
            s[(size_t)r * (cols / 128) + b] = quantize_block(v, 128, q + base);
        }
    return 0;
}

/* ---------------------------------------------------------------- routing */

typedef struct {
    float key;
    int idx;
} cand_t;

/* Order: larger key first; equal keys -> smaller index first. */
static int cand_cmp(const void* pa, const void* pb)
{
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

/* fp32 sigmoid defined as the fp64 sigmoid rounded once to fp32; near a
 * rounding midpoint the fp64 value is not trusted and long double decides. */
float oracle_sigmoid_f32(float l, int* hard)
{
    double v = 1.0 / (1.0 + exp(-(double)l));
    float f = (float)v;
    double up = 0.5 * ((double)f + (double)nextafterf(f, INFINITY));
    double dn = 0.5 * ((double)f + (double)nextafterf(f, -INFINITY));
    double tol = ldexp(fabs(v), -45);
    if (fabs(v - up) <= tol || fabs(v - dn) <= tol) {
        long double lv = 1.0L / (1.0L + expl(-(long double)l));
        f = (float)lv;
        if (hard) *hard += 1;
    }
    return f;
}

/* Routing of one token.  ids/scales receive k entries in selection order. */
static void route_token(const float* l, int E, int method, int k, int n_group,
                        int topk_group, const float* bias, double scaling,
                        int renorm, int32_t* ids, double* scales, int* hard,
                        cand_t* c /* scratch [E] */, float* sig /* scratch [E] */)
{
    if (method == ORACLE_DEEPSEEKV3) {
        /* scores = sigmoid(logits); biased keys decide selection only. */
        int gsz = E / n_group;
        cand_t gc[256];
        unsigned char gsel[256];
        float keyv[256];
        for (int e = 0; e < E; ++e) {
            sig[e] = oracle_sigmoid_f32(l[e], hard);
            keyv[e] = sig[e] + (bias ? bias[e] : 0.0f); /* one fp32 add */
        }
        /* group score = sum of the two largest biased keys of the group */
        for (int g = 0; g < n_group; ++g) {
            for (int i = 0; i < gsz; ++i) {
                c[i].key = keyv[g * gsz + i];
                c[i].idx = g * gsz + i;
            }
            qsort(c, (size_t)gsz, sizeof(cand_t), cand_cmp);
            gc[g].key = c[0].key + c[1].key; /* one fp32 add */
            gc[g].idx = g;
        }
        /* keep the topk_group best groups */
        qsort(gc, (size_t)n_group, sizeof(cand_t), cand_cmp);
        memset(gsel, 0, sizeof gsel);
        for (int i = 0; i < topk_group; ++i)
            gsel[gc[i].idx] = 1;
        /* top-k experts among the kept groups (others masked out) */
        int n = 0;
        for (int e = 0; e < E; ++e) {
            if (gsel[e / gsz]) {
                c[n].key = keyv[e];
                c[n].idx = e;
                ++n;
            }
        }
        qsort(c, (size_t)n, sizeof(cand_t), cand_cmp);
        /* weights from the unbiased scores of the chosen experts */
        double sum = 0.0;
        for (int j = 0; j < k; ++j)
            sum += (double)sig[c[j].idx];
        sum += 1e-20;
        for (int j = 0; j < k; ++j) {
            ids[j] = c[j].idx;
            scales[j] = (double)sig[c[j].idx] / sum * scaling;
        }
        return;
    }

    if (method == ORACLE_MINIMAX2 || method == ORACLE_SIGMOID_RENORM) {
        /* sigmoid scores; MiniMax2 adds the bias to the selection key only */
        for (int e = 0; e < E; ++e) {
            sig[e] = oracle_sigmoid_f32(l[e], hard);
            c[e].key = (method == ORACLE_MINIMAX2 && bias) ? sig[e] + bias[e] /* one fp32 add */
                                                           : sig[e];
            c[e].idx = e;
        }
        qsort(c, (size_t)E, sizeof(cand_t), cand_cmp);
        double sum = 0.0;
        for (int j = 0; j < k; ++j)
            sum += (double)sig[c[j].idx];
        for (int j = 0; j < k; ++j) {
            ids[j] = c[j].idx;
            scales[j] = (double)sig[c[j].idx] / sum * scaling;
        }
        return;
    }

    /* softmax family and Llama4: the top-k set is selected on the fp32 logits */
    for (int e = 0; e < E; ++e) {
        c[e].key = l[e];
        c[e].idx = e;
    }
    qsort(c, (size_t)E, sizeof(cand_t), cand_cmp);
    for (int j = 0; j < k; ++j)
        ids[j] = c[j].idx;

    if (method == ORACLE_LLAMA4) {
        /* Top1 -> Sigmoid: each kept expert weighs its own sigmoid */
        for (int j = 0; j < k; ++j)
            scales[j] = 1.0 / (1.0 + exp(-(double)c[j].key)) * scaling;
        return;
    }
    if (method == ORACLE_RENORMALIZE) {
        /* TopK -> Softmax over the selected logits only */
        double m = (double)c[0].key, z = 0.0;
        for (int j = 0; j < k; ++j)
            z += exp((double)c[j].key - m);
        for (int j = 0; j < k; ++j)
            scales[j] = exp((double)c[j].key - m) / z;
    } else {
        /* Default: Softmax over all experts -> TopK (-> renormalise when the
         * flag asks).  RenormalizeNaive: Softmax -> TopK -> Renormalize. */
        double m = (double)c[0].key, z = 0.0;
        for (int e = 0; e < E; ++e)
            z += exp((double)l[e] - m);
        double zs = 0.0;
        for (int j = 0; j < k; ++j) {
            scales[j] = exp((double)c[j].key - m) / z;
            zs += scales[j];
        }
        if (method == ORACLE_RENORMALIZE_NAIVE || renorm)
            for (int j = 0; j < k; ++j)
                scales[j] /= zs;
    }
    for (int j = 0; j < k; ++j)
        scales[j] *= scaling;
}

int oracle_route(const float* logits, int T, int E, int method, int k, int n_group,
                 int topk_group, const float* bias, double scaling, int renorm,
                 int32_t* ids, double* scales, int64_t* hard_cases)
{
    if (E < 1 || E > 256 || k < 1 || k > E)
        return -1;
    if (method == ORACLE_DEEPSEEKV3) {
        if (n_group < 1 || E % n_group || topk_group < 1 || topk_group > n_group ||
            E / n_group < 2 || k > topk_group * (E / n_group))
            return -1;
    } else if (method != ORACLE_DEFAULT && method != ORACLE_RENORMALIZE &&
               method != ORACLE_RENORMALIZE_NAIVE && method != ORACLE_LLAMA4 &&
               method != ORACLE_MINIMAX2 && method != ORACLE_SIGMOID_RENORM) {
        return -1;
    }
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)E);
    float* sig = (float*)malloc(sizeof(float) * (size_t)E);
    int hard = 0;
    for (int t = 0; t < T; ++t)
        route_token(logits + (size_t)t * E, E, method, k, n_group, topk_group, bias,
                    scaling, renorm, ids + (size_t)t * k, scales + (size_t)t * k, &hard, c,
                    sig);
    free(c);
    free(sig);
    if (hard_cases) *hard_cases = hard;
    return 0;
}

/* ---------------------------------------------------------------- permute */

/* Counting sort of the flat pairs p = t*k + j by expert id, stable in p.
 * offsets[g] = first row of group g; routed groups hold P rows in total,
 * shared group E+s holds rows P + s*T + t in token order. */
int oracle_permute(const int32_t* ids, int T, int k, int E, int n_shared,
                   int32_t* offsets, int32_t* permuted_pair, int32_t* unpermute)
{
    int P = T * k;
    int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int g = 0; g <= E + n_shared; ++g)
        offsets[g] = 0;
    for (int p = 0; p < P; ++p) {
        if (ids[p] < 0 || ids[p] >= E) {
            free(seen);
            return -1;
        }
        offsets[ids[p] + 1] += 1;
    }
    for (int e = 0; e < E; ++e)
        offsets[e + 1] += offsets[e];
    for (int s = 0; s < n_shared; ++s)
        offsets[E + s + 1] = offsets[E + s] + T;
    for (int p = 0; p < P; ++p) {
        int e = ids[p];
        int row = offsets[e] + seen[e]++;
        permuted_pair[row] = p;
        unpermute[p] = row;
    }
    free(seen);
    return 0;
}

/* ------------------------------------------------------------- expert FFN */

/* Weight of group g, matrix [rows, cols], element (r, c), dequantised. */
static double weight_at(const void* w, int wdt, const float* scale, int g, int rows, int cols,
                        int r, int c)
{
    size_t i = ((size_t)g * rows + r) * cols + c;
    double v = load_elem(w, wdt, i);
    if (wdt == ORACLE_FP8) {
        int sr = rows / 128, sc = cols / 128;
        v *= (double)scale[((size_t)g * sr + r / 128) * sc + c / 128];
    }
    return v;
}

/* Expert g applied to one activation row a[H]:
 *   gate = W1 a, up = W3 a (rows [0,I) and [I,2I) of w13[g]),
 *   h = silu(gate) * up, out = W2 h.  h (size I) receives h.  With fp8
 *   activations (quant_h), FC2 reads h rounded to fp32, quantised in 1x128
 *   blocks and dequantised: hq = e4m3 value * block scale. */
static void expert_apply(const oracle_weights* W, int g, const double* a, double* h,
                         double* out, int quant_h)
{
    int H = W->H, I = W->I;
    for (int i = 0; i < I; ++i) {
        double gate = 0.0, up = 0.0;
        for (int c = 0; c < H; ++c) {
            gate += weight_at(W->w13, W->wdt, W->w13_scale, g, 2 * I, H, i, c) * a[c];
            up += weight_at(W->w13, W->wdt, W->w13_scale, g, 2 * I, H, I + i, c) * a[c];
        }
        h[i] = gate / (1.0 + exp(-gate)) * up;
    }
    const double* hin = h;
    double* hq = NULL;
    if (quant_h) {
        hq = (double*)malloc(sizeof(double) * (size_t)I);
        float v[128];
        uint8_t q[128];
        for (int b = 0; b < I / 128; ++b) {
            for (int i = 0; i < 128; ++i)
                v[i] = (float)h[b * 128 + i];
            float s = quantize_block(v, 128, q);
            for (int i = 0; i < 128; ++i)
                hq[b * 128 + i] = oracle_decode_e4m3(q[i]) * (double)s;
        }
        hin = hq;
    }
    for (int o = 0; o < H; ++o) {
        double acc = 0.0;
        for (int i = 0; i < I; ++i)
            acc += weight_at(W->w2, W->wdt, W->w2_scale, g, H, I, o, i) * hin[i];
        out[o] = acc;
    }
    free(hq);
}

/* Activation row t, exact in fp64; fp8 codes are dequantised with their
 * row's 1x128 block scales x_scale [T, H/128]. */
static void load_row(const void* x, int act, const float* x_scale, int H, int t, double* a)
{
    for (int c = 0; c < H; ++c) {
        a[c] = load_elem(x, act, (size_t)t * H + c);
        if (act == ORACLE_FP8)
            a[c] *= (double)x_scale[(size_t)t * (H / 128) + c / 128];
    }
}

/* Output rows of the expert FFN for the permuted rows listed in `rows`:
 * row r belongs to the group g with offsets[g] <= r < offsets[g+1]; its token
 * is permuted_pair[r] / k for routed groups and r - offsets[g] for shared
 * ones.  out: [n_rows, H];  h_out (nullable): [n_rows, I]. */
int oracle_expert_rows(const oracle_weights* W, const void* x, int act, const float* x_scale,
                       int T, int k, int E,
                       int n_shared, const int32_t* offsets, const int32_t* permuted_pair,
                       const int32_t* rows, int n_rows, double* h_out, double* out)
{
    int G = E + n_shared;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int i = 0; i < n_rows; ++i) {
        int r = rows[i];
        int g = -1;
        for (int q = 0; q < G; ++q)
            if (offsets[q] <= r && r < offsets[q + 1]) g = q;
        if (g < 0) {
            bad += 1;
            continue;
        }
        int t = (g < E) ? permuted_pair[r] / k : r - offsets[g];
        double* a = (double*)malloc(sizeof(double) * (size_t)W->H);
        double* h = (double*)malloc(sizeof(double) * (size_t)W->I);
        load_row(x, act, x_scale, W->H, t, a);
        expert_apply(W, g, a, h, out + (size_t)i * W->H, act == ORACLE_FP8);
        if (h_out)
            memcpy(h_out + (size_t)i * W->I, h, sizeof(double) * (size_t)W->I);
        free(a);
        free(h);
    }
    (void)T;
    return bad ? -1 : 0;
}

/* The layer by its definition, for the tokens listed in `tokens`:
 *   y_t = sum_j scales[t,j] * E_{ids[t,j]}(x_t)  +  sum_s E_{E+s}(x_t).
 * No permute is involved.  y: [n_tokens, H]. */
int oracle_layer_tokens(const oracle_weights* W, const void* x, int act, const float* x_scale,
                        int T, int k, int E,
                        int n_shared, const int32_t* ids, const double* scales,
                        const int32_t* tokens, int n_tokens, double* y)
{
    int H = W->H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int i = 0; i < n_tokens; ++i) {
        int t = tokens[i];
        if (t < 0 || t >= T) {
            bad += 1;
            continue;
        }
        double* a = (double*)malloc(sizeof(double) * (size_t)H);
        double* h = (double*)malloc(sizeof(double) * (size_t)W->I);
        double* o = (double*)malloc(sizeof(double) * (size_t)H);
        double* yt = y + (size_t)i * H;
        load_row(x, act, x_scale, H, t, a);
        for (int c = 0; c < H; ++c)
            yt[c] = 0.0;
        for (int j = 0; j < k; ++j) {
            expert_apply(W, ids[(size_t)t * k + j], a, h, o, act == ORACLE_FP8);
            for (int c = 0; c < H; ++c)
                yt[c] += scales[(size_t)t * k + j] * o[c];
        }
        for (int s = 0; s < n_shared; ++s) {
            expert_apply(W, E + s, a, h, o, act == ORACLE_FP8);
            for (int c = 0; c < H; ++c)
                yt[c] += o[c];
        }
        free(a);
        free(h);
        free(o);
    }
    return bad ? -1 : 0;
}

/* ---------------------------------------------------------------- finalize */

/* y_t = sum_j scales[t,j] * fc2[unpermute[t*k+j]] + sum_s fc2[P + s*T + t].
 * fc2: [R, H] in `dt`; y: [T, H] fp64. */
int oracle_finalize(const void* fc2, int dt, const int32_t* unpermute, const double* scales,
                    int T, int k, int H, int n_shared, double* y)
{
    size_t P = (size_t)T * k;
    for (int t = 0; t < T; ++t) {
        double* yt = y + (size_t)t * H;
        for (int c = 0; c < H; ++c)
            yt[c] = 0.0;
        for (int j = 0; j < k; ++j) {
            size_t row = (size_t)unpermute[(size_t)t * k + j];
            for (int c = 0; c < H; ++c)
                yt[c] += scales[(size_t)t * k + j] * load_elem(fc2, dt, row * H + c);
        }
        for (int s = 0; s < n_shared; ++s) {
            size_t row = P + (size_t)s * T + t;
            for (int c = 0; c < H; ++c)
                yt[c] += load_elem(fc2, dt, row * H + c);
        }
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
