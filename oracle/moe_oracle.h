/* moe_oracle.h -- CPU oracle of the MoE layer forward (test infrastructure
 * only; never linked into the product library).  Definitions and the pages
 * they follow are documented in moe_oracle.c. */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_FP8 = 2 };
enum {
    ORACLE_DEFAULT = 0,
    ORACLE_RENORMALIZE = 1,
    ORACLE_DEEPSEEKV3 = 2,
    ORACLE_LLAMA4 = 3,
    ORACLE_RENORMALIZE_NAIVE = 4,
    ORACLE_MINIMAX2 = 5,
    ORACLE_SIGMOID_RENORM = 6
};

typedef struct {
    int H, I, wdt;
    const void* w13;        /* [G, 2I, H] */
    const void* w2;         /* [G, H, I]  */
    const float* w13_scale; /* [G, 2I/128, H/128] (fp8 only) */
    const float* w2_scale;  /* [G, H/128, I/128]  (fp8 only) */
} oracle_weights;

double oracle_decode_bf16(uint16_t bits);
double oracle_decode_e4m3(uint8_t bits);
uint8_t oracle_encode_e4m3(float f);
int oracle_quantize_fp8(const void* x, int dt, int rows, int cols, uint8_t* q, float* s);
float oracle_sigmoid_f32(float l, int* hard);

int oracle_route(const float* logits, int T, int E, int method, int k, int n_group,
                 int topk_group, const float* bias, double scaling, int renorm,
                 int32_t* ids, double* scales, int64_t* hard_cases);
int oracle_permute(const int32_t* ids, int T, int k, int E, int n_shared, int32_t* offsets,
                   int32_t* permuted_pair, int32_t* unpermute);
/* act == ORACLE_FP8: x holds e4m3 codes [T, H] with 1x128 scales x_scale [T, H/128]
 * (NULL otherwise), and h is quantised the same way before FC2. */
int oracle_expert_rows(const oracle_weights* W, const void* x, int act, const float* x_scale,
                       int T, int k, int E,
                       int n_shared, const int32_t* offsets, const int32_t* permuted_pair,
                       const int32_t* rows, int n_rows, double* h_out, double* out);
int oracle_layer_tokens(const oracle_weights* W, const void* x, int act, const float* x_scale,
                        int T, int k, int E,
                        int n_shared, const int32_t* ids, const double* scales,
                        const int32_t* tokens, int n_tokens, double* y);
int oracle_finalize(const void* fc2, int dt, const int32_t* unpermute, const double* scales,
                    int T, int k, int H, int n_shared, double* y);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
