/*
 * Declarations of the CPU oracle for the ThriftAttention forward pass.
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the HIP library.
 * Host pointers throughout; tensors are contiguous, [batch, head, seq, dim].
 */
#ifndef THRIFT_ORACLE_H
#define THRIFT_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#define THO_NVFP4 0 /* E2M1 + per-16 E4M3 block scale + per-slice fp32 scale */
#define THO_MX 1    /* E2M1 + per-32 E8M0 block scale */
#define THO_NVFP4_MXP 2 /* attention only: NVFP4 Q, K, V with P quantised MX-style */
#define THO_AXIS_D 0 /* groups along the head dimension (Q, K) */
#define THO_AXIS_S 1 /* groups along the sequence, stored transposed (V) */

double tho_half_to_double(uint16_t h);
double tho_round_to_half(double x);
double tho_e2m1_value(int code);
int tho_e2m1_encode(double x, double s);
double tho_e4m3_value(int code);
int tho_e4m3_encode_ratio(double num, double den);
int tho_mx_exponent(double amax);
int tho_group_size(int fmt);
int tho_pad_s(int S);

int tho_kmax(int S, int bq, int bk, int causal, int topk_count, int topk_bp);
int tho_kmax_kv(int Sq, int Sk, int bq, int bk, int causal, int topk_count, int topk_bp);
void tho_block_means(const uint16_t* x16, int B, int H, int S, int D, int blk, float* means);
float tho_block_score(const float* qm, const float* km, int D);
void tho_select(const uint16_t* q16, const uint16_t* k16, int B, int Hq, int Hkv, int S, int D,
                int bq, int bk, int causal, int topk_count, int topk_bp, int32_t* idx,
                int32_t* cnt, int kmax, float* scores);
/* Sq queries (the last Sq positions) against Sk keys; tho_select is Sq = Sk. */
void tho_select_kv(const uint16_t* q16, const uint16_t* k16, int B, int Hq, int Hkv, int Sq, int Sk,
                   int D, int bq, int bk, int causal, int topk_count, int topk_bp, int32_t* idx,
                   int32_t* cnt, int kmax, float* scores);
/* One budget per query head over all its valid pairs (K = ceil(P bp / 10^4)). */
void tho_select_head_kv(const uint16_t* q16, const uint16_t* k16, int B, int Hq, int Hkv, int Sq,
                        int Sk, int D, int bq, int bk, int causal, int topk_count, int topk_bp,
                        int32_t* idx, int32_t* cnt, int kmax);

void tho_quantize(const uint16_t* x16, int B, int H, int S, int D, int axis, int fmt,
                  uint8_t* codes, uint8_t* scales, float* tensor_scale);
void tho_dequant_row(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                     size_t bh, int S, int D, int s, int fmt, double* out);
void tho_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int B,
                    int H, int S, int D, int axis, int fmt, double* out);

void tho_attention(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                   const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                   const uint8_t* k4s, const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                   const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                   int B, int Hq, int Hkv, int S, int D, int bq, int bk, int causal,
                   double sm_scale, const int32_t* work, int nwork, double* o, double* lse,
                   int32_t* amb_row, double* amb_delta, int amb_cap, int* amb_n);
void tho_attention_kv(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                      const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                      const uint8_t* k4s, const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                      const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                      int B, int Hq, int Hkv, int S, int Sk, int D, int bq, int bk, int causal,
                      double sm_scale, const int32_t* work, int nwork, double* o, double* lse,
                      int32_t* amb_row, double* amb_delta, int amb_cap, int* amb_n);
/* Forward with Attn-QAT's high-precision output O' (ohp [B,Hq,S,D]); Sq = Sk. */
void tho_attention_hp(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                      const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                      const uint8_t* k4s, const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                      const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                      int B, int Hq, int Hkv, int S, int D, int bq, int bk, int causal,
                      double sm_scale, const int32_t* work, int nwork, double* o, double* lse,
                      double* ohp);
/* Backward (Attn-QAT): dq [B,Hq,S,D], dk and dv [B,Hkv,S,D] from the
 * forward's lse and O' and the output gradient do16; Sq = Sk. */
void tho_attention_bwd(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                       const uint8_t* q4c, const uint8_t* q4s, const float* q4t,
                       const uint8_t* k4c, const uint8_t* k4s, const float* k4t,
                       const uint8_t* v4c, const uint8_t* v4s, const float* v4t, int fmt,
                       const int32_t* idx, const int32_t* cnt, int kmax, int B, int Hq, int Hkv,
                       int S, int D, int bq, int bk, int causal, double sm_scale,
                       const double* lse, const double* ohp, const uint16_t* do16,
                       const int32_t* qwork, int nqwork, const int32_t* kwork, int nkwork,
                       double* dq, double* dk, double* dv, double* udv);
void tho_row_probs(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                   const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                   const uint8_t* k4s, const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                   const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                   int B, int Hq, int Hkv, int S, int D, int bq, int bk, int causal,
                   double sm_scale, const double* lse, int b, int hq, int r, int32_t* kind,
                   double* p, double* pt);
/* Middle precision tier (a variant; MX format): MXFP8 tensors and the
 * forward with the blocks idx2 lists and idx does not on the FP8 path. */
int tho_mx8_exponent(double amax);
int tho_e4m3_encode_signed(double x, double s);
void tho_quantize_fp8(const uint16_t* x16, int B, int H, int S, int D, int axis, uint8_t* codes,
                      uint8_t* scales);
void tho_dequant8_row(const uint8_t* codes, const uint8_t* scales, size_t bh, int S, int D, int s,
                      double* out);
void tho_dequantize_fp8(const uint8_t* codes, const uint8_t* scales, int B, int H, int S, int D,
                        int axis, double* out);
void tho_attention_tiers(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                         const uint8_t* q4c, const uint8_t* q4s, const uint8_t* k4c,
                         const uint8_t* k4s, const uint8_t* v4c, const uint8_t* v4s,
                         const uint8_t* q8c, const uint8_t* q8s, const uint8_t* k8c,
                         const uint8_t* k8s, const uint8_t* v8c, const uint8_t* v8s,
                         const int32_t* idx, const int32_t* cnt, int kmax, const int32_t* idx2,
                         const int32_t* cnt2, int kmax2, int B, int Hq, int Hkv, int S, int D,
                         int bq, int bk, int causal, double sm_scale, const int32_t* work,
                         int nwork, double* o, double* lse, int32_t* amb_row, double* amb_delta,
                         int amb_cap, int* amb_n);
void tho_fp4_scores(const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                    const uint8_t* k4s, const float* k4t, int fmt, int S, int D, int r, int c0,
                    int c1, double* out);

/* Relative evaluation-error bound of a tile value (path: 0 MX FP4, 1 NVFP4
 * FP4, 2 MXFP8 tier, 3 FP16, 4 NVFP4 tensors with MX-style P; b, bmax: the chain sums of the key's and the
 * tile maximum's scores, dt = t - mt, mt: log2 units). */
double tho_eval_rel(int path, double b, double bmax, double dt, double mt);

/* Test hook: values and decisions of one tile row (see the source). */
int tho_p_tile_decisions(const double* t, const double* tb, const int* mask, int n, int prec, int epath,
                         double* pq, int* k0, int* k1, double* dp, int maxf);

void tho_e2m1_encode_array(const double* x, const double* s, size_t n, uint8_t* out);
void tho_e4m3_encode_ratio_array(const double* num, const double* den, size_t n, uint8_t* out);
void tho_round_to_half_array(const double* x, size_t n, double* out);
void tho_half_to_double_array(const uint16_t* h, size_t n, double* out);
#endif
