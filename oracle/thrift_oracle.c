/*
 * Plain CPU oracle for the ThriftAttention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library: every number format, every rounding decision and every loop
 * below is written out again from the definitions.
 *
 * Source of the method: "ThriftAttention: Selective Mixed Precision for
 * Long-Context FP4 Attention" (gist.science summaries in Dutch and French,
 * sections "Methodologie" / "Méthodologie").  What the pages fix:
 *   - Q and K/V are cut into blocks; each (query block i, key block j) pair is
 *     scored by the dot product of the blocks' token means, S^_ij = qbar_i.kbar_j;
 *   - the top-k pairs run in FP16, every other pair in FP4 (NVFP4 micro-scaling);
 *   - both paths are merged by one online softmax in the style of
 *     FlashAttention-2, with a two-level quantisation of the probability
 *     blocks on the FP4 path (taken from SageAttention3);
 *   - the FP4 path runs first, the FP16 path over the promoted blocks second.
 * Everything else is a reading of where the pages are silent; each reading is
 * named at the function that takes it.
 *
 * Arithmetic: fp64 throughout, except where the method itself fixes a
 * precision (the FP4 / FP8 / FP16 roundings) and in the block-selection
 * scores, whose fp32 fused-multiply-add chain is the precision the selection
 * decision is taken in on both sides.  No fast-math, no contraction
 * (-ffp-contract=off): every rounding is the one written.
 *
 * Parity pins for each function live in tests/ (see the test files' headers).
 * Two readings are pinned only as implemented, since nothing on the pages
 * confirms or refutes them (parity unpinned as readings): the NVFP4
 * second-level scale taken per (batch, head) slice, and the row sum taken
 * over the unquantised probabilities on both paths.
 */
#include "thrift_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define THO_LOG2E 1.4426950408889634073599246810019
#define THO_LN2 0.69314718055994530941723212145818

/* ------------------------------------------------------------------ */
/* fp16 (IEEE binary16) decoding and rounding                          */
/* ------------------------------------------------------------------ */

double tho_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even (the value is
 * returned as a double).  Overflow gives +-inf, as IEEE rounding does. */
double tho_round_to_half(double x) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  double a = fabs(x);
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  int ulp_exp = e - 11; /* 11 significant bits */
  if (ulp_exp < -24) ulp_exp = -24; /* subnormal spacing */
  double q = nearbyint(ldexp(a, -ulp_exp)); /* default mode: ties to even */
  double r = ldexp(q, ulp_exp);
  if (r > 65504.0) r = INFINITY;
  return x < 0 ? -r : r;
}

/* ------------------------------------------------------------------ */
/* FP4 E2M1, FP8 E4M3 and E8M0 (OCP microscaling formats)              */
/* ------------------------------------------------------------------ */

/* E2M1: one sign bit, two exponent bits (bias 1), one mantissa bit.  The
 * pages give the bit split and the count of 15 distinct values; the values
 * themselves follow from the split: 0, 0.5 (subnormal), 1, 1.5, 2, 3, 4, 6. */
static const double tho_e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double tho_e2m1_value(int code) {
  double v = tho_e2m1_mag[code & 7];
  return (code & 8) ? -v : v;
}

/* Code of the E2M1 value nearest to x/s, ties to the even code, magnitudes
 * above 6 saturating to 6, the sign of x kept (so -0 and small negatives give
 * code 8).  s > 0.  The decision is exact: |x| is compared with midpoint*s,
 * and callers pass an s whose product with a 3-bit midpoint is exact in fp64. */
int tho_e2m1_encode(double x, double s) {
  static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  double a = fabs(x);
  int code = 0;
  for (int k = 0; k < 7; ++k) {
    double t = mid[k] * s;
    if (a > t || (a == t && ((k + 1) & 1) == 0)) code = k + 1;
  }
  return code | (signbit(x) ? 8 : 0);
}

/* E4M3 ("FN" variant): bias 7, three mantissa bits, no infinities, codes
 * 0x7F/0xFF are NaN, largest finite 448, subnormals m * 2^-9. */
double tho_e4m3_value(int code) {
  int e = (code >> 3) & 0xF;
  int m = code & 7;
  double v;
  if ((code & 0x7F) == 0x7F) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return (code & 0x80) ? -v : v;
}

/* Non-negative E4M3 code nearest to num/den (num >= 0, den > 0), ties to the
 * even code, saturating at 448.  Exact: num is compared with midpoint*den. */
int tho_e4m3_encode_ratio(double num, double den) {
  int c = 0;
  for (int k = 0; k < 126; ++k) {
    double mid = 0.5 * (tho_e4m3_value(k) + tho_e4m3_value(k + 1));
    double t = mid * den;
    if (num > t || (num == t && ((k + 1) & 1) == 0))
      c = k + 1;
    else
      break;
  }
  return c;
}

/* MX shared exponent for an E2M1 group: the largest power of two not above
 * amax, divided by 2^2 (the largest power of two in E2M1), clamped to the
 * E8M0 range.  amax == 0 gives the smallest scale, 2^-127. */
int tho_mx_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int e;
  frexp(amax, &e); /* amax in [2^(e-1), 2^e) */
  int x = (e - 1) - 2;
  if (x < -127) x = -127;
  if (x > 127) x = 127;
  return x;
}

/* MX shared exponent for an E4M3 group (MXFP8, the middle precision tier):
 * the largest power of two not above amax, divided by 2^8 (the largest power
 * of two among E4M3's finite values), clamped to the E8M0 range.  The group
 * maximum then lands in [256, 512) and values above 448 saturate. */
int tho_mx8_exponent(double amax) {
  if (!(amax > 0.0)) return -127;
  int e;
  frexp(amax, &e);
  int x = (e - 1) - 8;
  if (x < -127) x = -127;
  if (x > 127) x = 127;
  return x;
}

/* E4M3 code of x / s (s > 0) with the sign of x kept: the magnitude's code
 * from tho_e4m3_encode_ratio (ties to even, saturating at 448), bit 7 set
 * for a negative x or -0, as for E2M1. */
int tho_e4m3_encode_signed(double x, double s) {
  return tho_e4m3_encode_ratio(fabs(x), s) | (signbit(x) ? 0x80 : 0);
}

/* ------------------------------------------------------------------ */
/* Block selection (pages: "Heuristische Blokkenselectie")             */
/* ------------------------------------------------------------------ */

static int tho_cdiv(int a, int b) { return (a + b - 1) / b; }

/* Valid key blocks of query block i for Sq queries against Sk keys
 * (Sq <= Sk): every block for non-causal attention; for causal attention
 * every block holding at least one key not after the block's last query,
 * the queries being the last Sq positions of the key sequence (for Sq = Sk
 * the two sequences are aligned at their starts; for Sq < Sk, as when new
 * tokens attend to a cache, at their ends). */
static int tho_valid_blocks_kv(int i, int Sq, int Sk, int bq, int bk, int causal) {
  int nk = tho_cdiv(Sk, bk);
  if (!causal) return nk;
  int last_q = (i + 1) * bq < Sq ? (i + 1) * bq - 1 : Sq - 1;
  return (Sk - Sq + last_q) / bk + 1;
}


/* Budget of promoted blocks for a query block with n valid key blocks:
 * topk_count >= 0 is an absolute count, otherwise ceil(n * topk_bp / 10^4)
 * (basis points of the valid pairs of that query block); never above n. */
static int tho_budget(int n, int topk_count, int topk_bp) {
  long long k;
  if (topk_count >= 0)
    k = topk_count;
  else
    k = ((long long)n * topk_bp + 9999) / 10000;
  return (int)(k < n ? k : n);
}

int tho_kmax_kv(int Sq, int Sk, int bq, int bk, int causal, int topk_count, int topk_bp) {
  int nq = tho_cdiv(Sq, bq), km = 0;
  for (int i = 0; i < nq; ++i) {
    int k = tho_budget(tho_valid_blocks_kv(i, Sq, Sk, bq, bk, causal), topk_count, topk_bp);
    if (k > km) km = k;
  }
  return km;
}

int tho_kmax(int S, int bq, int bk, int causal, int topk_count, int topk_bp) {
  return tho_kmax_kv(S, S, bq, bk, causal, topk_count, topk_bp);
}

/* Token mean of each block of rows (reading of the pages' "token means":
 * the plain arithmetic mean over the block's valid rows, masked or not).
 * The sum is formed in fp64, which is exact whatever the order: every fp16
 * value is an integer multiple of 2^-24 below 2^16 in magnitude, so a sum of
 * up to 2^13 of them is an integer multiple of 2^-24 below 2^53.  It is then
 * divided by the row count in fp64 and rounded once to fp32.
 * means: [B, H, nblk, D]. */
void tho_block_means(const uint16_t* x16, int B, int H, int S, int D, int blk, float* means) {
  int nb = tho_cdiv(S, blk);
  for (int bh = 0; bh < B * H; ++bh) {
    const uint16_t* x = x16 + (size_t)bh * S * D;
    for (int j = 0; j < nb; ++j) {
      int r0 = j * blk, r1 = r0 + blk < S ? r0 + blk : S;
      for (int d = 0; d < D; ++d) {
        double sum = 0.0;
        for (int r = r0; r < r1; ++r) sum += tho_half_to_double(x[(size_t)r * D + d]);
        means[((size_t)bh * nb + j) * D + d] = (float)(sum / (double)(r1 - r0));
      }
    }
  }
}

/* Importance score of a block pair: the fp32 dot product of the two means,
 * one fused multiply-add per channel, channels in ascending order. */
float tho_block_score(const float* qm, const float* km, int D) {
  float s = 0.0f;
  for (int d = 0; d < D; ++d) s = fmaf(qm[d], km[d], s);
  return s;
}

typedef struct {
  float s;
  int j;
} tho_cand;

/* Higher score first; equal scores (with -0 == +0) by lower block index. */
static int tho_cand_cmp(const void* a, const void* b) {
  const tho_cand* x = (const tho_cand*)a;
  const tho_cand* y = (const tho_cand*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return x->j - y->j;
}

static int tho_int_cmp(const void* a, const void* b) {
  int x = *(const int*)a, y = *(const int*)b;
  return (x > y) - (x < y);
}

/* Per query block (reading of the pages' top-k over the best-scoring block
 * pairs: the budget is taken per query block, so that every query block gets
 * its share; the pages' 5% share of query-key blocks is then met per block
 * row), keep the
 * k_i best-scoring valid key blocks.  The query head hq reads key head
 * hq / (Hq / Hkv).  idx: [B, Hq, nQ, kmax], ascending, padded with -1;
 * cnt: [B, Hq, nQ].  scores (optional): [B, Hq, nQ, nK], NaN where invalid. */
void tho_select_kv(const uint16_t* q16, const uint16_t* k16, int B, int Hq, int Hkv, int Sq, int Sk,
                   int D, int bq, int bk, int causal, int topk_count, int topk_bp, int32_t* idx,
                   int32_t* cnt, int kmax, float* scores) {
  int nq = tho_cdiv(Sq, bq), nk = tho_cdiv(Sk, bk), G = Hq / Hkv;
  float* qm = (float*)malloc(sizeof(float) * (size_t)B * Hq * nq * D);
  float* km = (float*)malloc(sizeof(float) * (size_t)B * Hkv * nk * D);
  tho_block_means(q16, B, Hq, Sq, D, bq, qm);
  tho_block_means(k16, B, Hkv, Sk, D, bk, km);
  tho_cand* cand = (tho_cand*)malloc(sizeof(tho_cand) * (size_t)nk);
  int* sel = (int*)malloc(sizeof(int) * (size_t)nk);
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq) {
      int hk = hq / G;
      for (int i = 0; i < nq; ++i) {
        size_t row = ((size_t)b * Hq + hq) * nq + i;
        int n = tho_valid_blocks_kv(i, Sq, Sk, bq, bk, causal);
        int k = tho_budget(n, topk_count, topk_bp);
        const float* qv = qm + row * D;
        for (int j = 0; j < n; ++j) {
          cand[j].s = tho_block_score(qv, km + (((size_t)b * Hkv + hk) * nk + j) * D, D);
          cand[j].j = j;
        }
        if (scores)
          for (int j = 0; j < nk; ++j) scores[row * nk + j] = j < n ? cand[j].s : NAN;
        qsort(cand, (size_t)n, sizeof(tho_cand), tho_cand_cmp);
        for (int t = 0; t < k; ++t) sel[t] = cand[t].j;
        qsort(sel, (size_t)k, sizeof(int), tho_int_cmp);
        for (int t = 0; t < kmax; ++t) idx[row * kmax + t] = t < k ? sel[t] : -1;
        cnt[row] = k;
      }
    }
  free(sel);
  free(cand);
  free(km);
  free(qm);
}

typedef struct {
  float s;
  int i, j;
} tho_pair;

/* Higher score first; equal scores (with -0 == +0) by lower query block, then lower key block. */
static int tho_pair_cmp(const void* a, const void* b) {
  const tho_pair* x = (const tho_pair*)a;
  const tho_pair* y = (const tho_pair*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  if (x->i != y->i) return x->i - y->i;
  return x->j - y->j;
}

/* Per-head budget: the other reading of the pages' top-k over the best-scoring
 * block pairs (ThriftAttention summaries, "Heuristische Blokkenselectie"), one
 * budget over all valid pairs of a query head: K = min(P, topk_count) or
 * ceil(P * topk_bp / 10^4) of its P valid pairs, the K best-scoring pairs
 * kept.  Scores as tho_select_kv.  idx [B, Hq, nQ, kmax]: each query block's
 * kept key blocks ascending, padded with -1; cnt [B, Hq, nQ]: their number.
 * kmax must be at least the largest count (at most the largest n_i). */
void tho_select_head_kv(const uint16_t* q16, const uint16_t* k16, int B, int Hq, int Hkv, int Sq,
                        int Sk, int D, int bq, int bk, int causal, int topk_count, int topk_bp,
                        int32_t* idx, int32_t* cnt, int kmax) {
  int nq = tho_cdiv(Sq, bq), nk = tho_cdiv(Sk, bk), G = Hq / Hkv;
  float* qm = (float*)malloc(sizeof(float) * (size_t)B * Hq * nq * D);
  float* km = (float*)malloc(sizeof(float) * (size_t)B * Hkv * nk * D);
  tho_block_means(q16, B, Hq, Sq, D, bq, qm);
  tho_block_means(k16, B, Hkv, Sk, D, bk, km);
  tho_pair* cand = (tho_pair*)malloc(sizeof(tho_pair) * (size_t)nq * nk);
  unsigned char* keep = (unsigned char*)malloc((size_t)nq * nk);
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq) {
      int hk = hq / G;
      long long P = 0;
      for (int i = 0; i < nq; ++i) {
        const float* qv = qm + (((size_t)b * Hq + hq) * nq + i) * D;
        int n = tho_valid_blocks_kv(i, Sq, Sk, bq, bk, causal);
        for (int j = 0; j < n; ++j) {
          cand[P].s = tho_block_score(qv, km + (((size_t)b * Hkv + hk) * nk + j) * D, D);
          cand[P].i = i;
          cand[P].j = j;
          ++P;
        }
      }
      long long K = topk_count >= 0 ? (long long)topk_count : (P * topk_bp + 9999) / 10000;
      if (K > P) K = P;
      qsort(cand, (size_t)P, sizeof(tho_pair), tho_pair_cmp);
      memset(keep, 0, (size_t)nq * nk);
      for (long long t = 0; t < K; ++t) keep[(size_t)cand[t].i * nk + cand[t].j] = 1;
      for (int i = 0; i < nq; ++i) {
        size_t row = ((size_t)b * Hq + hq) * nq + i;
        int c = 0;
        for (int j = 0; j < nk; ++j)
          if (keep[(size_t)i * nk + j]) {
            if (c < kmax) idx[row * kmax + c] = j;
            ++c;
          }
        for (int t = c; t < kmax; ++t) idx[row * kmax + t] = -1;
        cnt[row] = c;
      }
    }
  free(keep);
  free(cand);
  free(km);
  free(qm);
}

void tho_select(const uint16_t* q16, const uint16_t* k16, int B, int Hq, int Hkv, int S, int D,
                int bq, int bk, int causal, int topk_count, int topk_bp, int32_t* idx,
                int32_t* cnt, int kmax, float* scores) {
  tho_select_kv(q16, k16, B, Hq, Hkv, S, S, D, bq, bk, causal, topk_count, topk_bp, idx, cnt, kmax,
                scores);
}

/* ------------------------------------------------------------------ */
/* FP4 quantisation of Q, K, V (pages: FP4 path in NVFP4 micro-scaling) */
/* ------------------------------------------------------------------ */

/* Encode one group of n values with the scale rule of the format.
 *  NVFP4-style (per-16 E4M3 block scale under a per-slice fp32 scale sg):
 *    block byte = E4M3(amax_g / (6 sg)), element = E2M1(x / (E4M3 value * sg));
 *    a block whose scale rounds to 0 gets all-zero codes.
 *  MXFP4 (per-32 E8M0): exponent X from the group maximum, element = E2M1(x / 2^X).
 * Codes go to out[] one per value (unpacked); the scale byte is returned. */
static int tho_encode_group(const double* x, int n, int fmt, double sg, uint8_t* out) {
  double amax = 0.0;
  for (int t = 0; t < n; ++t)
    if (fabs(x[t]) > amax) amax = fabs(x[t]);
  if (fmt == THO_NVFP4) {
    int sb = tho_e4m3_encode_ratio(amax, 6.0 * sg);
    double s = tho_e4m3_value(sb) * sg; /* exact: 4 x 24 significant bits */
    for (int t = 0; t < n; ++t) out[t] = (uint8_t)(s > 0.0 ? tho_e2m1_encode(x[t], s) : 0);
    return sb;
  } else {
    int X = tho_mx_exponent(amax);
    double s = ldexp(1.0, X);
    for (int t = 0; t < n; ++t) out[t] = (uint8_t)tho_e2m1_encode(x[t], s);
    return X + 127;
  }
}

/* The per-slice fp32 scale of the NVFP4-style format (reading: one scale per
 * (batch, head) slice, so that the largest block maps onto 6 * 448):
 * sg = amax / (6 * 448) rounded to fp32, or 1 for an all-zero slice. */
static float tho_slice_scale(const uint16_t* x, size_t n) {
  double amax = 0.0;
  for (size_t t = 0; t < n; ++t) {
    double v = fabs(tho_half_to_double(x[t]));
    if (v > amax) amax = v;
  }
  return amax > 0.0 ? (float)(amax / 2688.0) : 1.0f;
}

int tho_group_size(int fmt) { return fmt == THO_NVFP4 ? 16 : 32; }
int tho_pad_s(int S) { return tho_cdiv(S, 64) * 64; }

/* Quantise x16 [B, H, S, D].
 *  axis THO_AXIS_D (Q, K): groups run along D; codes [B,H,S,D/2], scales [B,H,S,D/g].
 *  axis THO_AXIS_S (V, stored transposed): groups run along the sequence;
 *    codes [B,H,D,Sp/2], scales [B,H,D,Sp/g], Sp = S rounded up to 64, the
 *    padding tokens being zeros.
 * Two codes per byte, the even element in the low nibble.  tensor_scale
 * [B,H] is written for the NVFP4-style format only. */
void tho_quantize(const uint16_t* x16, int B, int H, int S, int D, int axis, int fmt,
                  uint8_t* codes, uint8_t* scales, float* tensor_scale) {
  int g = tho_group_size(fmt);
  int Sp = tho_pad_s(S);
  double vals[32];
  uint8_t c[32];
  for (int bh = 0; bh < B * H; ++bh) {
    const uint16_t* x = x16 + (size_t)bh * S * D;
    double sg = 1.0;
    if (fmt == THO_NVFP4) {
      float f = tho_slice_scale(x, (size_t)S * D);
      tensor_scale[bh] = f;
      sg = f;
    }
    if (axis == THO_AXIS_D) {
      for (int s = 0; s < S; ++s)
        for (int gi = 0; gi < D / g; ++gi) {
          for (int t = 0; t < g; ++t) vals[t] = tho_half_to_double(x[(size_t)s * D + gi * g + t]);
          int sb = tho_encode_group(vals, g, fmt, sg, c);
          scales[((size_t)bh * S + s) * (D / g) + gi] = (uint8_t)sb;
          uint8_t* dst = codes + ((size_t)bh * S + s) * (D / 2) + gi * g / 2;
          for (int t = 0; t < g; t += 2) dst[t / 2] = (uint8_t)(c[t] | (c[t + 1] << 4));
        }
    } else {
      for (int d = 0; d < D; ++d)
        for (int gi = 0; gi < Sp / g; ++gi) {
          for (int t = 0; t < g; ++t) {
            int s = gi * g + t;
            vals[t] = s < S ? tho_half_to_double(x[(size_t)s * D + d]) : 0.0;
          }
          int sb = tho_encode_group(vals, g, fmt, sg, c);
          scales[((size_t)bh * D + d) * (Sp / g) + gi] = (uint8_t)sb;
          uint8_t* dst = codes + ((size_t)bh * D + d) * (Sp / 2) + gi * g / 2;
          for (int t = 0; t < g; t += 2) dst[t / 2] = (uint8_t)(c[t] | (c[t + 1] << 4));
        }
    }
  }
}

/* MXFP8 (the middle precision tier; reading: OCP MX with E4M3 elements, one
 * E8M0 scale per 32 elements along the same axes as the FP4 tensors).
 *  axis THO_AXIS_D (Q, K): codes [B,H,S,D] one byte each, scales [B,H,S,D/32];
 *  axis THO_AXIS_S (V, stored transposed): codes [B,H,D,Sp], scales
 *    [B,H,D,Sp/32], padding tokens zero.
 * Per group: X = tho_mx8_exponent(amax), element = E4M3(x / 2^X), sign kept. */
void tho_quantize_fp8(const uint16_t* x16, int B, int H, int S, int D, int axis, uint8_t* codes,
                      uint8_t* scales) {
  int Sp = tho_pad_s(S);
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh) {
    double vals[32];
    const uint16_t* x = x16 + (size_t)bh * S * D;
    int rows = axis == THO_AXIS_D ? S : D;
    int len = axis == THO_AXIS_D ? D : Sp;
    for (int r = 0; r < rows; ++r)
      for (int gi = 0; gi < len / 32; ++gi) {
        double amax = 0.0;
        for (int t = 0; t < 32; ++t) {
          int e = gi * 32 + t;
          double v;
          if (axis == THO_AXIS_D)
            v = tho_half_to_double(x[(size_t)r * D + e]);
          else
            v = e < S ? tho_half_to_double(x[(size_t)e * D + r]) : 0.0;
          vals[t] = v;
          if (fabs(v) > amax) amax = fabs(v);
        }
        int X = tho_mx8_exponent(amax);
        double sc = ldexp(1.0, X);
        scales[((size_t)bh * rows + r) * (len / 32) + gi] = (uint8_t)(X + 127);
        uint8_t* dst = codes + ((size_t)bh * rows + r) * len + gi * 32;
        for (int t = 0; t < 32; ++t) dst[t] = (uint8_t)tho_e4m3_encode_signed(vals[t], sc);
      }
  }
}

/* Row s of slice bh of an MXFP8 tensor quantised along D, decoded. */
void tho_dequant8_row(const uint8_t* codes, const uint8_t* scales, size_t bh, int S, int D, int s,
                      double* out) {
  for (int d = 0; d < D; ++d) {
    size_t row = (size_t)bh * S + s;
    out[d] = tho_e4m3_value(codes[row * D + d]) * ldexp(1.0, scales[row * (D / 32) + d / 32] - 127);
  }
}

/* An MXFP8 tensor back to fp64 in the [B, H, S, D] orientation. */
void tho_dequantize_fp8(const uint8_t* codes, const uint8_t* scales, int B, int H, int S, int D,
                        int axis, double* out) {
  int Sp = tho_pad_s(S);
  for (int bh = 0; bh < B * H; ++bh)
    for (int s = 0; s < S; ++s)
      for (int d = 0; d < D; ++d) {
        size_t e, si;
        if (axis == THO_AXIS_D) {
          e = ((size_t)bh * S + s) * D + d;
          si = ((size_t)bh * S + s) * (D / 32) + d / 32;
        } else {
          e = (size_t)bh * D * Sp + (size_t)d * Sp + s;
          si = ((size_t)bh * D + d) * (Sp / 32) + s / 32;
        }
        out[((size_t)bh * S + s) * D + d] = tho_e4m3_value(codes[e]) * ldexp(1.0, scales[si] - 127);
      }
}

/* Decoded scale of one group. */
static double tho_group_scale(int fmt, int byte, double sg) {
  return fmt == THO_NVFP4 ? tho_e4m3_value(byte) * sg : ldexp(1.0, byte - 127);
}

/* Dequantise row s of slice bh of a tensor quantised along D. */
void tho_dequant_row(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                     size_t bh, int S, int D, int s, int fmt, double* out) {
  int g = tho_group_size(fmt);
  double sg = fmt == THO_NVFP4 ? (double)tensor_scale[bh] : 1.0;
  for (int d = 0; d < D; ++d) {
    size_t e = ((size_t)bh * S + s) * D + d;
    size_t si = ((size_t)bh * S + s) * (D / g) + d / g;
    int code = (codes[e / 2] >> (4 * (e & 1))) & 0xF;
    out[d] = tho_e2m1_value(code) * tho_group_scale(fmt, scales[si], sg);
  }
}

/* Dequantise a tensor written by tho_quantize back to fp64, in the original
 * [B, H, S, D] orientation (padding dropped). */
void tho_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int B,
                    int H, int S, int D, int axis, int fmt, double* out) {
  int g = tho_group_size(fmt);
  int Sp = tho_pad_s(S);
  for (int bh = 0; bh < B * H; ++bh) {
    double sg = fmt == THO_NVFP4 ? (double)tensor_scale[bh] : 1.0;
    for (int s = 0; s < S; ++s)
      for (int d = 0; d < D; ++d) {
        size_t e, si;
        if (axis == THO_AXIS_D) {
          e = ((size_t)bh * S + s) * D + d;
          si = ((size_t)bh * S + s) * (D / g) + d / g;
        } else {
          e = ((size_t)bh * D + d) * Sp + s;
          si = ((size_t)bh * D + d) * (Sp / g) + s / g;
        }
        int code = (codes[e / 2] >> (4 * (e & 1))) & 0xF;
        out[((size_t)bh * S + s) * D + d] = tho_e2m1_value(code) * tho_group_scale(fmt, scales[si], sg);
      }
  }
}

/* ------------------------------------------------------------------ */
/* Attention forward (pages: "Gemengd-Precisie Berekening & Samenvoeging") */
/* ------------------------------------------------------------------ */

/* Probabilities of one key tile.  Reading of the pages' two-level
 * quantisation of the probability blocks (which they take from
 * SageAttention3), applied alike to every precision a tile runs in:
 *   level 1, per query row and key tile: the tile's scores t (log2 units)
 *     are exponentiated against the tile's own maximum mt, v = 2^(t - mt),
 *     so the tile's largest probability is exactly 1; the tile adds 2^mt
 *     times its level-2 values (times V) to the numerator of the output;
 *   level 2, by the tile's precision:
 *     NVFP4-style: v' = 2688 v (the maximum lands on 6 * 448); per 16 keys
 *       an E4M3 block scale s2 = E4M3(max v' / 6), codes E2M1(v' / s2),
 *       value code * s2 / 2688;
 *     MX: per 32 keys X = mx_exponent(max v), codes E2M1(v / 2^X), value
 *       code * 2^X;
 *     MXFP8 (the middle tier): per 32 keys X = mx8_exponent(max v), codes
 *       E4M3(v / 2^X), value code * 2^X;
 *     FP16: fp16(v).
 * Key groups follow the value tensor's groups along the keys.  A tile's
 * values then depend on its own scores only: not on the running maximum,
 * not on the order in which tiles are processed, and not on a constant
 * added to every score of a row (softmax's shift invariance holds exactly).
 * The row sum takes the unquantised probabilities 2^t. */

/* ---- decisions a device implementation may take either way ----
 * A device evaluates scores and exponentials in fp32.  A decision (a code, a
 * block scale, an fp16 rounding) whose exact input lies closer to its
 * rounding boundary than that evaluation error may come out either way; both
 * outcomes are then valid results of the method.  Evaluation-error model
 * (u = 2^-24):
 *  - a score s = q.k comes from a chain of matrix instructions over
 *    ascending slices of the contraction, each with exact products and
 *    returning within kappa u (|C| + sum over its slice of |product|) of the
 *    exact value (C the running accumulator), so s is within kappa u B of
 *    exact, B = sum over the slices of (|exact partial sum before the slice|
 *    + the slice's sum of |products|).  MX: the block-scaled FP4 instruction,
 *    64 channels each, kappa = 2.5; NVFP4 (decoded operands), the middle tier
 *    and FP16: the fp16 instruction, 16 channels each, kappa = 6.  The
 *    maxima measured on the device over 65,536 outputs each (random operands,
 *    block scales spread over 2^+-20, accumulators zero and not) are 1.99 and
 *    4.66: kappa is the measured maximum with a margin of about a quarter;
 *  - the softmax multiplier c = sm_scale log2(e) is an fp32 value carrying nc
 *    roundings (sm_scale to fp32, log2(e), the product: 3; NVFP4's two slice
 *    scales add 2), and the exponent's argument fma(s, c, -fl(c smax)) is
 *    within c (ds + dsmax) + (nc + 1) u |t - mt| + u |mt| of t - mt (log2
 *    units; B is taken in the same units, times sm_scale log2(e));
 *  - exp2 is within 2^-23 relative (one ulp);
 *  - NVFP4 adds four roundings to a value's decision input (the factor 2688,
 *    the block scale's reciprocal, the products).
 * tho_eval_rel is the resulting bound on the relative error of a tile value
 * v, times 1 + 2^-10 for second-order terms. */
#define THO_U 0x1p-24
#define THO_EXP_REL 0x1p-23
#define THO_PATH_MX4 0 /* FP4 path, MX format */
#define THO_PATH_NV4 1 /* FP4 path, NVFP4 format */
#define THO_PATH_F8 2  /* middle (MXFP8) tier */
#define THO_PATH_F16 3 /* FP16 path */
#define THO_PATH_NVMXP 4 /* FP4 path of the variant: NVFP4 tensors, P quantised MX-style */

/* Channels per matrix instruction of a path's scores. */
static int tho_path_slice(int path) { return path == THO_PATH_MX4 ? 64 : 16; }

/* Evaluation path of a tile's scores: FP4 tiles follow the tensors' format
 * (and the variant's P format), the other tiers their own. */
static int tho_eval_path(int prec, int fmt) {
  if (prec == THO_PATH_MX4 && fmt == THO_NVFP4) return THO_PATH_NVMXP;
  return prec;
}

/* b, bmax: the chain sums B of the key's score and of the tile maximum's
 * score (log2 units); dt = t - mt; mt the tile maximum (log2 units). */
double tho_eval_rel(int path, double b, double bmax, double dt, double mt) {
  double kappa = path == THO_PATH_MX4 ? 2.5 : 6.0;
  double nc = path == THO_PATH_NV4 || path == THO_PATH_NVMXP ? 5.0 : 3.0;
  double arg = kappa * THO_U * (b + bmax) + (nc + 1.0) * THO_U * fabs(dt) + THO_U * fabs(mt);
  double rel = THO_LN2 * arg + THO_EXP_REL + (path == THO_PATH_NV4 ? 4.0 * THO_U : 0.0);
  return rel * (1.0 + 0x1p-10);
}

/* The other outcome of rounding q to the nearest E2M1 magnitude (q >= 0) if q
 * lies within relative rel of a rounding midpoint; -1 otherwise. */
static double tho_e2m1_alt(double q, double rel) {
  static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  for (int k = 0; k < 7; ++k)
    if (fabs(q - mid[k]) <= rel * q) {
      double chosen = tho_e2m1_value(tho_e2m1_encode(q, 1.0));
      return chosen == tho_e2m1_mag[k] ? tho_e2m1_mag[k + 1] : tho_e2m1_mag[k];
    }
  return -1.0;
}

/* The same for the nearest finite E4M3 magnitude (q >= 0). */
static double tho_e4m3_alt(double q, double rel) {
  for (int k = 0; k < 126; ++k) {
    double lo = tho_e4m3_value(k), hi = tho_e4m3_value(k + 1);
    if (fabs(q - 0.5 * (lo + hi)) <= rel * q) {
      double chosen = tho_e4m3_value(tho_e4m3_encode_ratio(q, 1.0));
      return chosen == lo ? hi : lo;
    }
  }
  return -1.0;
}

/* The other outcomes of rounding q > 0 to fp16 when q may be off by a
 * relative rel: every fp16 value some point of [q (1 - rel), q (1 + rel)]
 * rounds to, other than fp16(q) (at most 8; returns their number). */
static int tho_half_alts(double q, double rel, double* alt) {
  if (!(q > 0.0)) return 0;
  double r = tho_round_to_half(q), lo = tho_round_to_half(q * (1.0 - rel)), hi = tho_round_to_half(q * (1.0 + rel));
  int n = 0;
  for (double x = lo; x <= hi && n < 8;) {
    if (x != r) alt[n++] = x;
    int e;
    frexp(x > 0.0 ? x : 0x1p-25, &e);
    int ue = e - 11 < -24 ? -24 : e - 11;
    x = x > 0.0 ? x + ldexp(1.0, ue) : 0x1p-24; /* the next fp16 value up */
  }
  return n;
}

/* One decision of a tile that may go either way: its other outcome changes
 * the values (relative to 2^mt) of keys [k0, k1) of the tile by dp[]. */
typedef struct {
  int k0, k1;
  double dp[64];
} tho_flip;

static int tho_add_flip(tho_flip* flips, int nf, int maxf, int k0, int k1, const double* dp) {
  if (!flips || nf >= maxf) return nf + (flips ? 1 : 0);
  flips[nf].k0 = k0;
  flips[nf].k1 = k1;
  for (int c = k0; c < k1; ++c) flips[nf].dp[c] = dp[c];
  return nf + 1;
}

/* Block scale of a level-2 group from its largest value vmax. */
static double tho_p_scale(int prec, double vmax) {
  if (prec == THO_PATH_NV4) return tho_e4m3_value(tho_e4m3_encode_ratio(vmax, 6.0));
  if (prec == THO_PATH_F8) return ldexp(1.0, tho_mx8_exponent(vmax));
  return ldexp(1.0, tho_mx_exponent(vmax));
}

/* Level-2 value of v under block scale s2 (relative to the level-1 unit). */
static double tho_p_value(int prec, double v, double s2) {
  if (prec == THO_PATH_NV4) return s2 > 0.0 ? tho_e2m1_value(tho_e2m1_encode(v, s2)) * s2 / 2688.0 : 0.0;
  if (prec == THO_PATH_F8) return tho_e4m3_value(tho_e4m3_encode_ratio(v, s2)) * s2;
  return tho_e2m1_value(tho_e2m1_encode(v, s2)) * s2;
}

/* Level-2 values pq[] (relative to 2^mt) of one tile row of n keys in
 * precision prec (THO_PATH_MX4, _NV4 or _F8) from scores t, chain sums ta
 * and mask (masked keys: value 0); epath is the scores' evaluation path.  With
 * flips != NULL also every decision within evaluation error of its boundary
 * (tho_eval_rel): element codes near a rounding midpoint, and block scales
 * whose group maximum lies near the scale rule's boundary.  A group holding
 * the tile maximum has its largest value exactly at the top of the scale
 * rule (1, or 2688 for NVFP4); its scale is decided unless a key outside it
 * could evaluate as the tile's maximum.  Returns the number of decisions
 * (at most maxf are stored). */
static int tho_quantize_p_tile(const double* t, const double* ta, const int* mask, int n, int prec,
                               int epath, double mt, double* pq, tho_flip* flips, int maxf) {
  int gs = prec == THO_PATH_NV4 ? 16 : 32;
  double top = prec == THO_PATH_NV4 ? 2688.0 : 1.0;
  double v[64], rel[64], dp[64];
  int imax = -1, nf = 0;
  for (int c = 0; c < n; ++c) {
    v[c] = mask[c] ? 0.0 : top * exp2(t[c] - mt);
    if (!mask[c] && t[c] == mt && imax < 0) imax = c;
  }
  for (int c = 0; c < n; ++c)
    rel[c] = mask[c] ? 0.0 : tho_eval_rel(epath, ta[c], ta[imax], t[c] - mt, mt);
  for (int g0 = 0; g0 < n; g0 += gs) {
    int g1 = g0 + gs < n ? g0 + gs : n;
    double amax = 0.0;
    int cm = -1;
    for (int c = g0; c < g1; ++c)
      if (v[c] > amax) {
        amax = v[c];
        cm = c;
      }
    double s2 = tho_p_scale(prec, amax);
    for (int c = g0; c < g1; ++c) pq[c] = mask[c] ? 0.0 : tho_p_value(prec, v[c], s2);
    if (!flips || cm < 0) continue;
    for (int c = g0; c < g1; ++c) {
      double alt = mask[c] ? -1.0
                   : prec == THO_PATH_F8 ? tho_e4m3_alt(v[c] / s2, rel[c])
                                         : (s2 > 0.0 ? tho_e2m1_alt(v[c] / s2, rel[c]) : -1.0);
      if (alt < 0.0) continue;
      for (int k = g0; k < g1; ++k) dp[k] = 0.0;
      dp[c] = alt * s2 / (prec == THO_PATH_NV4 ? 2688.0 : 1.0) - pq[c];
      nf = tho_add_flip(flips, nf, maxf, c, c + 1, dp);
    }
    int decided = t[cm] == mt;
    for (int c = 0; c < n && decided; ++c)
      if ((c < g0 || c >= g1) && !mask[c] && top - v[c] <= rel[c] * top) decided = 0;
    if (decided) continue;
    double lo = tho_p_scale(prec, amax * (1.0 - rel[cm])), hi = tho_p_scale(prec, amax * (1.0 + rel[cm]));
    double s2alt = lo != s2 ? lo : hi;
    if (s2alt == s2) continue;
    for (int c = g0; c < g1; ++c) dp[c] = mask[c] ? 0.0 : tho_p_value(prec, v[c], s2alt) - pq[c];
    nf = tho_add_flip(flips, nf, maxf, g0, g1, dp);
  }
  return nf;
}

/* FP16-path values of one tile row: pq[c] = fp16(2^(t - mt)), and the fp16
 * roundings within evaluation error of a midpoint. */
static int tho_quantize_p_tile16(const double* t, const double* ta, const int* mask, int n, double mt,
                                 double* pq, tho_flip* flips, int maxf) {
  double dp[64];
  int imax = -1, nf = 0;
  for (int c = 0; c < n; ++c)
    if (!mask[c] && t[c] == mt && imax < 0) imax = c;
  for (int c = 0; c < n; ++c) pq[c] = mask[c] ? 0.0 : tho_round_to_half(exp2(t[c] - mt));
  if (!flips) return 0;
  for (int c = 0; c < n; ++c) {
    if (mask[c]) continue;
    double alt[8];
    int na = tho_half_alts(exp2(t[c] - mt), tho_eval_rel(THO_PATH_F16, ta[c], ta[imax], t[c] - mt, mt), alt);
    for (int k = 0; k < na; ++k) {
      dp[c] = alt[k] - pq[c];
      nf = tho_add_flip(flips, nf, maxf, c, c + 1, dp);
    }
  }
  return nf;
}

typedef struct {
  int B, Hq, Hkv, S, Sk, D, bq, bk, causal, fmt, kmax; /* S: queries, Sk: keys */
  int pfmt; /* format of P's two-level quantisation (fmt, or MX for THO_NVFP4_MXP) */
  double sm_scale;
  const uint16_t *q16, *k16, *v16;
  const uint8_t *q4c, *q4s; /* FP4 query codes and scales as quantised */
  const float* q4t;
  const double *k4, *v4; /* dequantised FP4 keys and values, [B,Hkv,Sk,D] */
  const int32_t *idx, *cnt;
  /* middle (FP8) tier, NULL when absent: idx2/cnt2 list the blocks of the
   * FP16 and FP8 tiers together (the selection under the two budgets'
   * sum); a listed block that idx also lists stays on the FP16 path */
  const int32_t *idx2, *cnt2;
  int kmax2;
  const uint8_t *q8c, *q8s; /* MXFP8 queries as quantised */
  const double *k8, *v8;    /* dequantised MXFP8 keys and values, [B,Hkv,Sk,D] */
  /* decisions that may go either way (NULL: not wanted): row index
   * ((b * Hq + hq) * S + r) and the change of that row of O if the decision
   * takes its other outcome; *amb_n counts them (capacity amb_cap) */
  int32_t* amb_row;
  double* amb_delta;
  int amb_cap;
  int* amb_n;
} tho_attn_args;

#define THO_TILE_FLIPS 520 /* at most 64 keys x 8 fp16 outcomes, or 64 codes and 4 block scales, per tile */

/* Scores of query row r against the n keys of key block j from query qv and
 * keys kv ([keys, D], dequantised to fp64); masked keys get -inf.  tb[c]
 * receives the score's chain sum B for slices of `slice` channels (see the
 * evaluation-error model), in the same log2 units. */
static double tho_tile_scores(const tho_attn_args* a, const double* qv, const double* kv, int c0, int n,
                              int qpos, int slice, double* t, double* tb, int* mask) {
  int D = a->D;
  double mt = -INFINITY;
  for (int c = 0; c < n; ++c) {
    mask[c] = a->causal && (c0 + c > qpos);
    double s = 0.0, b = 0.0;
    if (!mask[c])
      for (int d0 = 0; d0 < D; d0 += slice) {
        double part = 0.0, sa = 0.0;
        for (int d = d0; d < d0 + slice && d < D; ++d) {
          double pr = qv[d] * kv[(size_t)c * D + d];
          part += pr;
          sa += fabs(pr);
        }
        b += fabs(s) + sa;
        s += part;
      }
    t[c] = mask[c] ? -INFINITY : s * a->sm_scale * THO_LOG2E;
    tb[c] = b * a->sm_scale * THO_LOG2E;
    if (t[c] > mt) mt = t[c];
  }
  return mt;
}

/* One query row r of query block i of head (b, hq). */
static void tho_attend_row(const tho_attn_args* a, int b, int hq, int i, int r, double* o_row,
                           double* lse_out, double* ohp_row) {
  int D = a->D, S = a->S, Sk = a->Sk, bk = a->bk;
  int hk = hq / (a->Hq / a->Hkv);
  int nq = tho_cdiv(S, a->bq);
  int qpos = Sk - S + r; /* the query's position in the key sequence */
  size_t qoff = (((size_t)b * a->Hq + hq) * S + r) * D;
  size_t kvbase = ((size_t)b * a->Hkv + hk) * Sk;
  const int32_t* sel = a->idx + (((size_t)b * a->Hq + hq) * nq + i) * a->kmax;
  int nsel = a->cnt[((size_t)b * a->Hq + hq) * nq + i];
  const int32_t* sel2 = a->idx2 ? a->idx2 + (((size_t)b * a->Hq + hq) * nq + i) * a->kmax2 : NULL;
  int nsel2 = a->idx2 ? a->cnt2[((size_t)b * a->Hq + hq) * nq + i] : 0;
  int nvalid = tho_valid_blocks_kv(i, S, Sk, a->bq, bk, a->causal);
  double t[64], ta[64], pq[64];
  int mask[64];
  double* acc = (double*)calloc((size_t)D, sizeof(double));
  /* the high-precision output O' (Attn-QAT): the same sum with the exact
   * probabilities in place of the quantised or fp16-rounded ones */
  double* hacc = (double*)calloc((size_t)D, sizeof(double));
  double* qh = (double*)malloc(sizeof(double) * (size_t)D);
  double* q4 = (double*)malloc(sizeof(double) * (size_t)D);
  double* q8 = (double*)malloc(sizeof(double) * (size_t)D);
  double* k16t = (double*)malloc(sizeof(double) * (size_t)bk * D);
  double* v16t = (double*)malloc(sizeof(double) * (size_t)bk * D);
  int want = a->amb_row != NULL;
  tho_flip* tf = want ? (tho_flip*)malloc(sizeof(tho_flip) * THO_TILE_FLIPS) : NULL;
  /* this row's decisions: the tile's level-1 exponent mt and the change of
   * the numerator (in units of 2^mt) if the decision flips */
  int nrf = 0, caprf = 0;
  double* rref = NULL;
  double* rvec = NULL;
  double m = -INFINITY, l = 0.0;
  tho_dequant_row(a->q4c, a->q4s, a->q4t, (size_t)b * a->Hq + hq, S, D, r, a->fmt, q4);
  if (nsel2 > 0) tho_dequant8_row(a->q8c, a->q8s, (size_t)b * a->Hq + hq, S, D, r, q8);
  if (nsel > 0)
    for (int d = 0; d < D; ++d) qh[d] = tho_half_to_double(a->q16[qoff + d]);

  /* Tiles in the pages' order: the FP4 path first, over every valid key
   * block that no higher tier lists, ascending; then the middle tier over
   * the blocks idx2 lists and idx does not; then the FP16 path over the
   * promoted blocks, ascending (the FP16 query row is read only then). */
  int npass = nvalid + nsel2 + nsel;
  int sp = 0, sp2 = 0;
  for (int step = 0; step < npass; ++step) {
    int j, prec;
    if (step < nvalid) {
      j = step;
      int listed = 0;
      if (sp < nsel && sel[sp] == j) {
        ++sp;
        listed = 1;
      }
      if (sp2 < nsel2 && sel2[sp2] == j) {
        ++sp2;
        listed = 1;
      }
      if (listed) continue;
      prec = a->pfmt == THO_NVFP4 ? THO_PATH_NV4 : THO_PATH_MX4;
    } else if (step < nvalid + nsel2) {
      j = sel2[step - nvalid];
      int in16 = 0;
      for (int p = 0; p < nsel; ++p)
        if (sel[p] == j) in16 = 1;
      if (in16) continue;
      prec = THO_PATH_F8;
    } else {
      j = sel[step - nvalid - nsel2];
      prec = THO_PATH_F16;
    }
    int c0 = j * bk, n = (c0 + bk < Sk ? c0 + bk : Sk) - c0;
    const double* vt;
    double mt;
    if (prec == THO_PATH_F16) {
      for (size_t e = 0; e < (size_t)n * D; ++e) {
        k16t[e] = tho_half_to_double(a->k16[(kvbase + c0) * D + e]);
        v16t[e] = tho_half_to_double(a->v16[(kvbase + c0) * D + e]);
      }
      mt = tho_tile_scores(a, qh, k16t, c0, n, qpos, tho_path_slice(THO_PATH_F16), t, ta, mask);
      vt = v16t;
    } else if (prec == THO_PATH_F8) {
      mt = tho_tile_scores(a, q8, a->k8 + (kvbase + c0) * D, c0, n, qpos, tho_path_slice(THO_PATH_F8), t, ta,
                           mask);
      vt = a->v8 + (kvbase + c0) * D;
    } else {
      mt = tho_tile_scores(a, q4, a->k4 + (kvbase + c0) * D, c0, n, qpos,
                           tho_path_slice(tho_eval_path(prec, a->fmt)), t, ta, mask);
      vt = a->v4 + (kvbase + c0) * D;
    }
    if (mt == -INFINITY) continue; /* every key of this block is masked for row r */
    /* the pages' FP4 tiles use the variant's P format for THO_NVFP4_MXP */
    int nf = prec == THO_PATH_F16 ? tho_quantize_p_tile16(t, ta, mask, n, mt, pq, tf, THO_TILE_FLIPS)
                                  : tho_quantize_p_tile(t, ta, mask, n, prec, tho_eval_path(prec, a->fmt), mt, pq,
                                                        tf, THO_TILE_FLIPS);
    double m_new = m > mt ? m : mt;
    double alpha = exp2(m - m_new); /* 0 when m = -inf */
    double w = exp2(mt - m_new);    /* level 1 relative to the running maximum */
    double psum = 0.0;
    for (int c = 0; c < n; ++c)
      if (!mask[c]) psum += exp2(t[c] - m_new);
    l = alpha * l + psum;
    for (int d = 0; d < D; ++d) {
      double pv = 0.0, hv = 0.0;
      for (int c = 0; c < n; ++c) {
        pv += pq[c] * vt[(size_t)c * D + d];
        if (!mask[c]) hv += exp2(t[c] - m_new) * vt[(size_t)c * D + d];
      }
      acc[d] = alpha * acc[d] + w * pv;
      hacc[d] = alpha * hacc[d] + hv;
    }
    m = m_new;
    if (want) {
      for (int f = 0; f < nf; ++f) {
        if (nrf == caprf) {
          caprf = caprf ? 2 * caprf : 16;
          rref = (double*)realloc(rref, sizeof(double) * (size_t)caprf);
          rvec = (double*)realloc(rvec, sizeof(double) * (size_t)caprf * D);
        }
        rref[nrf] = mt;
        for (int d = 0; d < D; ++d) {
          double s = 0.0;
          for (int c = tf[f].k0; c < tf[f].k1; ++c) s += tf[f].dp[c] * vt[(size_t)c * D + d];
          rvec[(size_t)nrf * D + d] = s;
        }
        ++nrf;
      }
    }
  }

  for (int d = 0; d < D; ++d) o_row[d] = acc[d] / l;
  if (ohp_row)
    for (int d = 0; d < D; ++d) ohp_row[d] = hacc[d] / l;
  if (lse_out) *lse_out = m * THO_LN2 + log(l);
  if (want && nrf > 0) {
    int base;
#pragma omp atomic capture
    {
      base = *a->amb_n;
      *a->amb_n += nrf;
    }
    for (int f = 0; f < nrf; ++f) {
      if (base + f >= a->amb_cap) break;
      a->amb_row[base + f] = (int32_t)(((size_t)b * a->Hq + hq) * S + r);
      double scale = exp2(rref[f] - m) / l;
      for (int d = 0; d < D; ++d) a->amb_delta[(size_t)(base + f) * D + d] = rvec[(size_t)f * D + d] * scale;
    }
  }
  free(rvec);
  free(rref);
  free(tf);
  free(v16t);
  free(k16t);
  free(q8);
  free(q4);
  free(qh);
  free(hacc);
  free(acc);
}

/* Full forward for a list of work items (b, hq, i) (NULL: all of them).
 * q4/k4/v4 are the FP4 tensors as written by tho_quantize (V along the
 * sequence axis); q16/k16/v16 may be NULL when no block is promoted.
 * o: [B, Hq, S, D] fp64, lse: [B, Hq, S] (may be NULL).  With amb_row !=
 * NULL every decision within evaluation error of its rounding boundary
 * (tho_eval_rel) is listed: amb_row[k] the row ((b * Hq + hq) * S + r) and
 * amb_delta[k * D ...] the change of that row of o if the decision takes its
 * other outcome; *amb_n receives their number, of which the first amb_cap
 * are stored.  Rows outside the work items are left untouched. */
static void tho_attention_impl(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                               const uint8_t* q4c, const uint8_t* q4s, const float* q4t,
                               const uint8_t* k4c, const uint8_t* k4s, const float* k4t,
                               const uint8_t* v4c, const uint8_t* v4s, const float* v4t, int fmt,
                               const int32_t* idx, const int32_t* cnt, int kmax,
                               const uint8_t* q8c, const uint8_t* q8s, const uint8_t* k8c,
                               const uint8_t* k8s, const uint8_t* v8c, const uint8_t* v8s,
                               const int32_t* idx2, const int32_t* cnt2, int kmax2, int B, int Hq,
                               int Hkv, int S, int Sk, int D, int bq, int bk, int causal,
                               double sm_scale, const int32_t* work, int nwork, double* o,
                               double* lse, int32_t* amb_row, double* amb_delta, int amb_cap,
                               int* amb_n, double* ohp) {
  tho_attn_args a;
  memset(&a, 0, sizeof a);
  a.amb_row = amb_row;
  a.amb_delta = amb_delta;
  a.amb_cap = amb_cap;
  a.amb_n = amb_n;
  if (amb_n) *amb_n = 0;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.Sk = Sk;
  a.D = D;
  a.bq = bq;
  a.bk = bk;
  a.causal = causal;
  /* THO_NVFP4_MXP: NVFP4 tensors, P quantised MX-style (a variant) */
  a.fmt = fmt == THO_NVFP4_MXP ? THO_NVFP4 : fmt;
  a.pfmt = fmt == THO_NVFP4_MXP ? THO_MX : fmt;
  a.kmax = kmax;
  a.sm_scale = sm_scale;
  a.q16 = q16;
  a.k16 = k16;
  a.v16 = v16;
  a.idx = idx;
  a.cnt = cnt;
  double* k4 = (double*)malloc(sizeof(double) * (size_t)B * Hkv * Sk * D);
  double* v4 = (double*)malloc(sizeof(double) * (size_t)B * Hkv * Sk * D);
  tho_dequantize(k4c, k4s, k4t, B, Hkv, Sk, D, THO_AXIS_D, a.fmt, k4);
  tho_dequantize(v4c, v4s, v4t, B, Hkv, Sk, D, THO_AXIS_S, a.fmt, v4);
  a.q4c = q4c;
  a.q4s = q4s;
  a.q4t = q4t;
  a.k4 = k4;
  a.v4 = v4;
  double *k8 = NULL, *v8 = NULL;
  if (idx2) {
    k8 = (double*)malloc(sizeof(double) * (size_t)B * Hkv * Sk * D);
    v8 = (double*)malloc(sizeof(double) * (size_t)B * Hkv * Sk * D);
    tho_dequantize_fp8(k8c, k8s, B, Hkv, Sk, D, THO_AXIS_D, k8);
    tho_dequantize_fp8(v8c, v8s, B, Hkv, Sk, D, THO_AXIS_S, v8);
    a.idx2 = idx2;
    a.cnt2 = cnt2;
    a.kmax2 = kmax2;
    a.q8c = q8c;
    a.q8s = q8s;
    a.k8 = k8;
    a.v8 = v8;
  }
  int nq = tho_cdiv(S, bq);
  int total = work ? nwork : B * Hq * nq;
#pragma omp parallel for schedule(dynamic, 1)
  for (int w = 0; w < total; ++w) {
    int b, hq, i;
    if (work) {
      b = work[3 * w];
      hq = work[3 * w + 1];
      i = work[3 * w + 2];
    } else {
      b = w / (Hq * nq);
      hq = (w / nq) % Hq;
      i = w % nq;
    }
    int r0 = i * bq, r1 = r0 + bq < S ? r0 + bq : S;
    for (int r = r0; r < r1; ++r) {
      size_t row = ((size_t)b * Hq + hq) * S + r;
      tho_attend_row(&a, b, hq, i, r, o + row * D, lse ? lse + row : NULL, ohp ? ohp + row * D : NULL);
    }
  }
  free(v8);
  free(k8);
  free(v4);
  free(k4);
}

void tho_attention_kv(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                      const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                      const uint8_t* k4s, const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                      const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                      int B, int Hq, int Hkv, int S, int Sk, int D, int bq, int bk, int causal,
                      double sm_scale, const int32_t* work, int nwork, double* o, double* lse,
                      int32_t* amb_row, double* amb_delta, int amb_cap, int* amb_n) {
  tho_attention_impl(q16, k16, v16, q4c, q4s, q4t, k4c, k4s, k4t, v4c, v4s, v4t, fmt, idx, cnt, kmax,
                     NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, B, Hq, Hkv, S, Sk, D, bq, bk,
                     causal, sm_scale, work, nwork, o, lse, amb_row, amb_delta, amb_cap, amb_n, NULL);
}

/* The forward with a middle precision tier (a variant): the blocks idx2
 * lists and idx does not run on MXFP8 (q8/k8/v8 as written by
 * tho_quantize_fp8, V along the sequence axis), between the FP4 path and the
 * FP16 path.  MX format only. */
void tho_attention_tiers(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                         const uint8_t* q4c, const uint8_t* q4s, const uint8_t* k4c,
                         const uint8_t* k4s, const uint8_t* v4c, const uint8_t* v4s,
                         const uint8_t* q8c, const uint8_t* q8s, const uint8_t* k8c,
                         const uint8_t* k8s, const uint8_t* v8c, const uint8_t* v8s,
                         const int32_t* idx, const int32_t* cnt, int kmax, const int32_t* idx2,
                         const int32_t* cnt2, int kmax2, int B, int Hq, int Hkv, int S, int D,
                         int bq, int bk, int causal, double sm_scale, const int32_t* work,
                         int nwork, double* o, double* lse, int32_t* amb_row, double* amb_delta,
                         int amb_cap, int* amb_n) {
  tho_attention_impl(q16, k16, v16, q4c, q4s, NULL, k4c, k4s, NULL, v4c, v4s, NULL, THO_MX, idx, cnt,
                     kmax, q8c, q8s, k8c, k8s, v8c, v8s, idx2, cnt2, kmax2, B, Hq, Hkv, S, S, D, bq,
                     bk, causal, sm_scale, work, nwork, o, lse, amb_row, amb_delta, amb_cap, amb_n, NULL);
}

/* The forward with Attn-QAT's extra output: ohp [B,Hq,S,D] receives O', the
 * attention output computed with the exact softmax probabilities (each key
 * and value in the precision of its block's path), which the backward uses
 * for its row term.  Sq = Sk (training shape). */
void tho_attention_hp(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                      const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                      const uint8_t* k4s, const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                      const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                      int B, int Hq, int Hkv, int S, int D, int bq, int bk, int causal,
                      double sm_scale, const int32_t* work, int nwork, double* o, double* lse,
                      double* ohp) {
  tho_attention_impl(q16, k16, v16, q4c, q4s, q4t, k4c, k4s, k4t, v4c, v4s, v4t, fmt, idx, cnt, kmax,
                     NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, B, Hq, Hkv, S, S, D, bq, bk,
                     causal, sm_scale, work, nwork, o, lse, NULL, NULL, 0, NULL, ohp);
}

void tho_attention(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                   const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                   const uint8_t* k4s, const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                   const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                   int B, int Hq, int Hkv, int S, int D, int bq, int bk, int causal,
                   double sm_scale, const int32_t* work, int nwork, double* o, double* lse,
                   int32_t* amb_row, double* amb_delta, int amb_cap, int* amb_n) {
  tho_attention_kv(q16, k16, v16, q4c, q4s, q4t, k4c, k4s, k4t, v4c, v4s, v4t, fmt, idx, cnt, kmax, B,
                   Hq, Hkv, S, S, D, bq, bk, causal, sm_scale, work, nwork, o, lse, amb_row, amb_delta,
                   amb_cap, amb_n);
}

/* ------------------------------------------------------------------ */
/* Backward pass (Attn-QAT, "Methodik": precision-consistent          */
/* recomputation of P from L, and the row term from O')               */
/* ------------------------------------------------------------------ */
/*
 * The gradient of the forward above with the selection (idx, cnt) held
 * fixed and every quantiser passed straight through (its derivative taken
 * as the identity), which is how quantisation-aware training differentiates
 * through fake quantisation.  For query row r (log2-domain log-sum-exp
 * L2 = lse * log2 e from the forward) and every key c of a valid pair, in
 * the precision of the path its block takes for this row's query block
 * (q4, k4, v4 dequantised on the FP4 path; the fp16 tensors on the FP16
 * path):
 *   t = sm_scale log2(e) q.k,  p = 2^(t - L2)          (exact probability)
 *   pt = the probability the forward's PV product used, recomputed from L:
 *        FP4 path: the two-level quantised value (relative to the tile's own
 *        maximum, so its codes do not depend on L) times 2^(ref - L2);
 *        FP16 path: fp16(p)
 *   dV[c] += pt dO[r]          dP = dO[r].v[c]
 *   Dr = dO[r].O'[r]           (O' from the forward: the exact-probability
 *                               output, so Dr = sum_c p dP)
 *   dS = p (dP - Dr)
 *   dQ[r] += sm_scale dS k[c]  dK[c] += sm_scale dS q[r]
 * Query heads sharing a key head add into the same dK, dV.
 */

/* Probabilities of query row r against key block j (the block must be
 * valid for r's query block): kind[c] 0 masked, 1 FP4 path, 2 FP16 path;
 * p, pt as above; dpt (may be NULL) the largest change in pt that decisions
 * within evaluation error of their rounding boundary can make (FP4: the
 * forward's decisions, tho_quantize_p_tile; FP16: the rounding of p, whose
 * input also carries the error of an fp32 log-sum-exp, allowed for as 2^-16
 * in log2 units).  q4 and qh are the row's dequantised FP4 and fp16 query;
 * k16d, v16d the fp16 keys and values as doubles.  Returns the number of keys
 * in the block. */
static int tho_tile_probs(const tho_attn_args* a, const double* k16d, int b, int hq, int r, int j,
                          double L2, const double* q4, const double* qh, int* kind, double* p,
                          double* pt, double* dpt) {
  int D = a->D, S = a->S, Sk = a->Sk, bk = a->bk;
  int i = r / a->bq, nq = tho_cdiv(S, a->bq);
  int hk = hq / (a->Hq / a->Hkv);
  int qpos = Sk - S + r;
  size_t kvbase = ((size_t)b * a->Hkv + hk) * Sk;
  const int32_t* sel = a->idx + (((size_t)b * a->Hq + hq) * nq + i) * a->kmax;
  int nsel = a->cnt[((size_t)b * a->Hq + hq) * nq + i];
  int prom = 0;
  for (int s = 0; s < nsel; ++s)
    if (sel[s] == j) prom = 1;
  int c0 = j * bk, n = (c0 + bk < Sk ? c0 + bk : Sk) - c0;
  double t[64], ta[64], pq[64];
  int mask[64];
  int fpath = a->pfmt == THO_NVFP4 ? THO_PATH_NV4 : THO_PATH_MX4;
  double mt = tho_tile_scores(a, prom ? qh : q4, (prom ? k16d : a->k4) + (kvbase + c0) * D, c0, n, qpos,
                              tho_path_slice(prom ? THO_PATH_F16 : tho_eval_path(fpath, a->fmt)), t, ta, mask);
  for (int c = 0; c < n; ++c) {
    kind[c] = 0;
    p[c] = pt[c] = 0.0;
    if (dpt) dpt[c] = 0.0;
  }
  if (mt == -INFINITY) return n;
  if (!prom) {
    tho_flip* tf = dpt ? (tho_flip*)malloc(sizeof(tho_flip) * THO_TILE_FLIPS) : NULL;
    int nf = tho_quantize_p_tile(t, ta, mask, n, fpath, tho_eval_path(fpath, a->fmt), mt, pq, tf, THO_TILE_FLIPS);
    for (int c = 0; c < n; ++c)
      if (!mask[c]) {
        kind[c] = 1;
        p[c] = exp2(t[c] - L2);
        pt[c] = pq[c] * exp2(mt - L2);
      }
    for (int f = 0; f < nf && dpt; ++f)
      for (int c = tf[f].k0; c < tf[f].k1; ++c) dpt[c] += fabs(tf[f].dp[c]) * exp2(mt - L2);
    free(tf);
  } else {
    for (int c = 0; c < n; ++c)
      if (!mask[c]) {
        kind[c] = 2;
        p[c] = exp2(t[c] - L2);
        pt[c] = tho_round_to_half(p[c]);
        if (dpt) {
          double rel = tho_eval_rel(THO_PATH_F16, ta[c], 0.0, t[c] - L2, L2) + THO_LN2 * 0x1p-16, alt[8];
          int na = tho_half_alts(p[c], rel, alt);
          for (int k = 0; k < na; ++k)
            if (fabs(alt[k] - pt[c]) > dpt[c]) dpt[c] = fabs(alt[k] - pt[c]);
        }
      }
  }
  return n;
}

static void tho_bwd_setup(tho_attn_args* a, const uint16_t* q16, const uint16_t* k16,
                          const uint16_t* v16, const uint8_t* q4c, const uint8_t* q4s,
                          const float* q4t, const uint8_t* k4c, const uint8_t* k4s,
                          const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                          const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt,
                          int kmax, int B, int Hq, int Hkv, int S, int D, int bq, int bk,
                          int causal, double sm_scale, double** k16d, double** v16d) {
  a->B = B;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->S = S;
  a->Sk = S;
  a->D = D;
  a->bq = bq;
  a->bk = bk;
  a->causal = causal;
  a->fmt = fmt;
  a->pfmt = fmt;
  a->kmax = kmax;
  a->sm_scale = sm_scale;
  a->q16 = q16;
  a->k16 = k16;
  a->v16 = v16;
  a->idx = idx;
  a->cnt = cnt;
  a->q4c = q4c;
  a->q4s = q4s;
  a->q4t = q4t;
  size_t nkv = (size_t)B * Hkv * S * D;
  double* k4 = (double*)malloc(sizeof(double) * nkv);
  double* v4 = (double*)malloc(sizeof(double) * nkv);
  tho_dequantize(k4c, k4s, k4t, B, Hkv, S, D, THO_AXIS_D, fmt, k4);
  tho_dequantize(v4c, v4s, v4t, B, Hkv, S, D, THO_AXIS_S, fmt, v4);
  a->k4 = k4;
  a->v4 = v4;
  *k16d = (double*)malloc(sizeof(double) * nkv);
  *v16d = (double*)malloc(sizeof(double) * nkv);
  for (size_t e = 0; e < nkv; ++e) {
    (*k16d)[e] = k16 ? tho_half_to_double(k16[e]) : 0.0;
    (*v16d)[e] = v16 ? tho_half_to_double(v16[e]) : 0.0;
  }
}

/* The row's query in both precisions and its term Dr = dO[r].O'[r]. */
static double tho_bwd_row(const tho_attn_args* a, int b, int hq, int r, const double* ohp,
                          const uint16_t* do16, double* q4, double* qh, double* dor) {
  int D = a->D, S = a->S;
  size_t row = ((size_t)b * a->Hq + hq) * S + r;
  tho_dequant_row(a->q4c, a->q4s, a->q4t, (size_t)b * a->Hq + hq, S, D, r, a->fmt, q4);
  double Dr = 0.0;
  for (int d = 0; d < D; ++d) {
    qh[d] = a->q16 ? tho_half_to_double(a->q16[row * D + d]) : 0.0;
    dor[d] = tho_half_to_double(do16[row * D + d]);
    Dr += dor[d] * ohp[row * D + d];
  }
  return Dr;
}

/* Backward pass.  lse [B,Hq,S] and ohp [B,Hq,S,D] come from the forward
 * (tho_attention_hp), do16 [B,Hq,S,D] is the output gradient.  dq
 * [B,Hq,S,D] is filled for the query blocks listed in qwork ((b, hq, i)
 * triples; NULL: all), dk and dv [B,Hkv,S,D] for the key blocks in kwork
 * ((b, hk, j) triples; NULL: all); udv (may be NULL) bounds what decisions
 * within fp32 evaluation error of their rounding boundary can change in dv.
 * Rows outside the work items are left untouched.  Sq = Sk. */
void tho_attention_bwd(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                       const uint8_t* q4c, const uint8_t* q4s, const float* q4t,
                       const uint8_t* k4c, const uint8_t* k4s, const float* k4t,
                       const uint8_t* v4c, const uint8_t* v4s, const float* v4t, int fmt,
                       const int32_t* idx, const int32_t* cnt, int kmax, int B, int Hq, int Hkv,
                       int S, int D, int bq, int bk, int causal, double sm_scale,
                       const double* lse, const double* ohp, const uint16_t* do16,
                       const int32_t* qwork, int nqwork, const int32_t* kwork, int nkwork,
                       double* dq, double* dk, double* dv, double* udv) {
  tho_attn_args a;
  memset(&a, 0, sizeof a);
  double *k16d, *v16d;
  tho_bwd_setup(&a, q16, k16, v16, q4c, q4s, q4t, k4c, k4s, k4t, v4c, v4s, v4t, fmt, idx, cnt, kmax,
                B, Hq, Hkv, S, D, bq, bk, causal, sm_scale, &k16d, &v16d);
  int nq = tho_cdiv(S, bq), nk = tho_cdiv(S, bk), G = Hq / Hkv;

  /* dQ, one query block at a time */
  int totq = qwork ? nqwork : B * Hq * nq;
#pragma omp parallel for schedule(dynamic, 1)
  for (int w = 0; w < totq; ++w) {
    int b = qwork ? qwork[3 * w] : w / (Hq * nq);
    int hq = qwork ? qwork[3 * w + 1] : (w / nq) % Hq;
    int i = qwork ? qwork[3 * w + 2] : w % nq;
    int hk = hq / G;
    size_t kvbase = ((size_t)b * Hkv + hk) * S;
    double *q4 = malloc(sizeof(double) * D), *qh = malloc(sizeof(double) * D);
    double* dor = malloc(sizeof(double) * D);
    double p[64], pt[64];
    int kind[64];
    int r1 = (i + 1) * bq < S ? (i + 1) * bq : S;
    int nvalid = tho_valid_blocks_kv(i, S, S, bq, bk, causal);
    for (int r = i * bq; r < r1; ++r) {
      size_t row = ((size_t)b * Hq + hq) * S + r;
      double Dr = tho_bwd_row(&a, b, hq, r, ohp, do16, q4, qh, dor);
      double L2 = lse[row] * THO_LOG2E;
      double* g = dq + row * D;
      for (int d = 0; d < D; ++d) g[d] = 0.0;
      for (int j = 0; j < nvalid; ++j) {
        int n = tho_tile_probs(&a, k16d, b, hq, r, j, L2, q4, qh, kind, p, pt, NULL);
        for (int c = 0; c < n; ++c) {
          if (!kind[c]) continue;
          size_t key = kvbase + (size_t)j * bk + c;
          const double* kv = (kind[c] == 1 ? a.k4 : k16d) + key * D;
          const double* vv = (kind[c] == 1 ? a.v4 : v16d) + key * D;
          double dP = 0.0;
          for (int d = 0; d < D; ++d) dP += dor[d] * vv[d];
          double dS = p[c] * (dP - Dr);
          for (int d = 0; d < D; ++d) g[d] += sm_scale * dS * kv[d];
        }
      }
    }
    free(dor);
    free(qh);
    free(q4);
  }

  /* dK and dV, one key block at a time, over every query row of the G
   * query heads of its key head whose query block sees it */
  int totk = kwork ? nkwork : B * Hkv * nk;
#pragma omp parallel for schedule(dynamic, 1)
  for (int w = 0; w < totk; ++w) {
    int b = kwork ? kwork[3 * w] : w / (Hkv * nk);
    int hk = kwork ? kwork[3 * w + 1] : (w / nk) % Hkv;
    int j = kwork ? kwork[3 * w + 2] : w % nk;
    size_t kvbase = ((size_t)b * Hkv + hk) * S;
    int c0 = j * bk, n = (c0 + bk < S ? c0 + bk : S) - c0;
    for (int c = 0; c < n; ++c)
      for (int d = 0; d < D; ++d) {
        dk[(kvbase + c0 + c) * D + d] = 0.0;
        dv[(kvbase + c0 + c) * D + d] = 0.0;
        if (udv) udv[(kvbase + c0 + c) * D + d] = 0.0;
      }
    double *q4 = malloc(sizeof(double) * D), *qh = malloc(sizeof(double) * D);
    double* dor = malloc(sizeof(double) * D);
    double p[64], pt[64], dpt[64];
    int kind[64];
    for (int hq = hk * G; hq < (hk + 1) * G; ++hq)
      for (int i = 0; i < nq; ++i) {
        if (j >= tho_valid_blocks_kv(i, S, S, bq, bk, causal)) continue;
        int r1 = (i + 1) * bq < S ? (i + 1) * bq : S;
        for (int r = i * bq; r < r1; ++r) {
          size_t row = ((size_t)b * Hq + hq) * S + r;
          double Dr = tho_bwd_row(&a, b, hq, r, ohp, do16, q4, qh, dor);
          double L2 = lse[row] * THO_LOG2E;
          tho_tile_probs(&a, k16d, b, hq, r, j, L2, q4, qh, kind, p, pt, udv ? dpt : NULL);
          for (int c = 0; c < n; ++c) {
            if (!kind[c]) continue;
            size_t key = kvbase + c0 + c;
            const double* vv = (kind[c] == 1 ? a.v4 : v16d) + key * D;
            const double* qv = kind[c] == 1 ? q4 : qh;
            double dP = 0.0;
            for (int d = 0; d < D; ++d) dP += dor[d] * vv[d];
            double dS = p[c] * (dP - Dr);
            for (int d = 0; d < D; ++d) {
              dk[key * D + d] += sm_scale * dS * qv[d];
              dv[key * D + d] += pt[c] * dor[d];
              if (udv) udv[key * D + d] += dpt[c] * fabs(dor[d]);
            }
          }
        }
      }
    free(dor);
    free(qh);
    free(q4);
  }
  free(v16d);
  free(k16d);
  free((void*)a.v4);
  free((void*)a.k4);
}

/* Test hook: the probabilities of query row r of head (b, hq) against every
 * key, as the backward recomputes them (kind, p, pt [S] each; keys outside
 * valid blocks get kind 0). */
void tho_row_probs(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16,
                   const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                   const uint8_t* k4s, const float* k4t, const uint8_t* v4c, const uint8_t* v4s,
                   const float* v4t, int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                   int B, int Hq, int Hkv, int S, int D, int bq, int bk, int causal,
                   double sm_scale, const double* lse, int b, int hq, int r, int32_t* kind,
                   double* p, double* pt) {
  tho_attn_args a;
  memset(&a, 0, sizeof a);
  double *k16d, *v16d;
  tho_bwd_setup(&a, q16, k16, v16, q4c, q4s, q4t, k4c, k4s, k4t, v4c, v4s, v4t, fmt, idx, cnt, kmax,
                B, Hq, Hkv, S, D, bq, bk, causal, sm_scale, &k16d, &v16d);
  double *q4 = malloc(sizeof(double) * D), *qh = malloc(sizeof(double) * D);
  size_t row = ((size_t)b * Hq + hq) * S + r;
  tho_dequant_row(q4c, q4s, q4t, (size_t)b * Hq + hq, S, D, r, fmt, q4);
  for (int d = 0; d < D; ++d) qh[d] = q16 ? tho_half_to_double(q16[row * D + d]) : 0.0;
  for (int c = 0; c < S; ++c) {
    kind[c] = 0;
    p[c] = pt[c] = 0.0;
  }
  int nvalid = tho_valid_blocks_kv(r / bq, S, S, bq, bk, causal);
  for (int j = 0; j < nvalid; ++j) {
    int kd[64];
    int n = tho_tile_probs(&a, k16d, b, hq, r, j, lse[row] * THO_LOG2E, q4, qh, kd, p + j * bk,
                           pt + j * bk, NULL);
    for (int c = 0; c < n; ++c) kind[j * bk + c] = kd[c];
  }
  free(qh);
  free(q4);
  free(v16d);
  free(k16d);
  free((void*)a.v4);
  free((void*)a.k4);
}

/* Scores of the FP4 path for one query row against keys [c0, c1) (test hook:
 * the raw dot products of the dequantised operands, before sm_scale). */
void tho_fp4_scores(const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c,
                    const uint8_t* k4s, const float* k4t, int fmt, int S, int D, int r, int c0,
                    int c1, double* out) {
  double* q = (double*)malloc(sizeof(double) * (size_t)S * D);
  double* k = (double*)malloc(sizeof(double) * (size_t)S * D);
  tho_dequantize(q4c, q4s, q4t, 1, 1, S, D, THO_AXIS_D, fmt, q);
  tho_dequantize(k4c, k4s, k4t, 1, 1, S, D, THO_AXIS_D, fmt, k);
  for (int c = c0; c < c1; ++c) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += q[(size_t)r * D + d] * k[(size_t)c * D + d];
    out[c - c0] = s;
  }
  free(k);
  free(q);
}

/* Test hook: the values and the decisions that may go either way of one
 * tile row of n <= 64 keys (t and tb in log2 units, mask != 0 for masked
 * keys) in precision prec (0 MX, 1 NVFP4, 2 MXFP8 tier, 3 FP16) with score
 * evaluation path epath.  pq[n] receives the values relative to 2^max t;
 * decision f changes keys [k0[f], k1[f]) by dp[f * 64 + c]; returns the
 * number of decisions (at most maxf are stored). */
int tho_p_tile_decisions(const double* t, const double* tb, const int* mask, int n, int prec, int epath,
                         double* pq, int* k0, int* k1, double* dp, int maxf) {
  double mt = -INFINITY;
  for (int c = 0; c < n; ++c)
    if (!mask[c] && t[c] > mt) mt = t[c];
  tho_flip* fl = (tho_flip*)malloc(sizeof(tho_flip) * THO_TILE_FLIPS);
  int nf = prec == THO_PATH_F16 ? tho_quantize_p_tile16(t, tb, mask, n, mt, pq, fl, THO_TILE_FLIPS)
                                : tho_quantize_p_tile(t, tb, mask, n, prec, epath, mt, pq, fl, THO_TILE_FLIPS);
  for (int f = 0; f < nf && f < maxf && f < THO_TILE_FLIPS; ++f) {
    k0[f] = fl[f].k0;
    k1[f] = fl[f].k1;
    for (int c = 0; c < 64; ++c) dp[f * 64 + c] = (c >= fl[f].k0 && c < fl[f].k1) ? fl[f].dp[c] : 0.0;
  }
  free(fl);
  return nf;
}

/* ------------------------------------------------------------------ */
/* Array forms of the scalar format routines (test sweeps)            */
/* ------------------------------------------------------------------ */

void tho_e2m1_encode_array(const double* x, const double* s, size_t n, uint8_t* out) {
  for (size_t t = 0; t < n; ++t) out[t] = (uint8_t)tho_e2m1_encode(x[t], s[t]);
}

void tho_e4m3_encode_ratio_array(const double* num, const double* den, size_t n, uint8_t* out) {
  for (size_t t = 0; t < n; ++t) out[t] = (uint8_t)tho_e4m3_encode_ratio(num[t], den[t]);
}

void tho_round_to_half_array(const double* x, size_t n, double* out) {
  for (size_t t = 0; t < n; ++t) out[t] = tho_round_to_half(x[t]);
}

void tho_half_to_double_array(const uint16_t* h, size_t n, double* out) {
  for (size_t t = 0; t < n; ++t) out[t] = tho_half_to_double(h[t]);
}
