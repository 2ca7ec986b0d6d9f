// Attn-QAT backward of the mixed FP4/FP16 attention, and the forward's
// high-precision output O' that it needs (Attn-QAT, "Methodik": the
// probabilities are recomputed from the forward's log-sum-exp in the forward's
// own precision, and the row term of the softmax gradient comes from O', the
// output with unquantised probabilities, not from the FP4 output).
//
// Every quantiser is passed straight through.  For query row r, key c of a
// valid pair, in the precision of the path the pair's block takes for r's
// query block (FP4-decoded Q, K, V on the FP4 path, fp16 on the FP16 path):
//   t = sm_scale log2(e) q.k, p = 2^(t - L2), L2 = lse log2(e)
//   pt = the forward's probability (FP4 path: two-level quantised, MX or
//        NVFP4; FP16 path: p rounded to fp16)
//   dV[c] += pt dO[r], dS = p (dO[r].v[c] - dO[r].O'[r]),
//   dQ[r] += sm_scale dS k[c], dK[c] += sm_scale dS q[r].
//
// All products run on the fp16 matrix cores: FP4-decoded operands are exact
// in fp16 (NVFP4's slice scales enter as fp32 factors).  After a preparation
// pass, the row kernel (one lane per query, as in the forward) computes O'
// or dQ, and the key kernel (one lane per key) computes dK and dV.
#include <hip/hip_runtime.h>

#include "common.h"

namespace thrift {
namespace {

constexpr int kBlkK = 64;  // key block
constexpr int kMaxS = 262144;
constexpr int kMaxKw = kMaxS / kBlkK / 32;  // promoted-bit words per query block row
constexpr float kLog2eB = 1.44269504088896341f;

typedef float v2f __attribute__((ext_vector_type(2)));

// The query-row counterpart of krow for one 32-row tile: row m reads query
// qperm(m), so register i of a lane of half hi holds query hi*16 + i.
__device__ inline int qperm(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, bytes, 0x00020000);
}
// 16 bytes at byte offset off; reads past the record count return zeros.
__device__ inline v8h ld8h(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(v8h, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

struct BwdArgs {
  const _Float16 *q16, *k16, *v16, *do16;  // [B,H,S,D]
  const _Float16 *qd, *kd;                 // FP4-decoded Q, K rows [B,H,S,D]
  const _Float16* vd;                      // FP4-decoded V rows [B,Hkv,Sp,D]
  const _Float16 *qt, *qdt, *dot;          // transposed [B,Hq,D,Sp]
  const _Float16 *kt, *kdt, *vt, *vdt;     // transposed [B,Hkv,D,Sp]
  const uint32_t* prom;                    // promoted-block bits [B,Hq,nq,nkw]
  const float *lse, *drow;                 // [B,Hq,S]
  const float *tq, *tk, *tv;               // NVFP4 slice scales [B,H] (NULL for MXFP4)
  float* out;                              // row kernel: O' or dQ [B,Hq,S,D]
  float *dk, *dv;                          // [B,Hkv,S,D]
  int B, Hq, Hkv, S, Sp, bq, nq, nkw, causal;
  float c;         // sm_scale * log2(e)
  float sm_scale;
};

// ---- preparation ------------------------------------------------------------------

// FP4 rows decoded to fp16: codes [R][L/2] (even element in the low
// nibble), block scales [R][L/g] (MXFP4: E8M0, g = 32; NVFP4: E4M3, g = 16);
// one thread per 8 elements.  Out [R][L]; or, with vD > 0, rows are V's
// stored (batch*head, 64-token block, channel) rows of L = 64 tokens and go
// to V^T [batch*head][vD][nb*64].  E2M1 times a power of two (MX) or times an
// E4M3 value (NVFP4, at most 6 significant bits, 2^-10 .. 2688) is exact in
// fp16; tsc (NVFP4 slice scales per batch*head of rows_per_bh rows, or
// NULL) multiplies in before the one rounding.
__global__ __launch_bounds__(256) void decode_fp4_kernel(const uint8_t* codes, const uint8_t* scales, size_t R,
                                                         int L, int fmt, const float* tsc, size_t rows_per_bh,
                                                         _Float16* out, int vD, int vnb) {
  const size_t e8 = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t n8 = R * (size_t)(L / 8);
  if (e8 >= n8) return;
  const size_t row = e8 / (L / 8);
  const int c8 = (int)(e8 % (L / 8)) * 8;
  const uint32_t cw = *(const uint32_t*)(codes + row * (L / 2) + c8 / 2);
  const int g = fmt == THRIFT_MXFP4 ? 32 : 16;
  const uint32_t sb = scales[row * (L / g) + c8 / g];
  float f = fmt == THRIFT_MXFP4 ? ldexpf(1.0f, (int)sb - 127) : e4m3_to_float(sb);
  if (tsc) f *= tsc[row / rows_per_bh];
  const v2f v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0),
                    __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1),
                    __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2),
                    __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3)};
  v8h o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (_Float16)(v[e / 2][e % 2] * f);
  size_t dst = row * L + c8;
  if (vD > 0) {
    const size_t d = row % vD, jb = (row / vD) % vnb, bh = row / ((size_t)vD * vnb);
    dst = (bh * vD + d) * ((size_t)vnb * 64) + jb * 64 + c8;
  }
  *(v8h*)(out + dst) = o;
}

// out[bh][c][r] = in[bh][r][c] (times tsc[bh] when tsc is not NULL, one
// rounding) for r < R, zero for R <= r < Rout; in rows of C halves.  64x64
// tiles through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const _Float16* in, int R, int C, int Rout,
                                                        const float* tsc, _Float16* out) {
  // 64x64 tile through LDS with 16-byte loads and stores: a thread reads 8
  // consecutive columns of one row and writes 8 consecutive rows of one
  // output row (C and Rout are multiples of 8, the tile origin of 64)
  __shared__ _Float16 tile[64][66];
  const size_t bh = blockIdx.y;
  const int ct = cdiv(C, 64);
  const int r0 = (blockIdx.x / ct) * 64, c0 = (blockIdx.x % ct) * 64;
  const int t = threadIdx.x, t8 = (t & 7) * 8, tr = t >> 3;
  const _Float16* src = in + bh * (size_t)R * C;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = h * 32 + tr, r = r0 + row, c = c0 + t8;
    v8h x = {};
    if (r < R && c < C) x = *(const v8h*)(src + (size_t)r * C + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) tile[row][t8 + u] = x[u];
  }
  __syncthreads();
  _Float16* dst = out + bh * (size_t)C * Rout;
  const float f = tsc ? tsc[bh] : 1.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int col = h * 32 + tr, c = c0 + col, r = r0 + t8;
    if (c < C && r < Rout) {
      v8h y;
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = tsc ? (_Float16)((float)tile[t8 + u][col] * f) : tile[t8 + u][col];
      *(v8h*)(dst + (size_t)c * Rout + r) = y;
    }
  }
}

// Promoted-block bits of each (batch, query head, query block).
__global__ __launch_bounds__(256) void prom_bits_kernel(const int32_t* idx, const int32_t* cnt, int nrows,
                                                        int kmax, int nk, int nkw, uint32_t* bits) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= nrows) return;
  uint32_t* w = bits + (size_t)row * nkw;
  for (int k = 0; k < nkw; ++k) w[k] = 0;
  const int n = min(max(cnt[row], 0), kmax);
  for (int s = 0; s < n; ++s) {
    const int j = idx[(size_t)row * kmax + s];
    if (j >= 0 && j < nk) w[j >> 5] |= 1u << (j & 31);
  }
}

// Row term dO[r] . O'[r]: D/8 lanes per row (a 16-byte load of dO and two of
// O' each), summed across those lanes; every lane reaches the shuffles.
template <int D>
__global__ __launch_bounds__(256) void row_term_kernel(const _Float16* do16, const float* ohp, size_t nrows,
                                                       float* drow) {
  constexpr int LPR = D / 8;  // lanes per row: 16 or 8, a divisor of the wave
  const size_t row = ((size_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int sub = threadIdx.x % LPR;
  float s = 0.0f;
  if (row < nrows) {
    const v8h h = *(const v8h*)(do16 + row * D + sub * 8);
    const float4 x = *(const float4*)(ohp + row * D + sub * 8), y = *(const float4*)(ohp + row * D + sub * 8 + 4);
    s = (float)h[0] * x.x + (float)h[1] * x.y + (float)h[2] * x.z + (float)h[3] * x.w + (float)h[4] * y.x +
        (float)h[5] * y.y + (float)h[6] * y.z + (float)h[7] * y.w;
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (row < nrows && sub == 0) drow[row] = s;
}

// ---- row kernel: one lane per query (O' or dQ) ---------------------------------

constexpr int kModeOhp = 0;
constexpr int kModeDq = 1;

// LDS stage of one key block for the row kernel: K rows, V rows (dQ mode)
// and the transposed operand of the second product (K^T or V^T).
template <int D>
struct RowLds {
  static constexpr int KR = D + 8;      // halves per K/V row
  static constexpr int TR = kBlkK + 8;  // halves per transposed row
  static constexpr int K = 0;
  static constexpr int V = K + kBlkK * KR * 2;
  static constexpr int T = V + kBlkK * KR * 2;
  static constexpr int SIZE = T + D * TR * 2;
};

// Workgroup = query block i of (batch, query head), one wave per 32 rows.
// Per valid key block j, in the precision of its path: S^T = K Q^T (keys in
// krow order), p = 2^(t - L2); then O'^T += V^T P^T, or dP^T = V dO^T,
// dS = p (dP - Dr) and dQ^T += K^T dS^T.  The waves share each key block's
// operands through one LDS stage; the next block's are loaded into
// registers while the current one is computed.
template <int D, int MODE, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_row_kernel(BwdArgs a) {
  using L = RowLds<D>;
  constexpr int NT = NW * 64;
  constexpr int PK = kBlkK * D / 8 / NT;  // 16-byte pieces of a K or V block per thread
  constexpr int PT = D * kBlkK / 8 / NT;  // of the transposed block
  __shared__ __attribute__((aligned(16))) char smem[L::SIZE];
  __shared__ uint32_t pmw[kMaxKw];  // this row of promoted-block bits
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), hi = lane >> 5, r32 = lane & 31;
  const int BHq = a.B * a.Hq, G = a.Hq / a.Hkv;
  const int x = blockIdx.x;
  const int i = a.causal ? a.nq - 1 - x / BHq : x / BHq;  // longest rows first
  const int bhq = x % BHq;
  const int b = bhq / a.Hq, hq = bhq % a.Hq;
  const size_t bhk = (size_t)b * a.Hkv + hq / G;
  const int S = a.S, Sp = a.Sp;
  const int q0 = i * a.bq + w * 32;
  const int qrow = q0 + r32;
  const bool qok = qrow < S;  // waves past S still pass every barrier

  const auto qrs = rsrc(a.q16 + (size_t)bhq * S * D, S * D * 2);
  const auto qdrs = rsrc(a.qd + (size_t)bhq * S * D, S * D * 2);
  v8h qh[D / 16], qd[D / 16], dh[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int off = (qrow * D + kk * 16 + hi * 8) * 2;
    qh[kk] = ld8h(qrs, off);
    qd[kk] = ld8h(qdrs, off);
  }
  if constexpr (MODE == kModeDq) {
    const auto drs = rsrc(a.do16 + (size_t)bhq * S * D, S * D * 2);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) dh[kk] = ld8h(drs, (qrow * D + kk * 16 + hi * 8) * 2);
  }
  const float L2 = qok ? a.lse[(size_t)bhq * S + qrow] * kLog2eB : 0.0f;
  const float Dr = (MODE == kModeDq && qok) ? a.drow[(size_t)bhq * S + qrow] : 0.0f;
  // NVFP4: FP4 pairs' scores and dP carry the slice scales (exact fp32 factors)
  const float cq4 = a.tq ? a.c * a.tq[bhq] * a.tk[bhk] : a.c;
  const float dpf4 = a.tv ? a.tv[bhk] : 1.0f;

  v16f acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = v16f{};

  const auto k16rs = rsrc(a.k16 + bhk * S * D, S * D * 2);
  const auto kdrs = rsrc(a.kd + bhk * S * D, S * D * 2);
  const auto v16rs = rsrc(a.v16 + bhk * S * D, S * D * 2);
  const auto vdrs = rsrc(a.vd + bhk * Sp * D, Sp * D * 2);
  const uint32_t* pm = a.prom + ((size_t)bhq * a.nq + i) * a.nkw;
  const int nvalid = valid_kv_blocks(i, S, a.bq, kBlkK, a.causal);
  for (int k = t; k < a.nkw; k += NT) pmw[k] = pm[k];
  __syncthreads();

  v4i pk[PK], pv[PK], pt[PT];
  auto promoted = [&](int j) { return ((pmw[j >> 5] >> (j & 31)) & 1u) != 0; };
  auto fetch = [&](int j) {
    const bool f16 = promoted(j);
    const auto krs = f16 ? k16rs : kdrs;
    const auto vrs = f16 ? v16rs : vdrs;
    const _Float16* T = (MODE == kModeOhp ? (f16 ? a.vt : a.vdt) : (f16 ? a.kt : a.kdt)) + bhk * D * Sp;
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int c = t + u * NT, row = c / (D / 8), c8 = c % (D / 8);
      const int off = ((j * kBlkK + row) * D + c8 * 8) * 2;
      pk[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
      if constexpr (MODE == kModeDq) pv[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int c = t + u * NT, d = c / (kBlkK / 8), k8 = c % (kBlkK / 8);
      pt[u] = *(const v4i*)(T + (size_t)d * Sp + j * kBlkK + k8 * 8);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int c = t + u * NT, row = c / (D / 8), c8 = c % (D / 8);
      *(v4i*)(smem + L::K + (row * L::KR + c8 * 8) * 2) = pk[u];
      if constexpr (MODE == kModeDq) *(v4i*)(smem + L::V + (row * L::KR + c8 * 8) * 2) = pv[u];
    }
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int c = t + u * NT, d = c / (kBlkK / 8), k8 = c % (kBlkK / 8);
      *(v4i*)(smem + L::T + (d * L::TR + k8 * 8) * 2) = pt[u];
    }
  };

  if (nvalid > 0) fetch(0);
  for (int j = 0; j < nvalid; ++j) {
    const bool f16 = promoted(j);
    __syncthreads();  // every wave is done with the previous block
    stash();
    __syncthreads();
    if (j + 1 < nvalid) fetch(j + 1);
    const _Float16* ks = (const _Float16*)(smem + L::K);
    v16f s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = v16f{};
      const _Float16* kr = ks + krow(mt, r32) * L::KR + hi * 8;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) s[mt] = mfma_f16(*(const v8h*)(kr + kk * 16), f16 ? qh[kk] : qd[kk], s[mt]);
    }
    v16f dp[2];
    if constexpr (MODE == kModeDq) {
      const _Float16* vs = (const _Float16*)(smem + L::V);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        dp[mt] = v16f{};
        const _Float16* vr = vs + krow(mt, r32) * L::KR + hi * 8;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) dp[mt] = mfma_f16(*(const v8h*)(vr + kk * 16), dh[kk], dp[mt]);
      }
    }
    // B operand of the second product: step st holds keys hi*32 + 8 st + u,
    // registers 8 (st % 2) + u of tile st / 2
    v8h pb[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int key = j * kBlkK + hi * 32 + mt * 16 + ii;
        const bool ok = qok && key < S && !(a.causal && key > qrow);
        const float p = ok ? exp2_fast(__builtin_fmaf(s[mt][ii], f16 ? a.c : cq4, -L2)) : 0.0f;
        float v = p;
        if constexpr (MODE == kModeDq) v = p * (dp[mt][ii] * (f16 ? 1.0f : dpf4) - Dr);
        pb[mt * 2 + ii / 8][ii % 8] = (_Float16)v;
      }
    const _Float16* ts = (const _Float16*)(smem + L::T);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const v8h tv = *(const v8h*)(ts + (dt * 32 + r32) * L::TR + hi * 32 + st * 8);
        acc[dt] = mfma_f16(tv, pb[st], acc[dt]);
      }
  }
  if (!qok) return;
  const float f = MODE == kModeDq ? a.sm_scale : 1.0f;
  float* dst = a.out + ((size_t)bhq * S + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = dt * 32 + i4 * 8 + hi * 4;
      *(float4*)(dst + d0) = make_float4(acc[dt][i4 * 4] * f, acc[dt][i4 * 4 + 1] * f, acc[dt][i4 * 4 + 2] * f,
                                         acc[dt][i4 * 4 + 3] * f);
    }
}

// ---- key kernel: one lane per key (dK, dV) -------------------------------------

// LDS stage of one 32-query step for the key kernel: query rows (fp16 and
// FP4-decoded, as needed), dO rows, their transposes, and the rows' LSE and
// row terms; plus each wave's per-query factors of P's quantisation.
template <int D>
struct KeyLds {  // (FA, FH: [wave][group][query]; HT: [wave][query] half-tile maxima, NVFP4)
  static constexpr int RR = D + 8;  // halves per query row
  static constexpr int TR = 32 + 8; // halves per transposed row (32 queries)
  static constexpr int QR16 = 0;
  static constexpr int QRD = QR16 + 32 * RR * 2;
  static constexpr int DOR = QRD + 32 * RR * 2;
  static constexpr int QT16 = DOR + 32 * RR * 2;
  static constexpr int QTD = QT16 + D * TR * 2;
  static constexpr int DOT = QTD + D * TR * 2;
  static constexpr int L2 = DOT + D * TR * 2;  // 32 floats
  static constexpr int DR = L2 + 32 * 4;       // 32 floats
  static constexpr int FA = DR + 32 * 4;
  static constexpr int FH = FA + 4 * 2 * 32 * 4;
  static constexpr int HT = FH + 4 * 2 * 32 * 4;
  static constexpr int SIZE = HT + 4 * 32 * 4;
};

// Workgroup = two key blocks (2 x 64 keys) of (batch, key head), four waves
// of 32 keys each, one lane per key.  Steps of 32 query rows run over the G
// query heads of the key head and the rows that see the blocks; each step's
// query rows, dO rows and their transposes come once into LDS for all four
// waves (the next step's are loaded into registers meanwhile).  Per step and
// wave: S = Q K^T and dP = dO V^T with this lane's key as the column, p and
// dS per element; on FP4 pairs the probability the forward used is rebuilt
// from its quantisation groups (MX: the wave's 32 keys; NVFP4: 16-key groups
// under the 64-key tile maximum, which the block's two waves exchange), whose
// maxima come from S^T = K Q^T (same operands swapped, one lane per query)
// and are handed to the key-major lanes through the wave's own LDS slot.
// Then dV += pt^T dO
// and dK += dS^T Q.  Only the K and V operands of the precision in use are
// held in registers; they are reloaded when a step switches path.
template <int D, int FMT>
__global__ __launch_bounds__(256) void bwd_key_kernel(BwdArgs a) {
  using L = KeyLds<D>;
  constexpr int PR = 32 * D / 8 / 256;  // 16-byte pieces of a 32-row tile per thread
  __shared__ __attribute__((aligned(16))) char smem[L::SIZE];
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), hi = lane >> 5, r32 = lane & 31;
  const int BHk = a.B * a.Hkv, G = a.Hq / a.Hkv;
  const int nk = cdiv(a.S, kBlkK);
  const int x = blockIdx.x;
  const int j0 = (x / BHk) * 2;  // causal: the lowest key blocks have the most rows
  const size_t bhk = x % BHk;
  const int b = (int)(bhk / a.Hkv), hk = (int)(bhk % a.Hkv);
  const int S = a.S, Sp = a.Sp;
  const int jb = j0 + (w >> 1);              // this wave's key block (waves w, w ^ 1 share it)
  const int key = jb * kBlkK + (w & 1) * 32 + r32;  // this lane's key (column of S)

  const auto k16rs = rsrc(a.k16 + bhk * S * D, S * D * 2);
  const auto kdrs = rsrc(a.kd + bhk * S * D, S * D * 2);
  const auto v16rs = rsrc(a.v16 + bhk * S * D, S * D * 2);
  const auto vdrs = rsrc(a.vd + bhk * Sp * D, Sp * D * 2);
  v8h kr[D / 16], vr[D / 16];
  int cur = -1;  // path whose K and V operands kr, vr hold (1 FP16, 0 FP4)
  auto load_kv = [&](bool f16) {
    const auto krs = f16 ? k16rs : kdrs;
    const auto vrs = f16 ? v16rs : vdrs;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int off = (key * D + kk * 16 + hi * 8) * 2;
      kr[kk] = ld8h(krs, off);
      vr[kk] = ld8h(vrs, off);
    }
    cur = f16;
  };
  v16f dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dk[dt] = dv[dt] = v16f{};
  const float dpf4 = a.tv ? a.tv[bhk] : 1.0f;

  // step sequence: for g < G, q0 from the first row that sees block j0, by 32
  const int qstart = a.causal ? (j0 * kBlkK / 32) * 32 : 0;
  const int nsteps_g = cdiv(S - qstart, 32);
  const int nsteps = G * nsteps_g;
  // steps advance (g, q0) incrementally; the promoted bits of blocks j0 and
  // j0+1 (one word: j0 is even) are loaded two steps ahead so that no step
  // waits for them
  const int bq_shift = a.bq == 128 ? 7 : 6;
  auto advance = [&](int& g, int& q0) {
    q0 += 32;
    if (q0 >= S) {
      q0 = qstart;
      ++g;
    }
  };
  auto word_addr = [&](int g, int q0) {
    const int bhq = b * a.Hq + hk * G + (g < G ? g : G - 1);
    return a.prom + ((size_t)bhq * a.nq + (q0 >> bq_shift)) * a.nkw + (j0 >> 5);
  };
  auto bit = [&](uint32_t word, int j) { return j < nk && ((word >> (j & 31)) & 1u) != 0; };
  v4i pq16[PR], pqd[PR], pdo[PR], pt16[PR], ptd[PR], pdt[PR];
  float pl = 0.0f, pr = 0.0f;
  auto fetch = [&](int g, int q0, uint32_t word) {
    const int bhq = b * a.Hq + hk * G + g;
    const bool f0 = bit(word, j0), f1 = bit(word, j0 + 1);
    const bool need16 = f0 || f1, needd = !f0 || !f1;
    const auto qrs = rsrc(a.q16 + (size_t)bhq * S * D, S * D * 2);
    const auto qdrs = rsrc(a.qd + (size_t)bhq * S * D, S * D * 2);
    const auto drs = rsrc(a.do16 + (size_t)bhq * S * D, S * D * 2);
    const size_t tb = (size_t)bhq * D * Sp;
#pragma unroll
    for (int u = 0; u < PR; ++u) {
      const int c = t + u * 256;
      const int row = c / (D / 8), c8 = c % (D / 8);  // row-major tiles
      const int off = ((q0 + row) * D + c8 * 8) * 2;
      if (need16) pq16[u] = __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0);
      if (needd) pqd[u] = __builtin_amdgcn_raw_buffer_load_b128(qdrs, off, 0, 0);
      pdo[u] = __builtin_amdgcn_raw_buffer_load_b128(drs, off, 0, 0);
      const int d = c / 4, c4 = c % 4;  // transposed tiles: row d, 8 queries
      const size_t toff = tb + (size_t)d * Sp + q0 + c4 * 8;
      if (need16) pt16[u] = *(const v4i*)(a.qt + toff);
      if (needd) ptd[u] = *(const v4i*)(a.qdt + toff);
      pdt[u] = *(const v4i*)(a.dot + toff);
    }
    if (t < 32) {
      const int q = q0 + t;
      pl = q < S ? a.lse[(size_t)bhq * S + q] * kLog2eB : 0.0f;
      pr = q < S ? a.drow[(size_t)bhq * S + q] : 0.0f;
    }
    return need16 * 2 + needd;
  };
  auto stash = [&](int need) {
#pragma unroll
    for (int u = 0; u < PR; ++u) {
      const int c = t + u * 256;
      const int row = c / (D / 8), c8 = c % (D / 8);
      const int ro = (row * L::RR + c8 * 8) * 2;
      if (need & 2) *(v4i*)(smem + L::QR16 + ro) = pq16[u];
      if (need & 1) *(v4i*)(smem + L::QRD + ro) = pqd[u];
      *(v4i*)(smem + L::DOR + ro) = pdo[u];
      const int d = c / 4, c4 = c % 4;
      const int to = (d * L::TR + c4 * 8) * 2;
      if (need & 2) *(v4i*)(smem + L::QT16 + to) = pt16[u];
      if (need & 1) *(v4i*)(smem + L::QTD + to) = ptd[u];
      *(v4i*)(smem + L::DOT + to) = pdt[u];
    }
    if (t < 32) {
      ((float*)(smem + L::L2))[t] = pl;
      ((float*)(smem + L::DR))[t] = pr;
    }
  };

  int g = 0, q0 = qstart;          // this step
  int g1 = 0, q01 = qstart;        // the next
  advance(g1, q01);
  int g2 = g1, q02 = q01;          // the one after
  advance(g2, q02);
  uint32_t wcur = nsteps > 0 ? __builtin_amdgcn_readfirstlane(*word_addr(g, q0)) : 0u;
  uint32_t wnext = nsteps > 1 ? *word_addr(g1, q01) : 0u;  // in flight
  int need = nsteps > 0 ? fetch(g, q0, wcur) : 0;
  float cq4 = a.c;  // scale of FP4 pairs' scores (NVFP4: times the head's slice scales)
  int cq_g = -1;
  for (int n = 0; n < nsteps; ++n) {
    const int bhq = b * a.Hq + hk * G + g;
    const bool f16 = bit(wcur, jb);
    if (g != cq_g) {
      cq4 = a.tq ? a.c * a.tq[bhq] * a.tk[bhk] : a.c;
      cq_g = g;
    }
    __syncthreads();  // every wave is done with the previous step
    stash(need);
    __syncthreads();
    if (n + 1 < nsteps) {
      const uint32_t w1 = __builtin_amdgcn_readfirstlane(wnext);
      wnext = *word_addr(g2, q02);
      need = fetch(g1, q01, w1);
      wcur = w1;
    }
    // (steps whose pairs are all masked for this wave add zeros: a branch
    // around the products would make the compiler copy the accumulators)
    if ((int)f16 != cur) load_kv(f16);
    const _Float16* qrow = (const _Float16*)(smem + (f16 ? L::QR16 : L::QRD)) + qperm(r32) * L::RR + hi * 8;
    const _Float16* drow = (const _Float16*)(smem + L::DOR) + qperm(r32) * L::RR + hi * 8;
    v16f s = v16f{}, dp = v16f{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      s = mfma_f16(*(const v8h*)(qrow + kk * 16), kr[kk], s);
      dp = mfma_f16(*(const v8h*)(drow + kk * 16), vr[kk], dp);
    }
    // FP4 pairs: per query and P group, p * fa is the element over its block
    // scale and pt = code * fh (this lane's key is in group grp of the wave)
    const float cj = f16 ? a.c : cq4;
    const int grp = FMT == THRIFT_MXFP4 ? 0 : r32 >> 4;
    const float* wa = (const float*)(smem + L::FA) + (w * 2 + grp) * 32;
    const float* wh = (const float*)(smem + L::FH) + (w * 2 + grp) * 32;
    float gm0 = -INFINITY, gm1 = -INFINITY, Lq = 0.0f;  // group maxima (raw scores) of query qperm(r32)
    if (!f16) {
      v16f st = v16f{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) st = mfma_f16(kr[kk], *(const v8h*)(qrow + kk * 16), st);
      // column r32 is query q0 + qperm(r32); register ii is key (ii/4)*8 + hi*4 + ii%4 of the wave's 32
      const int qm = q0 + qperm(r32);
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const int kx = jb * kBlkK + (w & 1) * 32 + (ii >> 2) * 8 + hi * 4 + (ii & 3);
        const bool ok = qm < S && kx < S && !(a.causal && kx > qm);
        const float v = ok ? st[ii] : -INFINITY;
        if (ii < 8)
          gm0 = fmaxf(gm0, v);
        else
          gm1 = fmaxf(gm1, v);
      }
      gm0 = pair_max(gm0);
      gm1 = pair_max(gm1);
      Lq = ((const float*)(smem + L::L2))[qperm(r32)];
      if constexpr (FMT == THRIFT_MXFP4) {
        // MX level 1 is any power of two (the E8M0 block scale absorbs it):
        // z = ceil(L2); block exponent from the group maximum's probability
        const float gm = fmaxf(gm0, gm1);
        const float z = ceilf(Lq);
        const uint32_t E = (__float_as_uint(exp2_fast(__builtin_fmaf(gm, cj, -z))) >> 23) & 0xFF;
        const int X = (int)(E > 3 ? E - 2 : 1) - 127;
        const float zx = z + (float)X;
        const bool any = gm > -INFINITY;
        if (hi == 0) {
          ((float*)wa)[qperm(r32)] = any ? exp2_fast(Lq - zx) : 0.0f;
          ((float*)wh)[qperm(r32)] = any ? exp2_fast(zx - Lq) : 0.0f;
        }
        // the wave reads back its own slot: its LDS operations complete in order
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      } else {
        if (hi == 0) ((float*)(smem + L::HT))[w * 32 + qperm(r32)] = fmaxf(gm0, gm1);
      }
    }
    if constexpr (FMT == THRIFT_NVFP4) {
      // level 1 of NVFP4 is the query's maximum over the whole 64-key tile:
      // the two waves of the block exchange their halves (every wave passes
      // this barrier on every step)
      __syncthreads();
      if (!f16) {
        const float tm = fmaxf(fmaxf(gm0, gm1), ((const float*)(smem + L::HT))[(w ^ 1) * 32 + qperm(r32)]);
        const float tml = tm * cj;
        // a tile more than 2^60 below the row's total contributes nothing
        const bool live = tm > -INFINITY && tml - Lq > -60.0f;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float gv = 2688.0f * exp2_fast(__builtin_fmaf(g ? gm1 : gm0, cj, -tml));
          v2s_t sb = {0, 0};
          sb = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(sb, fminf(gv * (1.0f / 6.0f), 448.0f), 0.0f, 1.0f, false);
          const float s2 = e4m3_to_float((uint32_t)sb[0] & 0xFF);
          const bool on = live && s2 > 0.0f;
          if (hi == 0) {
            float* fa = (float*)(smem + L::FA) + (w * 2 + g) * 32;
            float* fh = (float*)(smem + L::FH) + (w * 2 + g) * 32;
            fa[qperm(r32)] = on ? exp2_fast(Lq - tml) * (2688.0f / s2) : 0.0f;
            fh[qperm(r32)] = on ? s2 * exp2_fast(tml - Lq) * (1.0f / 2688.0f) : 0.0f;
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
    // A operands of the two products: step st holds queries hi*16 + 8 st + u;
    // this lane's queries are q0 + hi*16 + ii, four at a time
    v8h pA[2], sA[2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 l4 = *(const float4*)(smem + L::L2 + (hi * 16 + u * 4) * 4);
      const float4 r4 = *(const float4*)(smem + L::DR + (hi * 16 + u * 4) * 4);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
      float p[4], pt[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ii = u * 4 + e, q = q0 + hi * 16 + ii;
        const bool ok = q < S && key < S && !(a.causal && key > q);
        p[e] = ok ? exp2_fast(__builtin_fmaf(s[ii], cj, -lv[e])) : 0.0f;
        sA[ii / 8][ii % 8] = (_Float16)(p[e] * (dp[ii] * (f16 ? 1.0f : dpf4) - rv[e]));
        pt[e] = p[e];
      }
      if (!f16) {
        const float4 a4 = *(const float4*)(wa + hi * 16 + u * 4);
        const float4 h4 = *(const float4*)(wh + hi * 16 + u * 4);
        const uint32_t y0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, p[0] * a4.x, p[1] * a4.y, 1.0f, 0);
        const uint32_t y1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, p[2] * a4.z, p[3] * a4.w, 1.0f, 0);
        const v2f c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(y0, 1.0f, 0);
        const v2f c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(y1, 1.0f, 0);
        pt[0] = c0[0] * h4.x;
        pt[1] = c0[1] * h4.y;
        pt[2] = c1[0] * h4.z;
        pt[3] = c1[1] * h4.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pA[(u * 4 + e) / 8][(u * 4 + e) % 8] = (_Float16)pt[e];
    }
    const _Float16* qT = (const _Float16*)(smem + (f16 ? L::QT16 : L::QTD));
    const _Float16* oT = (const _Float16*)(smem + L::DOT);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int off = (dt * 32 + r32) * L::TR + hi * 16 + st * 8;
        dv[dt] = mfma_f16(pA[st], *(const v8h*)(oT + off), dv[dt]);
        dk[dt] = mfma_f16(sA[st], *(const v8h*)(qT + off), dk[dt]);
      }
    g = g1;
    q0 = q01;
    g1 = g2;
    q01 = q02;
    advance(g2, q02);
  }
  // C layout: column d = dt*32 + r32, register ii is key (ii/4)*8 + hi*4 + ii%4 of the wave's 32
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const int kx = jb * kBlkK + (w & 1) * 32 + (ii >> 2) * 8 + hi * 4 + (ii & 3);
      if (kx < S) {
        const size_t e = (bhk * S + kx) * D + dt * 32 + r32;
        a.dk[e] = dk[dt][ii] * a.sm_scale;
        a.dv[e] = dv[dt][ii];
      }
    }
}

// ---- host side -----------------------------------------------------------------------

struct BwdLayout {
  size_t qd, qt, qdt, dot, kd, kt, kdt, vd, vt, vdt, prom, drow, total;
};

inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }

BwdLayout bwd_layout(int B, int Hq, int Hkv, int S, int D, int bq) {
  const size_t Sp = (size_t)cdiv(S, kBlkK) * kBlkK;
  const size_t bhq = (size_t)B * Hq, bhk = (size_t)B * Hkv;
  const int nq = cdiv(S, bq), nkw = cdiv(cdiv(S, kBlkK), 32);
  BwdLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += al256(bytes);
    return at;
  };
  l.qd = take(bhq * S * D * 2);
  l.qt = take(bhq * D * Sp * 2);
  l.qdt = take(bhq * D * Sp * 2);
  l.dot = take(bhq * D * Sp * 2);
  l.kd = take(bhk * S * D * 2);
  l.kt = take(bhk * D * Sp * 2);
  l.kdt = take(bhk * D * Sp * 2);
  l.vd = take(bhk * Sp * D * 2);
  l.vt = take(bhk * D * Sp * 2);
  l.vdt = take(bhk * D * Sp * 2);
  l.prom = take(bhq * nq * nkw * 4);
  l.drow = take(bhq * S * 4);
  l.total = o;
  return l;
}

thrift_status check_bwd(const void* q16, const void* k16, const void* v16, const uint8_t* q4c,
                        const uint8_t* q4s, const float* q4t, const uint8_t* k4c, const uint8_t* k4s,
                        const float* k4t, const uint8_t* v4c, const uint8_t* v4s, const float* v4t,
                        thrift_format fmt, const int32_t* idx, const int32_t* cnt, int kmax,
                        int B, int Hq, int Hkv, int S, int D, int block_q, int block_k, int causal,
                        float sm_scale, const float* lse, const void* workspace, size_t workspace_bytes) {
  if (!q16 || !k16 || !v16 || !q4c || !q4s || !k4c || !k4s || !v4c || !v4s || !idx || !cnt || !lse ||
      !workspace)
    return THRIFT_EINVAL;
  if (fmt != THRIFT_NVFP4 && fmt != THRIFT_MXFP4) return THRIFT_EINVAL;
  if (fmt == THRIFT_NVFP4 && (!q4t || !k4t || !v4t)) return THRIFT_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || kmax < 1 || Hq % Hkv != 0 || (causal != 0 && causal != 1))
    return THRIFT_EINVAL;
  if (!(sm_scale > 0.0f) || !(sm_scale < 1e30f)) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if ((block_q != 64 && block_q != 128) || block_k != kBlkK || S > kMaxS) return THRIFT_EUNSUPPORTED;
  if ((size_t)S * D * 2 > 0x7fffffffu || (size_t)D * cdiv(S, kBlkK) * kBlkK * 2 > 0x7fffffffu)
    return THRIFT_EUNSUPPORTED;
  for (const void* p : {q16, k16, v16, (const void*)q4c, (const void*)k4c, (const void*)v4c, workspace})
    if (!aligned16(p)) return THRIFT_EALIGN;
  if (((uintptr_t)lse & 15) != 0) return THRIFT_EALIGN;
  if (workspace_bytes < bwd_layout(B, Hq, Hkv, S, D, block_q).total) return THRIFT_EWORKSPACE;
  return THRIFT_OK;
}

void launch_decode(const uint8_t* codes, const uint8_t* scales, size_t R, int L, int fmt, const float* tsc,
                   size_t rows_per_bh, _Float16* out, hipStream_t stream, int vD = 0, int vnb = 0) {
  const size_t n8 = R * (size_t)(L / 8);
  decode_fp4_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, stream>>>(codes, scales, R, L, fmt, tsc, rows_per_bh,
                                                                       out, vD, vnb);
}

void launch_transpose(const _Float16* in, int BH, int R, int C, int Rout, _Float16* out, hipStream_t stream,
                      const float* tsc = nullptr) {
  dim3 grid(cdiv(Rout > R ? Rout : R, 64) * cdiv(C, 64), BH);
  transpose_kernel<<<grid, 256, 0, stream>>>(in, R, C, Rout, tsc, out);
}

// Fills the FP4-decoded and transposed operands both entry points share.
// FP4-decoded operands keep NVFP4's slice scale out (exact fp16, the scale
// applied to the fp32 scores and dP); the transposed copies that are only
// ever the reduction-side operand (K^T for dQ, Q^T for dK, V^T for O')
// carry it, rounded once.
void prepare(BwdArgs& a, char* ws, const BwdLayout& l, const void* q16, const void* k16, const void* v16,
             const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c, const uint8_t* k4s,
             const float* k4t, const uint8_t* v4c, const uint8_t* v4s, const float* v4t, int fmt,
             const int32_t* idx, const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D, int block_q,
             int causal, float sm_scale, const float* lse, bool backward, hipStream_t stream) {
  const int Sp = cdiv(S, kBlkK) * kBlkK, nk = cdiv(S, kBlkK);
  a.q16 = (const _Float16*)q16;
  a.k16 = (const _Float16*)k16;
  a.v16 = (const _Float16*)v16;
  a.qd = (const _Float16*)(ws + l.qd);
  a.kd = (const _Float16*)(ws + l.kd);
  a.vd = (const _Float16*)(ws + l.vd);
  a.qt = (const _Float16*)(ws + l.qt);
  a.qdt = (const _Float16*)(ws + l.qdt);
  a.dot = (const _Float16*)(ws + l.dot);
  a.kt = (const _Float16*)(ws + l.kt);
  a.kdt = (const _Float16*)(ws + l.kdt);
  a.vt = (const _Float16*)(ws + l.vt);
  a.vdt = (const _Float16*)(ws + l.vdt);
  a.prom = (const uint32_t*)(ws + l.prom);
  a.lse = lse;
  a.drow = (const float*)(ws + l.drow);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.Sp = Sp;
  a.bq = block_q;
  a.nq = cdiv(S, block_q);
  a.nkw = cdiv(nk, 32);
  a.causal = causal;
  const bool nv = fmt == THRIFT_NVFP4;
  a.tq = nv ? q4t : nullptr;
  a.tk = nv ? k4t : nullptr;
  a.tv = nv ? v4t : nullptr;
  a.sm_scale = sm_scale;
  a.c = sm_scale * kLog2eB;
  const int BHq = B * Hq, BHk = B * Hkv;
  launch_decode(q4c, q4s, (size_t)BHq * S, D, fmt, nullptr, S, (_Float16*)a.qd, stream);
  launch_decode(k4c, k4s, (size_t)BHk * S, D, fmt, nullptr, S, (_Float16*)a.kd, stream);
  // V^T: with the slice scale for O' (reduction side), without for the rows of dP
  launch_decode(v4c, v4s, (size_t)BHk * nk * D, kBlkK, fmt, backward ? nullptr : a.tv, (size_t)nk * D,
                (_Float16*)a.vdt, stream, D, nk);
  const int nrows = BHq * a.nq;
  prom_bits_kernel<<<cdiv(nrows, 256), 256, 0, stream>>>(idx, cnt, nrows, kmax, nk, a.nkw, (uint32_t*)a.prom);
  if (backward) {
    launch_transpose(a.vdt, BHk, D, Sp, D, (_Float16*)a.vd, stream);  // [Sp][D]
    launch_transpose(a.q16, BHq, S, D, Sp, (_Float16*)a.qt, stream);
    launch_transpose(a.qd, BHq, S, D, Sp, (_Float16*)a.qdt, stream, a.tq);
    launch_transpose(a.k16, BHk, S, D, Sp, (_Float16*)a.kt, stream);
    launch_transpose(a.kd, BHk, S, D, Sp, (_Float16*)a.kdt, stream, a.tk);
  } else {
    launch_transpose(a.v16, BHk, S, D, Sp, (_Float16*)a.vt, stream);
  }
}

template <int D>
void launch_row(const BwdArgs& a, int mode, hipStream_t stream) {
  const int grid = a.B * a.Hq * a.nq;
  if (a.bq == 128) {
    if (mode == kModeOhp)
      bwd_row_kernel<D, kModeOhp, 4><<<grid, 256, 0, stream>>>(a);
    else
      bwd_row_kernel<D, kModeDq, 4><<<grid, 256, 0, stream>>>(a);
  } else {
    if (mode == kModeOhp)
      bwd_row_kernel<D, kModeOhp, 2><<<grid, 128, 0, stream>>>(a);
    else
      bwd_row_kernel<D, kModeDq, 2><<<grid, 128, 0, stream>>>(a);
  }
}

template __global__ void bwd_row_kernel<128, kModeOhp, 4>(BwdArgs);
template __global__ void bwd_row_kernel<128, kModeDq, 4>(BwdArgs);
template __global__ void bwd_row_kernel<64, kModeOhp, 4>(BwdArgs);
template __global__ void bwd_row_kernel<64, kModeDq, 4>(BwdArgs);
template __global__ void bwd_row_kernel<128, kModeOhp, 2>(BwdArgs);
template __global__ void bwd_row_kernel<128, kModeDq, 2>(BwdArgs);
template __global__ void bwd_row_kernel<64, kModeOhp, 2>(BwdArgs);
template __global__ void bwd_row_kernel<64, kModeDq, 2>(BwdArgs);
template __global__ void bwd_key_kernel<128, THRIFT_MXFP4>(BwdArgs);
template __global__ void bwd_key_kernel<64, THRIFT_MXFP4>(BwdArgs);
template __global__ void bwd_key_kernel<128, THRIFT_NVFP4>(BwdArgs);
template __global__ void bwd_key_kernel<64, THRIFT_NVFP4>(BwdArgs);
template __global__ void row_term_kernel<128>(const _Float16*, const float*, size_t, float*);
template __global__ void row_term_kernel<64>(const _Float16*, const float*, size_t, float*);

}  // namespace

}  // namespace thrift

using namespace thrift;

extern "C" size_t thrift_attention_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int block_q) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1 || block_q < 1) return 0;
  return bwd_layout(B, Hq, Hkv, S, D, block_q).total;
}

extern "C" thrift_status thrift_attention_fwd_hp(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes, const uint8_t* q4_scales,
    const float* q4_tscale, const uint8_t* k4_codes, const uint8_t* k4_scales, const float* k4_tscale,
    const uint8_t* v4_codes, const uint8_t* v4_scales, const float* v4_tscale, thrift_format fmt, const int32_t* idx, const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D,
    int block_q, int block_k, int causal, float sm_scale, const float* lse, float* ohp, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  thrift_status st = check_bwd(q16, k16, v16, q4_codes, q4_scales, q4_tscale, k4_codes, k4_scales, k4_tscale,
                               v4_codes, v4_scales, v4_tscale, fmt, idx, cnt, kmax, B, Hq, Hkv, S, D, block_q,
                               block_k, causal, sm_scale, lse, workspace, workspace_bytes);
  if (st != THRIFT_OK) return st;
  if (!ohp) return THRIFT_EINVAL;
  if (!aligned16(ohp)) return THRIFT_EALIGN;
  const BwdLayout l = bwd_layout(B, Hq, Hkv, S, D, block_q);
  BwdArgs a{};
  prepare(a, (char*)workspace, l, q16, k16, v16, q4_codes, q4_scales, q4_tscale, k4_codes, k4_scales, k4_tscale,
          v4_codes, v4_scales, v4_tscale, fmt, idx, cnt, kmax, B, Hq, Hkv, S, D, block_q, causal, sm_scale, lse,
          false, stream);
  a.out = ohp;
  if (D == 128)
    launch_row<128>(a, kModeOhp, stream);
  else
    launch_row<64>(a, kModeOhp, stream);
  return launch_status();
}

extern "C" thrift_status thrift_attention_bwd(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes, const uint8_t* q4_scales,
    const float* q4_tscale, const uint8_t* k4_codes, const uint8_t* k4_scales, const float* k4_tscale,
    const uint8_t* v4_codes, const uint8_t* v4_scales, const float* v4_tscale, thrift_format fmt, const int32_t* idx, const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D,
    int block_q, int block_k, int causal, float sm_scale, const float* lse, const float* ohp, const void* do16,
    float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  thrift_status st = check_bwd(q16, k16, v16, q4_codes, q4_scales, q4_tscale, k4_codes, k4_scales, k4_tscale,
                               v4_codes, v4_scales, v4_tscale, fmt, idx, cnt, kmax, B, Hq, Hkv, S, D, block_q,
                               block_k, causal, sm_scale, lse, workspace, workspace_bytes);
  if (st != THRIFT_OK) return st;
  if (!ohp || !do16 || !dq || !dk || !dv) return THRIFT_EINVAL;
  for (const void* p : {(const void*)ohp, do16, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(p)) return THRIFT_EALIGN;
  const BwdLayout l = bwd_layout(B, Hq, Hkv, S, D, block_q);
  BwdArgs a{};
  char* ws = (char*)workspace;
  prepare(a, ws, l, q16, k16, v16, q4_codes, q4_scales, q4_tscale, k4_codes, k4_scales, k4_tscale, v4_codes,
          v4_scales, v4_tscale, fmt, idx, cnt, kmax, B, Hq, Hkv, S, D, block_q, causal, sm_scale, lse, true, stream);
  const int Sp = a.Sp, BHq = B * Hq;
  a.do16 = (const _Float16*)do16;
  launch_transpose(a.do16, BHq, S, D, Sp, (_Float16*)a.dot, stream);
  const size_t nrows = (size_t)BHq * S;
  const unsigned rt_grid = (unsigned)((nrows * (size_t)(D / 8) + 255) / 256);
  if (D == 128)
    row_term_kernel<128><<<rt_grid, 256, 0, stream>>>(a.do16, ohp, nrows, (float*)a.drow);
  else
    row_term_kernel<64><<<rt_grid, 256, 0, stream>>>(a.do16, ohp, nrows, (float*)a.drow);
  a.out = dq;
  a.dk = dk;
  a.dv = dv;
  const int kgrid = B * Hkv * cdiv(cdiv(S, kBlkK), 2);
  const bool mx = fmt == THRIFT_MXFP4;
  if (D == 128) {
    launch_row<128>(a, kModeDq, stream);
    if (mx)
      bwd_key_kernel<128, THRIFT_MXFP4><<<kgrid, 256, 0, stream>>>(a);
    else
      bwd_key_kernel<128, THRIFT_NVFP4><<<kgrid, 256, 0, stream>>>(a);
  } else {
    launch_row<64>(a, kModeDq, stream);
    if (mx)
      bwd_key_kernel<64, THRIFT_MXFP4><<<kgrid, 256, 0, stream>>>(a);
    else
      bwd_key_kernel<64, THRIFT_NVFP4><<<kgrid, 256, 0, stream>>>(a);
  }
  return launch_status();
}
