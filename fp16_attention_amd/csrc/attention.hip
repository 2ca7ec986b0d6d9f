// Mixed FP4/FP16 attention forward of ThriftAttention on gfx950.
//
// Pages ("Gemengd-Precisie Berekening & Samenvoeging" / "Calcul a Precision
// Mixte et Fusion"): the unselected block pairs run through FP4 first, a
// separate FP16 routine then handles the promoted pairs, FP16 query tiles are
// loaded only when needed and units with no promoted pair skip the FP16 path;
// one FlashAttention-2 style online softmax merges both.  The pages' kernel
// is a single fused CUDA kernel for Blackwell NVFP4 tensor cores; this one is
// written for CDNA4:
//
//  * one workgroup = one (batch, query head, query block) of block_q rows;
//    one 64-wide wavefront per 32 query rows.  Each lane owns ONE query row:
//    scores are computed transposed, S^T = K Q^T, so the 32x32 MFMA output
//    puts a query in each lane column, and O^T = V^T P^T keeps it there.  The
//    softmax state (running max, running sum) is then one scalar per lane.
//  * The rows of the K operand are permuted so that the MFMA output hands
//    each lane 32 CONSECUTIVE keys of its query (lanes 0-31 keys 0-31 of the
//    tile, lanes 32-63 keys 32-63): that is one MX group of P, already in the
//    order the P^T operand of the second product wants, so the softmax and P
//    quantisation need no cross-lane traffic (the pair of lanes sharing a
//    query exchanges its maximum only when the running offset moves).
//  * MXFP4: both products use the block-scaled MFMA
//    v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and E8M0 scales per
//    32 elements of the contraction: Q/K groups run along D, V and P groups
//    along keys, exactly the micro-scaling layout of the quantised tensors,
//    so no dequantisation happens anywhere.
//  * NVFP4 (E4M3 scales per 16): no gfx950 matrix instruction takes E4M3
//    block scales, so tiles are dequantised exactly into fp16 in LDS (an
//    E2M1 x E4M3 product has at most 6 significant bits) and multiplied with
//    the FP16 MFMA v_mfma_f32_32x32x16_f16; the per-slice fp32 scales fold
//    into the softmax multiplier (Q, K) and into the accumulator (V).
//  * FP16 path: fp16 MFMA over the promoted tiles after all FP4 tiles.
//  * Online softmax with a lazy, integer running offset m (log2 units): the
//    accumulator is rescaled only when a tile's maximum exceeds m by more
//    than kTau, always by an exact power of two.  P codes do not depend on m
//    (MX: E8M0 scales absorb powers of two; NVFP4: level 1 normalises by the
//    tile maximum), so this is the pages' online softmax up to fp32 rounding.
//  * K/V tiles stream through double-buffered LDS, one barrier per tile; the
//    next tile's global loads are in flight while the current one computes.
#include "common.h"

namespace thrift {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kTau = 8.0f;        // lazy-rescale threshold, log2 units
constexpr float kMInit = -1.0e30f;  // running offset before the first key
constexpr int kBk = 64;             // key block

struct AttnArgs {
  const _Float16* q16;
  const _Float16* k16;
  const _Float16* v16;
  const uint8_t* q4c;
  const uint8_t* q4s;
  const float* q4t;
  const uint8_t* k4c;
  const uint8_t* k4s;
  const float* k4t;
  const uint8_t* v4c;
  const uint8_t* v4s;
  const float* v4t;
  const int32_t* idx;
  const int32_t* cnt;
  void* o;
  float* lse;
  int kmax, B, Hq, Hkv, S, Sp, nq, causal, o_fp32;
  float sm_log2;  // sm_scale * log2(e)
};

// ---- LDS layout --------------------------------------------------------------

template <int D>
struct Lds {
  // FP4 (MX) stage
  static constexpr int KROW4 = D / 2 + 16;  // bytes per key row of codes (padded)
  static constexpr int VROW4 = 32 + 16;     // bytes per V^T row of codes (64 keys)
  static constexpr int KC = 0;
  static constexpr int KS = KC + kBk * KROW4;  // u32 per key row: its D/32 scale bytes
  static constexpr int VC = KS + kBk * 4;
  static constexpr int VS = VC + D * VROW4;    // u32 [2][32]: byte dt = scale(dt*32+r, kb)
  static constexpr int STAGE4 = VS + 2 * 32 * 4;
  static constexpr int STAGE4R = (STAGE4 + 255) / 256 * 256;  // MX ring: three of these
  // fp16 stage (FP16 path, NVFP4 FP4 path)
  static constexpr int KROWH = D + 8;    // halves per key row
  static constexpr int VROWH = kBk + 8;  // halves per V^T row (16-byte aligned)
  static constexpr int KH = 0;
  static constexpr int VT = KH + kBk * KROWH * 2;
  static constexpr int STAGEH = VT + D * VROWH * 2;
  static constexpr int STAGE = ((STAGE4 > STAGEH ? STAGE4 : STAGEH) + 255) / 256 * 256;
  static constexpr int RING = (3 * STAGE4R > 2 * STAGE ? 3 * STAGE4R : 2 * STAGE);
  static constexpr int PROM = RING;  // int[kmax] promoted list
};

// ---- small helpers ---------------------------------------------------------------

__device__ inline v8i widen(v4i a) { return v8i{a.x, a.y, a.z, a.w, 0, 0, 0, 0}; }

template <int SA, int SB>
__device__ inline v16f mfma_fp4(v4i a, v4i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(a), widen(b), c, 4, 4, SA, sa, SB, sb);
}

__device__ inline v16f mfma_f16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ inline float xlane32(float v) { return __shfl_xor(v, 32, kWave); }
__device__ inline uint32_t xlane32u(uint32_t v) { return __shfl_xor(v, 32, kWave); }

// E4M3 byte -> value (finite codes only).
__device__ inline float e4m3_to_float(uint32_t b) {
  uint32_t e = (b >> 3) & 0xF, m = b & 7;
  return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120) << 23) | (m << 20));
}

// 4 E2M1 codes (2 bytes) -> 4 fp16 values, times an fp16 factor (exact when
// the factor has at most 4 significant bits and the products stay normal).
__device__ inline v4h fp4x4_to_h(uint32_t codes16, _Float16 f) {
  v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes16, 1.0f, 0);
  v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes16, 1.0f, 1);
  v2h ff = {f, f};
  a = a * ff;
  b = b * ff;
  return v4h{a.x, a.y, b.x, b.y};
}

// Key (within the 64-key tile) that A-operand row m of 32x32 S^T tile mt
// reads.  The MFMA output puts row (i/4)*8 + hi*4 + i%4 in register i of a
// lane of half hi, so register i of tile mt holds key hi*32 + mt*16 + i.
__device__ inline int krow(int mt, int m) { return ((m >> 2) & 1) * 32 + mt * 16 + (m >> 3) * 4 + (m & 3); }
// K tiles are stored in LDS in that read order (key krow(mt, m) at row
// mt*32 + m), so the 32 lanes of a half-wave read consecutive rows; kslot is
// the inverse map, key -> LDS row.
__device__ inline int kslot(int key) {
  const int h = key >> 5, mt = (key >> 4) & 1, i = key & 15;
  return mt * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
}
__device__ inline int key_of(int mt, int i, int hi) { return hi * 32 + mt * 16 + i; }

// Value of the other lane holding the same query (lane +- 32).
__device__ inline float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- online-softmax state ------------------------------------------------------

template <int D>
struct RowState {
  v16f acc[D / 32];  // O^T for this lane's query: d = dt*32 + (i/4)*8 + hi*4 + i%4
  float m;           // running integer offset (log2 units)
  float l;           // this lane's half of the running sum
  float g;           // acc holds O^T / g (NVFP4 FP4 path; 1 elsewhere)
};

// Lazy rescale: if the tile maximum (log2 units) of a query exceeds m +
// kTau, move m to its ceiling and rescale by the exact power of two.  own is
// this lane's half of the tile maximum (raw score units, c > 0); both lanes
// of the query decide on the pair's maximum, so they keep the same m.
template <int D>
__device__ inline void maybe_rescale(RowState<D>& st, float own, float c) {
  if (__builtin_amdgcn_ballot_w64(own * c > st.m + kTau)) {
    const float tml2 = pair_max(own) * c;
    const bool need = tml2 > st.m + kTau;
    const float mn = need ? ceilf(tml2) : st.m;
    const float f = need ? exp2f(st.m - mn) : 1.0f;  // integer difference: exact
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] *= f;
    st.l *= f;
    st.m = mn;
  }
}

// Causal / tail mask: keys past the query row or past S become -inf.
__device__ inline void mask_tile(v16f s[2], int key0, int qrow, int S, int causal, int hi) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int key = key0 + key_of(mt, i, hi);
      if (key >= S || (causal && key > qrow)) s[mt][i] = -INFINITY;
    }
}

__device__ inline float max16(const v16f& v) {
  float a = fmaxf(fmaxf(v[0], v[1]), v[2]);
  float b = fmaxf(fmaxf(v[3], v[4]), v[5]);
  float c = fmaxf(fmaxf(v[6], v[7]), v[8]);
  float d = fmaxf(fmaxf(v[9], v[10]), v[11]);
  float e = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), v[15]));
}

// ---- MX FP4 tile ------------------------------------------------------------------

// S^T = K Q^T for one MX tile: two 32-row tiles, D/64 contraction steps of
// 64 channels, block-scaled by the E8M0 bytes of K and Q.
template <int D>
__device__ inline void qk_mx(v16f s[2], const char* stage, const v4i* qB, uint32_t qsc, int lane) {
  using L = Lds<D>;
  const int hi = lane >> 5, r32 = lane & 31;
  const uint8_t* kc = (const uint8_t*)(stage + L::KC);
  const uint32_t* ks = (const uint32_t*)(stage + L::KS);
  uint32_t ksc[2];
  v4i a[2][D / 64];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = mt * 32 + r32;       // holds key krow(mt, r32)
    ksc[mt] = ks[row] >> (8 * hi);       // byte 2*kstep: this lane's 32-channel group
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) a[mt][kk] = *(const v4i*)(kc + row * L::KROW4 + kk * 32 + hi * 16);
  }
  s[0] = mfma_fp4<0, 0>(a[0][0], qB[0], v16f{}, ksc[0], qsc);
  s[1] = mfma_fp4<0, 0>(a[1][0], qB[0], v16f{}, ksc[1], qsc);
  if constexpr (D == 128) {
    s[0] = mfma_fp4<2, 2>(a[0][1], qB[1], s[0], ksc[0], qsc);
    s[1] = mfma_fp4<2, 2>(a[1][1], qB[1], s[1], ksc[1], qsc);
  }
}

// Softmax, two-level MX quantisation of P and O^T += V^T P^T for one tile.
template <int D>
__device__ inline void softmax_pv_mx(RowState<D>& st, v16f s[2], const char* stage, float c,
                                     int key0, int qrow, int S, int causal, bool need_mask,
                                     int lane) {
  using L = Lds<D>;
  const int hi = lane >> 5, r32 = lane & 31;
  const uint8_t* vc = (const uint8_t*)(stage + L::VC);
  const uint32_t* vs = (const uint32_t*)(stage + L::VS);
  if (need_mask) mask_tile(s, key0, qrow, S, causal, hi);

  // this lane's 32 keys are one P group: its maximum sets the E8M0 exponent
  const float gmax = fmaxf(max16(s[0]), max16(s[1]));
  maybe_rescale<D>(st, gmax, c);
  const float nm = -st.m;

  // probabilities relative to 2^m, unquantised row sum
  float lsum = 0.0f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2_fast(__builtin_fmaf(s[mt][i], c, nm));
      s[mt][i] = p;
      lsum += p;
    }
  st.l += lsum;

  // E8M0 exponent floor(log2(max p)) - 2 from the exponent field of the
  // group maximum's probability (computed like the elements' own)
  const uint32_t E = (__float_as_uint(exp2_fast(__builtin_fmaf(gmax, c, nm))) >> 23) & 0xFF;
  const uint32_t psc = E > 3 ? E - 2 : 1;
  const float sf = __uint_as_float(psc << 23);

  // P^T operand: nibble n of this lane = key hi*32 + n = register n%16 of tile n/16
  v4i P;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const v16f& v = s[r >> 1];
    const int o = (r & 1) * 8;
    uint32_t x = 0;
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[o + 0], v[o + 1], sf, 0);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[o + 2], v[o + 3], sf, 1);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[o + 4], v[o + 5], sf, 2);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, v[o + 6], v[o + 7], sf, 3);
    P[r] = (int)x;
  }

  // O^T += V^T P^T
  const uint32_t vsw = vs[hi * 32 + r32];
  const uint8_t* vrow = vc + r32 * L::VROW4 + hi * 16;
  st.acc[0] = mfma_fp4<0, 0>(*(const v4i*)(vrow), P, st.acc[0], vsw, psc);
  st.acc[1] = mfma_fp4<1, 0>(*(const v4i*)(vrow + 32 * L::VROW4), P, st.acc[1], vsw, psc);
  if constexpr (D == 128) {
    st.acc[2] = mfma_fp4<2, 0>(*(const v4i*)(vrow + 64 * L::VROW4), P, st.acc[2], vsw, psc);
    st.acc[3] = mfma_fp4<3, 0>(*(const v4i*)(vrow + 96 * L::VROW4), P, st.acc[3], vsw, psc);
  }
}

// ---- fp16-MFMA tile (FP16 path, and the FP4 path of the NVFP4 format) ----------

// S^T = K Q^T from the fp16 stage.
template <int D>
__device__ inline void qk_f16(v16f s[2], const char* stage, const v8h* qh, int lane) {
  using L = Lds<D>;
  const int hi = lane >> 5, r32 = lane & 31;
  const _Float16* kh = (const _Float16*)(stage + L::KH);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const _Float16* row = kh + (mt * 32 + r32) * L::KROWH + hi * 8;  // key krow(mt, r32)
    s[mt] = v16f{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) s[mt] = mfma_f16(*(const v8h*)(row + kk * 16), qh[kk], s[mt]);
  }
}

// O^T += V^T P^T over four 16-key steps; in step st this lane supplies
// keys hi*32 + 8*st + u (u = 0..7), its registers 8*(st%2)+u of tile st/2.
template <int D>
__device__ inline void pv_f16(RowState<D>& st, const char* stage, const v8h* pB, int lane) {
  using L = Lds<D>;
  const int hi = lane >> 5, r32 = lane & 31;
  const _Float16* vt = (const _Float16*)(stage + L::VT);
#pragma unroll
  for (int stp = 0; stp < 4; ++stp)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const v8h a = *(const v8h*)(vt + (dt * 32 + r32) * L::VROWH + hi * 32 + stp * 8);
      st.acc[dt] = mfma_f16(a, pB[stp], st.acc[dt]);
    }
}

// Promoted tile: fp16 scores, probabilities rounded to fp16.
template <int D>
__device__ inline void fp16_tile(RowState<D>& st, const char* stage, const v8h* qh, float c, int key0,
                                 int qrow, int S, int causal, bool need_mask, int lane) {
  const int hi = lane >> 5;
  v16f s[2];
  qk_f16<D>(s, stage, qh, lane);
  if (need_mask) mask_tile(s, key0, qrow, S, causal, hi);
  maybe_rescale<D>(st, fmaxf(max16(s[0]), max16(s[1])), c);
  const float nm = -st.m;
  float lsum = 0.0f;
  v8h pB[4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2_fast(__builtin_fmaf(s[mt][i], c, nm));
      lsum += p;
      pB[mt * 2 + i / 8][i % 8] = (_Float16)p;
    }
  st.l += lsum;
  pv_f16<D>(st, stage, pB, lane);
}

// NVFP4 FP4 tile: scores from the dequantised fp16 stage, P quantised in two
// levels (level 1 per row and tile: v = 2688 p / p_max; level 2 per 16 keys:
// E4M3 scale s2, E2M1 codes of v / s2).  The product with V uses code * s2,
// which fp16 holds exactly, so the per-row level-1 factor p_max / 2688 (and
// V's per-slice scale) is carried in the accumulator scale g instead of being
// rounded into P: acc becomes acc * g / f before the tile and g becomes f.
template <int D>
__device__ inline void fp4_nv_tile(RowState<D>& st, const char* stage, const v8h* qh, float c,
                                   float sv, int key0, int qrow, int S, int causal, bool need_mask,
                                   int lane) {
  const int hi = lane >> 5;
  v16f s[2];
  qk_f16<D>(s, stage, qh, lane);
  if (need_mask) mask_tile(s, key0, qrow, S, causal, hi);
  const float gm0 = max16(s[0]), gm1 = max16(s[1]);  // this lane's two 16-key groups
  maybe_rescale<D>(st, fmaxf(gm0, gm1), c);
  const float tm = pair_max(fmaxf(gm0, gm1));  // the query's tile maximum (level 1)
  const float nm = -st.m;
  float lsum = 0.0f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2_fast(__builtin_fmaf(s[mt][i], c, nm));
      s[mt][i] = p;
      lsum += p;
    }
  st.l += lsum;
  const float em = exp2_fast(__builtin_fmaf(tm, c, nm));  // probability of the tile maximum
  // a tile more than 2^60 below the running maximum contributes nothing
  const bool live = em > 0x1p-60f;
  const float r = live ? 2688.0f / em : 0.0f;  // level 1: maximum -> 6 * 448
  const float f = live ? em * (sv * (1.0f / 2688.0f)) : st.g;
  const float ratio = st.g / f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] *= ratio;
  st.g = f;
  v8h pB[4];
#pragma unroll
  for (int g = 0; g < 2; ++g) {  // group g = keys hi*32 + 16g .. +15 = registers of tile g
    const v16f& v = s[g];
    const float gm = exp2_fast(__builtin_fmaf(g ? gm1 : gm0, c, nm)) * r;
    // level 2: E4M3 block scale (the conversion does not saturate: clamp)
    v2s_t sb = {0, 0};
    sb = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(sb, fminf(gm * (1.0f / 6.0f), 448.0f), 0.0f, 1.0f, false);
    const float s2 = e4m3_to_float((uint32_t)sb[0] & 0xFF);
    const float k = s2 > 0.0f ? r / s2 : 0.0f;
    const _Float16 s2h = (_Float16)(live ? s2 : 0.0f);  // exact: E4M3 has 4 significant bits
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // 8 keys per P^T operand
      const int o = h * 8;
      uint32_t cw = 0;
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[o + 0] * k, v[o + 1] * k, 1.0f, 0);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[o + 2] * k, v[o + 3] * k, 1.0f, 1);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[o + 4] * k, v[o + 5] * k, 1.0f, 2);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[o + 6] * k, v[o + 7] * k, 1.0f, 3);
      v4h lo = fp4x4_to_h(cw & 0xFFFFu, s2h);
      v4h hi4 = fp4x4_to_h(cw >> 16, s2h);
      pB[g * 2 + h] = v8h{lo.x, lo.y, lo.z, lo.w, hi4.x, hi4.y, hi4.z, hi4.w};
    }
  }
  pv_f16<D>(st, stage, pB, lane);
}

}  // namespace thrift

namespace thrift {

// ---- staging: global -> registers (next tile) -> LDS --------------------------

// MX FP4 tile: K codes [64 keys][D/2 B], K scales (one u32 per key row),
// V^T codes [D][32 B], V^T scales regrouped so that a lane reads the scale
// bytes of its four d-tiles with one 32-bit load.  Loads are unconditional:
// key rows past S (last tile only) read row S-1 instead, and their scores
// are masked anyway.
template <int D, int NT>
struct Mx4Stager {
  static constexpr int NKC = kBk * D / 32;  // 16-byte chunks of K codes
  static constexpr int NVC = D * 2;         // 16-byte chunks of V^T codes
  static constexpr int PK = (NKC + NT - 1) / NT, PV = (NVC + NT - 1) / NT;
  v4i kc[PK], vc[PV];
  uint32_t ksc, vsc;

  struct Base {  // per-workgroup bases of the key head's FP4 tensors
    const uint8_t *kc, *ks, *vc, *vs;
    int S, Sp;
  };

  __device__ static Base base(const AttnArgs& a, size_t bhk) {
    return Base{a.k4c + bhk * a.S * (D / 2), a.k4s + bhk * a.S * (D / 32),
                a.v4c + bhk * D * (a.Sp / 2), a.v4s + bhk * D * (a.Sp / 32), a.S, a.Sp};
  }

  // Every thread issues the same number of loads on every tile (threads past
  // a table re-read an in-range entry and drop it), so the compiler can wait
  // for exactly the older tile's loads and leave the newer ones in flight.
  __device__ void load(const Base& g, int j, int t) {
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      const int c = (t + p * NT) % NKC;
      const int row = c / (D / 32), col = c % (D / 32);
      const uint32_t key = (uint32_t)min(j * kBk + row, g.S - 1);
      kc[p] = *(const v4i*)(g.kc + (key * (D / 2) + col * 16));
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      const int c = (t + p * NT) % NVC;
      vc[p] = *(const v4i*)(g.vc + ((uint32_t)(c / 2) * (uint32_t)(g.Sp / 2) + j * 32 + (c % 2) * 16));
    }
    {
      const uint32_t key = (uint32_t)min(j * kBk + t % kBk, g.S - 1);
      const uint8_t* p = g.ks + key * (D / 32);
      ksc = D == 128 ? *(const uint32_t*)p : (uint32_t)(*(const uint16_t*)p);
    }
    vsc = *(const uint16_t*)(g.vs + ((uint32_t)(t % D) * (uint32_t)(g.Sp / 32) + j * 2));
  }

  __device__ void store(char* stage, int t) const {
    using L = Lds<D>;
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      const int c = t + p * NT;
      if (NKC % NT == 0 || c < NKC) {
        const int row = c / (D / 32), col = c % (D / 32);
        *(v4i*)(stage + L::KC + kslot(row) * L::KROW4 + col * 16) = kc[p];
      }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      const int c = t + p * NT;
      if (NVC % NT == 0 || c < NVC) *(v4i*)(stage + L::VC + (c / 2) * L::VROW4 + (c % 2) * 16) = vc[p];
    }
    if (t < kBk) ((uint32_t*)(stage + L::KS))[kslot(t)] = ksc;
    if (t < D) {
      uint8_t* vs = (uint8_t*)(stage + L::VS);
      vs[((0 * 32) + (t & 31)) * 4 + (t >> 5)] = (uint8_t)(vsc & 0xFF);
      vs[((1 * 32) + (t & 31)) * 4 + (t >> 5)] = (uint8_t)(vsc >> 8);
    }
  }
};

// fp16 tile of the promoted path: K row-major (rows in MFMA read order), V
// transposed into V^T.  The transpose goes through registers: a thread takes
// two consecutive keys x 8 channels and writes eight 4-byte (key pair) words,
// so a wavefront's stores hit consecutive words of one V^T row.
template <int D, int NT>
struct F16Stager {
  static constexpr int NK = kBk * D / 8;        // 16-byte chunks of K
  static constexpr int NV = (kBk / 2) * (D / 8);  // (key pair, 8 channels) items of V
  static constexpr int PK = (NK + NT - 1) / NT, PV = (NV + NT - 1) / NT;
  v8h kr[PK], v0[PV], v1[PV];

  __device__ void load(const AttnArgs& a, size_t bhk, int j, int t) {
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      int c = t + p * NT;
      kr[p] = v8h{};
      if (c < NK) {
        int row = c / (D / 8), col = (c % (D / 8)) * 8, key = j * kBk + row;
        if (key < a.S) kr[p] = *(const v8h*)(a.k16 + (bhk * a.S + key) * D + col);
      }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      int c = t + p * NT;
      v0[p] = v8h{};
      v1[p] = v8h{};
      if (c < NV) {
        int kp = c % (kBk / 2), col = (c / (kBk / 2)) * 8, key = j * kBk + 2 * kp;
        const _Float16* src = a.v16 + (bhk * a.S + key) * D + col;
        if (key < a.S) v0[p] = *(const v8h*)src;
        if (key + 1 < a.S) v1[p] = *(const v8h*)(src + D);
      }
    }
  }

  __device__ void store(char* stage, int t) const {
    using L = Lds<D>;
    _Float16* kh = (_Float16*)(stage + L::KH);
    _Float16* vt = (_Float16*)(stage + L::VT);
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      int c = t + p * NT;
      if (c < NK) {
        int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *(v8h*)(kh + kslot(row) * L::KROWH + col) = kr[p];
      }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      int c = t + p * NT;
      if (c < NV) {
        int kp = c % (kBk / 2), col = (c / (kBk / 2)) * 8;
        const v4i a = __builtin_bit_cast(v4i, v0[p]), b = __builtin_bit_cast(v4i, v1[p]);
        uint32_t* dst = (uint32_t*)(vt + col * L::VROWH + 2 * kp);
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // channels 2w, 2w+1: (key, key+1) half pairs
          dst[(2 * w) * (L::VROWH / 2)] = __builtin_amdgcn_perm((uint32_t)b[w], (uint32_t)a[w], 0x05040100u);
          dst[(2 * w + 1) * (L::VROWH / 2)] = __builtin_amdgcn_perm((uint32_t)b[w], (uint32_t)a[w], 0x07060302u);
        }
      }
    }
  }
};

// NVFP4 tile: codes and E4M3 block scales, dequantised exactly to fp16 in LDS
// (K row-major, V already transposed).  Per-slice scales are applied elsewhere.
template <int D, int NT>
struct Nv4Stager {
  static constexpr int NKC = kBk * D / 32;  // 16-byte chunks = 32 elements = 2 groups
  static constexpr int NVC = D * 2;
  static constexpr int PK = (NKC + NT - 1) / NT, PV = (NVC + NT - 1) / NT;
  v4i kc[PK], vc[PV];
  uint32_t ks[PK], vs[PV];

  __device__ void load(const AttnArgs& a, size_t bhk, int j, int t) {
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      int c = t + p * NT;
      kc[p] = v4i{};
      ks[p] = 0;
      if (c < NKC) {
        int row = c / (D / 32), col = c % (D / 32), key = j * kBk + row;
        if (key < a.S) {
          kc[p] = *(const v4i*)(a.k4c + ((bhk * a.S + key) * (D / 2)) + col * 16);
          ks[p] = *(const uint16_t*)(a.k4s + (bhk * a.S + key) * (D / 16) + col * 2);
        }
      }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      int c = t + p * NT;
      vc[p] = v4i{};
      vs[p] = 0;
      if (c < NVC) {
        int d = c / 2, h = c % 2;
        vc[p] = *(const v4i*)(a.v4c + (bhk * D + d) * (a.Sp / 2) + j * 32 + h * 16);
        vs[p] = *(const uint16_t*)(a.v4s + (bhk * D + d) * (a.Sp / 16) + j * 4 + h * 2);
      }
    }
  }

  __device__ static void expand(_Float16* dst, v4i codes, uint32_t sc2) {
    const _Float16 f0 = (_Float16)e4m3_to_float(sc2 & 0xFF);
    const _Float16 f1 = (_Float16)e4m3_to_float((sc2 >> 8) & 0xFF);
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // 8 elements per dword; dwords 0-1 group 0, 2-3 group 1
      const _Float16 f = q < 2 ? f0 : f1;
      v4h lo = fp4x4_to_h((uint32_t)codes[q] & 0xFFFFu, f);
      v4h hi = fp4x4_to_h((uint32_t)codes[q] >> 16, f);
      *(v8h*)(dst + q * 8) = v8h{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  }

  __device__ void store(char* stage, int t) const {
    using L = Lds<D>;
    _Float16* kh = (_Float16*)(stage + L::KH);
    _Float16* vt = (_Float16*)(stage + L::VT);
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      int c = t + p * NT;
      if (c < NKC) expand(kh + kslot(c / (D / 32)) * L::KROWH + (c % (D / 32)) * 32, kc[p], ks[p]);
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      int c = t + p * NT;
      if (c < NVC) expand(vt + (c / 2) * L::VROWH + (c % 2) * 32, vc[p], vs[p]);
    }
  }
};

// ---- the kernel ----------------------------------------------------------------------

// Work item of workgroup `id`.  Workgroups are dispatched round-robin over
// the 8 XCDs (id % 8), each with its own L2; items are mapped so that one XCD
// streams the K/V of one key head (all its query blocks and the query heads
// that share it), heaviest causal blocks first, which keeps that head's FP4
// K/V resident in the XCD's L2:
//  - B*Hkv a multiple of 8: XCD x takes key heads x, x+8, ...;
//  - B*Hkv dividing 8: key head x % (B*Hkv), every (8/(B*Hkv))-th block of it;
//  - otherwise: plain heaviest-first order.
// The grid is a multiple of 8; workgroups past the last item return.
constexpr int kXcds = 8;
__device__ inline bool work_item(const AttnArgs& a, int id, int& i, int& bhq) {
  const int G = a.Hq / a.Hkv, nbh = a.B * a.Hkv, per_head = G * a.nq;
  const int N = a.B * a.Hq * a.nq;
  int h, p;  // key head (b*Hkv + hk) and position in its heaviest-first list
  if (nbh % kXcds == 0) {
    const int x = id % kXcds, k = id / kXcds, heads = nbh / kXcds;
    if (k >= heads * per_head) return false;
    h = x + kXcds * (k / per_head);
    p = k % per_head;
  } else if (kXcds % nbh == 0) {
    const int x = id % kXcds, k = id / kXcds, st = kXcds / nbh;
    h = x % nbh;
    p = k * st + x / nbh;
    if (p >= per_head) return false;
  } else {
    if (id >= N) return false;
    const int BHq = a.B * a.Hq;
    i = a.causal ? a.nq - 1 - id / BHq : id / BHq;
    bhq = id % BHq;
    return true;
  }
  const int ii = p / G, g = p % G;  // query block rank (heaviest first), head in group
  i = a.causal ? a.nq - 1 - ii : ii;
  bhq = (h / a.Hkv) * a.Hq + (h % a.Hkv) * G + g;
  return true;
}

template <int D, int NW, int FMT>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(AttnArgs a) {
  using L = Lds<D>;
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, hi = lane >> 5;
  const int S = a.S;
  int i, bhq;
  if (!work_item(a, blockIdx.x, i, bhq)) return;
  const int b = bhq / a.Hq, hq = bhq % a.Hq;
  const size_t bhk = (size_t)b * a.Hkv + hq / (a.Hq / a.Hkv);
  const int q0 = __builtin_amdgcn_readfirstlane(i * BQ + w * 32);  // wave-uniform
  const int qrow = q0 + (lane & 31);
  const bool qvalid = qrow < S;
  const int nvalid = valid_kv_blocks(i, S, BQ, kBk, a.causal);
  const size_t rowid = (size_t)bhq * a.nq + i;
  int ncnt = a.cnt[rowid];
  ncnt = ncnt < 0 ? 0 : (ncnt > a.kmax ? a.kmax : ncnt);
  int* prom = (int*)(smem + L::PROM);
  uint32_t* pbits = (uint32_t*)prom + a.kmax;  // bit j: key block j is promoted
  const int nwords = (nvalid + 31) >> 5;
  for (int e = t; e < nwords; e += NT) pbits[e] = 0;
  __syncthreads();
  for (int e = t; e < ncnt; e += NT) {
    const int j = a.idx[rowid * a.kmax + e];
    prom[e] = j;
    if (j >= 0 && j < nvalid) atomicOr(&pbits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();

  RowState<D> st;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] = v16f{};
  st.m = kMInit;
  st.l = 0.0f;
  st.g = 1.0f;

  // ---------------- FP4 path: every valid key block not promoted ----------------
  int pj = 0;
  auto next_fp4 = [&](int j) {
    while (pj < ncnt && prom[pj] < j) ++pj;
    while (j < nvalid && pj < ncnt && prom[pj] == j) {
      ++j;
      ++pj;
    }
    return j;
  };
  {
    const size_t qoff = (size_t)bhq * S + (qvalid ? qrow : 0);
    int jc = next_fp4(0);
    if constexpr (FMT == THRIFT_MXFP4) {
      v4i qB[D / 64];
      uint32_t qsc = 0x7F7F7F7Fu;
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk)
        qB[kk] = qvalid ? *(const v4i*)(a.q4c + qoff * (D / 2) + kk * 32 + hi * 16) : v4i{};
      if (qvalid) {
        const uint8_t* p = a.q4s + qoff * (D / 32);
        qsc = D == 128 ? *(const uint32_t*)p : (uint32_t)(*(const uint16_t*)p);
      }
      qsc >>= 8 * hi;
      const float c = a.sm_log2;
      // Three-stage LDS ring over every valid key block in order, one barrier
      // per block; promoted blocks are staged but not computed (their FP16
      // pass comes later), which keeps the load stream regular.  Iteration n
      // issues the loads of block n+2 into registers, the QK MFMAs of block
      // n+1 (K from ring slot n+1) before the softmax of block n, so the
      // matrix core works while this wave's VALU does, the PV product of
      // block n (V from slot n), and finally stores block n+2 into slot n+2,
      // whose previous block (n-1) every wave finished before the last
      // barrier.
      using Stg = Mx4Stager<D, NT>;
      const typename Stg::Base g = Stg::base(a, bhk);
      Stg stg;
      constexpr int R = L::STAGE4R;
      const uint32_t* pbits = (const uint32_t*)(smem + L::PROM) + a.kmax;
      auto active_of = [&](int j) {
        return j < nvalid && !((pbits[j >> 5] >> (j & 31)) & 1u) && (!a.causal || j * kBk <= q0 + 31);
      };
      auto mask_of = [&](int j) {
        const int key0 = j * kBk;
        return (a.causal && key0 + kBk - 1 > q0) || key0 + kBk > S;
      };
      if (ncnt < nvalid) {
        int jc = 0;
        stg.load(g, 0, t);
        stg.store(smem, t);
        if (1 < nvalid) {
          stg.load(g, 1, t);
          stg.store(smem + R, t);
        }
        __syncthreads();
        v16f sA[2], sB[2];
        bool actc = active_of(0);
        if (actc) qk_mx<D>(sA, smem, qB, qsc, lane);
        int b = 0;
        // cur/nxt: score registers of blocks n, n+1
        auto step = [&](v16f (&cur)[2], v16f (&nxt)[2]) -> bool {
          const bool more2 = jc + 2 < nvalid;
          if (more2) stg.load(g, jc + 2, t);
          const int b1 = b == 2 ? 0 : b + 1, b2 = b1 == 2 ? 0 : b1 + 1;
          const bool actn = active_of(jc + 1);
          if (actn) qk_mx<D>(nxt, smem + b1 * R, qB, qsc, lane);
          if (actc)
            softmax_pv_mx<D>(st, cur, smem + b * R, c, jc * kBk, qrow, S, a.causal, mask_of(jc), lane);
          if (more2) stg.store(smem + b2 * R, t);
          __syncthreads();
          ++jc;
          actc = actn;
          b = b1;
          return jc < nvalid;
        };
        while (step(sA, sB) && step(sB, sA)) {
        }
      }
    } else {
      v8h qh[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        qh[kk] = v8h{};
        if (qvalid) {
          uint32_t cw = *(const uint32_t*)(a.q4c + qoff * (D / 2) + kk * 8 + hi * 4);
          _Float16 f = (_Float16)e4m3_to_float(a.q4s[qoff * (D / 16) + kk]);
          v4h lo = fp4x4_to_h(cw & 0xFFFFu, f), h4 = fp4x4_to_h(cw >> 16, f);
          qh[kk] = v8h{lo.x, lo.y, lo.z, lo.w, h4.x, h4.y, h4.z, h4.w};
        }
      }
      const float c = a.sm_log2 * a.q4t[bhq] * a.k4t[bhk];
      const float sv = a.v4t[bhk];
      Nv4Stager<D, NT> stg;
      if (jc < nvalid) {
        stg.load(a, bhk, jc, t);
        stg.store(smem, t);
      }
      __syncthreads();
      int buf = 0;
      while (jc < nvalid) {
        const int jn = next_fp4(jc + 1);
        if (jn < nvalid) stg.load(a, bhk, jn, t);
        const int key0 = jc * kBk;
        const bool active = !a.causal || key0 <= q0 + 31;
        const bool need_mask = (a.causal && key0 + kBk - 1 > q0) || key0 + kBk > S;
        if (active)
          fp4_nv_tile<D>(st, smem + buf * L::STAGE, qh, c, sv, key0, qrow, S, a.causal, need_mask, lane);
        if (jn < nvalid) stg.store(smem + (buf ^ 1) * L::STAGE, t);
        __syncthreads();
        buf ^= 1;
        jc = jn;
      }
      // back to plain units: acc holds O^T / g
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] *= st.g;
      st.g = 1.0f;
    }
  }

  // ---------------- FP16 path: promoted blocks only ----------------
  if (ncnt > 0) {
    v8h qh[D / 16];
    const size_t qoff = ((size_t)bhq * S + qrow) * D + hi * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qh[kk] = qvalid ? *(const v8h*)(a.q16 + qoff + kk * 16) : v8h{};
    F16Stager<D, NT> stg;
    auto valid_j = [&](int p) { int j = prom[p]; return j >= 0 && j < nvalid ? j : -1; };
    int jc = valid_j(0);
    if (jc >= 0) stg.load(a, bhk, jc, t);
    stg.store(smem, t);
    __syncthreads();
    int buf = 0;
    for (int p = 0; p < ncnt; ++p) {
      const bool more = p + 1 < ncnt;
      const int jn = more ? valid_j(p + 1) : -1;
      if (more) {
        if (jn >= 0) stg.load(a, bhk, jn, t);
      }
      if (jc >= 0) {
        const int key0 = jc * kBk;
        const bool active = !a.causal || key0 <= q0 + 31;
        const bool need_mask = (a.causal && key0 + kBk - 1 > q0) || key0 + kBk > S;
        if (active)
          fp16_tile<D>(st, smem + buf * L::STAGE, qh, a.sm_log2, key0, qrow, S, a.causal, need_mask, lane);
      }
      if (more && jn >= 0) stg.store(smem + (buf ^ 1) * L::STAGE, t);
      __syncthreads();
      buf ^= 1;
      jc = jn;
    }
  }

  // ---------------- epilogue: O = acc / l, LSE ----------------
  const float lt = st.l + xlane32(st.l);
  if (qvalid) {
    const float inv = 1.0f / lt;
    const size_t obase = ((size_t)bhq * S + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = dt * 32 + i4 * 8 + hi * 4;
        float x0 = st.acc[dt][i4 * 4 + 0] * inv, x1 = st.acc[dt][i4 * 4 + 1] * inv;
        float x2 = st.acc[dt][i4 * 4 + 2] * inv, x3 = st.acc[dt][i4 * 4 + 3] * inv;
        if (a.o_fp32) {
          *(float4*)((float*)a.o + obase + d0) = make_float4(x0, x1, x2, x3);
        } else {
          *(v4h*)((_Float16*)a.o + obase + d0) = v4h{(_Float16)x0, (_Float16)x1, (_Float16)x2, (_Float16)x3};
        }
      }
    if (a.lse && hi == 0) a.lse[(size_t)bhq * S + qrow] = (st.m + log2f(lt)) * kLn2;
  }
}

template <int D, int NW, int FMT>
static thrift_status launch_attn(const AttnArgs& a, hipStream_t stream) {
  using L = Lds<D>;
  const size_t lds = (size_t)L::PROM + (size_t)a.kmax * 4 + (size_t)((a.S + 64 * 32 - 1) / (64 * 32)) * 4;
  static bool configured = false;
  if (!configured) {
    if (hipFuncSetAttribute((const void*)attn_fwd_kernel<D, NW, FMT>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
      return THRIFT_EHIP;
    configured = true;
  }
  const int items = a.B * a.Hq * a.nq;
  const int grid = (items + kXcds - 1) / kXcds * kXcds;
  attn_fwd_kernel<D, NW, FMT><<<grid, NW * 64, lds, stream>>>(a);
  return launch_status();
}

}  // namespace thrift

using namespace thrift;

extern "C" thrift_status thrift_attention_fwd(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes,
    const uint8_t* q4_scales, const float* q4_tscale, const uint8_t* k4_codes,
    const uint8_t* k4_scales, const float* k4_tscale, const uint8_t* v4_codes,
    const uint8_t* v4_scales, const float* v4_tscale, thrift_format fmt, const int32_t* idx,
    const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D, int block_q, int block_k,
    int causal, float sm_scale, void* o, int o_is_fp32, float* lse, hipStream_t stream) {
  if (!q4_codes || !q4_scales || !k4_codes || !k4_scales || !v4_codes || !v4_scales || !idx ||
      !cnt || !o)
    return THRIFT_EINVAL;
  if (fmt != THRIFT_NVFP4 && fmt != THRIFT_MXFP4) return THRIFT_EINVAL;
  if (fmt == THRIFT_NVFP4 && (!q4_tscale || !k4_tscale || !v4_tscale)) return THRIFT_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || kmax < 1 || (causal != 0 && causal != 1)) return THRIFT_EINVAL;
  if (Hq % Hkv != 0 || (o_is_fp32 != 0 && o_is_fp32 != 1)) return THRIFT_EINVAL;
  if (!(sm_scale > 0.0f) || !(sm_scale < 1e30f)) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if ((block_q != 64 && block_q != 128) || block_k != 64) return THRIFT_EUNSUPPORTED;
  if (S > 262144 || kmax > cdiv(S, block_k)) return THRIFT_EUNSUPPORTED;
  const bool any16 = q16 || k16 || v16;
  if (any16 && !(q16 && k16 && v16)) return THRIFT_EINVAL;
  for (const void* p : {(const void*)q4_codes, (const void*)k4_codes, (const void*)v4_codes, (const void*)o})
    if (!aligned16(p)) return THRIFT_EALIGN;
  if (any16 && (!aligned16(q16) || !aligned16(k16) || !aligned16(v16))) return THRIFT_EALIGN;
  if (((uintptr_t)q4_scales | (uintptr_t)k4_scales | (uintptr_t)v4_scales) & 3) return THRIFT_EALIGN;
  AttnArgs a;
  a.q16 = (const _Float16*)q16;
  a.k16 = (const _Float16*)k16;
  a.v16 = (const _Float16*)v16;
  a.q4c = q4_codes;
  a.q4s = q4_scales;
  a.q4t = q4_tscale;
  a.k4c = k4_codes;
  a.k4s = k4_scales;
  a.k4t = k4_tscale;
  a.v4c = v4_codes;
  a.v4s = v4_scales;
  a.v4t = v4_tscale;
  a.idx = idx;
  a.cnt = cnt;
  a.o = o;
  a.lse = lse;
  a.kmax = kmax;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = S;
  a.Sp = cdiv(S, 64) * 64;
  a.nq = cdiv(S, block_q);
  a.causal = causal;
  a.o_fp32 = o_is_fp32;
  a.sm_log2 = sm_scale * 1.4426950408889634f;
  if (fmt == THRIFT_MXFP4) {
    if (D == 128) return block_q == 128 ? launch_attn<128, 4, THRIFT_MXFP4>(a, stream) : launch_attn<128, 2, THRIFT_MXFP4>(a, stream);
    return block_q == 128 ? launch_attn<64, 4, THRIFT_MXFP4>(a, stream) : launch_attn<64, 2, THRIFT_MXFP4>(a, stream);
  }
  if (D == 128) return block_q == 128 ? launch_attn<128, 4, THRIFT_NVFP4>(a, stream) : launch_attn<128, 2, THRIFT_NVFP4>(a, stream);
  return block_q == 128 ? launch_attn<64, 4, THRIFT_NVFP4>(a, stream) : launch_attn<64, 2, THRIFT_NVFP4>(a, stream);
}

extern "C" const char* thrift_status_string(thrift_status s) {
  switch (s) {
    case THRIFT_OK: return "ok";
    case THRIFT_EINVAL: return "invalid argument";
    case THRIFT_EUNSUPPORTED: return "unsupported shape";
    case THRIFT_EALIGN: return "pointer not 16-byte aligned";
    case THRIFT_EWORKSPACE: return "workspace missing or too small";
    case THRIFT_EHIP: return "HIP launch error";
  }
  return "unknown status";
}
