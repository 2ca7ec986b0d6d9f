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
//  * Two-level P (the pages take it from SageAttention3): level 1 of every
//    tile is the tile's own maximum, so each tile's probabilities are
//    2^(t - mt) with the largest exactly 1, quantised in the tile's
//    precision (level 2); the accumulator and row sum follow each tile's
//    level-1 unit (one rescale per tile), so the online softmax merges tiles
//    whose values do not depend on the running maximum or the order.
//  * Three workgroups per compute unit (12 waves, at most 168 VGPRs each):
//    the per-tile accumulator rescale of the two-level P makes the FP4 path
//    VALU-bound, and the third wave per SIMD hides one wave's MFMA and LDS
//    latency behind the others' VALU work.  MX K/V tiles stream through a
//    three-slot LDS ring of direct global->LDS loads, one barrier per two
//    blocks; the fp16 tiles (FP16 path, NVFP4, the middle tier) go through
//    one LDS stage inside the same space, loaded after the previous tile's
//    compute so that no registers are held across it.
#include <type_traits>

#include "common.h"

namespace thrift {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kMInit = -1.0e30f;  // unit and running maximum before the first key
constexpr float kDead = 60.0f;      // tiles this far (log2) below the running maximum add nothing
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
  // middle (MXFP8) tier, read by the three-tier kernels only: codes one byte
  // per element (Q, K [B,H,S,D]; V^T [B,H,D,Sp]) and E8M0 scales per 32;
  // idx2/cnt2 list the FP16 and FP8 tiers' blocks together
  const uint8_t* q8c;
  const uint8_t* q8s;
  const uint8_t* k8c;
  const uint8_t* k8s;
  const uint8_t* v8c;
  const uint8_t* v8s;
  const int32_t* idx2;
  const int32_t* cnt2;
  int kmax2;
};

// ---- MX stage layout -------------------------------------------------------
// A stage holds two 64-key blocks, filled by direct global->LDS loads (each
// lane of a load writes 16 consecutive bytes, so the layout is dense and the
// lanes' source addresses choose it).  K rows are in MFMA read order (row r =
// mt*32 + m holds key krow(mt, m)), 16-byte chunks XOR-swizzled by the row so
// that eight lanes reading eight rows hit eight different bank groups; V^T
// rows likewise.  Scales: K one u32 (D/32 bytes) per row in read order; V a
// [2][32] u32 table whose byte dt is the scale of (d = dt*32 + r, group kb).
template <int D>
struct MxStage {
  static constexpr int CPR = D / 32;        // 16-byte chunks per K row
  static constexpr int KCODE = kBk * D / 2;  // bytes of K codes per block
  static constexpr int VCODE = D * 32;       // bytes of V^T codes per block
  static constexpr int KSB = D / 32;         // K scale bytes per row
  static constexpr int KC = 0;                          // [2][KCODE]
  static constexpr int VC = KC + 2 * KCODE;             // [2][VCODE]
  static constexpr int KS = VC + 2 * VCODE;             // [2][64][KSB]
  static constexpr int VS = KS + 2 * kBk * KSB;         // [2][2][32] u32
  static constexpr int SIZE = (VS + 2 * 256 + 255) / 256 * 256;
  // Swizzled chunk of K row r / V^T row d.  A half-wave reads one chunk of
  // 16 consecutive rows: with 64 four-byte banks, 16 rows x 16 bytes must
  // land on 16 distinct 16-byte slots modulo 256 bytes (and any 8 of them
  // on distinct slots modulo 128 bytes).
  __device__ static int kswz(int r, int c) {
    return CPR == 4 ? c ^ (((r >> 1) ^ (r >> 3)) & 3) : c ^ (((r >> 2) ^ (r >> 3)) & 1);
  }
  __device__ static int vswz(int d, int h) { return h ^ (((d >> 2) ^ (d >> 3)) & 1); }
};

// ---- LDS layout --------------------------------------------------------------

template <int D>
struct Lds {
  // fp16 stage (FP16 path, NVFP4 FP4 path)
  static constexpr int KROWH = D + 8;    // halves per key row
  static constexpr int VROWH = kBk + 8;  // halves per V^T row (16-byte aligned)
  static constexpr int KH = 0;
  static constexpr int VT = KH + kBk * KROWH * 2;
  static constexpr int STAGEH = VT + D * VROWH * 2;
  static constexpr int STAGE = (STAGEH + 255) / 256 * 256;
  static constexpr int RING = (3 * MxStage<D>::SIZE > STAGE ? 3 * MxStage<D>::SIZE : STAGE);
  static constexpr int PROM = RING;  // int[kmax] promoted list
};

// ---- small helpers ---------------------------------------------------------------

__device__ inline v8i widen(v4i a) { return v8i{a.x, a.y, a.z, a.w, 0, 0, 0, 0}; }

template <int SA, int SB>
__device__ inline v16f mfma_fp4(v4i a, v4i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(a), widen(b), c, 4, 4, SA, sa, SB, sb);
}

__device__ inline float xlane32(float v) { return __shfl_xor(v, 32, kWave); }
__device__ inline uint32_t xlane32u(uint32_t v) { return __shfl_xor(v, 32, kWave); }

// 8 E2M1 codes (one dword, low nibble first) -> 8 fp16 values, times an
// fp16 factor (exact when the factor has at most 4 significant bits and the
// products stay normal).
__device__ inline v8h fp4x8_to_h(uint32_t cw, _Float16 f) {
  const v2h ff = {f, f};
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * ff;
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * ff;
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * ff;
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * ff;
  return v8h{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// K tiles are stored in LDS in krow's read order (key krow(mt, m) at row
// mt*32 + m), so the 32 lanes of a half-wave read consecutive rows; kslot is
// the inverse map, key -> LDS row.
__device__ inline int kslot(int key) {
  const int h = key >> 5, mt = (key >> 4) & 1, i = key & 15;
  return mt * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
}
__device__ inline int key_of(int mt, int i, int hi) { return hi * 32 + mt * 16 + i; }

// ---- online-softmax state ------------------------------------------------------

// acc and l are held in units of 2^lu.  lu is the level-1 exponent of the
// latest tile (its maximum in log2 units, plus the log2 of any factor its
// values carry, see tile_unit); mrun is the running maximum of the tiles'
// maxima.  Both lanes of a query (halves hi = 0, 1 of its keys and of its
// output channels) hold the same lu and mrun.
template <int D>
struct RowState {
  v16f acc[D / 32];  // O^T for this lane's query: d = dt*32 + (i/4)*8 + hi*4 + i%4
  float lu;          // log2 of the unit of acc and l
  float mrun;        // running maximum of the tiles' maxima (log2 units)
  float l;           // this lane's half of the running sum
};

template <int D>
__device__ inline void init_state(RowState<D>& st) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] = v16f{};
  st.lu = kMInit;
  st.mrun = kMInit;
  st.l = 0.0f;
}

// Level 1 of a tile whose maximum is mtc (log2 units): acc and l move to the
// unit 2^(mtc + lk), lk the log2 of the factor the tile's quantised values
// carry beyond 2^mtc (NVFP4 tensors: V's slice scale, and 1/2688 on the FP4
// path; 0 elsewhere).  A tile more than kDead below the running maximum adds
// nothing (it is below the row sum's fp32 resolution); the return value says
// whether the tile contributes.
template <int D>
__device__ inline bool tile_unit(RowState<D>& st, float mtc, float lk) {
  const bool live = mtc > st.mrun - kDead;
  const float nu = mtc + lk;
  const float r = live ? exp2_fast(st.lu - nu) : 1.0f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.acc[dt] *= r;
  st.l *= r;
  st.lu = live ? nu : st.lu;
  st.mrun = fmaxf(st.mrun, mtc);
  return live;
}

// Whether some row of the wave keeps the tile (tile_unit's test).  A tile
// that every row drops adds exactly nothing (its probabilities are all 0 and
// the state's unit does not move), so the wave skips the rest of it.
template <int D>
__device__ inline bool wave_live(const RowState<D>& st, float mtc) {
  return __builtin_amdgcn_ballot_w64(mtc > st.mrun - kDead) != 0;
}

// Causal / tail mask: keys past the query row or past S become -inf.  A
// lane's 32 keys are consecutive (key_of), so both conditions are one
// threshold on the element index: one compare and one select per element.
__device__ inline void mask_tile(v16f s[2], int key0, int qrow, int S, int causal, int hi) {
  const int last = causal && qrow < S - 1 ? qrow : S - 1;  // the last key the row sees
  const int lim = last - (key0 + key_of(0, 0, hi));       // elements past lim are masked
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (mt * 16 + i > lim) s[mt][i] = -INFINITY;
}

__device__ inline float max16(const v16f& v) {
  float a = fmaxf(fmaxf(v[0], v[1]), v[2]);
  float b = fmaxf(fmaxf(v[3], v[4]), v[5]);
  float c = fmaxf(fmaxf(v[6], v[7]), v[8]);
  float d = fmaxf(fmaxf(v[9], v[10]), v[11]);
  float e = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), v[15]));
}

// MFMA operands of one MX block read from LDS into registers ahead of use.
template <int D>
struct MxKOps {
  v4i a[2][D / 64];  // K codes of S^T tiles mt = 0, 1
  uint32_t sc[2];    // their E8M0 scales (this lane's contraction half)
};
template <int D>
struct MxVOps {
  v4i a[D / 32];  // V^T codes, one 32-row tile per dt
  uint32_t sc;    // byte dt: scale of V^T row dt*32 + r, key group hi
};

template <int D>
__device__ inline void load_k_mx(MxKOps<D>& k, const char* stage, int t, int lane) {
  using M = MxStage<D>;
  const int hi = lane >> 5, r32 = lane & 31;
  const uint8_t* kc = (const uint8_t*)(stage + M::KC + t * M::KCODE);
  const uint8_t* ks = (const uint8_t*)(stage + M::KS + t * kBk * M::KSB);
  // the scales' address from an opaque copy of the lane index: computed once
  // and held across the key sweep it was spilled, and each reload from
  // scratch waited for the ring's direct loads in flight
  int lo = lane;
  asm volatile("" : "+v"(lo));
  const uint8_t* ksl = ks + (lo & 31) * (D == 128 ? 4 : 2);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int row = mt * 32 + r32;  // holds key krow(mt, r32)
    k.sc[mt] = (D == 128 ? *(const uint32_t*)(ksl + mt * 128) : (uint32_t)(*(const uint16_t*)(ksl + mt * 64))) >> (8 * hi);
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk)
      k.a[mt][kk] = *(const v4i*)(kc + row * (D / 2) + M::kswz(row, kk * 2 + hi) * 16);
  }
}

template <int D>
__device__ inline void load_v_mx(MxVOps<D>& v, const char* stage, int t, int lane) {
  using M = MxStage<D>;
  const int hi = lane >> 5, r32 = lane & 31;
  const uint8_t* vc = (const uint8_t*)(stage + M::VC + t * M::VCODE);
  v.sc = ((const uint32_t*)(stage + M::VS + t * 256))[hi * 32 + r32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int d = dt * 32 + r32;
    v.a[dt] = *(const v4i*)(vc + d * 32 + M::vswz(d, hi) * 16);
  }
}

// S^T = K Q^T: two 32-row tiles, D/64 contraction steps of 64 channels,
// block-scaled by the E8M0 bytes of K and Q.
template <int D>
__device__ inline void qk_mx(v16f s[2], const MxKOps<D>& k, const v4i* qB, uint32_t qsc) {
  s[0] = mfma_fp4<0, 0>(k.a[0][0], qB[0], v16f{}, k.sc[0], qsc);
  s[1] = mfma_fp4<0, 0>(k.a[1][0], qB[0], v16f{}, k.sc[1], qsc);
  if constexpr (D == 128) {
    s[0] = mfma_fp4<2, 2>(k.a[0][1], qB[1], s[0], k.sc[0], qsc);
    s[1] = mfma_fp4<2, 2>(k.a[1][1], qB[1], s[1], k.sc[1], qsc);
  }
}

// Softmax, two-level MX quantisation of P and O^T += V^T P^T for one block.
template <int D>
__device__ inline void softmax_pv_mx(RowState<D>& st, v16f s[2], const MxVOps<D>& v, float c, int key0,
                                     int qrow, int S, int causal, bool need_mask, int lane) {
  const int hi = lane >> 5;
  if (need_mask) mask_tile(s, key0, qrow, S, causal, hi);

  // this lane's 32 keys are one P group (level 2); level 1 is the query's
  // tile maximum over both lane halves
  const float gmax = fmaxf(max16(s[0]), max16(s[1]));
  const float tmax = pair_max(gmax);
  const float mtc = tmax * c;
  if (!wave_live<D>(st, mtc)) return;
  const float nm = tile_unit<D>(st, mtc, -0.0f) ? -mtc : -INFINITY;  // dead tile: every p = 0

  // probabilities relative to the tile maximum, unquantised row sum
  float lsum = -0.0f;  // x + -0 folds to x
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2_fast(__builtin_fmaf(s[mt][i], c, nm));
      s[mt][i] = p;
      lsum += p;
    }
  st.l += lsum;

  // E8M0 exponent floor(log2(max p)) - 2: -2 for the group holding the tile
  // maximum (its p is 1 up to the rounding of mtc), else from the exponent
  // field of the group maximum's probability, computed like the elements'
  const uint32_t E = gmax == tmax ? 127u : (__float_as_uint(exp2_fast(__builtin_fmaf(gmax, c, nm))) >> 23) & 0xFF;
  const uint32_t psc = E > 3 ? E - 2 : 1;
  const float sf = __uint_as_float(psc << 23);

  // P^T operand: nibble n of this lane = key hi*32 + n = register n%16 of tile n/16
  v4i P;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const v16f& x = s[r >> 1];
    const int o = (r & 1) * 8;
    uint32_t y = __float_as_uint(x[o]);  // every byte is written below
    y = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(y, x[o + 0], x[o + 1], sf, 0);
    y = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(y, x[o + 2], x[o + 3], sf, 1);
    y = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(y, x[o + 4], x[o + 5], sf, 2);
    y = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(y, x[o + 6], x[o + 7], sf, 3);
    P[r] = (int)y;
  }

  // O^T += V^T P^T
  st.acc[0] = mfma_fp4<0, 0>(v.a[0], P, st.acc[0], v.sc, psc);
  st.acc[1] = mfma_fp4<1, 0>(v.a[1], P, st.acc[1], v.sc, psc);
  if constexpr (D == 128) {
    st.acc[2] = mfma_fp4<2, 0>(v.a[2], P, st.acc[2], v.sc, psc);
    st.acc[3] = mfma_fp4<3, 0>(v.a[3], P, st.acc[3], v.sc, psc);
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
__device__ inline void pv_f16(RowState<D>& st, const _Float16* vt, const v8h* pB, int lane) {
  using L = Lds<D>;
  const int hi = lane >> 5, r32 = lane & 31;
#pragma unroll
  for (int stp = 0; stp < 4; ++stp)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const v8h a = *(const v8h*)(vt + (dt * 32 + r32) * L::VROWH + hi * 32 + stp * 8);
      st.acc[dt] = mfma_f16(a, pB[stp], st.acc[dt]);
    }
}

// Promoted tile after its scores: mask, probabilities relative to the tile
// maximum rounded to fp16 (pB, the P^T operand: step st holds keys
// hi*32 + 8*st + u), the row sum; false when every row of the wave drops
// the tile (nothing to add).
template <int D>
__device__ inline bool fp16_probs(RowState<D>& st, v16f s[2], v8h pB[4], float c, int key0, int qrow, int S,
                                  int causal, bool need_mask, int lane) {
  const int hi = lane >> 5;
  if (need_mask) mask_tile(s, key0, qrow, S, causal, hi);
  // probabilities relative to the tile maximum (level 1), rounded to fp16
  const float mtc = pair_max(fmaxf(max16(s[0]), max16(s[1]))) * c;
  if (!wave_live<D>(st, mtc)) return false;
  const float nm = tile_unit<D>(st, mtc, -0.0f) ? -mtc : -INFINITY;
  float lsum = -0.0f;  // x + -0 folds to x
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2_fast(__builtin_fmaf(s[mt][i], c, nm));
      lsum += p;
      pB[mt * 2 + i / 8][i % 8] = (_Float16)p;
    }
  st.l += lsum;
  return true;
}

// Promoted tile after its scores: mask, probabilities rounded to fp16, times
// fp16 V^T (vt: D rows of Lds<D>::VROWH halves).
template <int D>
__device__ inline void fp16_softmax_pv(RowState<D>& st, v16f s[2], const _Float16* vt, float c, int key0,
                                       int qrow, int S, int causal, bool need_mask, int lane) {
  v8h pB[4];
  if (fp16_probs<D>(st, s, pB, c, key0, qrow, S, causal, need_mask, lane)) pv_f16<D>(st, vt, pB, lane);
}

// NVFP4 FP4 tile: scores from the dequantised fp16 stage, P quantised in two
// levels (level 1 per row and tile: v = 2688 p / p_max, p_max the tile
// maximum's probability, so the maximum lands on 6 * 448; level 2 per 16
// keys: E4M3 scale s2, E2M1 codes of v / s2).  The product with V uses
// code * s2, which fp16 holds exactly; the factor p_max / 2688 and V's slice
// scale are the tile's unit (lk = log2(sv / 2688)), so P is never rounded
// beyond the method.  ilk = 2688 / sv brings the row sum to that unit.
template <int D>
__device__ inline void fp4_nv_softmax_pv(RowState<D>& st, v16f s[2], const char* stage, float c, float lk,
                                         float ilk, int key0, int qrow, int S, int causal, bool need_mask,
                                         int lane) {
  const int hi = lane >> 5;
  if (need_mask) mask_tile(s, key0, qrow, S, causal, hi);
  const float gm0 = max16(s[0]), gm1 = max16(s[1]);  // this lane's two 16-key groups
  const float tmax = pair_max(fmaxf(gm0, gm1));      // the query's tile maximum (level 1)
  const float mtc = tmax * c;
  if (!wave_live<D>(st, mtc)) return;
  const float nm = tile_unit<D>(st, mtc, lk) ? -mtc : -INFINITY;
  float lsum = -0.0f;  // x + -0 folds to x
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2_fast(__builtin_fmaf(s[mt][i], c, nm));
      s[mt][i] = p;
      lsum += p;
    }
  st.l += lsum * ilk;
  v8h pB[4];
#pragma unroll
  for (int g = 0; g < 2; ++g) {  // group g = keys hi*32 + 16g .. +15 = registers of tile g
    const v16f& v = s[g];
    const float gmg = g ? gm1 : gm0;
    // level 2: E4M3 block scale of the group's largest value / 6 (the group
    // holding the tile maximum: 2688 / 6 = 448); the conversion does not
    // saturate: clamp
    const float gv = gmg == tmax ? 2688.0f : 2688.0f * exp2_fast(__builtin_fmaf(gmg, c, nm));
    v2s_t sb = {0, 0};
    sb = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(sb, fminf(gv * (1.0f / 6.0f), 448.0f), 0.0f, 1.0f, false);
    const float s2 = e4m3_to_float((uint32_t)sb[0] & 0xFF);
    const float k = nv_p_factor(s2);
    const _Float16 s2h = (_Float16)s2;  // exact: E4M3 has 4 significant bits
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // 8 keys per P^T operand
      const int o = h * 8;
      uint32_t cw = 0;
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[o + 0] * k, v[o + 1] * k, 1.0f, 0);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[o + 2] * k, v[o + 3] * k, 1.0f, 1);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[o + 4] * k, v[o + 5] * k, 1.0f, 2);
      cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, v[o + 6] * k, v[o + 7] * k, 1.0f, 3);
      pB[g * 2 + h] = fp4x8_to_h(cw, s2h);
    }
  }
  pv_f16<D>(st, (const _Float16*)(stage + Lds<D>::VT), pB, lane);
}

// The variant's FP4 tile: NVFP4 Q, K, V (dequantised to fp16 in the stage),
// P quantised MX-style: level 1 the tile maximum, level 2 an E8M0 scale per
// 32 keys (this lane's keys are one group), codes back to fp16 (code * 2^X,
// exact down to fp16's subnormal range) for the fp16 PV product.  V's slice
// scale is part of the tile's unit (lk = log2 sv, ilk = 1 / sv).
template <int D>
__device__ inline void fp4_nvmxp_tile(RowState<D>& st, const char* stage, const v8h* qh, float c, float lk,
                                      float ilk, int key0, int qrow, int S, int causal, bool need_mask, int lane) {
  const int hi = lane >> 5;
  v16f s[2];
  qk_f16<D>(s, stage, qh, lane);
  if (need_mask) mask_tile(s, key0, qrow, S, causal, hi);
  const float gmax = fmaxf(max16(s[0]), max16(s[1]));
  const float tmax = pair_max(gmax);
  const float mtc = tmax * c;
  if (!wave_live<D>(st, mtc)) return;
  const float nm = tile_unit<D>(st, mtc, lk) ? -mtc : -INFINITY;
  float lsum = -0.0f;  // x + -0 folds to x
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2_fast(__builtin_fmaf(s[mt][i], c, nm));
      s[mt][i] = p;
      lsum += p;
    }
  st.l += lsum * ilk;
  // E8M0 exponent floor(log2(max p)) - 2, as on the MX path
  const uint32_t E = gmax == tmax ? 127u : (__float_as_uint(exp2_fast(__builtin_fmaf(gmax, c, nm))) >> 23) & 0xFF;
  const uint32_t psc = E > 3 ? E - 2 : 1;
  const float sf = __uint_as_float(psc << 23);
  v8h pB[4];
#pragma unroll
  for (int stp = 0; stp < 4; ++stp) {  // keys hi*32 + 8 stp + u: registers 8 (stp % 2) + u of tile stp / 2
    const v16f& x = s[stp >> 1];
    const int o = (stp & 1) * 8;
    uint32_t cw = 0;
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, x[o + 0], x[o + 1], sf, 0);
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, x[o + 2], x[o + 3], sf, 1);
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, x[o + 4], x[o + 5], sf, 2);
    cw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(cw, x[o + 6], x[o + 7], sf, 3);
    const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sf, 0);
    const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sf, 1);
    const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sf, 2);
    const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, sf, 3);
    pB[stp] = v8h{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
  }
  pv_f16<D>(st, (const _Float16*)(stage + Lds<D>::VT), pB, lane);
}

template <int D>
__device__ inline void fp4_nv_tile(RowState<D>& st, const char* stage, const v8h* qh, float c, float lk,
                                   float ilk, int key0, int qrow, int S, int causal, bool need_mask, int lane) {
  v16f s[2];
  qk_f16<D>(s, stage, qh, lane);
  fp4_nv_softmax_pv<D>(st, s, stage, c, lk, ilk, key0, qrow, S, causal, need_mask, lane);
}

}  // namespace thrift

namespace thrift {

// ---- staging: global -> registers -> LDS ----------------------------------------

// MX stage fill.  K codes, V^T codes and (D = 128) K scales go global -> LDS
// directly with buffer loads (buffer_load_dwordx4 / _dword ... lds: no
// registers, no LDS store instructions); V scales (two bytes per V^T row and
// block) and the D = 64 K scales go through registers.  Every per-lane source
// offset is fixed for the whole key sweep; the block moves only the base of
// the buffer resource (scalar work).  The resource's record count ends at the
// tensor's end, so key rows past S (last block) read as out of range and
// never touch memory; their scores are masked.
// ---- middle-tier (MXFP8) tile ------------------------------------------------------
//
// gfx950's block-scaled matrix instruction does not sum E4M3 products exactly:
// its error reaches about 2^-12.6 of the sum of the products' magnitudes
// (measured on random E4M3 operands), where E2M1 products, spanning few
// binades, come out exact.  The middle tier therefore runs like NVFP4's FP4
// path: its tiles are decoded to fp16 in LDS (an E4M3 value times a power of
// two has 4 significant bits, exact in fp16 for every group whose maximum is
// at least 2^-7; the elements of smaller groups round to fp16's 2^-24 grid)
// and multiplied on the fp16 matrix cores; P is quantised to E4M3 and held
// as the fp16 value code * 2^exponent.

// 8 E4M3 codes (two dwords, byte u = element u) times the power of two
// `scale`, to fp16 by the scaled FP8 -> fp16 conversion (two values per
// instruction; exact wherever fp16 holds the product).
__device__ inline v8h fp8x8_to_h(uint32_t lo, uint32_t hi, float scale) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)lo, scale, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)lo, scale, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)hi, scale, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)hi, scale, true);
  return v8h{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Promoted tile on the middle tier: scores from the decoded fp16 stage; this
// lane's 32 keys are one P group (its E8M0 exponent floor(log2(max p)) - 8);
// elements clamped to 448 times the scale, rounded to E4M3 by the scaled FP8
// conversion (nearest even) and decoded back exactly; times the decoded V^T.
template <int D>
__device__ inline void fp8_tile(RowState<D>& st, const char* stage, const v8h* qh, float c, int key0, int qrow,
                                int S, int causal, bool need_mask, int lane) {
  const int hi = lane >> 5;
  v16f s[2];
  qk_f16<D>(s, stage, qh, lane);
  if (need_mask) mask_tile(s, key0, qrow, S, causal, hi);
  const float gmax = fmaxf(max16(s[0]), max16(s[1]));
  const float tmax = pair_max(gmax);  // level 1: the tile maximum
  const float mtc = tmax * c;
  if (!wave_live<D>(st, mtc)) return;
  const float nm = tile_unit<D>(st, mtc, -0.0f) ? -mtc : -INFINITY;
  float lsum = -0.0f;  // x + -0 folds to x
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = exp2_fast(__builtin_fmaf(s[mt][i], c, nm));
      s[mt][i] = p;
      lsum += p;
    }
  st.l += lsum;
  // E8M0 exponent floor(log2(max p)) - 8 (-8 for the tile maximum's group)
  const uint32_t E = gmax == tmax ? 127u : (__float_as_uint(exp2_fast(__builtin_fmaf(gmax, c, nm))) >> 23) & 0xFF;
  const uint32_t psc = E > 9 ? E - 8 : 1;
  const float sf = __uint_as_float(psc << 23);
  const float cap = 448.0f * sf;
  // P^T operand as pv_f16 takes it: step st, element u = key hi*32 + 8*st + u
  v8h pB[4];
#pragma unroll
  for (int stp = 0; stp < 4; ++stp) {
    const v16f& x = s[stp >> 1];
    const int o = (stp & 1) * 8;
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v2s_t y = {0, 0};
      y = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(y, fminf(x[o + 4 * h], cap), fminf(x[o + 4 * h + 1], cap), sf, false);
      y = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(y, fminf(x[o + 4 * h + 2], cap), fminf(x[o + 4 * h + 3], cap), sf,
                                                    true);
      w[h] = __builtin_bit_cast(uint32_t, y);
    }
    pB[stp] = fp8x8_to_h(w[0], w[1], sf);
  }
  pv_f16<D>(st, (const _Float16*)(stage + Lds<D>::VT), pB, lane);
}

template <int D, int NW>
struct MxDma {
  using M = MxStage<D>;
  static constexpr int KINST = M::KCODE / 1024;  // wave loads (64 lanes x 16 B) per block of K codes
  static constexpr int VINST = M::VCODE / 1024;  // ... of V^T codes
  static constexpr int NK = 2 * KINST / NW;      // per wave and stage
  static constexpr int NV = 2 * VINST / NW;
  static_assert(NK * NW == 2 * KINST && NV * NW == 2 * VINST, "wave loads must split evenly");
  static constexpr int NT = NW * 64;
  static constexpr int NVS = 2 * D;  // V scale entries (one per V^T row and block) per stage
  static constexpr int NVR = (NVS + NT - 1) / NT;
  static constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

  __amdgpu_buffer_rsrc_t kc, ks, vc, vs;  // this head's tensors, record counts ending at their ends
  int nv, w;
  uint32_t koff[NK], voff[NV], ksoff, vsoff[NVR];
  uint32_t vreg[NVR], kreg;

  __device__ static __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcWord3);
  }
  __device__ static __attribute__((address_space(3))) void* lds(char* p) {
    return (__attribute__((address_space(3))) void*)p;
  }

  __device__ MxDma(const AttnArgs& a, size_t bhk, int nv_, int w_, int lane, int t)
      : kc(rsrc(a.k4c + bhk * a.S * (D / 2), a.S * (D / 2))),
        ks(rsrc(a.k4s + bhk * a.S * (D / 32), a.S * (D / 32))),
        vc(rsrc(a.v4c + bhk * D * (a.Sp / 2), D * (a.Sp / 2))),
        vs(rsrc(a.v4s + bhk * D * (a.Sp / 32), D * (a.Sp / 32))),
        nv(nv_), w(w_) {
#pragma unroll
    for (int k = 0; k < NK; ++k) {  // LDS chunk ci of the block -> row r, swizzled chunk
      const int ci = ((w * NK + k) % KINST) * 64 + lane, r = ci / M::CPR;
      const int c = M::kswz(r, ci % M::CPR);  // the swizzle is an involution per row
      koff[k] = krow(r >> 5, r & 31) * (D / 2) + c * 16;
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int ci = ((w * NV + k) % VINST) * 64 + lane, d = ci / 2;
      voff[k] = d * 32 + M::vswz(d, ci % 2) * 16;  // key-block-major V^T
    }
    ksoff = krow(lane >> 5, lane & 31) * (D / 32);
#pragma unroll
    for (int p = 0; p < NVR; ++p) {
      const int e = t + p * NT;
      vsoff[p] = (e % D) * 2 + ((e / D) & 1) * (2 * D);
    }
  }

  // Issue the loads of blocks j0 and j0+1 into `stage` (a block past the last
  // valid one reloads the last one; it is never computed).  The block offset
  // goes into the per-lane offset, which the resource's record count checks.
  __device__ void issue(char* stage, int j0) {
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      const int g = w * NK + k, jj = min(j0 + g / KINST, nv - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kc, lds(stage + M::KC + g * 1024), 16, koff[k] + jj * M::KCODE,
                                               0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int g = w * NV + k, jj = min(j0 + g / VINST, nv - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vc, lds(stage + M::VC + g * 1024), 16, voff[k] + jj * M::VCODE,
                                               0, 0, 0);
    }
    if (w < 2) {  // K scales of block j0 + w, rows in read order
      const uint32_t o = ksoff + min(j0 + w, nv - 1) * (kBk * (D / 32));
      if constexpr (D == 128)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ks, lds(stage + M::KS + w * kBk * 4), 4, o, 0, 0, 0);
      else
        kreg = __builtin_amdgcn_raw_buffer_load_b16(ks, o, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < NVR; ++p) vreg[p] = __builtin_amdgcn_raw_buffer_load_b16(vs, vsoff[p] + j0 * (2 * D), 0, 0);
  }

  // Store what issue() loaded into registers (after the compute, before the barrier).
  __device__ void finish(char* stage, int t) const {
    if constexpr (D == 64)
      if (w < 2) ((uint16_t*)(stage + M::KS + w * kBk * 2))[t & 63] = (uint16_t)kreg;
#pragma unroll
    for (int p = 0; p < NVR; ++p) {
      const int e = t + p * NT;
      if (NVS % NT != 0 && e >= NVS) continue;
      const int tb = (e / D) & 1, d = e % D;
      uint8_t* vsb = (uint8_t*)(stage + M::VS + tb * 256);
      vsb[(d & 31) * 4 + (d >> 5)] = (uint8_t)(vreg[p] & 0xFF);
      vsb[(32 + (d & 31)) * 4 + (d >> 5)] = (uint8_t)(vreg[p] >> 8);
    }
  }
};

// ---- the FP16 path's pipelined stage ------------------------------------------
typedef short v4s_t __attribute__((ext_vector_type(4)));
//
// K and V rows of a promoted block go from HBM straight into LDS
// (buffer_load_dwordx4 ... lds: no staging registers, no LDS stores).  Two K
// buffers and one V buffer: while a block's scores and probabilities are
// computed, the next block's V and the one after's K are in flight.  Each
// buffer is chunk-column-major: 16-byte chunk c of row r at c * CS + r * 16,
// one direct wave load per chunk column (K rows in MFMA read order, row r
// holding key krow(r >> 5, r & 31); V rows in key order).  The column stride
// CS = 1024 + 64 bytes staggers the columns by 64 bytes across the banks, so
// that both the K reads (16 rows of one chunk per half-wave) and the
// transposed V reads (ds_read_b64_tr_b16: per 16 lanes, 4 keys of 16
// channels, two chunk columns) are free of bank conflicts, and every address
// is a per-lane base plus an immediate.  The buffers take the ring's memory,
// free once the FP4 pass is done.
template <int D>
struct F16Pipe {
  static constexpr int CS = 1024 + 64;         // bytes per chunk column (64 rows + stagger)
  static constexpr int TILE = (D / 8) * CS;    // one K or V block
  static constexpr int KB = 0;                 // [2][TILE]
  static constexpr int VB = 2 * TILE;          // [TILE]
  static constexpr int SIZE = 3 * TILE;
};

// This wave's share of one block's direct loads: chunk columns w*NI ..
// w*NI + NI - 1 of the K or V buffer, one wave load (64 rows x 16 bytes) each.
template <int D, int NW>
struct F16Dma {
  using P = F16Pipe<D>;
  static constexpr int NI = (D / 8) / NW;  // chunk columns per wave and tensor
  static_assert(NI * NW == D / 8, "chunk columns must split evenly over the waves");
  static constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
  __amdgpu_buffer_rsrc_t kr, vr;                 // this head's fp16 K and V; rows past S read as zeros
  uint32_t koff, voff;                           // this lane's row: key krow(lane) of K, key lane of V
  int w;

  __device__ F16Dma(const AttnArgs& a, size_t bhk, int w_, int lane) : w(w_) {
    const int bytes = a.S * D * 2;
    kr = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k16 + bhk * a.S * D), 0, bytes, kRsrcWord3);
    vr = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + bhk * a.S * D), 0, bytes, kRsrcWord3);
    koff = krow(lane >> 5, lane & 31) * (D * 2) + w * NI * 16;
    voff = lane * (D * 2) + w * NI * 16;
  }
  __device__ static __attribute__((address_space(3))) void* lds(char* p) {
    return (__attribute__((address_space(3))) void*)p;
  }
  __device__ void issue_k(char* buf, int j) const {
#pragma unroll
    for (int k = 0; k < NI; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, lds(buf + (w * NI + k) * P::CS), 16,
                                               koff + j * (kBk * D * 2) + k * 16, 0, 0, 0);
  }
  __device__ void issue_v(char* buf, int j) const {
#pragma unroll
    for (int k = 0; k < NI; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, lds(buf + (w * NI + k) * P::CS), 16,
                                               voff + j * (kBk * D * 2) + k * 16, 0, 0, 0);
  }
};

// S^T = K Q^T from a K buffer: lane (r32, hi) reads chunk kk*2 + hi of row
// mt*32 + r32.
template <int D>
__device__ inline void qk_f16p(v16f s[2], const char* kb, const v8h* qh, int lane) {
  using P = F16Pipe<D>;
  const int hi = lane >> 5, r32 = lane & 31;
  const char* base = kb + hi * P::CS + r32 * 16;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    s[mt] = v16f{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      s[mt] = mfma_f16(*(const v8h*)(base + kk * 2 * P::CS + mt * 32 * 16), qh[kk], s[mt]);
  }
}

// O^T += V^T P^T with the V^T operand read transposed from the V buffer:
// ds_read_b64_tr_b16 gives lane i of each 16 lanes element i % 4 of the
// 8-byte pieces that lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12 address;
// so lane r addresses key key0 + r / 4, channels d0 + 4 (r % 4) .. + 3, and
// lane i receives channel d0 + i of keys key0 .. key0 + 3.  In step st this
// lane supplies keys hi*32 + 8*st + u of channel dt*32 + r32.
template <int D>
__device__ inline void pv_f16p(RowState<D>& st, const char* vb, const v8h* pB, int lane) {
  using P = F16Pipe<D>;
  const int hi = lane >> 5, r32 = lane & 31, r = r32 & 15;
  const int col = (r32 >> 4) * 16 + 4 * (r & 3);  // channel within a 32-channel tile
  const char* base = vb + (col >> 3) * P::CS + (hi * 32 + (r >> 2)) * 16 + (col & 7) * 2;
#pragma unroll
  for (int stp = 0; stp < 4; ++stp)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const char* q = base + dt * 4 * P::CS + stp * 8 * 16;
      const v4h lo = __builtin_bit_cast(
          v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(char*)q));
      const v4h up = __builtin_bit_cast(
          v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(char*)(q + 64)));
      const v8h av = {lo.x, lo.y, lo.z, lo.w, up.x, up.y, up.z, up.w};
      st.acc[dt] = mfma_f16(av, pB[stp], st.acc[dt]);
    }
}

// MXFP8 tile of key block j decoded to the fp16 stage (K rows at kslot, V^T
// rows, the fp16 stage's layout): each thread takes 16-byte chunks of codes
// with the E8M0 byte of their group.  K rows past S read as zeros; V^T rows
// are padded to Sp with zeros by the quantiser.
template <int D, int NT>
struct F8Stager {
  static constexpr int NK = kBk * D / 16;  // 16-code chunks of K (row, 16 channels)
  static constexpr int NV = D * kBk / 16;  // 16-code chunks of V^T (d, 16 keys)
  static constexpr int PK = (NK + NT - 1) / NT, PV = (NV + NT - 1) / NT;
  v4i kr[PK], vr[PV];
  uint8_t ks[PK], vs[PV];

  __device__ void load(const AttnArgs& a, size_t bhk, int j, int t) {
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      const int c = t + p * NT, row = c / (D / 16), col = (c % (D / 16)) * 16, key = j * kBk + row;
      kr[p] = v4i{};
      ks[p] = 127;
      if (c < NK && key < a.S) {
        kr[p] = *(const v4i*)(a.k8c + (bhk * a.S + key) * D + col);
        ks[p] = a.k8s[(bhk * a.S + key) * (D / 32) + col / 32];
      }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      const int c = t + p * NT, d = c / (kBk / 16), k0 = (c % (kBk / 16)) * 16;
      vr[p] = v4i{};
      vs[p] = 127;
      if (c < NV) {
        vr[p] = *(const v4i*)(a.v8c + (bhk * D + d) * a.Sp + j * kBk + k0);
        vs[p] = a.v8s[(bhk * D + d) * (a.Sp / 32) + (j * kBk + k0) / 32];
      }
    }
  }

  __device__ void store(char* stage, int t) const {
    using L = Lds<D>;
    _Float16* kh = (_Float16*)(stage + L::KH);
    _Float16* vt = (_Float16*)(stage + L::VT);
#pragma unroll
    for (int p = 0; p < PK; ++p) {
      const int c = t + p * NT;
      if (c < NK) {
        const float sc = __uint_as_float((uint32_t)ks[p] << 23);
        _Float16* dst = kh + kslot(c / (D / 16)) * L::KROWH + (c % (D / 16)) * 16;
        *(v8h*)dst = fp8x8_to_h((uint32_t)kr[p].x, (uint32_t)kr[p].y, sc);
        *(v8h*)(dst + 8) = fp8x8_to_h((uint32_t)kr[p].z, (uint32_t)kr[p].w, sc);
      }
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      const int c = t + p * NT;
      if (c < NV) {
        const float sc = __uint_as_float((uint32_t)vs[p] << 23);
        _Float16* dst = vt + (c / (kBk / 16)) * L::VROWH + (c % (kBk / 16)) * 16;
        *(v8h*)dst = fp8x8_to_h((uint32_t)vr[p].x, (uint32_t)vr[p].y, sc);
        *(v8h*)(dst + 8) = fp8x8_to_h((uint32_t)vr[p].z, (uint32_t)vr[p].w, sc);
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
        const size_t blk = bhk * (a.Sp / 64) + j;  // key-block-major V^T
        vc[p] = *(const v4i*)(a.v4c + (blk * D + d) * 32 + h * 16);
        vs[p] = *(const uint16_t*)(a.v4s + (blk * D + d) * 4 + h * 2);
      }
    }
  }

  __device__ static void expand(_Float16* dst, v4i codes, uint32_t sc2) {
    const _Float16 f0 = (_Float16)e4m3_to_float(sc2 & 0xFF);
    const _Float16 f1 = (_Float16)e4m3_to_float((sc2 >> 8) & 0xFF);
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // 8 elements per dword; dwords 0-1 group 0, 2-3 group 1
      const _Float16 f = q < 2 ? f0 : f1;
      *(v8h*)(dst + q * 8) = fp4x8_to_h((uint32_t)codes[q], f);
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

// NVFP4 FP4 pass through LDS twice: one block's codes and scales come by
// direct loads into a raw buffer (a byte copy of the block's stretch of each
// tensor: K codes, V^T codes, K scales, V^T scales, all contiguous per
// block), are decoded from there into the fp16 stage, and the raw buffer
// then takes the next block's loads while the current block is computed.
// The raw buffer sits after the fp16 stage in the ring's memory.
template <int D>
struct NvRaw {
  static constexpr int KC = Lds<D>::STAGE;        // [kBk][D/2]
  static constexpr int VC = KC + kBk * D / 2;      // [D][32]
  static constexpr int KS = VC + D * 32;           // [kBk][D/16]
  static constexpr int VS = KS + kBk * D / 16;     // [D][4]
  static constexpr int END = VS + D * 4;
  static_assert(END <= Lds<D>::RING, "the raw buffer must fit the ring");
  // wave loads per block: 1 KB of codes (64 lanes x 16 B) or 256 B of
  // scales (64 lanes x 4 B) each
  static constexpr int NCODE = D / 32;  // per tensor
  static constexpr int NSC = D / 64;    // per tensor
  static constexpr int NLOAD = 2 * NCODE + 2 * NSC;
};

template <int D, int NW>
struct NvDma {
  using R = NvRaw<D>;
  static constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
  // this head's tensors; record counts end at their ends, so K rows past S
  // read as zeros
  __amdgpu_buffer_rsrc_t kc, ks, vc, vs;
  int w, lane;

  __device__ static __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, kRsrcWord3);
  }
  __device__ static __attribute__((address_space(3))) void* lds(char* p) {
    return (__attribute__((address_space(3))) void*)p;
  }
  __device__ NvDma(const AttnArgs& a, size_t bhk, int w_, int lane_)
      : kc(rsrc(a.k4c + bhk * a.S * (D / 2), a.S * (D / 2))),
        ks(rsrc(a.k4s + bhk * a.S * (D / 16), a.S * (D / 16))),
        vc(rsrc(a.v4c + bhk * (a.Sp / 64) * D * 32, (a.Sp / 64) * D * 32)),
        vs(rsrc(a.v4s + bhk * (a.Sp / 64) * D * 4, (a.Sp / 64) * D * 4)),
        w(w_), lane(lane_) {}

  // Wave w issues loads w, w + NW, ... of block j's NLOAD.
  __device__ void issue(char* smem, int j) const {
#pragma unroll
    for (int g = 0; g < R::NLOAD; ++g) {
      if (g % NW != w) continue;
      if (g < R::NCODE)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kc, lds(smem + R::KC + g * 1024), 16,
                                                 j * (kBk * D / 2) + g * 1024 + lane * 16, 0, 0, 0);
      else if (g < 2 * R::NCODE)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vc, lds(smem + R::VC + (g - R::NCODE) * 1024), 16,
                                                 j * (D * 32) + (g - R::NCODE) * 1024 + lane * 16, 0, 0, 0);
      else if (g < 2 * R::NCODE + R::NSC)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ks, lds(smem + R::KS + (g - 2 * R::NCODE) * 256), 4,
                                                 j * (kBk * D / 16) + (g - 2 * R::NCODE) * 256 + lane * 4, 0, 0,
                                                 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vs, lds(smem + R::VS + (g - 2 * R::NCODE - R::NSC) * 256), 4,
                                                 j * (D * 4) + (g - 2 * R::NCODE - R::NSC) * 256 + lane * 4, 0,
                                                 0, 0);
    }
  }
};

// Raw buffer -> fp16 stage, in Nv4Stager's layout: thread t decodes 16-byte
// chunks t, t + NT, ... of the K codes (row c / (D/32), 32 channels) and of
// the V^T codes (row c / 2, 32 keys).
template <int D, int NT>
__device__ inline void nv_decode(char* smem, int t) {
  using R = NvRaw<D>;
  using L = Lds<D>;
  using St = Nv4Stager<D, NT>;
  _Float16* kh = (_Float16*)(smem + L::KH);
  _Float16* vt = (_Float16*)(smem + L::VT);
#pragma unroll
  for (int p = 0; p < St::PK; ++p) {
    const int c = t + p * NT;
    if (c < St::NKC) {
      const int row = c / (D / 32), col = c % (D / 32);
      const v4i codes = *(const v4i*)(smem + R::KC + c * 16);
      const uint32_t sc = *(const uint16_t*)(smem + R::KS + row * (D / 16) + col * 2);
      St::expand(kh + kslot(row) * L::KROWH + col * 32, codes, sc);
    }
  }
#pragma unroll
  for (int p = 0; p < St::PV; ++p) {
    const int c = t + p * NT;
    if (c < St::NVC) {
      const v4i codes = *(const v4i*)(smem + R::VC + c * 16);
      const uint32_t sc = *(const uint16_t*)(smem + R::VS + c * 2);
      St::expand(vt + (c / 2) * L::VROWH + (c % 2) * 32, codes, sc);
    }
  }
}

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

// T8: the three-tier variant (MX only): the blocks idx2 lists and idx does
// not run on the middle MXFP8 tier, between the FP4 and FP16 paths.
template <int D, int NW, int FMT, bool T8 = false>
__global__ __launch_bounds__(NW * 64, 3) void attn_fwd_kernel(AttnArgs a) {
  static_assert(!T8 || FMT == THRIFT_MXFP4, "the middle tier is built for the MX format");
  using L = Lds<D>;
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), hi = lane >> 5;
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
  int ncnt2 = 0;
  if constexpr (T8) {
    ncnt2 = a.cnt2[rowid];
    ncnt2 = ncnt2 < 0 ? 0 : (ncnt2 > a.kmax2 ? a.kmax2 : ncnt2);
  }
  int* prom = (int*)(smem + L::PROM);
  int* prom2 = prom + a.kmax;  // three-tier kernels: int[kmax2], the idx2 list
  // bit j: key block j leaves the FP4 path (promoted to a higher tier)
  uint32_t* pbits = (uint32_t*)prom2 + (T8 ? a.kmax2 : 0);
  const int nwords = (nvalid + 31) >> 5;
  uint32_t* pbits16 = pbits + nwords;  // three-tier kernels: bit j: block j is FP16
  for (int e = t; e < nwords; e += NT) {
    pbits[e] = 0;
    if constexpr (T8) pbits16[e] = 0;
  }
  __syncthreads();
  for (int e = t; e < ncnt; e += NT) {
    const int j = a.idx[rowid * a.kmax + e];
    prom[e] = j;
    if (j >= 0 && j < nvalid) {
      atomicOr(&pbits[j >> 5], 1u << (j & 31));
      if constexpr (T8) atomicOr(&pbits16[j >> 5], 1u << (j & 31));
    }
  }
  if constexpr (T8)
    for (int e = t; e < ncnt2; e += NT) {
      const int j = a.idx2[rowid * a.kmax2 + e];
      prom2[e] = j;
      if (j >= 0 && j < nvalid) atomicOr(&pbits[j >> 5], 1u << (j & 31));
    }
  __syncthreads();

  RowState<D> st;
  init_state<D>(st);

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
      // Three-stage LDS ring of two-block stages over every valid key block in
      // order, one barrier per stage; promoted blocks are loaded but not
      // computed (their FP16 pass comes later), which keeps the load stream
      // regular.  Iteration s issues the direct loads of stage s+2 into ring
      // slot s+2 (whose previous stage, s-1, every wave finished before the
      // last barrier) and computes blocks 2s and 2s+1, each QK product right
      // before its softmax (one score tile in registers: the other waves of
      // the SIMD cover the product's latency).
      using Dma = MxDma<D, NW>;
      using M = MxStage<D>;
      Dma dma(a, bhk, nvalid, w, lane, t);
      auto active_of = [&](int j) {
        return j < nvalid && !((pbits[j >> 5] >> (j & 31)) & 1u) && (!a.causal || j * kBk <= q0 + 31);
      };
      auto mask_of = [&](int j) {
        const int key0 = j * kBk;
        return (a.causal && key0 + kBk - 1 > q0) || key0 + kBk > S;
      };
      auto slot = [&](int k) { return smem + (k % 3) * M::SIZE; };
      if (T8 || ncnt < nvalid) {
        const int nst = (nvalid + 1) / 2;  // stages
        dma.issue(slot(0), 0);
        dma.finish(slot(0), t);
        if (nst > 1) {
          dma.issue(slot(1), 2);
          dma.finish(slot(1), t);
        }
        __syncthreads();
        v16f sA[2];
        MxKOps<D> kop;
        MxVOps<D> vop;
        int sg = 0;
        // one stage; the ring slot is a compile-time constant so that every
        // LDS address is a per-lane base plus an immediate offset
        auto stage_step = [&](auto slot_c) {
          constexpr int SL = decltype(slot_c)::value;
          char* const cur = smem + SL * M::SIZE;
          char* const fut = smem + ((SL + 2) % 3) * M::SIZE;
          const int j0 = 2 * sg;
          const bool more = sg + 2 < nst;
          if (more) dma.issue(fut, j0 + 4);
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            if (active_of(j0 + tb)) {
              load_k_mx<D>(kop, cur, tb, lane);
              qk_mx<D>(sA, kop, qB, qsc);
              load_v_mx<D>(vop, cur, tb, lane);
              softmax_pv_mx<D>(st, sA, vop, c, (j0 + tb) * kBk, qrow, S, a.causal, mask_of(j0 + tb), lane);
            }
          }
          if (more) dma.finish(fut, t);
          __syncthreads();
          return ++sg < nst;
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        while (stage_step(I0{}) && stage_step(I1{}) && stage_step(I2{})) {
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
          qh[kk] = fp4x8_to_h(cw, f);
        }
      }
      const float c = a.sm_log2 * a.q4t[bhq] * a.k4t[bhk];
      // the tiles' unit carries V's slice scale (and NVFP4's 1/2688 of level 1)
      const float sv = a.v4t[bhk];
      const float lk = FMT == THRIFT_NVFP4 ? log2f(sv) - log2f(2688.0f) : log2f(sv);
      const float ilk = FMT == THRIFT_NVFP4 ? 2688.0f / sv : 1.0f / sv;
      // the next block's codes arrive in the raw buffer while this one is computed
      NvDma<D, NW> dma(a, bhk, w, lane);
      if (jc < nvalid) dma.issue(smem, jc);
      while (jc < nvalid) {
        const int jn = next_fp4(jc + 1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();  // the raw buffer holds block jc; the fp16 stage is free
        nv_decode<D, NT>(smem, t);
        __syncthreads();  // the stage holds block jc; the raw buffer is free
        if (jn < nvalid) dma.issue(smem, jn);
        const int key0 = jc * kBk;
        const bool active = !a.causal || key0 <= q0 + 31;
        const bool need_mask = (a.causal && key0 + kBk - 1 > q0) || key0 + kBk > S;
        if (active) {
          if constexpr (FMT == THRIFT_NVFP4)
            fp4_nv_tile<D>(st, smem, qh, c, lk, ilk, key0, qrow, S, a.causal, need_mask, lane);
          else
            fp4_nvmxp_tile<D>(st, smem, qh, c, lk, ilk, key0, qrow, S, a.causal, need_mask, lane);
        }
        jc = jn;
      }
      __syncthreads();  // every wave is done with the stage
    }
  }

  // ---------------- middle tier (MXFP8): idx2's blocks not on the FP16 path ----------------
  if constexpr (T8) {
    if (ncnt2 > 0) {
      // the query row decoded to fp16 in the fp16 path's operand order
      const size_t qoff = (size_t)bhq * S + (qvalid ? qrow : 0);
      v8h qh8[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        qh8[kk] = v8h{};
        if (qvalid) {
          const int ch = kk * 16 + hi * 8;
          const uint2 cw = *(const uint2*)(a.q8c + qoff * D + ch);
          qh8[kk] = fp8x8_to_h(cw.x, cw.y, __uint_as_float((uint32_t)a.q8s[qoff * (D / 32) + ch / 32] << 23));
        }
      }
      auto tier8_j = [&](int p) {
        const int j = prom2[p];
        return j >= 0 && j < nvalid && !((pbits16[j >> 5] >> (j & 31)) & 1u) ? j : -1;
      };
      F8Stager<D, NT> stg;
      for (int p = 0; p < ncnt2; ++p) {
        const int jc = tier8_j(p);
        if (jc >= 0) stg.load(a, bhk, jc, t);
        if (jc >= 0) stg.store(smem, t);
        __syncthreads();
        if (jc >= 0) {
          const int key0 = jc * kBk;
          const bool active = !a.causal || key0 <= q0 + 31;
          const bool need_mask = (a.causal && key0 + kBk - 1 > q0) || key0 + kBk > S;
          if (active)
            fp8_tile<D>(st, smem, qh8, a.sm_log2, key0, qrow, S, a.causal, need_mask, lane);
        }
        __syncthreads();
      }
    }
  }

  // ---------------- FP16 path: promoted blocks only ----------------
  // Pipelined through F16Pipe's buffers (the ring's memory: the passes before
  // ended with a barrier).  Block p: its scores and probabilities (K[p % 2]),
  // a barrier (V_p in LDS), PV, a barrier (every wave done with V and K[p % 2];
  // K_{p+1} in LDS), then the loads of V_{p+1} and K_{p+2} go out, in flight
  // during block p+1's scores and probabilities.  Every wave waits for its own
  // direct loads before each barrier.
  if (ncnt > 0) {
    using FP = F16Pipe<D>;
    static_assert(FP::SIZE <= L::RING, "the fp16 pipeline's buffers fit in the ring");
    v8h qh[D / 16];
    const size_t qoff = ((size_t)bhq * S + qrow) * D + hi * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qh[kk] = qvalid ? *(const v8h*)(a.q16 + qoff + kk * 16) : v8h{};
    F16Dma<D, NW> fd(a, bhk, w, lane);
    auto prom_j = [&](int p) {
      const int j = p < ncnt ? prom[p] : -1;
      return j >= 0 && j < nvalid ? j : -1;
    };
    auto kbuf = [&](int p) { return smem + FP::KB + (p & 1) * FP::TILE; };
    {
      const int j0 = prom_j(0), j1 = prom_j(1);
      if (j0 >= 0) {
        fd.issue_k(kbuf(0), j0);
        fd.issue_v(smem + FP::VB, j0);
      }
      if (j1 >= 0) fd.issue_k(kbuf(1), j1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    for (int p = 0; p < ncnt; ++p) {
      const int jc = prom_j(p);
      const int key0 = jc * kBk;
      const bool active = jc >= 0 && (!a.causal || key0 <= q0 + 31);
      const bool need_mask = (a.causal && key0 + kBk - 1 > q0) || key0 + kBk > S;
      v8h pB[4];
      bool live = false;
      if (active) {
        v16f sc[2];
        qk_f16p<D>(sc, kbuf(p), qh, lane);
        live = fp16_probs<D>(st, sc, pB, a.sm_log2, key0, qrow, S, a.causal, need_mask, lane);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // V_p in LDS
      if (live) pv_f16p<D>(st, smem + FP::VB, pB, lane);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // V and K[p % 2] free; K_{p+1} in LDS
      const int jn = prom_j(p + 1), jn2 = prom_j(p + 2);
      if (jn >= 0) fd.issue_v(smem + FP::VB, jn);
      if (jn2 >= 0) fd.issue_k(kbuf(p), jn2);
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
    if (a.lse && hi == 0) a.lse[(size_t)bhq * S + qrow] = (st.lu + log2f(lt)) * kLn2;
  }
}

template <int D, int NW, int FMT, bool T8 = false>
static thrift_status launch_attn(const AttnArgs& a, hipStream_t stream) {
  using L = Lds<D>;
  const size_t nwords = (size_t)((a.S + 64 * 32 - 1) / (64 * 32));
  const size_t lds = (size_t)L::PROM + (size_t)a.kmax * 4 + (T8 ? (size_t)a.kmax2 * 4 + nwords * 4 : 0) + nwords * 4;
  static std::atomic<uint64_t> configured{0};
  if (once_per_device(configured, [] {
        return hipFuncSetAttribute((const void*)attn_fwd_kernel<D, NW, FMT, T8>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) == hipSuccess
                   ? THRIFT_OK
                   : THRIFT_EHIP;
      }) != THRIFT_OK)
    return THRIFT_EHIP;
  const int items = a.B * a.Hq * a.nq;
  const int grid = (items + kXcds - 1) / kXcds * kXcds;
  attn_fwd_kernel<D, NW, FMT, T8><<<grid, NW * 64, lds, stream>>>(a);
  return launch_status();
}

// ---- decode-shaped forward: Sq new queries against an Sk-key cache ------------
//
// The new queries are the last Sq positions (causal masks aligned at the
// sequence ends).  One query block holds all of them, so each query head has
// one promoted list.  The G query heads sharing a key head and their Sq rows
// are packed as the query columns of the transposed products (column c =
// g*Sq + r), 32 per column group, so one K/V tile serves 32 columns of the
// group (a workgroup takes one column group; with more than 32 columns the
// key head's K/V are read once per group); the key range is split
// across workgroups and, inside one, across its four waves (each wave its own
// blocks of the shared stages), every wave leaving a partial (m, l, acc)
// per column.  Promoted blocks run in one-wave units of their own (one per
// query head and promoted block) and a last kernel merges all partials of a
// row by their log-sum-exp.  Order does not change the result: codes and
// fp16 roundings of P do not depend on the running maximum.

struct DecodeArgs {
  AttnArgs kv;     // K/V (S = Sk keys), Q pointers with Sq rows, idx/cnt of the one query block
  int Sq, G, nsplit, bpw, nvalid;
  int ncg;         // column groups: ceil(G*Sq / 32)
  float* part4;    // [B*Hkv*nsplit*4][G*Sq][D + 4]: acc[D], m, l, 2 pad
  float* part16;   // [B*Hq*kmax][Sq][D + 4]
};

template <int D>
constexpr int kPartStride = D + 4;  // floats per partial row (16-byte aligned)

constexpr int kDecWaves = 4;

template <int D>
__device__ inline void store_partial(float* dst, const RowState<D>& st, int lane) {
  // dst = this column's partial row; lanes c and c + 32 hold alternate d groups
  const int hi = lane >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = dt * 32 + i4 * 8 + hi * 4;
      *(float4*)(dst + d0) = make_float4(st.acc[dt][i4 * 4 + 0], st.acc[dt][i4 * 4 + 1],
                                         st.acc[dt][i4 * 4 + 2], st.acc[dt][i4 * 4 + 3]);
    }
  const float lt = st.l + xlane32(st.l);
  if (hi == 0) {
    dst[D] = st.lu;
    dst[D + 1] = lt;
  }
}

template <int D>
__device__ inline void decode_fp4_body(const DecodeArgs& d, int unit, char* smem) {
  using M = MxStage<D>;
  constexpr int NT = kDecWaves * 64;
  const AttnArgs& a = d.kv;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), hi = lane >> 5;
  const int sidx = unit % d.nsplit, cg = (unit / d.nsplit) % d.ncg;
  const size_t bhk = unit / d.nsplit / d.ncg;
  const int b = (int)(bhk / a.Hkv), hk = (int)(bhk % a.Hkv);
  const int Sk = a.S, Sq = d.Sq, G = d.G, ncol = G * Sq;
  const int jb = sidx * d.bpw, je = min(jb + d.bpw, d.nvalid);
  const int col = cg * 32 + (lane & 31), g = col / Sq, r = col % Sq;
  const bool col_ok = col < ncol;
  const int hq = hk * G + (col_ok ? g : 0);
  const int qpos = Sk - Sq + r;

  // promoted-block bits of the group's heads: [G][nwords]
  const int nwords = (d.nvalid + 31) >> 5;
  uint32_t* pb = (uint32_t*)(smem + 4 * M::SIZE);
  for (int e = t; e < G * nwords; e += NT) pb[e] = 0;
  __syncthreads();
  for (int e = t; e < G * a.kmax; e += NT) {
    const int gg = e / a.kmax, p = e % a.kmax;
    const size_t row = (size_t)b * a.Hq + hk * G + gg;
    const int c = min(max(a.cnt[row], 0), a.kmax);
    const int j = p < c ? a.idx[row * a.kmax + p] : -1;
    if (j >= 0 && j < d.nvalid) atomicOr(&pb[gg * nwords + (j >> 5)], 1u << (j & 31));
  }

  // this column's FP4 query operand
  v4i qB[D / 64];
  uint32_t qsc = 0x7F7F7F7Fu;
  const size_t qoff = ((size_t)b * a.Hq + hq) * Sq + r;
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk)
    qB[kk] = col_ok ? *(const v4i*)(a.q4c + qoff * (D / 2) + kk * 32 + hi * 16) : v4i{};
  if (col_ok) {
    const uint8_t* pq = a.q4s + qoff * (D / 32);
    qsc = D == 128 ? *(const uint32_t*)pq : (uint32_t)(*(const uint16_t*)pq);
  }
  qsc >>= 8 * hi;

  RowState<D> st;
  init_state<D>(st);

  // Two ring halves of four blocks (two MX stages each); wave w computes
  // block j0 + w of every super-stage.
  MxDma<D, kDecWaves> dma0(a, bhk, d.nvalid, w, lane, t), dma1(a, bhk, d.nvalid, w, lane, t);
  const int nss = je > jb ? cdiv(je - jb, 4) : 0;
  auto half = [&](int k) { return smem + (k & 1) * 2 * M::SIZE; };
  if (nss > 0) {
    dma0.issue(half(0), jb);
    dma1.issue(half(0) + M::SIZE, jb + 2);
    dma0.finish(half(0), t);
    dma1.finish(half(0) + M::SIZE, t);
  }
  __syncthreads();
  MxKOps<D> kop;
  MxVOps<D> vop;
  v16f sc[2];
  for (int k = 0; k < nss; ++k) {
    char* h = half(k);
    const bool more = k + 1 < nss;
    // next super-stage: issue now, store its register part after the compute
    if (more) {
      dma0.issue(half(k + 1), jb + 4 * (k + 1));
      dma1.issue(half(k + 1) + M::SIZE, jb + 4 * (k + 1) + 2);
    }
    const int j = jb + 4 * k + w;
    if (j < je) {
      const char* stg = h + (w >> 1) * M::SIZE;
      const int tb = w & 1;
      load_k_mx<D>(kop, stg, tb, lane);
      qk_mx<D>(sc, kop, qB, qsc);
      const bool prom = col_ok && ((pb[g * nwords + (j >> 5)] >> (j & 31)) & 1u);
      // Columns whose head promotes this block (the FP16 units take it) or
      // that hold no query get probability 0.  Branch-free on purpose: a
      // lane-divergent branch here would let the compiler sink the QK MFMAs
      // into it, and an MFMA under a partial EXEC mask drops the inactive
      // lanes' operands for every column.
      const float lim = (!col_ok || prom) ? -INFINITY : INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[mt][i] = fminf(sc[mt][i], lim);
      const int key0 = j * kBk;
      const bool need_mask = (a.causal && key0 + kBk - 1 > Sk - Sq) || key0 + kBk > Sk;
      load_v_mx<D>(vop, stg, tb, lane);
      softmax_pv_mx<D>(st, sc, vop, a.sm_log2, key0, qpos, Sk, a.causal, need_mask, lane);
    }
    if (more) {
      dma0.finish(half(k + 1), t);
      dma1.finish(half(k + 1) + M::SIZE, t);
    }
    __syncthreads();
  }
  if (col_ok) {
    const size_t u4 = (bhk * d.nsplit + sidx) * kDecWaves + w;
    store_partial<D>(d.part4 + (u4 * ncol + col) * kPartStride<D>, st, lane);
  }
}

// FP4 pass of the decode shape, NVFP4: the same work split as the MXFP4
// kernel (wave w takes blocks jb + w + 4n).  gfx950 has no matrix
// instruction with E4M3 block scales, so each wave dequantises its block
// exactly to fp16 in its own LDS stage (the next block's codes already in
// registers) and runs the NVFP4 tile of the prefill kernel on the fp16
// matrix cores.  Each column's score scale carries its own head's Q slice
// scale.
// Orders this wave's LDS accesses before and after it (its lanes' writes
// before its later reads, its reads before its later writes); no other wave
// takes part.
__device__ inline void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D>
__global__ __launch_bounds__(kDecWaves * 64, 1) void decode_nv4_kernel(DecodeArgs d) {
  using L = Lds<D>;
  constexpr int NT = kDecWaves * 64;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const AttnArgs& a = d.kv;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), hi = lane >> 5;
  const int unit = blockIdx.x, sidx = unit % d.nsplit, cg = (unit / d.nsplit) % d.ncg;
  const size_t bhk = unit / d.nsplit / d.ncg;
  const int b = (int)(bhk / a.Hkv), hk = (int)(bhk % a.Hkv);
  const int Sk = a.S, Sq = d.Sq, G = d.G, ncol = G * Sq;
  const int jb = sidx * d.bpw, je = min(jb + d.bpw, d.nvalid);
  const int col = cg * 32 + (lane & 31), g = col / Sq, r = col % Sq;
  const bool col_ok = col < ncol;
  const int hq = hk * G + (col_ok ? g : 0);
  const int qpos = Sk - Sq + r;
  char* stage = smem + w * L::STAGE;  // this wave's fp16 stage

  // promoted-block bits of the group's heads: [G][nwords]
  const int nwords = (d.nvalid + 31) >> 5;
  uint32_t* pb = (uint32_t*)(smem + kDecWaves * L::STAGE);
  for (int e = t; e < G * nwords; e += NT) pb[e] = 0;
  __syncthreads();
  for (int e = t; e < G * a.kmax; e += NT) {
    const int gg = e / a.kmax, p = e % a.kmax;
    const size_t row = (size_t)b * a.Hq + hk * G + gg;
    const int c = min(max(a.cnt[row], 0), a.kmax);
    const int j = p < c ? a.idx[row * a.kmax + p] : -1;
    if (j >= 0 && j < d.nvalid) atomicOr(&pb[gg * nwords + (j >> 5)], 1u << (j & 31));
  }

  // this column's query, dequantised exactly to fp16, and its score scale
  v8h qh[D / 16];
  const size_t qoff = ((size_t)b * a.Hq + hq) * Sq + r;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qh[kk] = v8h{};
    if (col_ok) {
      const uint32_t cw = *(const uint32_t*)(a.q4c + qoff * (D / 2) + kk * 8 + hi * 4);
      const _Float16 f = (_Float16)e4m3_to_float(a.q4s[qoff * (D / 16) + kk]);
      qh[kk] = fp4x8_to_h(cw, f);
    }
  }
  const float c = a.sm_log2 * a.q4t[(size_t)b * a.Hq + hq] * a.k4t[bhk];
  const float sv = a.v4t[bhk];
  const float lk = log2f(sv) - log2f(2688.0f), ilk = 2688.0f / sv;  // the FP4 tiles' unit factor

  RowState<D> st;
  init_state<D>(st);

  // each wave fills and reads only its own stage, and one wave's LDS
  // operations complete in order, so the waves order their stages with
  // wavefront-scope fences instead of workgroup barriers
  const int nss = je > jb ? cdiv(je - jb, kDecWaves) : 0;
  Nv4Stager<D, 64> stg;
  if (nss > 0 && jb + w < je) {
    stg.load(a, bhk, jb + w, lane);
    stg.store(stage, lane);
  }
  wave_lds_fence();
  for (int k = 0; k < nss; ++k) {
    const int j = jb + kDecWaves * k + w, jn = j + kDecWaves;
    const bool next = k + 1 < nss && jn < je;
    if (next) stg.load(a, bhk, jn, lane);  // registers, while this block is computed
    if (j < je) {
      v16f sc[2];
      qk_f16<D>(sc, stage, qh, lane);
      const bool prom = col_ok && ((pb[g * nwords + (j >> 5)] >> (j & 31)) & 1u);
      // promoted blocks of this column's head and columns without a query:
      // probability 0, branch-free (see the MXFP4 kernel)
      const float lim = (!col_ok || prom) ? -INFINITY : INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[mt][i] = fminf(sc[mt][i], lim);
      const int key0 = j * kBk;
      const bool need_mask = (a.causal && key0 + kBk - 1 > Sk - Sq) || key0 + kBk > Sk;
      fp4_nv_softmax_pv<D>(st, sc, stage, c, lk, ilk, key0, qpos, Sk, a.causal, need_mask, lane);
    }
    wave_lds_fence();
    if (next) stg.store(stage, lane);
    wave_lds_fence();
  }
  if (col_ok) {
    const size_t u4 = (bhk * d.nsplit + sidx) * kDecWaves + w;
    store_partial<D>(d.part4 + (u4 * ncol + col) * kPartStride<D>, st, lane);
  }
}

// One FP16 unit per wave: (batch, query head, promoted slot) `unit`, V^T
// staged in this wave's LDS slice vt_smem.  Every wave of the workgroup
// passes the one barrier, also with no unit (unit < 0 or past cnt).
template <int D>
__device__ inline void decode_f16_body(const DecodeArgs& d, int unit, char* vt_smem) {
  const AttnArgs& a = d.kv;
  const int lane = threadIdx.x & 63, hi = lane >> 5;
  const int p = unit >= 0 ? unit % a.kmax : 0;
  const size_t bhq = unit >= 0 ? unit / a.kmax : 0;
  const int ncnt = unit >= 0 ? min(max(a.cnt[bhq], 0), a.kmax) : 0;
  const bool live = p < ncnt;  // the merge reads units p < cnt only
  const int b = (int)(bhq / a.Hq), hq = (int)(bhq % a.Hq);
  const size_t bhk = (size_t)b * a.Hkv + hq / d.G;
  const int Sk = a.S, Sq = d.Sq;
  const int col = lane & 31, r = col < Sq ? col : 0;
  const int qpos = Sk - Sq + r;
  const int j = live ? a.idx[bhq * a.kmax + p] : -1;
  const bool act = j >= 0 && j < d.nvalid;

  RowState<D> st;
  init_state<D>(st);
  using L = Lds<D>;
  _Float16* vt = (_Float16*)vt_smem;  // V^T: D rows of VROWH halves
  v8h qh[D / 16], ka[2][D / 16];
  if (act) {
    // Every load goes out first: the query rows; K in MFMA operand order
    // (the rows krow(mt, r32), 16-byte chunks straight into registers, no
    // LDS); V as (key pair, 8 channels) items, transposed into LDS below.
    // Rows past the cache's end read as zeros through the buffer resources'
    // record counts (their scores are masked).
    constexpr int w3 = 0x00020000;  // raw buffer, 32-bit data format
    const int r32 = lane & 31;
    const auto krs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.k16 + bhk * Sk * D), 0, Sk * D * 2, w3);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.v16 + bhk * Sk * D), 0, Sk * D * 2, w3);
    const size_t qoff = (bhq * Sq + r) * D + hi * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qh[kk] = col < Sq ? *(const v8h*)(a.q16 + qoff + kk * 16) : v8h{};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        ka[mt][kk] = __builtin_bit_cast(
            v8h, __builtin_amdgcn_raw_buffer_load_b128(krs, ((j * kBk + krow(mt, r32)) * D + kk * 16 + hi * 8) * 2, 0, 0));
    constexpr int PV = (kBk / 2) * (D / 8) / 64;
    v4i v0[PV], v1[PV];
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      const int c = lane + p * 64, kp = c % (kBk / 2), cv = (c / (kBk / 2)) * 8, key = j * kBk + 2 * kp;
      v0[p] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(vrs, (key * D + cv) * 2, 0, 0));
      v1[p] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(vrs, ((key + 1) * D + cv) * 2, 0, 0));
    }
#pragma unroll
    for (int p = 0; p < PV; ++p) {
      const int c = lane + p * 64, kp = c % (kBk / 2), cv = (c / (kBk / 2)) * 8;
      uint32_t* dst = (uint32_t*)(vt + cv * L::VROWH + 2 * kp);
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // channels 2w, 2w+1: (key, key+1) half pairs
        dst[(2 * w) * (L::VROWH / 2)] = __builtin_amdgcn_perm((uint32_t)v1[p][w], (uint32_t)v0[p][w], 0x05040100u);
        dst[(2 * w + 1) * (L::VROWH / 2)] = __builtin_amdgcn_perm((uint32_t)v1[p][w], (uint32_t)v0[p][w], 0x07060302u);
      }
    }
  }
  __syncthreads();
  if (act) {
    v16f sc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sc[mt] = v16f{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) sc[mt] = mfma_f16(ka[mt][kk], qh[kk], sc[mt]);
    }
    const int key0 = j * kBk;
    const bool need_mask = (a.causal && key0 + kBk - 1 > Sk - Sq) || key0 + kBk > Sk;
    fp16_softmax_pv<D>(st, sc, vt, a.sm_log2, key0, qpos, Sk, a.causal, need_mask, lane);
  }
  if (live && col < Sq) store_partial<D>(d.part16 + ((bhq * a.kmax + p) * Sq + col) * kPartStride<D>, st, lane);
}

template <int D>
__global__ __launch_bounds__(64) void decode_f16_kernel(DecodeArgs d) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  decode_f16_body<D>(d, blockIdx.x, smem);
}

// MXFP4 decode forward in one launch: the first n4wg workgroups are the FP4
// splits (the long chains, so they start first); the rest hold four FP16
// units each, one per wave, and fill the compute units as the splits drain
// instead of waiting for the last of them.  Units past n16 do nothing.
template <int D>
__global__ __launch_bounds__(kDecWaves * 64, 2) void decode_mx_fused_kernel(DecodeArgs d, int n4wg, int n16) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int x = blockIdx.x;
  if (x < n4wg) {
    decode_fp4_body<D>(d, x, smem);
    return;
  }
  const int w = threadIdx.x >> 6, unit = (x - n4wg) * kDecWaves + w;
  decode_f16_body<D>(d, unit < n16 ? unit : -1, smem + w * (D * Lds<D>::VROWH * 2));
}

constexpr int kMergeThreads = 256;

// O and LSE of one (batch, query head, row) from every partial that holds it:
// one workgroup per row.  Thread t takes float4 column t % (D/4) of the
// partials u = t / (D/4), + 256/(D/4), ...; loads of several partials are in
// flight at once, and the per-group sums meet in LDS.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs d) {
  constexpr int C4 = D / 4, PG = kMergeThreads / C4, NW = kMergeThreads / 64;
  __shared__ float red_m[NW];
  __shared__ __attribute__((aligned(16))) float red_acc[PG][D];
  __shared__ float red_l[PG];
  const AttnArgs& a = d.kv;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const size_t row = blockIdx.x;  // (b*Hq + hq)*Sq + r
  const int r = (int)(row % d.Sq);
  const size_t bhq = row / d.Sq;
  const int b = (int)(bhq / a.Hq), hq = (int)(bhq % a.Hq);
  const size_t bhk = (size_t)b * a.Hkv + hq / d.G;
  const int ncol = d.G * d.Sq, col = (hq % d.G) * d.Sq + r;
  const int n4 = d.nsplit * kDecWaves;
  const int n = n4 + min(max(a.cnt[bhq], 0), a.kmax);
  auto part = [&](int u) -> const float* {
    return u < n4 ? d.part4 + ((bhk * n4 + u) * ncol + col) * kPartStride<D>
                  : d.part16 + ((bhq * a.kmax + (u - n4)) * d.Sq + r) * kPartStride<D>;
  };
  float M = kMInit;
  for (int u = t; u < n; u += kMergeThreads) M = fmaxf(M, part(u)[D]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (lane == 0) red_m[w] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) M = fmaxf(M, red_m[i]);

  const int c4 = t % C4, pg = t / C4;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float l = 0.0f;
#pragma unroll 4
  for (int u = pg; u < n; u += PG) {
    const float* q = part(u);
    const float2 ml = *(const float2*)(q + D);
    const float4 x = *(const float4*)(q + 4 * c4);
    const float f = exp2f(ml.x - M);  // the partial's unit relative to the largest
    l += f * ml.y;
    acc.x += f * x.x;
    acc.y += f * x.y;
    acc.z += f * x.z;
    acc.w += f * x.w;
  }
  *(float4*)&red_acc[pg][4 * c4] = acc;
  if (c4 == 0) red_l[pg] = l;
  __syncthreads();
  if (t < D) {
    float o = 0.0f, lt = 0.0f;
#pragma unroll
    for (int g = 0; g < PG; ++g) {
      o += red_acc[g][t];
      lt += red_l[g];
    }
    const float x = o / lt;
    if (a.o_fp32)
      ((float*)a.o)[row * D + t] = x;
    else
      ((_Float16*)a.o)[row * D + t] = (_Float16)x;
    if (a.lse && t == 0) a.lse[row] = (M + log2f(lt)) * kLn2;
  }
}

// Work split: about two workgroups per compute unit, at least one block per
// wave, a multiple of four blocks per workgroup.
inline void decode_split(int B, int Hkv, int nvalid, int& nsplit, int& bpw) {
  int want = cdiv(512, B * Hkv);
  want = want < 1 ? 1 : want;
  const int most = cdiv(nvalid, kDecWaves);
  want = want > most ? most : want;
  bpw = cdiv(cdiv(nvalid, want), kDecWaves) * kDecWaves;
  nsplit = cdiv(nvalid, bpw);
}

// Every kernel the entry points launch, instantiated explicitly (the host
// compiler does not always emit the launch stubs of templates used only
// through launch helpers).
template __global__ void attn_fwd_kernel<128, 4, THRIFT_MXFP4>(AttnArgs);
template __global__ void attn_fwd_kernel<128, 2, THRIFT_MXFP4>(AttnArgs);
template __global__ void attn_fwd_kernel<64, 4, THRIFT_MXFP4>(AttnArgs);
template __global__ void attn_fwd_kernel<64, 2, THRIFT_MXFP4>(AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, THRIFT_NVFP4>(AttnArgs);
template __global__ void attn_fwd_kernel<128, 2, THRIFT_NVFP4>(AttnArgs);
template __global__ void attn_fwd_kernel<64, 4, THRIFT_NVFP4>(AttnArgs);
template __global__ void attn_fwd_kernel<64, 2, THRIFT_NVFP4>(AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, THRIFT_NVFP4_MXP>(AttnArgs);
template __global__ void attn_fwd_kernel<128, 2, THRIFT_NVFP4_MXP>(AttnArgs);
template __global__ void attn_fwd_kernel<64, 4, THRIFT_NVFP4_MXP>(AttnArgs);
template __global__ void attn_fwd_kernel<64, 2, THRIFT_NVFP4_MXP>(AttnArgs);
template __global__ void attn_fwd_kernel<128, 4, THRIFT_MXFP4, true>(AttnArgs);
template __global__ void attn_fwd_kernel<128, 2, THRIFT_MXFP4, true>(AttnArgs);
template __global__ void attn_fwd_kernel<64, 4, THRIFT_MXFP4, true>(AttnArgs);
template __global__ void attn_fwd_kernel<64, 2, THRIFT_MXFP4, true>(AttnArgs);
template __global__ void decode_mx_fused_kernel<128>(DecodeArgs, int, int);
template __global__ void decode_mx_fused_kernel<64>(DecodeArgs, int, int);
template __global__ void decode_nv4_kernel<128>(DecodeArgs);
template __global__ void decode_nv4_kernel<64>(DecodeArgs);
template __global__ void decode_f16_kernel<128>(DecodeArgs);
template __global__ void decode_f16_kernel<64>(DecodeArgs);
template __global__ void decode_merge_kernel<128>(DecodeArgs);
template __global__ void decode_merge_kernel<64>(DecodeArgs);

}  // namespace thrift

using namespace thrift;

static thrift_status make_attn_args(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes,
    const uint8_t* q4_scales, const float* q4_tscale, const uint8_t* k4_codes,
    const uint8_t* k4_scales, const float* k4_tscale, const uint8_t* v4_codes,
    const uint8_t* v4_scales, const float* v4_tscale, int fmt, const int32_t* idx,
    const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D, int block_q, int block_k,
    int causal, float sm_scale, void* o, int o_is_fp32, float* lse, AttnArgs& a) {
  if (!q4_codes || !q4_scales || !k4_codes || !k4_scales || !v4_codes || !v4_scales || !idx ||
      !cnt || !o)
    return THRIFT_EINVAL;
  if (fmt != THRIFT_NVFP4 && fmt != THRIFT_MXFP4 && fmt != THRIFT_NVFP4_MXP) return THRIFT_EINVAL;
  if (fmt != THRIFT_MXFP4 && (!q4_tscale || !k4_tscale || !v4_tscale)) return THRIFT_EINVAL;
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
  a = AttnArgs{};
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
  return THRIFT_OK;
}

extern "C" thrift_status thrift_attention_fwd(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes,
    const uint8_t* q4_scales, const float* q4_tscale, const uint8_t* k4_codes,
    const uint8_t* k4_scales, const float* k4_tscale, const uint8_t* v4_codes,
    const uint8_t* v4_scales, const float* v4_tscale, int fmt, const int32_t* idx,
    const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D, int block_q, int block_k,
    int causal, float sm_scale, void* o, int o_is_fp32, float* lse, hipStream_t stream) {
  AttnArgs a;
  const thrift_status st = make_attn_args(q16, k16, v16, q4_codes, q4_scales, q4_tscale, k4_codes, k4_scales,
                                          k4_tscale, v4_codes, v4_scales, v4_tscale, fmt, idx, cnt, kmax, B, Hq,
                                          Hkv, S, D, block_q, block_k, causal, sm_scale, o, o_is_fp32, lse, a);
  if (st != THRIFT_OK) return st;
  if (fmt == THRIFT_MXFP4) {
    if (D == 128) return block_q == 128 ? launch_attn<128, 4, THRIFT_MXFP4>(a, stream) : launch_attn<128, 2, THRIFT_MXFP4>(a, stream);
    return block_q == 128 ? launch_attn<64, 4, THRIFT_MXFP4>(a, stream) : launch_attn<64, 2, THRIFT_MXFP4>(a, stream);
  }
  if (fmt == THRIFT_NVFP4_MXP) {
    if (D == 128) return block_q == 128 ? launch_attn<128, 4, THRIFT_NVFP4_MXP>(a, stream) : launch_attn<128, 2, THRIFT_NVFP4_MXP>(a, stream);
    return block_q == 128 ? launch_attn<64, 4, THRIFT_NVFP4_MXP>(a, stream) : launch_attn<64, 2, THRIFT_NVFP4_MXP>(a, stream);
  }
  if (D == 128) return block_q == 128 ? launch_attn<128, 4, THRIFT_NVFP4>(a, stream) : launch_attn<128, 2, THRIFT_NVFP4>(a, stream);
  return block_q == 128 ? launch_attn<64, 4, THRIFT_NVFP4>(a, stream) : launch_attn<64, 2, THRIFT_NVFP4>(a, stream);
}

extern "C" thrift_status thrift_attention_fwd_tiered(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes, const uint8_t* q4_scales,
    const uint8_t* k4_codes, const uint8_t* k4_scales, const uint8_t* v4_codes, const uint8_t* v4_scales,
    const uint8_t* q8_codes, const uint8_t* q8_scales, const uint8_t* k8_codes, const uint8_t* k8_scales,
    const uint8_t* v8_codes, const uint8_t* v8_scales, const int32_t* idx, const int32_t* cnt, int kmax,
    const int32_t* idx2, const int32_t* cnt2, int kmax2, int B, int Hq, int Hkv, int S, int D, int block_q,
    int block_k, int causal, float sm_scale, void* o, int o_is_fp32, float* lse, hipStream_t stream) {
  if (!q8_codes || !q8_scales || !k8_codes || !k8_scales || !v8_codes || !v8_scales || !idx2 || !cnt2)
    return THRIFT_EINVAL;
  if (kmax2 < 1) return THRIFT_EINVAL;
  AttnArgs a;
  const thrift_status st = make_attn_args(q16, k16, v16, q4_codes, q4_scales, nullptr, k4_codes, k4_scales,
                                          nullptr, v4_codes, v4_scales, nullptr, THRIFT_MXFP4, idx, cnt, kmax, B,
                                          Hq, Hkv, S, D, block_q, block_k, causal, sm_scale, o, o_is_fp32, lse, a);
  if (st != THRIFT_OK) return st;
  if (kmax2 > cdiv(S, block_k)) return THRIFT_EUNSUPPORTED;
  for (const void* p : {(const void*)q8_codes, (const void*)k8_codes, (const void*)v8_codes})
    if (!aligned16(p)) return THRIFT_EALIGN;
  if (((uintptr_t)q8_scales | (uintptr_t)k8_scales | (uintptr_t)v8_scales) & 3) return THRIFT_EALIGN;
  a.q8c = q8_codes;
  a.q8s = q8_scales;
  a.k8c = k8_codes;
  a.k8s = k8_scales;
  a.v8c = v8_codes;
  a.v8s = v8_scales;
  a.idx2 = idx2;
  a.cnt2 = cnt2;
  a.kmax2 = kmax2;
  if (D == 128)
    return block_q == 128 ? launch_attn<128, 4, THRIFT_MXFP4, true>(a, stream)
                          : launch_attn<128, 2, THRIFT_MXFP4, true>(a, stream);
  return block_q == 128 ? launch_attn<64, 4, THRIFT_MXFP4, true>(a, stream)
                        : launch_attn<64, 2, THRIFT_MXFP4, true>(a, stream);
}

static size_t decode_part_floats(int B, int Hq, int Hkv, int Sq, int Sk, int D, int kmax,
                                 size_t* n4_out) {
  int nsplit, bpw;
  decode_split(B, Hkv, cdiv(Sk, 64), nsplit, bpw);
  const size_t stride = (size_t)D + 4;
  const size_t n4 = (size_t)B * Hkv * nsplit * kDecWaves * (Hq / Hkv) * Sq * stride;
  const size_t n16 = (size_t)B * Hq * kmax * Sq * stride;
  if (n4_out) *n4_out = n4;
  return n4 + n16;
}

extern "C" size_t thrift_attention_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                                          int kmax) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq < 1 || Sk < Sq || D < 1 || kmax < 1) return 0;
  return decode_part_floats(B, Hq, Hkv, Sq, Sk, D, kmax, nullptr) * sizeof(float);
}

template <int D>
static thrift_status launch_decode(DecodeArgs& d, int fmt, hipStream_t stream) {
  using M = MxStage<D>;
  const AttnArgs& a = d.kv;
  static std::atomic<uint64_t> configured{0};
  if (once_per_device(configured, [] {
        for (const void* kf : {(const void*)decode_mx_fused_kernel<D>, (const void*)decode_nv4_kernel<D>,
                               (const void*)decode_f16_kernel<D>})
          if (hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024) != hipSuccess)
            return THRIFT_EHIP;
        return THRIFT_OK;
      }) != THRIFT_OK)
    return THRIFT_EHIP;
  // the split kernels' LDS: their stages and the group's promoted-bit table
  // (G words per 32 key blocks); shapes it does not fit launch nothing
  const size_t pbytes = (size_t)d.G * ((d.nvalid + 31) / 32) * 4;
  const size_t lsplit = (fmt == THRIFT_MXFP4 ? 4 * (size_t)M::SIZE : kDecWaves * (size_t)Lds<D>::STAGE) + pbytes;
  if (lsplit > 160 * 1024) return THRIFT_EUNSUPPORTED;
  const int n4wg = a.B * a.Hkv * d.ncg * d.nsplit, n16 = a.B * a.Hq * a.kmax;
  if (fmt == THRIFT_MXFP4) {
    const size_t l4 = 4 * (size_t)M::SIZE + pbytes, l16 = (size_t)kDecWaves * D * Lds<D>::VROWH * 2;
    const size_t lds = l4 > l16 ? l4 : l16;
    decode_mx_fused_kernel<D><<<n4wg + cdiv(n16, kDecWaves), kDecWaves * 64, lds, stream>>>(d, n4wg, n16);
  } else {
    decode_nv4_kernel<D><<<n4wg, kDecWaves * 64, kDecWaves * (size_t)Lds<D>::STAGE + pbytes, stream>>>(d);
    decode_f16_kernel<D><<<n16, 64, D * Lds<D>::VROWH * 2, stream>>>(d);
  }
  decode_merge_kernel<D><<<a.B * a.Hq * d.Sq, kMergeThreads, 0, stream>>>(d);
  return launch_status();
}

extern "C" thrift_status thrift_attention_decode(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes,
    const uint8_t* q4_scales, const float* q4_tscale, const uint8_t* k4_codes,
    const uint8_t* k4_scales, const float* k4_tscale, const uint8_t* v4_codes,
    const uint8_t* v4_scales, const float* v4_tscale, int fmt, const int32_t* idx,
    const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int Sq, int Sk, int D, int block_k,
    int causal, float sm_scale, void* o, int o_is_fp32, float* lse, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  if (!q16 || !k16 || !v16 || !q4_codes || !q4_scales || !k4_codes || !k4_scales || !v4_codes ||
      !v4_scales || !idx || !cnt || !o || !workspace)
    return THRIFT_EINVAL;
  if (fmt != THRIFT_NVFP4 && fmt != THRIFT_MXFP4) return THRIFT_EINVAL;
  if (fmt == THRIFT_NVFP4 && (!q4_tscale || !k4_tscale || !v4_tscale)) return THRIFT_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < Sq || kmax < 1 || (causal != 0 && causal != 1))
    return THRIFT_EINVAL;
  if (Hq % Hkv != 0 || (o_is_fp32 != 0 && o_is_fp32 != 1)) return THRIFT_EINVAL;
  if (!(sm_scale > 0.0f) || !(sm_scale < 1e30f)) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if (block_k != 64 || Sq > 32 || (Hq / Hkv) * Sq > 128) return THRIFT_EUNSUPPORTED;
  if (Sk > 262144 || kmax > cdiv(Sk, block_k)) return THRIFT_EUNSUPPORTED;
  for (const void* p : {q16, k16, v16, (const void*)q4_codes, (const void*)k4_codes,
                        (const void*)v4_codes, (const void*)o, (const void*)workspace})
    if (!aligned16(p)) return THRIFT_EALIGN;
  if (((uintptr_t)q4_scales | (uintptr_t)k4_scales | (uintptr_t)v4_scales) & 3) return THRIFT_EALIGN;
  size_t n4 = 0;
  const size_t need = decode_part_floats(B, Hq, Hkv, Sq, Sk, D, kmax, &n4) * sizeof(float);
  if (workspace_bytes < need) return THRIFT_EWORKSPACE;
  DecodeArgs d;
  AttnArgs& a = d.kv;
  a.q16 = (const _Float16*)q16;
  a.k16 = (const _Float16*)k16;
  a.v16 = (const _Float16*)v16;
  a.q4c = q4_codes;
  a.q4s = q4_scales;
  a.q4t = fmt == THRIFT_NVFP4 ? q4_tscale : nullptr;
  a.k4c = k4_codes;
  a.k4s = k4_scales;
  a.k4t = fmt == THRIFT_NVFP4 ? k4_tscale : nullptr;
  a.v4c = v4_codes;
  a.v4s = v4_scales;
  a.v4t = fmt == THRIFT_NVFP4 ? v4_tscale : nullptr;
  a.idx = idx;
  a.cnt = cnt;
  a.o = o;
  a.lse = lse;
  a.kmax = kmax;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.S = Sk;
  a.Sp = cdiv(Sk, 64) * 64;
  a.nq = 1;
  a.causal = causal;
  a.o_fp32 = o_is_fp32;
  a.sm_log2 = sm_scale * 1.4426950408889634f;
  d.Sq = Sq;
  d.G = Hq / Hkv;
  d.ncg = cdiv(d.G * Sq, 32);
  d.nvalid = valid_kv_blocks_kv(0, Sq, Sk, 128, 64, causal);
  decode_split(B, Hkv, d.nvalid, d.nsplit, d.bpw);
  d.part4 = (float*)workspace;
  d.part16 = (float*)workspace + n4;
  return D == 128 ? launch_decode<128>(d, fmt, stream) : launch_decode<64>(d, fmt, stream);
}

// ---- decode without allocation --------------------------------------------------
//
// The split partials of thrift_attention_decode_noalloc live in a file-scope
// device array instead of a caller workspace: THRIFT_DECODE_SCRATCH_BYTES per
// GPU, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress once per device, with that device
// current, and is kept per device.  Every call on one GPU shares the array;
// nothing in it has to start at zero (each partial the merge reads is written
// by the same call first), and calls that overlap on one GPU race.
static __device__ __align__(256) float scratch[THRIFT_DECODE_SCRATCH_BYTES / sizeof(float)];
static float* scratch_ptr[64];
static std::atomic<uint64_t> scratch_ready{0};

extern "C" thrift_status thrift_attention_decode_noalloc(
    const void* q16, const void* k16, const void* v16, const uint8_t* q4_codes,
    const uint8_t* q4_scales, const float* q4_tscale, const uint8_t* k4_codes,
    const uint8_t* k4_scales, const float* k4_tscale, const uint8_t* v4_codes,
    const uint8_t* v4_scales, const float* v4_tscale, int fmt, const int32_t* idx,
    const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int Sq, int Sk, int D, int block_k,
    int causal, float sm_scale, void* o, int o_is_fp32, float* lse, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return THRIFT_EHIP;
  if (once_per_device(scratch_ready, [dev] {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return THRIFT_EHIP;
        scratch_ptr[dev] = (float*)ptr;
        return THRIFT_OK;
      }) != THRIFT_OK)
    return THRIFT_EHIP;
  if (B >= 1 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && Sq >= 1 && Sk >= Sq && D >= 1 && kmax >= 1 &&
      thrift_attention_decode_workspace_bytes(B, Hq, Hkv, Sq, Sk, D, kmax) > THRIFT_DECODE_SCRATCH_BYTES)
    return THRIFT_EWORKSPACE;
  return thrift_attention_decode(q16, k16, v16, q4_codes, q4_scales, q4_tscale, k4_codes, k4_scales, k4_tscale,
                                 v4_codes, v4_scales, v4_tscale, fmt, idx, cnt, kmax, B, Hq, Hkv, Sq, Sk, D,
                                 block_k, causal, sm_scale, o, o_is_fp32, lse, scratch_ptr[dev],
                                 THRIFT_DECODE_SCRATCH_BYTES, stream);
}

extern "C" const char* thrift_status_string(int s) {
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
