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
// or dQ, and the key kernel (one lane per key) computes dV in one launch and
// dK in another.  Every kernel streams its operand tiles into LDS by direct
// loads one step ahead and reads the transposed operands of its second
// product from those row tiles (ds_read_b64_tr_b16).
#include <hip/hip_runtime.h>

#include "common.h"

namespace thrift {
namespace {

constexpr int kBlkK = 64;  // key block
constexpr int kMaxS = 262144;
constexpr int kMaxKw = kMaxS / kBlkK / 32;  // promoted-bit words per query block row
constexpr float kLog2eB = 1.44269504088896341f;
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt at their maxima), as an instruction
// the compiler's wait insertion sees (an inline-asm wait it cannot read)
constexpr int kWaitVm0 = 0x0F70;

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
  const _Float16* qds;                     // FP4-decoded Q times its slice scale (NVFP4) [B,Hq,S,D]
  const _Float16* vd;                      // FP4-decoded V rows [B,Hkv,Sp,D]
  const uint32_t* prom;                    // promoted-block bits [B,Hq,nq,nkw]
  const float *lse, *drow, *lse2;          // [B,Hq,S]; lse2 = lse * log2(e)
  const float *tq, *tk, *tv;               // NVFP4 slice scales [B,H] (NULL for MXFP4)
  float* out;                              // row kernel: O' or dQ [B,Hq,S,D]
  float *dk, *dv;                          // [B,Hkv,S,D]
  int B, Hq, Hkv, S, Sp, bq, nq, nkw, causal;
  float c;         // sm_scale * log2(e)
  float sm_scale;
};

// ---- preparation ------------------------------------------------------------------
//
// One launch fills every operand the backward kernels read.  Its workgroups
// take, in blockIdx order, these roles:
//   V    one per (batch*head, 64-key block): the block's stored V^T codes
//        (key-block-major) decoded and written as 64 rows of D channels
//        through an LDS tile, so no transposed copy is written;
//   Q, K FP4 rows decoded to fp16 rows, one thread per 8 elements;
//   QS   (NVFP4 backward) the decoded Q rows times Q's slice scale;
//   RT   (backward) the row term dO[r] . O'[r] and the LSE in log2 units;
//   PB   the promoted-block bits of each (batch, query head, query block).
// E2M1 times a power of two (MX) or times an E4M3 value (NVFP4, at most 6
// significant bits, 2^-10 .. 2688) is exact in fp16; a slice scale
// multiplies in before the one rounding.

struct PrepArgs {
  const uint8_t *q4c, *q4s, *k4c, *k4s, *v4c, *v4s;
  const float* tq;  // NVFP4 slice scales of Q (QS role)
  const int32_t *idx, *cnt;
  const _Float16* do16;
  const float *ohp, *lse;
  _Float16 *qd, *kd, *vd, *qds;
  uint32_t* prom;
  float *drow, *lse2;
  int fmt, S, nk, kmax, nkw;
  size_t rq, rk, nrows_rt;  // rows of Q, of K, and of the row term
  int nrows_pb;
  // first workgroup of each role (V starts at 0); end is the grid size
  unsigned wq, wk, wqs, wrt, wpb, wend;
};

// 8 FP4 elements of a row of L (codes [R][L/2], block scales [R][L/g]) at
// element c8, times f0 (the slice scale, or 1), to fp16.
__device__ inline v8h decode8(const uint8_t* codes, const uint8_t* scales, size_t row, int L, int c8, int fmt,
                              float f0) {
  const uint32_t cw = *(const uint32_t*)(codes + row * (L / 2) + c8 / 2);
  const int g = fmt == THRIFT_MXFP4 ? 32 : 16;
  const uint32_t sb = scales[row * (L / g) + c8 / g];
  float f = fmt == THRIFT_MXFP4 ? ldexpf(1.0f, (int)sb - 127) : e4m3_to_float(sb);
  f *= f0;
  const v2f v[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0),
                    __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1),
                    __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2),
                    __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3)};
  v8h o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (_Float16)(v[e / 2][e % 2] * f);
  return o;
}

// Rows [0, R) of L = D elements: thread e8 decodes elements 8*(e8 % (D/8))..
// of row e8 / (D/8); tsc (or NULL) holds one slice scale per S rows.
template <int D>
__device__ inline void decode_rows(const uint8_t* codes, const uint8_t* scales, size_t R, int fmt, const float* tsc,
                                   int S, _Float16* out, size_t e8) {
  if (e8 >= R * (size_t)(D / 8)) return;
  const size_t row = e8 / (D / 8);
  const int c8 = (int)(e8 % (D / 8)) * 8;
  const float f0 = tsc ? tsc[row / (size_t)S] : 1.0f;
  *(v8h*)(out + row * D + c8) = decode8(codes, scales, row, D, c8, fmt, f0);
}

template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(PrepArgs a) {
  const unsigned wg = blockIdx.x;
  const int t = threadIdx.x;
  if (wg < a.wq) {
    // V: stored block blk = bh * nk + j holds, per channel d, the codes of
    // its 64 keys (32 bytes) and their block scales.  Thread (dp, kq)
    // decodes channels 2dp and 2dp+1 of keys kq*KPG .. kq*KPG+KPG-1 and
    // writes each key's channel pair as one word of the LDS tile [key][d]
    // (a wave's lanes cover every bank once); the tile then goes out as
    // rows, 16 bytes per thread and step.
    constexpr int NP = D / 2, KPG = 64 / (256 / NP);  // channel pairs; keys per thread (16 or 8)
    constexpr int RS = D + 8;                         // tile row stride in halves
    __shared__ __attribute__((aligned(16))) _Float16 tile[64 * RS];
    const size_t blk = wg;
    const int j = (int)(blk % (size_t)a.nk);
    const size_t bh = blk / (size_t)a.nk;
    const int dp = t % NP, kq = t / NP;
    v8h h[2][KPG / 8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < KPG / 8; ++q) h[u][q] = decode8(a.v4c, a.v4s, blk * D + 2 * dp + u, 64, kq * KPG + q * 8, a.fmt, 1.0f);
#pragma unroll
    for (int e = 0; e < KPG; ++e) {
      const v2h pr = {h[0][e / 8][e % 8], h[1][e / 8][e % 8]};
      *(v2h*)(tile + (kq * KPG + e) * RS + 2 * dp) = pr;
    }
    __syncthreads();
    _Float16* dst = a.vd + (bh * (size_t)a.nk + (size_t)j) * 64 * D;
#pragma unroll
    for (int it = 0; it < (64 * D / 8) / 256; ++it) {
      const int c = t + it * 256, r = c / (D / 8), c8 = (c % (D / 8)) * 8;
      *(v8h*)(dst + (size_t)r * D + c8) = *(const v8h*)(tile + r * RS + c8);
    }
    return;
  }
  // the other roles: element e of the role's range
  const unsigned w0 = wg < a.wk ? a.wq : wg < a.wqs ? a.wk : wg < a.wrt ? a.wqs : wg < a.wpb ? a.wrt : a.wpb;
  const size_t e = (size_t)(wg - w0) * 256 + t;
  if (wg < a.wk) {
    decode_rows<D>(a.q4c, a.q4s, a.rq, a.fmt, nullptr, a.S, a.qd, e);
  } else if (wg < a.wqs) {
    decode_rows<D>(a.k4c, a.k4s, a.rk, a.fmt, nullptr, a.S, a.kd, e);
  } else if (wg < a.wrt) {
    decode_rows<D>(a.q4c, a.q4s, a.rq, a.fmt, a.tq, a.S, a.qds, e);
  } else if (wg < a.wpb) {
    // row term: D/8 lanes per row (a 16-byte load of dO and two of O'
    // each), summed across those lanes; every lane reaches the shuffles
    constexpr int LPR = D / 8;  // 16 or 8, a divisor of the wave
    const size_t row = e / LPR;
    const int sub = t % LPR;
    float s = 0.0f;
    if (row < a.nrows_rt) {
      const v8h h = *(const v8h*)(a.do16 + row * D + sub * 8);
      const float4 x = *(const float4*)(a.ohp + row * D + sub * 8),
                   y = *(const float4*)(a.ohp + row * D + sub * 8 + 4);
      s = (float)h[0] * x.x + (float)h[1] * x.y + (float)h[2] * x.z + (float)h[3] * x.w + (float)h[4] * y.x +
          (float)h[5] * y.y + (float)h[6] * y.z + (float)h[7] * y.w;
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
    if (row < a.nrows_rt && sub == 0) {
      a.drow[row] = s;
      a.lse2[row] = a.lse[row] * kLog2eB;
    }
  } else {
    const size_t row = e;
    if (row >= (size_t)a.nrows_pb) return;
    uint32_t* w = a.prom + row * a.nkw;
    for (int k = 0; k < a.nkw; ++k) w[k] = 0;
    const int n = min(max(a.cnt[row], 0), a.kmax);
    for (int s = 0; s < n; ++s) {
      const int jj = a.idx[row * a.kmax + s];
      if (jj >= 0 && jj < a.nk) w[jj >> 5] |= 1u << (jj & 31);
    }
  }
}

// ---- row kernel: one lane per query (O' or dQ) ---------------------------------

__device__ inline __attribute__((address_space(3))) void* lds_ptr(char* p) {
  return (__attribute__((address_space(3))) void*)p;
}

// Eight halves of a transposed operand: ds_read_b64_tr_b16 at tile + o0 and
// tile + o1 (elements 0-3 and 4-7).
__device__ inline v8h tr_read(const char* tile, uint32_t o0, uint32_t o1) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4s* lp;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(tile + o0));
  const v4s up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(tile + o1));
  return __builtin_bit_cast(v8h, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}


constexpr int kModeOhp = 0;
constexpr int kModeDq = 1;

// Row kernel LDS: two stages of one key block each (the next block's K and
// V rows arrive by direct loads while a block is computed).  Each tile holds
// the block's 64 key rows in krow order (slot mt*32 + m holds key
// krow(mt, m)), chunk-column-major: 16-byte chunk c of slot r at
// c * 1088 + r * 16, one direct wave load per chunk column.  The 64-byte
// stagger per column keeps both reads free of bank conflicts: the rows as
// the A operand of S^T = K Q^T and dP^T = V dO^T (16 slots of one chunk per
// half-wave) and the transposed reads of the K^T and V^T operands
// (ds_read_b64_tr_b16: per 16 lanes, 4 keys of 16 channels).
template <int D>
struct RowStage {
  static constexpr int CS = 1024 + 64;
  static constexpr int TILE = (D / 8) * CS;
  static constexpr int K = 0;
  static constexpr int V = TILE;
  static constexpr int SIZE = 2 * TILE;
};

// Slot of key k (0..63) in krow order.
__device__ constexpr int kslot_of(int k) {
  return ((k >> 4) & 1) * 32 + ((k >> 2) & 3) * 8 + ((k >> 5) & 1) * 4 + (k & 3);
}

// One key block's K and V rows into a row-kernel stage: wave w loads chunk
// columns w, w + NW, ... of each tile (lane l: the row of slot l, source
// byte offset o plus the column's 16 bytes).
template <int D, int NW>
__device__ inline void row_issue(char* buf, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs, uint32_t o,
                                 int w) {
  using R = RowStage<D>;
#pragma unroll
  for (int k = 0; k < (D / 8) / NW; ++k) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, lds_ptr(buf + R::K + (w + k * NW) * R::CS), 16, o + k * NW * 16, 0,
                                             0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, lds_ptr(buf + R::V + (w + k * NW) * R::CS), 16, o + k * NW * 16, 0,
                                             0, 0);
  }
}

// Workgroup = query block i of (batch, query head), one wave per 32 rows,
// one lane per query.  The valid key blocks run FP4 blocks first, then the
// promoted ones, each ascending.  Per block, in the precision of its path:
// S^T = K Q^T (keys in krow order), p = 2^(t - L2); then O'^T += V^T P^T,
// or dP^T = V dO^T, dS = p (dP - Dr) and dQ^T += K^T dS^T.  K^T and V^T are
// read transposed from the row tiles; NVFP4's slice scale of K (dQ) or V
// (O') multiplies the accumulator once, after the FP4 blocks.
template <int D, int MODE, int NW>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void bwd_row_kernel(BwdArgs a) {
  using R = RowStage<D>;
  // one LDS object: the two stages, then this row of promoted-block bits
  // (with a second __shared__ array the compiler waited for the next
  // stage's direct loads before every read of the current one)
  __shared__ __attribute__((aligned(16))) char smem[2 * R::SIZE + kMaxKw * 4];
  uint32_t* const pmw = (uint32_t*)(smem + 2 * R::SIZE);
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

  // B operands: Q of the current path (FP4-decoded first), dO (dQ mode)
  const auto qrs = rsrc(a.q16 + (size_t)bhq * S * D, S * D * 2);
  const auto qdrs = rsrc(a.qd + (size_t)bhq * S * D, S * D * 2);
  v8h qx[D / 16], dh[MODE == kModeDq ? D / 16 : 1];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) qx[kk] = ld8h(qdrs, (qrow * D + kk * 16 + hi * 8) * 2);
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
  const float tacc = MODE == kModeDq ? (a.tk ? a.tk[bhk] : 1.0f) : dpf4;  // the FP4 blocks' operand scale

  v16f acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = v16f{};

  const auto k16rs = rsrc(a.k16 + bhk * S * D, S * D * 2);  // rows past S read as zeros
  const auto kdrs = rsrc(a.kd + bhk * S * D, S * D * 2);
  const auto v16rs = rsrc(a.v16 + bhk * S * D, S * D * 2);
  const auto vdrs = rsrc(a.vd + bhk * Sp * D, Sp * D * 2);
  const uint32_t* pm = a.prom + ((size_t)bhq * a.nq + i) * a.nkw;
  const int nvalid = valid_kv_blocks(i, S, a.bq, kBlkK, a.causal);
  for (int k = t; k < a.nkw; k += NW * 64) pmw[k] = pm[k];
  __syncthreads();

  // the first block j' >= j of path ph (1: promoted), or nvalid; the last
  // bit word read stays in a register
  int cwi = -1;
  uint32_t cw = 0;
  auto next_blk = [&](int j, int ph) {
    while (j < nvalid) {
      if ((j >> 5) != cwi) {
        cwi = j >> 5;
        cw = __builtin_amdgcn_readfirstlane(pmw[cwi]);
      }
      const uint32_t wd = (ph ? cw : ~cw) & (~0u << (j & 31));
      if (wd) {
        const int jj = (j & ~31) + __builtin_ctz(wd);
        return jj < nvalid ? jj : nvalid;
      }
      j = (j & ~31) + 32;
    }
    return nvalid;
  };
  // this lane's direct-load source row (key krow(hi, r32) of a block, chunk
  // column w of the tile) and its transposed-read base (see below)
  const uint32_t loff = krow(hi, r32) * (D * 2) + w * 16;
  const int rr = r32 & 15;
  const uint32_t tb = (2 * (r32 >> 4) + ((rr & 3) >> 1)) * R::CS + (hi * 4 + (rr >> 2)) * 16 + (rr & 1) * 8;
  auto issue = [&](char* buf, int j, int ph) {
    row_issue<D, NW>(buf, ph ? k16rs : kdrs, ph ? v16rs : vdrs, loff + j * (kBlkK * D * 2), w);
  };

  int jc = next_blk(0, 0), pc = 0;
  if (jc >= nvalid) {
    jc = next_blk(0, 1);
    pc = 1;
  }
  int qph = 0;  // path whose Q operand qx holds
  if (jc < nvalid) issue(smem, jc, pc);
  for (int n = 0; jc < nvalid; ++n) {
    int jn = next_blk(jc + 1, pc), pn = pc;
    if (jn >= nvalid && pc == 0) {
      jn = next_blk(0, 1);
      pn = 1;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // this block's tiles are in; every wave is done with the previous block
    // the Q operand's reload completes inside its branch, before the next
    // block's direct loads go out: left pending, it made the compiler wait
    // at the products of every step (switching or not) for every load in
    // flight, the prefetch included
    if (pc != qph) {  // from the FP4 blocks to the promoted ones
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= tacc;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qx[kk] = ld8h(qrs, (qrow * D + kk * 16 + hi * 8) * 2);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      qph = pc;
    }
    if (jn < nvalid) issue(smem + ((n + 1) & 1) * R::SIZE, jn, pn);
    const bool f16 = pc != 0;
    const char* buf = smem + (n & 1) * R::SIZE;
    // S^T (and dP^T): lane (r32, hi) reads chunk 2 kk + hi of slot mt*32 + r32
    const char* kb = buf + R::K + hi * R::CS + r32 * 16;
    const char* vb = buf + R::V + hi * R::CS + r32 * 16;
    v16f s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = v16f{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) s[mt] = mfma_f16(*(const v8h*)(kb + kk * 2 * R::CS + mt * 512), qx[kk], s[mt]);
    }
    if constexpr (MODE == kModeDq) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        dp[mt] = v16f{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          dp[mt] = mfma_f16(*(const v8h*)(vb + kk * 2 * R::CS + mt * 512), dh[kk], dp[mt]);
      }
    }
    // causal and tail mask, on the diagonal and tail blocks only: a lane's 32
    // keys are consecutive, so both conditions are one threshold (rows past
    // S keep their values: their outputs are never written)
    if ((a.causal && jc * kBlkK + kBlkK - 1 > q0) || jc * kBlkK + kBlkK > S) {
      const int last = a.causal && qrow < S - 1 ? qrow : S - 1;
      const int lim = last - (jc * kBlkK + hi * 32);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ii = 0; ii < 16; ++ii)
          if (mt * 16 + ii > lim) s[mt][ii] = -INFINITY;
    }
    // B operand of the second product: step st holds keys hi*32 + 8 st + u,
    // registers 8 (st % 2) + u of tile st / 2
    v8h pb[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ii = 0; ii < 16; ++ii) {
        const float p = exp2_fast(__builtin_fmaf(s[mt][ii], f16 ? a.c : cq4, -L2));
        float v = p;
        if constexpr (MODE == kModeDq) v = p * (dp[mt][ii] * (f16 ? 1.0f : dpf4) - Dr);
        pb[mt * 2 + ii / 8][ii % 8] = (_Float16)v;
      }
    // A operand K^T (dQ) or V^T (O') read transposed: lane r of each 16
    // addresses key hi*32 + 8 st + 4 h2 + r / 4 (slot kslot_of) and channels
    // dt*32 + 16 (r32 / 16) + 4 (r % 4) .. + 3; it receives channel
    // dt*32 + r32 of 4 keys per read (h2 = 0, 1: the step's 8 keys)
    const char* tt = buf + (MODE == kModeDq ? R::K : R::V) + tb;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int o0 = 4 * dt * R::CS + kslot_of(8 * st) * 16;
        const int o1 = 4 * dt * R::CS + kslot_of(8 * st + 4) * 16;
        acc[dt] = mfma_f16(tr_read(tt, o0, o1), pb[st], acc[dt]);
      }
    jc = jn;
    pc = pn;
  }
  if (qph == 0) {  // only FP4 blocks (or none)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= tacc;
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

// The key kernels: one for dV, one for dK (each holds one set of
// accumulators, which keeps them at two or three waves per SIMD).
constexpr int kKeyDv = 0, kKeyDk = 1;

// Key kernel LDS: two stages of one 32-query step each (the next step's
// tiles arrive by direct loads while a step is computed); the dV kernel adds
// each wave's per-query factors of P's quantisation.  A stage holds tiles of
// 32 query rows (fp16 Q, FP4-decoded Q, for NVFP4's dK the decoded Q times
// its slice scale, dO) and the rows' LSE (log2 units) and row terms.  Tile
// layout: 16-byte chunk c of the row at slot m (query q0 + qperm(m)) sits at
// c * 512 + ((m + 4c) % 32) * 16: chunk-column-major with the rows rotated
// by four slots per column.  One direct wave load fills two chunk columns
// (lanes 0-31 column 2p, lanes 32-63 column 2p + 1), and both reads are free
// of bank conflicts: the row reads of the S and dP products (a half-wave
// reads 16 slots of one chunk) and the transposed reads of the dV and dK
// products (ds_read_b64_tr_b16: per 16 lanes, 4 queries of 16 channels).
template <int D, int FMT, int MODE>
struct KeyStage {
  static constexpr bool QSCALED = FMT == THRIFT_NVFP4 && MODE == kKeyDk;
  static constexpr int TILE = (D / 8) * 512;
  static constexpr int NTL = QSCALED ? 4 : 3;
  static constexpr int Q16 = 0;
  static constexpr int QD = TILE;
  static constexpr int QS = QSCALED ? 2 * TILE : TILE;  // dK's operand on FP4 pairs
  static constexpr int DO = (NTL - 1) * TILE;
  static constexpr int L2 = NTL * TILE;  // 32 floats, query order
  static constexpr int DR = L2 + 128;    // 32 floats, query order
  static constexpr int SIZE = DR + 128;
};
template <int D, int FMT, int MODE>
struct KeyLds {  // (FA, FH: [wave][group][query]; HT: [wave][query] half-tile maxima)
  static constexpr int FA = 2 * KeyStage<D, FMT, MODE>::SIZE;
  static constexpr int FH = FA + 4 * 2 * 32 * 4;
  static constexpr int HT = FH + 4 * 2 * 32 * 4;
  static constexpr int SIZE = MODE == kKeyDv ? HT + 4 * 32 * 4 : FA;
};

// The direct loads of one step (query head bhq, rows q0 .. q0 + 31) into
// stage buffer buf: the Q tiles the step's paths need (f0, f1: the two key
// blocks are on the FP16 path), dO, the rows' LSE (wave 0) and, for dK,
// their row terms (wave 1).  Wave w loads chunk-column pairs w + 4k of every
// tile, lane l the row at slot l % 32 of column 2p + l / 32 (voff).  Rows
// past S read as zeros (each tensor's buffer resource ends at its end).
template <int D, int FMT, int MODE>
__device__ inline void key_issue(const BwdArgs& a, char* buf, size_t bhq, int q0, bool f0, bool f1,
                                 const uint32_t* voff, int w, int lane) {
  using St = KeyStage<D, FMT, MODE>;
  constexpr int PW = D / 64;
  const int S = a.S;
  const uint32_t qo = q0 * (D * 2);
  auto tile = [&](const _Float16* base, int at) {
    const auto rs = rsrc(base + bhq * S * D, S * D * 2);
#pragma unroll
    for (int k = 0; k < PW; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(buf + at + (w + 4 * k) * 1024), 16, voff[k] + qo, 0, 0, 0);
  };
  if (f0 || f1) tile(a.q16, St::Q16);
  if (!f0 || !f1) {
    tile(a.qd, St::QD);
    if constexpr (St::QSCALED) tile(a.qds, St::QS);
  }
  tile(a.do16, St::DO);
  auto rows = [&](const float* base, int at) {
    // the row's base made visibly uniform (the load sits under a lane mask)
    const uint64_t p = (uint64_t)(base + bhq * S);
    const uint32_t ph = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t pl = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);  // (int: no sign extension)
    const uint64_t pu = (uint64_t)ph << 32 | pl;
    const auto rs = rsrc((const void*)pu, S * 4);
    if (lane < 32) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_ptr(buf + at), 4, (q0 + lane) * 4, 0, 0, 0);
  };
  if (w == 0) rows(a.lse2, St::L2);
  if (MODE == kKeyDk && w == 1) rows(a.drow, St::DR);
}

// Workgroup = two key blocks (2 x 64 keys) of (batch, key head), four waves
// of 32 keys each, one lane per key.  Steps of 32 query rows run over the G
// query heads of the key head and the rows that see the blocks; each step's
// query rows and dO rows come once into LDS for all four waves, by direct
// loads one step ahead.  Per step and wave, with this lane's key as the
// column of S = Q K^T:
//  - dV (MODE kKeyDv): p per element; on FP4 pairs the probability the
//    forward used is rebuilt from its quantisation groups (MX: the wave's 32
//    keys; NVFP4: 16-key groups) under the 64-key tile maximum, which the
//    block's two waves exchange; the maxima come from S^T = K Q^T (same
//    operands swapped, one lane per query), and the per-query factors reach
//    the key-major lanes through the wave's own LDS slot; then dV += pt^T dO;
//  - dK (MODE kKeyDk): dP = dO V^T, dS = p (dP - Dr); dK += dS^T Q.
// The dV and dK products read their dO and Q operands transposed from the
// row tiles.  Only the K (and for dK the V) operands of the precision in use
// are held in registers; they are reloaded when a step switches path.
template <int D, int FMT, int MODE>
__global__ __launch_bounds__(256, MODE == kKeyDv ? 3 : 2) void bwd_key_kernel(BwdArgs a) {
  using L = KeyLds<D, FMT, MODE>;
  using St = KeyStage<D, FMT, MODE>;
  constexpr bool DV = MODE == kKeyDv;
  constexpr int PW = D / 64;  // chunk-column pairs per wave and tile
  __shared__ __attribute__((aligned(16))) char smem[L::SIZE];
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6), hi = lane >> 5, r32 = lane & 31;
  const int BHk = a.B * a.Hkv, G = a.Hq / a.Hkv;
  const int nk = cdiv(a.S, kBlkK);
  const int x = blockIdx.x;
  const int j0 = (x / BHk) * 2;  // causal: the lowest key blocks have the most rows
  const size_t bhk = x % BHk;
  const int b = (int)(bhk / a.Hkv), hk = (int)(bhk % a.Hkv);
  const int S = a.S;
  const int jb = j0 + (w >> 1);              // this wave's key block (waves w, w ^ 1 share it)
  const int key = jb * kBlkK + (w & 1) * 32 + r32;  // this lane's key (column of S)

  const auto k16rs = rsrc(a.k16 + bhk * S * D, S * D * 2);
  const auto kdrs = rsrc(a.kd + bhk * S * D, S * D * 2);
  const auto v16rs = rsrc(a.v16 + bhk * S * D, S * D * 2);
  const auto vdrs = rsrc(a.vd + bhk * a.Sp * D, a.Sp * D * 2);
  v8h kr[D / 16], vr[DV ? 1 : D / 16];
  int cur = -1;  // path whose K (and V) operands kr, vr hold (1 FP16, 0 FP4)
  auto load_kv = [&](bool f16) {
    const auto krs = f16 ? k16rs : kdrs;
    const auto vrs = f16 ? v16rs : vdrs;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int off = (key * D + kk * 16 + hi * 8) * 2;
      kr[kk] = ld8h(krs, off);
      if constexpr (!DV) vr[kk] = ld8h(vrs, off);
    }
    cur = f16;
  };
  v16f acc[D / 32];  // dV or dK (unscaled)
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = v16f{};
  const float dpf4 = a.tv ? a.tv[bhk] : 1.0f;

  // this lane's byte offsets: direct-load sources (row of slot r32 of column
  // 2p + hi, p = w + 4k), row reads (column 2kk + hi, by kk % 4) and
  // transposed reads (by (2 st + h2 + 2 dt) % 4, see below).  They are
  // recomputed where used from an opaque copy of the lane index: held across
  // the loop they were spilled, and each reload from scratch waited for the
  // step's direct loads in flight before it.
  uint32_t voff[PW], rrow[4], rtr[4];
  auto lane_offsets = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int h = ln >> 5, l32 = ln & 31, r = l32 & 15, g = l32 >> 4;
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const int c = 2 * (w + 4 * k) + h;
      voff[k] = qperm((l32 - 4 * c) & 31) * (D * 2) + c * 16;
    }
    const int xq = h * 4 + (r >> 2) + 8 * g + 4 * ((r & 3) >> 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      rrow[k] = h * 512 + ((l32 + 8 * k + 4 * h) & 31) * 16;
      rtr[k] = ((xq + 8 * k) & 31) * 16 + (2 * g + ((r & 3) >> 1)) * 512 + (r & 1) * 8;
    }
  };
  lane_offsets();

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

  int g = 0, q0 = qstart;          // this step
  int g1 = 0, q01 = qstart;        // the next
  advance(g1, q01);
  int g2 = g1, q02 = q01;          // the one after
  advance(g2, q02);
  uint32_t wcur = nsteps > 0 ? __builtin_amdgcn_readfirstlane(*word_addr(g, q0)) : 0u;
  uint32_t wnext = nsteps > 1 ? *word_addr(g1, q01) : 0u;  // in flight
  if (nsteps > 0)
    key_issue<D, FMT, MODE>(a, smem, b * a.Hq + hk * G + g, q0, bit(wcur, j0), bit(wcur, j0 + 1), voff, w, lane);
  float cq4 = a.c;  // scale of FP4 pairs' scores (NVFP4: times the head's slice scales)
  int cq_g = -1;
  for (int n = 0; n < nsteps; ++n) {
    const int bhq = b * a.Hq + hk * G + g;
    const bool f16 = bit(wcur, jb);
    if (g != cq_g) {
      cq4 = a.tq ? a.c * a.tq[bhq] * a.tk[bhk] : a.c;
      cq_g = g;
    }
    char* const buf = smem + (n & 1) * St::SIZE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // this step's tiles are in; every wave is done with the previous step
    lane_offsets();
    // a path switch reloads the K (and V) operands and waits for them
    // before the next step's direct loads go out: left pending, the reload
    // made the compiler wait at the products of every step for every load
    // in flight, the prefetch included
    if ((int)f16 != cur) {
      load_kv(f16);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    uint32_t wn = 0;
    if (n + 1 < nsteps) {
      wn = __builtin_amdgcn_readfirstlane(wnext);
      wnext = *word_addr(g2, q02);
      key_issue<D, FMT, MODE>(a, smem + ((n + 1) & 1) * St::SIZE, b * a.Hq + hk * G + g1, q01, bit(wn, j0),
                              bit(wn, j0 + 1), voff, w, lane);
    }
    // (steps whose pairs are all masked for this wave add zeros: a branch
    // around the products would make the compiler copy the accumulators)
    const char* qrows = buf + (f16 ? St::Q16 : St::QD);
    const char* dob = buf + St::DO;
    const float* l2 = (const float*)(buf + St::L2);
    const float cj = f16 ? a.c : cq4;
    // causal and tail mask, on diagonal and tail steps only: register ii of
    // S holds query q0 + hi*16 + ii, so the valid queries of this lane's key
    // are one range of ii
    const int kw0 = jb * kBlkK + (w & 1) * 32;  // the wave's first key
    const bool need_mask = (a.causal && kw0 + 31 > q0) || q0 + 31 >= S || kw0 + 31 >= S;
    auto mask_s = [&](v16f& sc) {
      const int qb = q0 + hi * 16;
      const int lo = a.causal ? key - qb : 0, up = key < S ? S - 1 - qb : -1;
#pragma unroll
      for (int ii = 0; ii < 16; ++ii)
        if (ii < lo || ii > up) sc[ii] = -INFINITY;
    };
    v8h opA[2];  // A operand of the product: pt (dV) or dS (dK); step st holds queries hi*16 + 8 st + u
    if constexpr (DV) {
      // FP4 pairs: per query and P group, p * fa is the element over its
      // block scale and pt = code * fh (this lane's key is in group grp)
      const int grp = FMT == THRIFT_MXFP4 ? 0 : r32 >> 4;
      const float* wa = (const float*)(smem + L::FA) + (w * 2 + grp) * 32;
      const float* wh = (const float*)(smem + L::FH) + (w * 2 + grp) * 32;
      float gm0 = -INFINITY, gm1 = -INFINITY, Lq = 0.0f;  // group maxima (raw scores) of query qperm(r32)
      if (!f16) {
        v16f st = v16f{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          st = mfma_f16(kr[kk], *(const v8h*)(qrows + kk * 1024 + rrow[kk & 3]), st);
        // column r32 is query q0 + qperm(r32); register ii is key (ii/4)*8 + hi*4 + ii%4 of the wave's 32
        const int qm = q0 + qperm(r32);
        if (need_mask) {  // keys past the query (causal) or past S, queries past S
          const int lim = qm < S ? (a.causal && qm < S - 1 ? qm : S - 1) - kw0 : -1;
#pragma unroll
          for (int ii = 0; ii < 16; ++ii)
            if ((ii >> 2) * 8 + hi * 4 + (ii & 3) > lim) st[ii] = -INFINITY;
        }
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          if (ii < 8)
            gm0 = fmaxf(gm0, st[ii]);
          else
            gm1 = fmaxf(gm1, st[ii]);
        }
        gm0 = pair_max(gm0);
        gm1 = pair_max(gm1);
        Lq = l2[qperm(r32)];
        if (hi == 0) ((float*)(smem + L::HT))[w * 32 + qperm(r32)] = fmaxf(gm0, gm1);
      }
      v16f s = v16f{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) s = mfma_f16(*(const v8h*)(qrows + kk * 1024 + rrow[kk & 3]), kr[kk], s);
      if (need_mask) mask_s(s);
      // level 1 is the query's maximum over the whole 64-key tile: the two
      // waves of the block exchange their halves (every wave passes this
      // barrier on every step)
      __syncthreads();
      if (!f16) {
        const float tm = fmaxf(fmaxf(gm0, gm1), ((const float*)(smem + L::HT))[(w ^ 1) * 32 + qperm(r32)]);
        const float tml = tm * cj;
        // a tile more than 2^60 below the row's total contributes nothing
        const bool live = tm > -INFINITY && tml - Lq > -60.0f;
        if constexpr (FMT == THRIFT_MXFP4) {
          // level 2: this wave's 32 keys are one group; E8M0 exponent
          // floor(log2(max p)) - 2 relative to the tile maximum (-2 for the
          // group holding it)
          const float gm = fmaxf(gm0, gm1);
          const uint32_t E =
              gm == tm ? 127u : (__float_as_uint(exp2_fast(__builtin_fmaf(gm, cj, -tml))) >> 23) & 0xFF;
          const float X = (float)((int)(E > 3 ? E - 2 : 1) - 127);
          const bool on = live && gm > -INFINITY;
          if (hi == 0) {
            ((float*)wa)[qperm(r32)] = on ? exp2_fast(Lq - tml - X) : 0.0f;
            ((float*)wh)[qperm(r32)] = on ? exp2_fast(X + tml - Lq) : 0.0f;
          }
        } else {
#pragma unroll
          for (int gg = 0; gg < 2; ++gg) {
            const float gmg = gg ? gm1 : gm0;
            const float gv = gmg == tm ? 2688.0f : 2688.0f * exp2_fast(__builtin_fmaf(gmg, cj, -tml));
            v2s_t sb = {0, 0};
            sb = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(sb, fminf(gv * (1.0f / 6.0f), 448.0f), 0.0f, 1.0f, false);
            const float s2 = e4m3_to_float((uint32_t)sb[0] & 0xFF);
            const bool on = live && s2 > 0.0f;
            if (hi == 0) {
              float* fa = (float*)(smem + L::FA) + (w * 2 + gg) * 32;
              float* fh = (float*)(smem + L::FH) + (w * 2 + gg) * 32;
              fa[qperm(r32)] = on ? exp2_fast(Lq - tml) * nv_p_factor(s2) : 0.0f;
              fh[qperm(r32)] = on ? s2 * exp2_fast(tml - Lq) * (1.0f / 2688.0f) : 0.0f;
            }
          }
        }
        // the wave reads back its own slot: its LDS operations complete in order
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      // this lane's queries are q0 + hi*16 + ii, four at a time
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 l4 = *(const float4*)(l2 + hi * 16 + u * 4);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        float pt[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pt[e] = exp2_fast(__builtin_fmaf(s[u * 4 + e], cj, -lv[e]));
        if (!f16) {
          const float4 a4 = *(const float4*)(wa + hi * 16 + u * 4);
          const float4 h4 = *(const float4*)(wh + hi * 16 + u * 4);
          const uint32_t y0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, pt[0] * a4.x, pt[1] * a4.y, 1.0f, 0);
          const uint32_t y1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, pt[2] * a4.z, pt[3] * a4.w, 1.0f, 0);
          const v2f c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(y0, 1.0f, 0);
          const v2f c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(y1, 1.0f, 0);
          pt[0] = c0[0] * h4.x;
          pt[1] = c0[1] * h4.y;
          pt[2] = c1[0] * h4.z;
          pt[3] = c1[1] * h4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) opA[(u * 4 + e) / 8][(u * 4 + e) % 8] = (_Float16)pt[e];
      }
    } else {
      v16f s = v16f{}, dp = v16f{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = mfma_f16(*(const v8h*)(qrows + kk * 1024 + rrow[kk & 3]), kr[kk], s);
        dp = mfma_f16(*(const v8h*)(dob + kk * 1024 + rrow[kk & 3]), vr[kk], dp);
      }
      if (need_mask) mask_s(s);
      const float* dr = (const float*)(buf + St::DR);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 l4 = *(const float4*)(l2 + hi * 16 + u * 4);
        const float4 r4 = *(const float4*)(dr + hi * 16 + u * 4);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ii = u * 4 + e;
          const float p = exp2_fast(__builtin_fmaf(s[ii], cj, -lv[e]));
          opA[ii / 8][ii % 8] = (_Float16)(p * (dp[ii] * (f16 ? 1.0f : dpf4) - rv[e]));
        }
      }
    }
    // B operand read transposed: in step st, lane (r32, hi) takes channel
    // dt*32 + r32 of queries hi*16 + 8 st + 4 h2 + (0..3) from two
    // ds_read_b64_tr_b16, h2 = 0, 1 (rtr's index (2 st + h2 + 2 dt) % 4):
    // dO for dV, Q for dK
    const char* opB = DV ? dob : buf + (f16 ? St::Q16 : St::QS);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int k0 = (2 * st + 2 * dt) & 3, k1 = (2 * st + 1 + 2 * dt) & 3;
        acc[dt] = mfma_f16(opA[st], tr_read(opB + dt * 2048, rtr[k0], rtr[k1]), acc[dt]);
      }
    wcur = wn;
    g = g1;
    q0 = q01;
    g1 = g2;
    q01 = q02;
    advance(g2, q02);
  }
  // C layout: column d = dt*32 + r32, register ii is key (ii/4)*8 + hi*4 + ii%4 of the wave's 32
  float* out = DV ? a.dv : a.dk;
  const float osc = DV ? 1.0f : a.sm_scale;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
      const int kx = jb * kBlkK + (w & 1) * 32 + (ii >> 2) * 8 + hi * 4 + (ii & 3);
      if (kx < S) out[(bhk * S + kx) * D + dt * 32 + r32] = acc[dt][ii] * osc;
    }
}

// ---- host side -----------------------------------------------------------------------

struct BwdLayout {
  size_t qd, qds, kd, vd, prom, drow, lse2, total;
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
  l.qds = take(bhq * S * D * 2);
  l.kd = take(bhk * S * D * 2);
  l.vd = take(bhk * Sp * D * 2);
  l.prom = take(bhq * nq * nkw * 4);
  l.drow = take(bhq * S * 4);
  l.lse2 = take(bhq * S * 4);
  l.total = o;
  return l;
}

thrift_status check_bwd(const void* q16, const void* k16, const void* v16, const uint8_t* q4c,
                        const uint8_t* q4s, const float* q4t, const uint8_t* k4c, const uint8_t* k4s,
                        const float* k4t, const uint8_t* v4c, const uint8_t* v4s, const float* v4t,
                        int fmt, const int32_t* idx, const int32_t* cnt, int kmax,
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

// Fills the FP4-decoded operands both entry points share.  They keep
// NVFP4's slice scale out (exact fp16): the scale multiplies the fp32 scores
// and dP, and the row kernel's accumulator after its FP4 blocks; only the
// key kernel's dK operand, the decoded Q rows times Q's slice scale, carries
// it, rounded once.
void prepare(BwdArgs& a, char* ws, const BwdLayout& l, const void* q16, const void* k16, const void* v16,
             const uint8_t* q4c, const uint8_t* q4s, const float* q4t, const uint8_t* k4c, const uint8_t* k4s,
             const float* k4t, const uint8_t* v4c, const uint8_t* v4s, const float* v4t, int fmt,
             const int32_t* idx, const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D, int block_q,
             int causal, float sm_scale, const float* lse, const void* do16, const float* ohp, hipStream_t stream) {
  const bool backward = do16 != nullptr;
  const int Sp = cdiv(S, kBlkK) * kBlkK, nk = cdiv(S, kBlkK);
  a.q16 = (const _Float16*)q16;
  a.k16 = (const _Float16*)k16;
  a.v16 = (const _Float16*)v16;
  a.do16 = (const _Float16*)do16;
  a.qd = (const _Float16*)(ws + l.qd);
  a.kd = (const _Float16*)(ws + l.kd);
  a.vd = (const _Float16*)(ws + l.vd);
  a.qds = (const _Float16*)(ws + l.qds);
  a.prom = (const uint32_t*)(ws + l.prom);
  a.lse = lse;
  a.drow = (const float*)(ws + l.drow);
  a.lse2 = (const float*)(ws + l.lse2);
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
  const size_t BHq = (size_t)B * Hq, BHk = (size_t)B * Hkv;
  PrepArgs p{};
  p.q4c = q4c;
  p.q4s = q4s;
  p.k4c = k4c;
  p.k4s = k4s;
  p.v4c = v4c;
  p.v4s = v4s;
  p.tq = a.tq;
  p.idx = idx;
  p.cnt = cnt;
  p.do16 = a.do16;
  p.ohp = ohp;
  p.lse = lse;
  p.qd = (_Float16*)a.qd;
  p.kd = (_Float16*)a.kd;
  p.vd = (_Float16*)a.vd;
  p.qds = (_Float16*)a.qds;
  p.prom = (uint32_t*)a.prom;
  p.drow = (float*)a.drow;
  p.lse2 = (float*)a.lse2;
  p.fmt = fmt;
  p.S = S;
  p.nk = nk;
  p.kmax = kmax;
  p.nkw = a.nkw;
  p.rq = BHq * S;
  p.rk = BHk * S;
  p.nrows_rt = backward ? BHq * S : 0;
  p.nrows_pb = (int)BHq * a.nq;
  auto wgs = [](size_t threads) { return (unsigned)((threads + 255) / 256); };
  p.wq = (unsigned)(BHk * nk);
  p.wk = p.wq + wgs(p.rq * (D / 8));
  p.wqs = p.wk + wgs(p.rk * (D / 8));
  p.wrt = p.wqs + (backward && nv ? wgs(p.rq * (D / 8)) : 0);
  p.wpb = p.wrt + wgs(p.nrows_rt * (D / 8));
  p.wend = p.wpb + wgs((size_t)p.nrows_pb);
  if (D == 128)
    bwd_prep_kernel<128><<<p.wend, 256, 0, stream>>>(p);
  else
    bwd_prep_kernel<64><<<p.wend, 256, 0, stream>>>(p);
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

template <int D, int FMT>
void launch_key(const BwdArgs& a, int kgrid, hipStream_t stream) {
  bwd_key_kernel<D, FMT, kKeyDv><<<kgrid, 256, 0, stream>>>(a);
  bwd_key_kernel<D, FMT, kKeyDk><<<kgrid, 256, 0, stream>>>(a);
}

template __global__ void bwd_row_kernel<128, kModeOhp, 4>(BwdArgs);
template __global__ void bwd_row_kernel<128, kModeDq, 4>(BwdArgs);
template __global__ void bwd_row_kernel<64, kModeOhp, 4>(BwdArgs);
template __global__ void bwd_row_kernel<64, kModeDq, 4>(BwdArgs);
template __global__ void bwd_row_kernel<128, kModeOhp, 2>(BwdArgs);
template __global__ void bwd_row_kernel<128, kModeDq, 2>(BwdArgs);
template __global__ void bwd_row_kernel<64, kModeOhp, 2>(BwdArgs);
template __global__ void bwd_row_kernel<64, kModeDq, 2>(BwdArgs);

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
    const uint8_t* v4_codes, const uint8_t* v4_scales, const float* v4_tscale, int fmt, const int32_t* idx, const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D,
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
          nullptr, nullptr, stream);
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
    const uint8_t* v4_codes, const uint8_t* v4_scales, const float* v4_tscale, int fmt, const int32_t* idx, const int32_t* cnt, int kmax, int B, int Hq, int Hkv, int S, int D,
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
          v4_scales, v4_tscale, fmt, idx, cnt, kmax, B, Hq, Hkv, S, D, block_q, causal, sm_scale, lse, do16, ohp,
          stream);
  a.out = dq;
  a.dk = dk;
  a.dv = dv;
  const int kgrid = B * Hkv * cdiv(cdiv(S, kBlkK), 2);
  const bool mx = fmt == THRIFT_MXFP4;
  if (D == 128) {
    launch_row<128>(a, kModeDq, stream);
    if (mx)
      launch_key<128, THRIFT_MXFP4>(a, kgrid, stream);
    else
      launch_key<128, THRIFT_NVFP4>(a, kgrid, stream);
  } else {
    launch_row<64>(a, kModeDq, stream);
    if (mx)
      launch_key<64, THRIFT_MXFP4>(a, kgrid, stream);
    else
      launch_key<64, THRIFT_NVFP4>(a, kgrid, stream);
  }
  return launch_status();
}
