// FP4 quantisation of Q, K and V on gfx950 (the FP4 path of ThriftAttention
// uses NVFP4 micro-scaling; MXFP4 is the layout of gfx950's block-scaled
// matrix instructions).  Streaming kernels, bound by HBM: each fp16 element
// is read once (NVFP4 reads the slice twice, once for its maximum) and each
// code nibble and scale byte written once, with 16-byte loads and stores.
//
// Every rounding decision is exact:
//  - MXFP4 divides by a power of two (exact in fp32) and uses gfx950's
//    scaled FP4 conversion, which rounds to nearest even and saturates at 6;
//  - NVFP4's block scale is E4M3(amax / (6 sg)): the fp64 quotient of an
//    11-bit and a 26-bit significand can only land on a 5-bit E4M3 midpoint
//    if the exact quotient is that midpoint, so rounding the fp64 quotient
//    is exact; element codes compare |x| (fp16, exact in fp32) against the
//    seven E2M1 midpoints times the block scale, each midpoint rounded down
//    to fp32 with a flag telling whether it was exact, which decides every
//    comparison (and every tie) exactly.
#include "common.h"

namespace thrift {

constexpr int kQThreads = 256;
constexpr int kAmaxChunk = 65536;  // elements reduced per workgroup

// ---- per-slice maxima (NVFP4 only) ------------------------------------------

__global__ __launch_bounds__(kQThreads) void slice_amax_kernel(const _Float16* __restrict__ x,
                                                               size_t slice, int nchunk,
                                                               float* __restrict__ part) {
  __shared__ float red[kQThreads / kWave];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const _Float16* base = x + (size_t)bh * slice;
  size_t e0 = (size_t)c * kAmaxChunk, e1 = e0 + kAmaxChunk < slice ? e0 + kAmaxChunk : slice;
  float m = 0.0f;
  for (size_t e = e0 + (size_t)t * 8; e < e1; e += kQThreads * 8) {
    v8h v = *reinterpret_cast<const v8h*>(base + e);  // slice sizes are multiples of 8
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, fabsf((float)v[u]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  if (t % kWave == 0) red[t / kWave] = m;
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < kQThreads / kWave; ++w) m = fmaxf(m, red[w]);
    part[(size_t)bh * nchunk + c] = m;
  }
}

// sg = fp32(amax / 2688) (fp64 division, one rounding), or 1 for an all-zero slice.
__global__ void slice_scale_kernel(const float* __restrict__ part, int nchunk, int BH,
                                   float* __restrict__ tscale) {
  int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= BH) return;
  float m = 0.0f;
  for (int c = 0; c < nchunk; ++c) m = fmaxf(m, part[(size_t)bh * nchunk + c]);
  tscale[bh] = m > 0.0f ? (float)((double)m / 2688.0) : 1.0f;
}

// ---- exact roundings ---------------------------------------------------------

// Non-negative E4M3 code nearest to q (ties to even), saturating at 448.
__device__ inline int e4m3_rne(double q) {
  if (!(q > 0.0)) return 0;
  if (q >= 448.0) return 126;
  int e;
  double f = frexp(q, &e);  // q = f 2^e, f in [0.5, 1)
  int E = e - 1;            // q in [2^E, 2^(E+1))
  if (E < -6) {             // subnormal range: multiples of 2^-9
    int m = (int)rint(ldexp(q, 9));
    return m;               // m == 8 is the smallest normal, code 8
  }
  int m = (int)rint((f * 2.0 - 1.0) * 8.0);  // 3 mantissa bits
  int code = ((E + 7) << 3) + m;             // m == 8 carries into the exponent
  return code > 126 ? 126 : code;
}

__device__ inline double e4m3_value(int code) {
  int e = code >> 3, m = code & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

// Largest fp32 value <= x (x >= 0), and whether it equals x.
__device__ inline float round_down_f32(double x, bool* exact) {
  float f = (float)x;  // nearest
  if ((double)f > x) f = nextafterf(f, 0.0f);
  *exact = (double)f == x;
  return f;
}

// E2M1 code of x / s from the seven midpoint thresholds m_k * s.
struct E2m1Thresholds {
  float t[7];
  unsigned exact;  // bit k: t[k] == m_k * s exactly
};

__device__ inline E2m1Thresholds make_thresholds(double s) {
  const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  E2m1Thresholds th;
  th.exact = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    bool ex;
    th.t[k] = round_down_f32(mid[k] * s, &ex);
    th.exact |= (unsigned)ex << k;
  }
  return th;
}

__device__ inline uint32_t e2m1_code_exact(float x, const E2m1Thresholds& th) {
  float a = fabsf(x);
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    // above the midpoint, or on it exactly and the upper neighbour is even
    bool up = a > th.t[k] || (a == th.t[k] && ((th.exact >> k) & 1u) && ((k + 1) & 1) == 0);
    c += up ? 1u : 0u;
  }
  return c | (__float_as_uint(x) >> 31 << 3);
}

// ---- encoders -------------------------------------------------------------------

// NVFP4-style group of 16: returns the block scale byte, fills 8 code bytes.
__device__ inline uint32_t encode_nvfp4_16(const float* v, float sg, uint32_t* w /*2 dwords*/) {
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 16; ++u) amax = fmaxf(amax, fabsf(v[u]));
  int sb = e4m3_rne((double)amax / (6.0 * (double)sg));
  double s = e4m3_value(sb) * (double)sg;
  w[0] = w[1] = 0;
  if (s > 0.0) {
    E2m1Thresholds th = make_thresholds(s);
#pragma unroll
    for (int u = 0; u < 16; ++u) w[u / 8] |= e2m1_code_exact(v[u], th) << (4 * (u % 8));
  }
  return (uint32_t)sb;
}

// MXFP4 group of 32: returns the E8M0 byte, fills 4 code dwords.
__device__ inline uint32_t encode_mx_32(const float* v, uint32_t* w /*4 dwords*/) {
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 32; ++u) amax = fmaxf(amax, fabsf(v[u]));
  // floor(log2 amax) - 2 from the exponent field (fp16 values are normal fp32)
  int X = amax > 0.0f ? (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 2 : -127;
  float scale = amax > 0.0f ? __uint_as_float((uint32_t)(X + 127) << 23) : 1.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* p = v + q * 8;
    uint32_t d = 0;  // byte u holds elements 2u (low nibble) and 2u+1
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, p[0], p[1], scale, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, p[2], p[3], scale, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, p[4], p[5], scale, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, p[6], p[7], scale, 3);
    w[q] = d;
  }
  return (uint32_t)(X + 127);
}

// ---- groups along D (Q, K) -----------------------------------------------------

// Thread li encodes group gi = (li / range) * groups_per_slice + first + li % range:
// `range` groups from group `first` of every (batch, head) slice (the whole
// slice when range == groups_per_slice and first == 0).
// Group gi (g consecutive elements along D) of x: its code bytes and scale byte.
template <int FMT>
__device__ inline void quant_d_group(const _Float16* __restrict__ x, size_t gi, int groups_per_slice,
                                     const float* __restrict__ tscale, uint8_t* __restrict__ codes,
                                     uint8_t* __restrict__ scales) {
  constexpr int g = FMT == THRIFT_NVFP4 ? 16 : 32;
  float v[g];
  const v8h* src = reinterpret_cast<const v8h*>(x + gi * g);
#pragma unroll
  for (int q = 0; q < g / 8; ++q) {
    v8h h = src[q];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[q * 8 + u] = (float)h[u];
  }
  if (FMT == THRIFT_NVFP4) {
    uint32_t w[2];
    float sg = tscale[gi / groups_per_slice];
    scales[gi] = (uint8_t)encode_nvfp4_16(v, sg, w);
    *reinterpret_cast<uint2*>(codes + gi * 8) = make_uint2(w[0], w[1]);
  } else {
    uint32_t w[4];
    scales[gi] = (uint8_t)encode_mx_32(v, w);
    *reinterpret_cast<uint4*>(codes + gi * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int FMT>
__global__ __launch_bounds__(kQThreads) void quant_d_kernel(const _Float16* __restrict__ x,
                                                            size_t ngroups, int groups_per_slice,
                                                            int range, int first,
                                                            const float* __restrict__ tscale,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const size_t li = (size_t)blockIdx.x * kQThreads + threadIdx.x;
  if (li >= ngroups) return;
  const size_t gi = range == groups_per_slice
                        ? li
                        : (li / range) * groups_per_slice + first + li % range;
  quant_d_group<FMT>(x, gi, groups_per_slice, tscale, codes, scales);
}

// ---- groups along S (V, stored transposed) -------------------------------------

constexpr int kVTile = 128;  // tokens per workgroup

// Tile tt (kVTile positions) of slice bh of x, staged through tile[][] (LDS).
template <int FMT, int D>
__device__ inline void quant_s_tile(const _Float16* __restrict__ x, int S, int Sp, int tt, int bh, int t,
                                    _Float16 (*tile)[D + 2], const float* __restrict__ tscale,
                                    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int g = FMT == THRIFT_NVFP4 ? 16 : 32;
  constexpr int GPT = kVTile / g;  // groups per d in this tile
  const int s0 = tt * kVTile;
  const _Float16* base = x + (size_t)bh * S * D;
  // stage kVTile x D fp16 (zeros past S)
  for (int e = t; e < kVTile * D / 8; e += kQThreads) {
    int r = e / (D / 8), c = (e % (D / 8)) * 8;
    v8h h = {};
    if (s0 + r < S) h = *reinterpret_cast<const v8h*>(base + (size_t)(s0 + r) * D + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) tile[r][c + u] = h[u];
  }
  __syncthreads();
  const float sg = FMT == THRIFT_NVFP4 ? tscale[bh] : 1.0f;
  for (int e = t; e < D * GPT; e += kQThreads) {
    const int d = e / GPT, gq = e % GPT;
    const int tok0 = s0 + gq * g;
    if (tok0 >= Sp) continue;
    float v[g];
#pragma unroll
    for (int u = 0; u < g; ++u) v[u] = (float)tile[gq * g + u][d];
    // key-block-major: block jb = tok0 / 64 holds [D][32 B] codes, [D][64/g] scales
    const size_t blk = (size_t)bh * (Sp / 64) + tok0 / 64;
    const size_t crow = (blk * D + d) * 32 + (tok0 % 64) / 2;
    const size_t srow = (blk * D + d) * (64 / g) + (tok0 % 64) / g;
    if (FMT == THRIFT_NVFP4) {
      uint32_t w[2];
      scales[srow] = (uint8_t)encode_nvfp4_16(v, sg, w);
      *reinterpret_cast<uint2*>(codes + crow) = make_uint2(w[0], w[1]);
    } else {
      uint32_t w[4];
      scales[srow] = (uint8_t)encode_mx_32(v, w);
      *reinterpret_cast<uint4*>(codes + crow) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

template <int FMT, int D>
__global__ __launch_bounds__(kQThreads) void quant_s_kernel(const _Float16* __restrict__ x, int S,
                                                            int Sp, int tile0,
                                                            const float* __restrict__ tscale,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  __shared__ _Float16 tile[kVTile][D + 2];
  quant_s_tile<FMT, D>(x, S, Sp, tile0 + blockIdx.x, blockIdx.y, threadIdx.x, tile, tscale, codes, scales);
}

// ---- KV-cache update: what new positions change, in one launch ----------------------

// For new positions s0 <= s < s1 of a cache slice (blockIdx.y): workgroups
// [0, nmeans) compute the mean of key block j0 + blockIdx.x (as
// block_means_kernel: fp64 column sums, one rounding); the next ndg encode
// K's groups along D of rows s0..s1-1 (as quant_d_kernel); the rest encode
// the V tiles from t0 on (as quant_s_kernel).  The branch is uniform per
// workgroup.
template <int FMT, int D>
__global__ __launch_bounds__(kQThreads) void cache_update_kernel(
    const _Float16* __restrict__ k16, const _Float16* __restrict__ v16, int S, int blk, int nb, int j0,
    int nmeans, int s0, int s1, int ndg, int t0, float* __restrict__ kbar, const float* __restrict__ k4t,
    uint8_t* __restrict__ k4c, uint8_t* __restrict__ k4s, const float* __restrict__ v4t,
    uint8_t* __restrict__ v4c, uint8_t* __restrict__ v4s) {
  constexpr int CG = D / 8, RP = kQThreads / CG;
  constexpr int g = FMT == THRIFT_NVFP4 ? 16 : 32;
  __shared__ double red[RP][D + 1];
  __shared__ _Float16 tile[kVTile][D + 2];
  const int x = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  if (x < nmeans) {
    const int j = j0 + x, cg = t % CG, rp = t / CG;
    const int r0 = j * blk, r1 = min(S, r0 + blk);
    const _Float16* base = k16 + (size_t)bh * S * D + cg * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = r0 + rp; r < r1; r += RP) {
      const v8h h = *reinterpret_cast<const v8h*>(base + (size_t)r * D);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += (double)(float)h[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rp][cg * 8 + e] = acc[e];
    __syncthreads();
    if (t < D) {
      double sum = 0.0;
      for (int k = 0; k < RP; ++k) sum += red[k][t];
      kbar[((size_t)bh * nb + j) * D + t] = (float)(sum / (double)(r1 - r0));
    }
  } else if (x < nmeans + ndg) {
    const int gpr = D / g, li = (x - nmeans) * kQThreads + t;
    if (li < (s1 - s0) * gpr)
      quant_d_group<FMT>(k16, (size_t)bh * S * gpr + (size_t)s0 * gpr + li, S * gpr, k4t, k4c, k4s);
  } else {
    quant_s_tile<FMT, D>(v16, S, cdiv(S, 64) * 64, t0 + (x - nmeans - ndg), bh, t, tile, v4t, v4c, v4s);
  }
}

// ---- block means and FP4 along D in one read (Q, K) -------------------------------

// One workgroup per (slice, block of blk rows); thread t holds the 16-byte
// column chunk cg = t % (D/8) of rows rp, rp + RP, ... (rp = t / (D/8)), so
// the four lanes of a 32-element MX group are adjacent and share their rows.
//  - Block means as block_means_kernel computes them (fp64 column sums in
//    any order are exact; one rounding to fp32).
//  - MXFP4: the group maximum by two lane exchanges, then each lane encodes
//    its 8 elements with the group's E8M0 scale, exactly as quant_d_kernel.
//  - NVFP4: the block's absolute maximum goes to part[bh * nb + j] for the
//    slice scale; the codes follow in quant_d_kernel (a second read).
template <int D, int FMT>
__global__ __launch_bounds__(kQThreads) void means_quant_kernel(const _Float16* __restrict__ x, int S,
                                                                int blk, int nb,
                                                                float* __restrict__ means,
                                                                uint8_t* __restrict__ codes,
                                                                uint8_t* __restrict__ scales,
                                                                float* __restrict__ part) {
  constexpr int CG = D / 8;              // 16-byte column chunks per row
  constexpr int RP = kQThreads / CG;     // row phases
  static_assert(CG % 4 == 0, "an MX group is four chunks");
  __shared__ double red[RP][D + 1];
  __shared__ float redm[kQThreads / kWave];
  const int j = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int cg = t % CG, rp = t / CG;
  const int r0 = j * blk, r1 = min(S, r0 + blk);
  const size_t row0 = (size_t)bh * S;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float amax = 0.0f;
  for (int r = r0 + rp; r < r1; r += RP) {
    const v8h h = *reinterpret_cast<const v8h*>(x + (row0 + r) * D + cg * 8);
    float f[8];
    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      f[u] = (float)h[u];
      acc[u] += (double)f[u];
      m = fmaxf(m, fabsf(f[u]));
    }
    if constexpr (FMT == THRIFT_MXFP4) {
      m = fmaxf(m, __shfl_xor(m, 1, kWave));  // the group's four chunks
      m = fmaxf(m, __shfl_xor(m, 2, kWave));
      // floor(log2 amax) - 2 from the exponent field (fp16 values are normal fp32)
      const int X = m > 0.0f ? (int)((__float_as_uint(m) >> 23) & 0xFF) - 127 - 2 : -127;
      const float scale = m > 0.0f ? __uint_as_float((uint32_t)(X + 127) << 23) : 1.0f;
      uint32_t d = 0;  // byte u holds elements 2u (low nibble) and 2u+1
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[0], f[1], scale, 0);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[2], f[3], scale, 1);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[4], f[5], scale, 2);
      d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, f[6], f[7], scale, 3);
      *reinterpret_cast<uint32_t*>(codes + (row0 + r) * (D / 2) + cg * 4) = d;
      if ((cg & 3) == 0) scales[(row0 + r) * (D / 32) + cg / 4] = (uint8_t)(X + 127);
    } else {
      amax = fmaxf(amax, m);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rp][cg * 8 + e] = acc[e];
  if constexpr (FMT == THRIFT_NVFP4) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    if (t % kWave == 0) redm[t / kWave] = amax;
  }
  __syncthreads();
  if (t < D) {
    double sum = 0.0;
    for (int k = 0; k < RP; ++k) sum += red[k][t];
    means[((size_t)bh * nb + j) * D + t] = (float)(sum / (double)(r1 - r0));
  }
  if constexpr (FMT == THRIFT_NVFP4)
    if (t == 0) {
      for (int w = 1; w < kQThreads / kWave; ++w) amax = fmaxf(amax, redm[w]);
      part[(size_t)bh * nb + j] = amax;
    }
}

// ---- MXFP8 (the middle precision tier) ------------------------------------------
//
// E4M3 elements under one E8M0 scale per 32: exponent floor(log2 amax) - 8
// from the fp32 exponent field of amax (fp16 inputs are normal in fp32), so
// the group maximum lands in [256, 512).  Elements are clamped to +-448 * 2^X
// (the largest finite E4M3 value, which is where round-to-nearest-even with
// saturation sends everything above it) and converted by gfx950's scaled FP8
// conversion, which divides by the power of two exactly and rounds to nearest
// even, keeping the sign (so -0 and negatives that round to zero give 0x80).

// Group of 32: returns the E8M0 byte, fills 8 code dwords (byte u = element u).
__device__ inline uint32_t encode_mx8_32(const float* v, uint32_t* w /*8 dwords*/) {
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < 32; ++u) amax = fmaxf(amax, fabsf(v[u]));
  const int X = amax > 0.0f ? (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127 - 8 : -127;
  const float scale = amax > 0.0f ? __uint_as_float((uint32_t)(X + 127) << 23) : 1.0f;
  const float cap = 448.0f * scale;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float* p = v + q * 4;
    v2s_t y = {0, 0};
    y = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(y, __builtin_amdgcn_fmed3f(p[0], -cap, cap),
                                                  __builtin_amdgcn_fmed3f(p[1], -cap, cap), scale, false);
    y = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(y, __builtin_amdgcn_fmed3f(p[2], -cap, cap),
                                                  __builtin_amdgcn_fmed3f(p[3], -cap, cap), scale, true);
    w[q] = __builtin_bit_cast(uint32_t, y);
  }
  return (uint32_t)(X + 127);
}

// Groups along D (Q, K): thread gi encodes elements [32 gi, 32 gi + 32).
__global__ __launch_bounds__(kQThreads) void quant8_d_kernel(const _Float16* __restrict__ x, size_t ngroups,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const size_t gi = (size_t)blockIdx.x * kQThreads + threadIdx.x;
  if (gi >= ngroups) return;
  float v[32];
  const v8h* src = reinterpret_cast<const v8h*>(x + gi * 32);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v8h h = src[q];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[q * 8 + u] = (float)h[u];
  }
  uint32_t w[8];
  scales[gi] = (uint8_t)encode_mx8_32(v, w);
  uint4* dst = reinterpret_cast<uint4*>(codes + gi * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// Groups along S (V): codes [B,H,D,Sp] and scales [B,H,D,Sp/32], the tile of
// kVTile positions staged through LDS so that the reads stay row-contiguous.
template <int D>
__global__ __launch_bounds__(kQThreads) void quant8_s_kernel(const _Float16* __restrict__ x, int S, int Sp,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  __shared__ _Float16 tile[kVTile][D + 2];
  const int t = threadIdx.x, bh = blockIdx.y, s0 = blockIdx.x * kVTile;
  const _Float16* base = x + (size_t)bh * S * D;
  for (int e = t; e < kVTile * D / 8; e += kQThreads) {
    int r = e / (D / 8), c = (e % (D / 8)) * 8;
    v8h h = {};
    if (s0 + r < S) h = *reinterpret_cast<const v8h*>(base + (size_t)(s0 + r) * D + c);
#pragma unroll
    for (int u = 0; u < 8; ++u) tile[r][c + u] = h[u];
  }
  __syncthreads();
  constexpr int GPT = kVTile / 32;
  for (int e = t; e < D * GPT; e += kQThreads) {
    const int d = e / GPT, gq = e % GPT, tok0 = s0 + gq * 32;
    if (tok0 >= Sp) continue;
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = (float)tile[gq * 32 + u][d];
    uint32_t w[8];
    const size_t row = (size_t)bh * D + d;
    scales[row * (Sp / 32) + tok0 / 32] = (uint8_t)encode_mx8_32(v, w);
    uint4* dst = reinterpret_cast<uint4*>(codes + row * Sp + tok0);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

}  // namespace thrift

using namespace thrift;

static int pad_s(int S) { return cdiv(S, 64) * 64; }

extern "C" size_t thrift_quantize_workspace_bytes(int B, int H, int S, int D, int fmt) {
  if (B < 1 || H < 1 || S < 1 || D < 1) return 0;
  if (fmt != THRIFT_NVFP4) return 0;
  size_t nchunk = ((size_t)S * D + kAmaxChunk - 1) / kAmaxChunk;
  return (size_t)B * H * nchunk * sizeof(float);
}

extern "C" thrift_status thrift_quantize_fp4(const void* x16, int B, int H, int S, int D,
                                             int axis, int fmt,
                                             uint8_t* codes, uint8_t* scales, float* tensor_scale,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream) {
  if (!x16 || !codes || !scales) return THRIFT_EINVAL;
  if (B < 1 || H < 1 || S < 1) return THRIFT_EINVAL;
  if (fmt != THRIFT_NVFP4 && fmt != THRIFT_MXFP4) return THRIFT_EINVAL;
  if (axis != THRIFT_GROUP_D && axis != THRIFT_GROUP_S) return THRIFT_EINVAL;
  if (fmt == THRIFT_NVFP4 && !tensor_scale) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if (S > 262144) return THRIFT_EUNSUPPORTED;
  if (!aligned16(x16) || !aligned16(codes)) return THRIFT_EALIGN;
  const size_t need = thrift_quantize_workspace_bytes(B, H, S, D, fmt);
  if (need && (!workspace || workspace_bytes < need)) return THRIFT_EWORKSPACE;
  const int BH = B * H;
  auto x = (const _Float16*)x16;
  if (fmt == THRIFT_NVFP4) {
    const size_t slice = (size_t)S * D;
    const int nchunk = (int)((slice + kAmaxChunk - 1) / kAmaxChunk);
    float* part = (float*)workspace;
    slice_amax_kernel<<<dim3(nchunk, BH), kQThreads, 0, stream>>>(x, slice, nchunk, part);
    slice_scale_kernel<<<cdiv(BH, 256), 256, 0, stream>>>(part, nchunk, BH, tensor_scale);
  }
  if (axis == THRIFT_GROUP_D) {
    const int g = fmt == THRIFT_NVFP4 ? 16 : 32;
    const size_t ngroups = (size_t)BH * S * (D / g);
    const int blocks = (int)((ngroups + kQThreads - 1) / kQThreads);
    const int gps = S * (D / g);
    if (fmt == THRIFT_NVFP4)
      quant_d_kernel<THRIFT_NVFP4><<<blocks, kQThreads, 0, stream>>>(x, ngroups, gps, gps, 0,
                                                                       tensor_scale, codes, scales);
    else
      quant_d_kernel<THRIFT_MXFP4><<<blocks, kQThreads, 0, stream>>>(x, ngroups, gps, gps, 0,
                                                                       tensor_scale, codes, scales);
  } else {
    const int Sp = pad_s(S);
    dim3 grid(cdiv(Sp, kVTile), BH);
    if (fmt == THRIFT_NVFP4) {
      if (D == 128)
        quant_s_kernel<THRIFT_NVFP4, 128><<<grid, kQThreads, 0, stream>>>(x, S, Sp, 0, tensor_scale, codes, scales);
      else
        quant_s_kernel<THRIFT_NVFP4, 64><<<grid, kQThreads, 0, stream>>>(x, S, Sp, 0, tensor_scale, codes, scales);
    } else {
      if (D == 128)
        quant_s_kernel<THRIFT_MXFP4, 128><<<grid, kQThreads, 0, stream>>>(x, S, Sp, 0, tensor_scale, codes, scales);
      else
        quant_s_kernel<THRIFT_MXFP4, 64><<<grid, kQThreads, 0, stream>>>(x, S, Sp, 0, tensor_scale, codes, scales);
    }
  }
  return launch_status();
}

extern "C" thrift_status thrift_quantize_fp4_range(const void* x16, int B, int H, int S, int D,
                                                   int axis, int fmt, int s0,
                                                   int s1, uint8_t* codes, uint8_t* scales,
                                                   const float* tensor_scale, hipStream_t stream) {
  if (!x16 || !codes || !scales) return THRIFT_EINVAL;
  if (B < 1 || H < 1 || S < 1 || s0 < 0 || s1 > S || s0 >= s1) return THRIFT_EINVAL;
  if (fmt != THRIFT_NVFP4 && fmt != THRIFT_MXFP4) return THRIFT_EINVAL;
  if (axis != THRIFT_GROUP_D && axis != THRIFT_GROUP_S) return THRIFT_EINVAL;
  if (fmt == THRIFT_NVFP4 && !tensor_scale) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if (S > 262144) return THRIFT_EUNSUPPORTED;
  if (!aligned16(x16) || !aligned16(codes)) return THRIFT_EALIGN;
  const int BH = B * H;
  auto x = (const _Float16*)x16;
  const bool nv = fmt == THRIFT_NVFP4;
  if (axis == THRIFT_GROUP_D) {
    const int gpr = D / (nv ? 16 : 32);  // groups per row
    const int gps = S * gpr, range = (s1 - s0) * gpr;
    const size_t ngroups = (size_t)BH * range;
    const int blocks = (int)((ngroups + kQThreads - 1) / kQThreads);
    if (nv)
      quant_d_kernel<THRIFT_NVFP4><<<blocks, kQThreads, 0, stream>>>(x, ngroups, gps, range, s0 * gpr,
                                                                       tensor_scale, codes, scales);
    else
      quant_d_kernel<THRIFT_MXFP4><<<blocks, kQThreads, 0, stream>>>(x, ngroups, gps, range, s0 * gpr,
                                                                       nullptr, codes, scales);
  } else {
    const int Sp = pad_s(S), t0 = s0 / kVTile, t1 = cdiv(s1, kVTile);
    dim3 grid(t1 - t0, BH);
    if (nv) {
      if (D == 128)
        quant_s_kernel<THRIFT_NVFP4, 128><<<grid, kQThreads, 0, stream>>>(x, S, Sp, t0, tensor_scale, codes, scales);
      else
        quant_s_kernel<THRIFT_NVFP4, 64><<<grid, kQThreads, 0, stream>>>(x, S, Sp, t0, tensor_scale, codes, scales);
    } else {
      if (D == 128)
        quant_s_kernel<THRIFT_MXFP4, 128><<<grid, kQThreads, 0, stream>>>(x, S, Sp, t0, nullptr, codes, scales);
      else
        quant_s_kernel<THRIFT_MXFP4, 64><<<grid, kQThreads, 0, stream>>>(x, S, Sp, t0, nullptr, codes, scales);
    }
  }
  return launch_status();
}

extern "C" size_t thrift_quantize_means_workspace_bytes(int B, int H, int S, int D, int fmt,
                                                        int blk) {
  if (B < 1 || H < 1 || S < 1 || D < 1 || blk < 1) return 0;
  if (fmt != THRIFT_NVFP4) return 0;
  return (size_t)B * H * cdiv(S, blk) * sizeof(float);
}

extern "C" thrift_status thrift_quantize_fp4_means(const void* x16, int B, int H, int S, int D,
                                                   int fmt, int blk, uint8_t* codes,
                                                   uint8_t* scales, float* tensor_scale, float* means,
                                                   void* workspace, size_t workspace_bytes,
                                                   hipStream_t stream) {
  if (!x16 || !codes || !scales || !means) return THRIFT_EINVAL;
  if (B < 1 || H < 1 || S < 1 || blk < 1) return THRIFT_EINVAL;
  if (fmt != THRIFT_NVFP4 && fmt != THRIFT_MXFP4) return THRIFT_EINVAL;
  if (fmt == THRIFT_NVFP4 && !tensor_scale) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if (S > 262144 || B * H > 65535) return THRIFT_EUNSUPPORTED;
  if (!aligned16(x16) || !aligned16(codes) || !aligned16(means)) return THRIFT_EALIGN;
  const size_t need = thrift_quantize_means_workspace_bytes(B, H, S, D, fmt, blk);
  if (need && (!workspace || workspace_bytes < need)) return THRIFT_EWORKSPACE;
  const int BH = B * H, nb = cdiv(S, blk);
  auto x = (const _Float16*)x16;
  dim3 grid(nb, BH);
  if (fmt == THRIFT_MXFP4) {
    if (D == 128)
      means_quant_kernel<128, THRIFT_MXFP4><<<grid, kQThreads, 0, stream>>>(x, S, blk, nb, means, codes, scales, nullptr);
    else
      means_quant_kernel<64, THRIFT_MXFP4><<<grid, kQThreads, 0, stream>>>(x, S, blk, nb, means, codes, scales, nullptr);
  } else {
    float* part = (float*)workspace;
    if (D == 128)
      means_quant_kernel<128, THRIFT_NVFP4><<<grid, kQThreads, 0, stream>>>(x, S, blk, nb, means, codes, scales, part);
    else
      means_quant_kernel<64, THRIFT_NVFP4><<<grid, kQThreads, 0, stream>>>(x, S, blk, nb, means, codes, scales, part);
    slice_scale_kernel<<<cdiv(BH, 256), 256, 0, stream>>>(part, nb, BH, tensor_scale);
    const size_t ngroups = (size_t)BH * S * (D / 16);
    const int blocks = (int)((ngroups + kQThreads - 1) / kQThreads);
    const int gps = S * (D / 16);
    quant_d_kernel<THRIFT_NVFP4><<<blocks, kQThreads, 0, stream>>>(x, ngroups, gps, gps, 0, tensor_scale,
                                                                     codes, scales);
  }
  return launch_status();
}

extern "C" thrift_status thrift_cache_update(const void* k16, const void* v16, int B, int H, int S, int D,
                                             int block_k, int s0, int s1, int fmt, float* kbar,
                                             uint8_t* k4_codes, uint8_t* k4_scales, const float* k4_tscale,
                                             uint8_t* v4_codes, uint8_t* v4_scales, const float* v4_tscale,
                                             hipStream_t stream) {
  if (!k16 || !v16 || !kbar || !k4_codes || !k4_scales || !v4_codes || !v4_scales) return THRIFT_EINVAL;
  if (B < 1 || H < 1 || S < 1 || block_k < 1 || s0 < 0 || s1 > S || s0 >= s1) return THRIFT_EINVAL;
  if (fmt != THRIFT_NVFP4 && fmt != THRIFT_MXFP4) return THRIFT_EINVAL;
  if (fmt == THRIFT_NVFP4 && (!k4_tscale || !v4_tscale)) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if (S > 262144 || B * H > 65535) return THRIFT_EUNSUPPORTED;
  if (!aligned16(k16) || !aligned16(v16) || !aligned16(kbar) || !aligned16(k4_codes) || !aligned16(v4_codes))
    return THRIFT_EALIGN;
  const int g = fmt == THRIFT_NVFP4 ? 16 : 32;
  const int j0 = s0 / block_k, nmeans = (s1 - 1) / block_k - j0 + 1, nb = cdiv(S, block_k);
  const int ndg = cdiv((s1 - s0) * (D / g), kQThreads);
  const int t0 = s0 / kVTile, ntiles = cdiv(s1, kVTile) - t0;
  const dim3 grid(nmeans + ndg + ntiles, B * H);
  auto k = (const _Float16*)k16;
  auto v = (const _Float16*)v16;
#define THRIFT_CACHE_UPDATE(F, DD)                                                                          \
  cache_update_kernel<F, DD><<<grid, kQThreads, 0, stream>>>(k, v, S, block_k, nb, j0, nmeans, s0, s1, ndg, t0, \
                                                            kbar, k4_tscale, k4_codes, k4_scales, v4_tscale,   \
                                                            v4_codes, v4_scales)
  if (fmt == THRIFT_MXFP4) {
    if (D == 128)
      THRIFT_CACHE_UPDATE(THRIFT_MXFP4, 128);
    else
      THRIFT_CACHE_UPDATE(THRIFT_MXFP4, 64);
  } else {
    if (D == 128)
      THRIFT_CACHE_UPDATE(THRIFT_NVFP4, 128);
    else
      THRIFT_CACHE_UPDATE(THRIFT_NVFP4, 64);
  }
#undef THRIFT_CACHE_UPDATE
  return launch_status();
}

extern "C" thrift_status thrift_quantize_fp8(const void* x16, int B, int H, int S, int D, int axis,
                                             uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (!x16 || !codes || !scales) return THRIFT_EINVAL;
  if (B < 1 || H < 1 || S < 1) return THRIFT_EINVAL;
  if (axis != THRIFT_GROUP_D && axis != THRIFT_GROUP_S) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if (S > 262144 || B * H > 65535) return THRIFT_EUNSUPPORTED;
  if (!aligned16(x16) || !aligned16(codes)) return THRIFT_EALIGN;
  auto x = (const _Float16*)x16;
  if (axis == THRIFT_GROUP_D) {
    const size_t ngroups = (size_t)B * H * S * (D / 32);
    quant8_d_kernel<<<(int)((ngroups + kQThreads - 1) / kQThreads), kQThreads, 0, stream>>>(x, ngroups, codes,
                                                                                          scales);
  } else {
    const int Sp = pad_s(S);
    const dim3 grid(cdiv(Sp, kVTile), B * H);
    if (D == 128)
      quant8_s_kernel<128><<<grid, kQThreads, 0, stream>>>(x, S, Sp, codes, scales);
    else
      quant8_s_kernel<64><<<grid, kQThreads, 0, stream>>>(x, S, Sp, codes, scales);
  }
  return launch_status();
}
