// Block selection of ThriftAttention on gfx950: block means, pair scores and
// the per-query-block top-k (ThriftAttention summaries, "Heuristische
// Blokkenselectie": S^_ij = qbar_i . kbar_j, the top-k pairs go to FP16).
//
// Both kernels are HBM/L2-bound and tiny next to the attention kernel:
//  - block_means reads every fp16 element of Q and K once (coalesced 16-byte
//    loads) and sums in fp64, which is exact in any order, so the means are
//    bit-identical to any other exact summation;
//  - score_topk gives one workgroup to each (batch, key head, query block),
//    scoring all query heads of the GQA group against key-block means staged
//    through LDS (each kbar is read once per group, not once per head), then
//    gives each head's row of scores to one wavefront, which finds the k-th
//    largest (score, block) key with wavefront reductions only (k rounds of
//    argmax below the previous one for small k, a bitwise search from the
//    top bit otherwise) and writes the blocks at or above it in ascending
//    order by ballot compaction: no workgroup barrier in the selection.
#include "common.h"

namespace thrift {

constexpr int kMeansThreads = 256;

// means[bh][j][d] = fp32( sum_{rows of block j} x[bh][row][d] / rows ), sum in fp64.
template <int D>
__global__ __launch_bounds__(kMeansThreads) void block_means_kernel(const _Float16* __restrict__ x,
                                                                    int S, int blk, int nb,
                                                                    float* __restrict__ means) {
  constexpr int CG = D / 8;                   // 16-byte column groups per row
  constexpr int RP = kMeansThreads / CG;      // row phases
  __shared__ double red[RP][D + 1];
  const int j = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int cg = t % CG, rp = t / CG;
  const int r0 = j * blk, r1 = min(S, r0 + blk);
  const _Float16* base = x + (size_t)bh * S * D + cg * 8;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0 + rp; r < r1; r += RP) {
    v8h v = *reinterpret_cast<const v8h*>(base + (size_t)r * D);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += (double)(float)v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rp][cg * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    double s = 0.0;
    for (int k = 0; k < RP; ++k) s += red[k][t];
    means[((size_t)bh * nb + j) * D + t] = (float)(s / (double)(r1 - r0));
  }
}

// Total order on (score, block): higher score first, then lower block index.
// -0 is treated as +0.  The returned key is larger for the preferred pair.
__device__ inline uint64_t pair_key(float s, int j) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ inline int wave_sum_i32(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// One wavefront selects the k best of the n scores srow[0..n) (LDS) and
// writes them ascending into out[0..k), -1 into out[k..kmax).  The
// (score, block) keys are unique, so the k-th largest key is a threshold
// that selects exactly k blocks.
__device__ inline void wave_topk(const float* srow, int n, int k, int32_t* __restrict__ out, int kmax,
                                 int lane) {
  if (k >= n) {
    for (int e = lane; e < kmax; e += kWave) out[e] = e < n ? e : -1;
    return;
  }
  const int nc = cdiv(n, kWave);  // this lane's candidates: j = c*64 + lane
  uint64_t thr = ~0ull;
  if (k == 0) {
  } else if (k <= 32) {  // k rounds: the largest key below the previous round's
    uint64_t prev = ~0ull;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
      for (int c = 0; c < nc; ++c) {
        const int j = c * kWave + lane;
        if (j < n) {
          const uint64_t key = pair_key(srow[j], j);
          if (key < prev && key > best) best = key;
        }
      }
      prev = wave_max_u64(best);
    }
    thr = prev;
  } else {  // the largest t with at least k keys >= t, one bit at a time
    uint64_t prefix = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t cand = prefix | (1ull << bit);
      int cntv = 0;
      for (int c = 0; c < nc; ++c) {
        const int j = c * kWave + lane;
        cntv += (j < n && pair_key(srow[j], j) >= cand) ? 1 : 0;
      }
      if (wave_sum_i32(cntv) >= k) prefix = cand;
    }
    thr = prefix;
  }
  int base = 0;
  for (int c = 0; c < nc; ++c) {
    const int j = c * kWave + lane;
    const bool sel = k > 0 && j < n && pair_key(srow[j], j) >= thr;
    const uint64_t bal = __ballot(sel);
    if (sel) out[base + __popcll(bal & ((1ull << lane) - 1))] = j;
    base += __popcll(bal);
  }
  for (int e = k + lane; e < kmax; e += kWave) out[e] = -1;
}

constexpr int kTopkThreads = 256;
constexpr int kHeadChunk = 4;     // query heads scored together per pass
constexpr int kKeyChunk = 256;    // key blocks staged per pass (one per thread)
constexpr int kDimChunk = 32;     // channels staged per pass

template <int D>
__global__ __launch_bounds__(kTopkThreads) void score_topk_kernel(
    const float* __restrict__ qm, const float* __restrict__ km, int Hq, int Hkv, int Sq, int Sk, int bq,
    int bk, int causal, int topk_count, int topk_bp, int32_t* __restrict__ idx,
    int32_t* __restrict__ cnt, int kmax) {
  extern __shared__ float sc[];  // [kHeadChunk][nK] scores
  __shared__ float qv[kHeadChunk][D];
  __shared__ float kst[kKeyChunk][kDimChunk + 1];

  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int i = blockIdx.x, bhk = blockIdx.y;
  const int b = bhk / Hkv, hk = bhk % Hkv, G = Hq / Hkv;
  const int nq = cdiv(Sq, bq), nK = cdiv(Sk, bk);
  const int n = valid_kv_blocks_kv(i, Sq, Sk, bq, bk, causal);
  const int k = topk_budget(n, topk_count, topk_bp);
  const float* kbase = km + (size_t)bhk * nK * D;

  for (int h0 = 0; h0 < G; h0 += kHeadChunk) {
    const int nh = min(kHeadChunk, G - h0);
    __syncthreads();
    for (int e = t; e < kHeadChunk * D; e += kTopkThreads) {
      int h = e / D, d = e % D;
      int hq = hk * G + h0 + h;
      qv[h][d] = h < nh ? qm[(((size_t)b * Hq + hq) * nq + i) * D + d] : 0.0f;
    }
    // scores: one key block per thread, fp32 FMA chain over ascending channels
    for (int jc = 0; jc < n; jc += kKeyChunk) {
      float s[kHeadChunk];
#pragma unroll
      for (int h = 0; h < kHeadChunk; ++h) s[h] = 0.0f;
      for (int dc = 0; dc < D; dc += kDimChunk) {
        __syncthreads();
        for (int e = t; e < kKeyChunk * kDimChunk; e += kTopkThreads) {
          int kk = e / kDimChunk, dd = e % kDimChunk;
          kst[kk][dd] = (jc + kk < n) ? kbase[(size_t)(jc + kk) * D + dc + dd] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int dd = 0; dd < kDimChunk; ++dd) {
          float kvv = kst[t][dd];
#pragma unroll
          for (int h = 0; h < kHeadChunk; ++h) s[h] = __builtin_fmaf(qv[h][dc + dd], kvv, s[h]);
        }
      }
      if (jc + t < n)
        for (int h = 0; h < nh; ++h) sc[h * nK + jc + t] = s[h];
    }
    __syncthreads();

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    for (int h = wave_u; h < nh; h += kTopkThreads / kWave) {  // one wavefront per head row
      const int hq = hk * G + h0 + h;
      const size_t row = ((size_t)b * Hq + hq) * nq + i;
      wave_topk(sc + h * nK, n, k, idx + row * kmax, kmax, lane);
      if (lane == 0) cnt[row] = k;
    }
  }
}

}  // namespace thrift

using namespace thrift;

extern "C" int thrift_select_kmax_kv(int Sq, int Sk, int block_q, int block_k, int causal,
                                     int topk_count, int topk_bp) {
  if (Sq < 1 || Sk < Sq || block_q < 1 || block_k < 1 || (topk_count < 0 && topk_bp < 0)) return -1;
  int nq = cdiv(Sq, block_q), km = 0;
  for (int i = 0; i < nq; ++i) {
    int k = topk_budget(valid_kv_blocks_kv(i, Sq, Sk, block_q, block_k, causal), topk_count, topk_bp);
    km = k > km ? k : km;
  }
  return km;
}

extern "C" int thrift_select_kmax(int S, int block_q, int block_k, int causal, int topk_count,
                                  int topk_bp) {
  return thrift_select_kmax_kv(S, S, block_q, block_k, causal, topk_count, topk_bp);
}

extern "C" size_t thrift_select_workspace_bytes_kv(int B, int Hq, int Hkv, int Sq, int Sk, int D,
                                                   int block_q, int block_k) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1 || block_q < 1 || block_k < 1) return 0;
  size_t qbytes = (size_t)B * Hq * cdiv(Sq, block_q) * D * sizeof(float);
  size_t kbytes = (size_t)B * Hkv * cdiv(Sk, block_k) * D * sizeof(float);
  return ((qbytes + 255) / 256) * 256 + kbytes;
}

extern "C" size_t thrift_select_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int block_q,
                                                int block_k) {
  return thrift_select_workspace_bytes_kv(B, Hq, Hkv, S, S, D, block_q, block_k);
}

extern "C" thrift_status thrift_select_blocks_kv(const void* q16, const void* k16, int B, int Hq,
                                                 int Hkv, int Sq, int Sk, int D, int block_q,
                                                 int block_k, int causal, int topk_count,
                                                 int topk_bp, int32_t* idx, int32_t* cnt, int kmax,
                                                 void* workspace, size_t workspace_bytes,
                                                 hipStream_t stream) {
  if (!q16 || !k16 || !idx || !cnt || !workspace) return THRIFT_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < Sq || (causal != 0 && causal != 1)) return THRIFT_EINVAL;
  if (Hq % Hkv != 0) return THRIFT_EINVAL;
  if (topk_count < 0 && (topk_bp < 0 || topk_bp > 10000)) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if ((block_q != 64 && block_q != 128) || block_k != 64) return THRIFT_EUNSUPPORTED;
  if (Sk > 262144) return THRIFT_EUNSUPPORTED;
  int need = thrift_select_kmax_kv(Sq, Sk, block_q, block_k, causal, topk_count, topk_bp);
  if (kmax < need || kmax < 1) return THRIFT_EINVAL;
  if (!aligned16(q16) || !aligned16(k16) || !aligned16(workspace)) return THRIFT_EALIGN;
  if (workspace_bytes < thrift_select_workspace_bytes_kv(B, Hq, Hkv, Sq, Sk, D, block_q, block_k))
    return THRIFT_EWORKSPACE;
  const int nq = cdiv(Sq, block_q), nk = cdiv(Sk, block_k);
  float* qm = (float*)workspace;
  size_t qbytes = (size_t)B * Hq * nq * D * sizeof(float);
  float* km = (float*)((char*)workspace + ((qbytes + 255) / 256) * 256);
  auto q = (const _Float16*)q16;
  auto k = (const _Float16*)k16;
  const size_t lds = (size_t)kHeadChunk * nk * sizeof(float);
  static bool configured = false;  // allow more than the default dynamic LDS for long S
  if (!configured) {
    if (hipFuncSetAttribute((const void*)score_topk_kernel<128>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024) != hipSuccess ||
        hipFuncSetAttribute((const void*)score_topk_kernel<64>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024) != hipSuccess)
      return THRIFT_EHIP;
    configured = true;
  }
  if (D == 128) {
    block_means_kernel<128><<<dim3(nq, B * Hq), kMeansThreads, 0, stream>>>(q, Sq, block_q, nq, qm);
    block_means_kernel<128><<<dim3(nk, B * Hkv), kMeansThreads, 0, stream>>>(k, Sk, block_k, nk, km);
    score_topk_kernel<128><<<dim3(nq, B * Hkv), kTopkThreads, lds, stream>>>(
        qm, km, Hq, Hkv, Sq, Sk, block_q, block_k, causal, topk_count, topk_bp, idx, cnt, kmax);
  } else {
    block_means_kernel<64><<<dim3(nq, B * Hq), kMeansThreads, 0, stream>>>(q, Sq, block_q, nq, qm);
    block_means_kernel<64><<<dim3(nk, B * Hkv), kMeansThreads, 0, stream>>>(k, Sk, block_k, nk, km);
    score_topk_kernel<64><<<dim3(nq, B * Hkv), kTopkThreads, lds, stream>>>(
        qm, km, Hq, Hkv, Sq, Sk, block_q, block_k, causal, topk_count, topk_bp, idx, cnt, kmax);
  }
  return launch_status();
}

extern "C" thrift_status thrift_select_blocks(const void* q16, const void* k16, int B, int Hq,
                                              int Hkv, int S, int D, int block_q, int block_k,
                                              int causal, int topk_count, int topk_bp,
                                              int32_t* idx, int32_t* cnt, int kmax,
                                              void* workspace, size_t workspace_bytes,
                                              hipStream_t stream) {
  return thrift_select_blocks_kv(q16, k16, B, Hq, Hkv, S, S, D, block_q, block_k, causal, topk_count,
                                 topk_bp, idx, cnt, kmax, workspace, workspace_bytes, stream);
}
