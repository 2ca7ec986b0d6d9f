// Block selection of ThriftAttention on gfx950: block means, pair scores and
// the per-query-block top-k (ThriftAttention summaries, "Heuristische
// Blokkenselectie": S^_ij = qbar_i . kbar_j, the top-k pairs go to FP16).
//
// Both kernels are HBM/L2-bound and tiny next to the attention kernel:
//  - block_means reads every fp16 element of Q and K once (coalesced 16-byte
//    loads) and sums in fp64, which is exact in any order, so the means are
//    bit-identical to any other exact summation;
//  - score_topk gives one workgroup to each (batch, key head, run of up to
//    four query blocks); each thread scores one key block against up to four
//    query heads of the GQA group in each of those query blocks (each kbar
//    row read once per sixteen score rows, all of it in flight at once), then each head's row of scores goes to one wavefront,
//    which finds the k-th largest score by a bitwise search counted with
//    ballots, breaks ties at it by lower block index, and writes the blocks
//    in ascending order by ballot compaction: no workgroup barrier in the
//    selection.
#include "common.h"

namespace thrift {

constexpr int kMeansThreads = 256;

// means[bh][j][d] = fp32( sum_{rows of block j} x[bh][row][d] / rows ), sum in fp64.
template <int D>
__global__ __launch_bounds__(kMeansThreads) void block_means_kernel(const _Float16* __restrict__ x,
                                                                    int S, int blk, int nb, int j0,
                                                                    float* __restrict__ means) {
  constexpr int CG = D / 8;                   // 16-byte column groups per row
  constexpr int RP = kMeansThreads / CG;      // row phases
  __shared__ double red[RP][D + 1];
  const int j = j0 + blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
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

// Scores as unsigned keys with the order of the floats: -0 maps to +0, and
// every finite score maps above 0, so 0 can stand for "no block here".
__device__ inline uint32_t score_key(float s) {
  const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The keys of the first kRegChunks chunks of a row stay in registers during
// the search; chunks beyond (rows of more than 512 blocks) are re-read from LDS.
constexpr int kRegChunks = 8;

// One wavefront selects the k best of the n scores srow[0..n) (LDS): higher
// score first, equal scores by lower block index.  It writes them ascending
// into out[0..k) and -1 into out[k..kmax).
//   1. T = the k-th largest key: the largest t with at least k keys >= t,
//      found one bit at a time from the top; each count is a sum of ballot
//      popcounts over the row's chunks (lane l of chunk c holds block c*64+l).
//      The search stops early at a prefix with exactly k keys at or above
//      it: those keys are then the selection whatever the lower bits of T.
//   2. Every block with key > T is selected (fewer than k of them); of the
//      blocks with key == T the lowest-indexed k - count(> T) are selected,
//      ranked by a running ballot prefix in ascending block order.
__device__ inline void wave_topk(const float* srow, int n, int k, int32_t* __restrict__ out, int kmax,
                                 int lane) {
  if (k >= n) {
    for (int e = lane; e < kmax; e += kWave) out[e] = e < n ? e : -1;
    return;
  }
  const int nc = cdiv(n, kWave);
  const uint64_t below = (1ull << lane) - 1;
  auto key_at = [&](int c) -> uint32_t {
    const int j = c * kWave + lane;
    return j < n ? score_key(srow[j]) : 0u;
  };
  uint32_t kr[kRegChunks];
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) kr[c] = c < nc ? key_at(c) : 0u;
  auto count_ge = [&](uint32_t t) {
    int m = 0;
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c)
      if (c < nc) m += __popcll(__ballot(kr[c] >= t));
    for (int c = kRegChunks; c < nc; ++c) m += __popcll(__ballot(key_at(c) >= t));
    return m;
  };
  uint32_t thr = 0;
  if (k > 0)
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      const int m = count_ge(cand);
      if (m >= k) {
        thr = cand;
        if (m == k) break;  // step 2 then takes every key >= thr
      }
    }
  // k > 0: thr >= the smallest finite key > 0, so padding (key 0) never ties
  const int need = k > 0 ? k - (thr == 0xFFFFFFFFu ? 0 : count_ge(thr + 1)) : 0;
  int base = 0, eq_seen = 0;
  auto emit = [&](int c, uint32_t u) {
    const uint64_t eq = __ballot(k > 0 && u == thr);
    const bool sel = k > 0 && (u > thr || (u == thr && eq_seen + __popcll(eq & below) < need));
    const uint64_t bal = __ballot(sel);
    if (sel) out[base + __popcll(bal & below)] = c * kWave + lane;
    base += __popcll(bal);
    eq_seen += __popcll(eq);
  };
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c)
    if (c < nc) emit(c, kr[c]);
  for (int c = kRegChunks; c < nc; ++c) emit(c, key_at(c));
  for (int e = k + lane; e < kmax; e += kWave) out[e] = -1;
}

constexpr int kTopkThreads = 256;
constexpr int kHeadChunk = 4;  // query heads scored together per pass

// QB consecutive query blocks share a workgroup, so each k̄ row is read once
// for QB x (up to) four query-head rows.  With OUT (per-head budgets) the
// scores of the valid pairs go to scores_out [B,Hq,nQ,nK] instead of a
// per-row top-k.
template <int D, int QB, bool OUT = false, int HC = kHeadChunk>
__global__ __launch_bounds__(kTopkThreads) void score_topk_kernel(
    const float* __restrict__ qm, const float* __restrict__ km, int Hq, int Hkv, int Sq, int Sk, int bq,
    int bk, int causal, int topk_count, int topk_bp, int32_t* __restrict__ idx,
    int32_t* __restrict__ cnt, int kmax, float* __restrict__ scores_out = nullptr) {
  // HC query heads per pass; with HC < kHeadChunk the group's heads are
  // spread over blockIdx.z (more workgroups when there are few query blocks)
  constexpr int NR = QB * HC;  // score rows per pass: (query block, head)
  extern __shared__ float sc[];         // [NR][nK] scores
  __shared__ __attribute__((aligned(16))) float qv[NR][D];

  const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
  const int i0 = blockIdx.x * QB, bhk = blockIdx.y;
  const int b = bhk / Hkv, hk = bhk % Hkv, G = Hq / Hkv;
  const int nq = cdiv(Sq, bq), nK = cdiv(Sk, bk);
  const int nqb = min(QB, nq - i0);  // query blocks of this workgroup
  // valid key blocks grow with the query block under causal masking
  const int nmax = valid_kv_blocks_kv(i0 + nqb - 1, Sq, Sk, bq, bk, causal);
  const float* kbase = km + (size_t)bhk * nK * D;

  const int hz = HC < kHeadChunk ? (int)blockIdx.z * HC : 0;
  const int hend = HC < kHeadChunk ? min(G, hz + HC) : G;
  for (int h0 = hz; h0 < hend; h0 += HC) {
    const int nh = min(HC, hend - h0);
    __syncthreads();
    for (int e = t; e < NR * D; e += kTopkThreads) {
      const int rr = e / D, d = e % D, qb = rr / HC, h = rr % HC;
      const int hq = hk * G + h0 + h;
      qv[rr][d] = (h < nh && qb < nqb) ? qm[(((size_t)b * Hq + hq) * nq + i0 + qb) * D + d] : 0.0f;
    }
    __syncthreads();
    // scores: one key block per thread, its whole mean row loaded at once
    // (independent loads, one memory latency per 256 blocks), then an fp32
    // FMA chain over ascending channels per (query block, head) row
    for (int jc = 0; jc < nmax; jc += kTopkThreads) {
      const int j = jc + t;
      if (j < nmax) {
        const float4* kr = reinterpret_cast<const float4*>(kbase + (size_t)j * D);
        float s[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) s[r] = 0.0f;
        float4 kv[D / 4];
#pragma unroll
        for (int c = 0; c < D / 4; ++c) kv[c] = kr[c];
        // the scheduling barriers keep the compiler from reading every
        // query mean (NR x D floats) ahead of the FMAs, which would not fit
        // in registers
#pragma unroll
        for (int c = 0; c < D / 4; ++c) {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const float4 qq = *reinterpret_cast<const float4*>(&qv[r][4 * c]);
            s[r] = __builtin_fmaf(qq.x, kv[c].x, s[r]);
            s[r] = __builtin_fmaf(qq.y, kv[c].y, s[r]);
            s[r] = __builtin_fmaf(qq.z, kv[c].z, s[r]);
            s[r] = __builtin_fmaf(qq.w, kv[c].w, s[r]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // every row of sc is written (rows past the valid ones are never
        // read): a conditional store would let the compiler sink the FMA
        // chains below all the query-mean reads
#pragma unroll
        for (int r = 0; r < NR; ++r) sc[r * nK + j] = s[r];
      }
    }
    __syncthreads();

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    for (int rr = wave_u; rr < NR; rr += kTopkThreads / kWave) {  // one wavefront per row
      const int qb = rr / HC, h = rr % HC;
      if (qb >= nqb || h >= nh) continue;
      const int i = i0 + qb, hq = hk * G + h0 + h;
      const int n = valid_kv_blocks_kv(i, Sq, Sk, bq, bk, causal);
      const int k = topk_budget(n, topk_count, topk_bp);
      const size_t row = ((size_t)b * Hq + hq) * nq + i;
      if constexpr (OUT) {
        for (int j = lane; j < n; j += kWave) scores_out[row * nK + j] = sc[rr * nK + j];
      } else {
        wave_topk(sc + rr * nK, n, k, idx + row * kmax, kmax, lane);
        if (lane == 0) cnt[row] = k;
      }
    }
  }
}

// ---- per-head budget: one top-k over all valid pairs of a query head ----------

// The K-th largest key T of each head's valid pairs, by a most-significant-
// digit-first radix select over the flat [nQ][nK] score array: four 8-bit
// digits, each pass a 256-bin histogram of the keys that match the digits
// fixed so far.  Every pass runs over many workgroups per head (LDS
// histograms, added into the head's global one), then one small kernel per
// pass picks the digit.  Per head, hs[bh] = {prefix, mask, kk, K}: the
// digits fixed so far, their mask, how many keys are still to take below
// the fixed prefix, and the budget.
constexpr int kHistChunk = 4096;  // flat entries per histogram workgroup

__device__ inline long long head_pairs(int Sq, int Sk, int bq, int bk, int causal) {
  long long P = 0;
  for (int i = 0, nq = cdiv(Sq, bq); i < nq; ++i) P += valid_kv_blocks_kv(i, Sq, Sk, bq, bk, causal);
  return P;
}

// hs[bh] = {0, 0, K, K}; the global histograms cleared.
__global__ __launch_bounds__(256) void head_init_kernel(int Sq, int Sk, int bq, int bk, int causal, int topk_count,
                                                        int topk_bp, uint32_t* __restrict__ hs,
                                                        uint32_t* __restrict__ ghist) {
  const int bh = blockIdx.x, t = threadIdx.x;
  ghist[(size_t)bh * 256 + t] = 0;
  if (t == 0) {
    const long long P = head_pairs(Sq, Sk, bq, bk, causal);
    long long K = topk_count >= 0 ? (long long)topk_count : (P * topk_bp + 9999) / 10000;
    K = K < P ? K : P;
    hs[4 * bh + 0] = 0;
    hs[4 * bh + 1] = 0;
    hs[4 * bh + 2] = (uint32_t)K;
    hs[4 * bh + 3] = (uint32_t)K;
  }
}

// One pass: the histogram of digit `shift` over the keys matching hs's prefix.
__global__ __launch_bounds__(256) void head_hist_kernel(const float* __restrict__ scores, int Sq, int Sk, int bq,
                                                        int bk, int causal, int shift,
                                                        const uint32_t* __restrict__ hs,
                                                        uint32_t* __restrict__ ghist) {
  __shared__ uint32_t hist[256];
  const int t = threadIdx.x, bh = blockIdx.y;
  const int nq = cdiv(Sq, bq), nK = cdiv(Sk, bk), total = nq * nK;
  const uint32_t prefix = hs[4 * bh + 0], mask = hs[4 * bh + 1];
  if (hs[4 * bh + 3] == 0) return;  // K == 0: nothing to select
  hist[t] = 0;
  __syncthreads();
  const float* sh = scores + (size_t)bh * nq * nK;
  const int e_end = min(total, (blockIdx.x + 1) * kHistChunk);
  for (int e0 = blockIdx.x * kHistChunk + t; e0 < e_end; e0 += 8 * 256) {
    uint32_t u[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {  // eight independent loads in flight
      const int e = e0 + r * 256;
      u[r] = 0u;
      if (e < e_end) {
        const int i = e / nK;
        if (e - i * nK < valid_kv_blocks_kv(i, Sq, Sk, bq, bk, causal)) u[r] = score_key(sh[e]);
      }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (u[r] != 0u && (u[r] & mask) == prefix) atomicAdd(&hist[(u[r] >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (hist[t]) atomicAdd(&ghist[(size_t)bh * 256 + t], hist[t]);
}

// One pass: the digit where the count from the top reaches kk; hs updated,
// the global histogram cleared for the next pass.
__global__ __launch_bounds__(256) void head_pick_kernel(int shift, uint32_t* __restrict__ hs,
                                                        uint32_t* __restrict__ ghist) {
  __shared__ uint32_t h[256];
  const int t = threadIdx.x, bh = blockIdx.x;
  h[t] = ghist[(size_t)bh * 256 + t];
  ghist[(size_t)bh * 256 + t] = 0;
  __syncthreads();
  if (t == 0 && hs[4 * bh + 3] != 0) {
    const uint32_t kk = hs[4 * bh + 2];
    uint32_t cum = 0;
    int dsel = 0;
    for (int d = 255; d >= 0; --d) {
      if (cum + h[d] >= kk) {
        dsel = d;
        break;
      }
      cum += h[d];
    }
    hs[4 * bh + 0] |= (uint32_t)dsel << shift;
    hs[4 * bh + 1] |= 255u << shift;
    hs[4 * bh + 2] = kk - cum;
  }
}

// Ties at T (= the full prefix): each query block's count of keys equal to
// T, one wavefront per (batch, query head, query block).
__global__ __launch_bounds__(256) void head_eqcount_kernel(const float* __restrict__ scores, int rows, int nq,
                                                           int Sq, int Sk, int bq, int bk, int causal,
                                                           const uint32_t* __restrict__ hs,
                                                           int32_t* __restrict__ eqc) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const int bh = row / nq, i = row % nq, nK = cdiv(Sk, bk);
  const int n = valid_kv_blocks_kv(i, Sq, Sk, bq, bk, causal);
  const uint32_t T = hs[4 * bh + 0];
  const float* sr = scores + (size_t)row * nK;
  int c = 0;
  if (hs[4 * bh + 3] != 0)
    for (int j = lane; j - lane < n; j += kWave) c += __popcll(__ballot(j < n && score_key(sr[j]) == T));
  if (lane == 0) eqc[row] = c;
}

// Exclusive prefix of the tie counts over each head's query blocks (ties go
// to the lower query block, then the lower key block).
__global__ __launch_bounds__(1024) void head_scan_kernel(int nq, int32_t* __restrict__ eq) {
  __shared__ int part[1024];
  const int t = threadIdx.x, bh = blockIdx.x;
  int32_t* e = eq + (size_t)bh * nq;
  const int per = cdiv(nq, 1024), i0 = min(nq, t * per), i1 = min(nq, i0 + per);
  int mine = 0;
  for (int i = i0; i < i1; ++i) mine += e[i];
  part[t] = mine;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan of the segment sums
    const int v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t > 0 ? part[t - 1] : 0;
  for (int i = i0; i < i1; ++i) {
    const int c = e[i];
    e[i] = run;
    run += c;
  }
}

// One wavefront per (batch, query head, query block): the kept key blocks
// ascending, by ballot compaction (key > T, or key == T within the head's
// first `need` ties; state = hs after the last pass).
__global__ __launch_bounds__(256) void head_emit_kernel(const float* __restrict__ scores, int rows, int nq,
                                                         int Sq, int Sk, int bq, int bk, int causal,
                                                         const uint32_t* __restrict__ state,
                                                         const int32_t* __restrict__ eqbase,
                                                         int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ cnt, int kmax) {
  const int lane = threadIdx.x % kWave;
  const int row = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (row >= rows) return;
  const int bh = row / nq, i = row % nq, nK = cdiv(Sk, bk);
  const int n = valid_kv_blocks_kv(i, Sq, Sk, bq, bk, causal);
  const uint32_t T = state[4 * bh + 3] != 0 ? state[4 * bh + 0] : 0xFFFFFFFFu;
  const int need = state[4 * bh + 3] != 0 ? (int)state[4 * bh + 2] : 0;
  const int eq0 = eqbase[row];
  const float* sr = scores + (size_t)row * nK;
  int32_t* out = idx + (size_t)row * kmax;
  const uint64_t below = (1ull << lane) - 1;
  int base = 0, eq_seen = 0;
  for (int c = 0; c * kWave < n; ++c) {
    const int j = c * kWave + lane;
    const uint32_t u = j < n ? score_key(sr[j]) : 0u;
    const uint64_t eq = __ballot(j < n && u == T);
    const bool sel = j < n && (u > T || (u == T && eq0 + eq_seen + __popcll(eq & below) < need));
    const uint64_t bal = __ballot(sel);
    if (sel) out[base + __popcll(bal & below)] = j;
    base += __popcll(bal);
    eq_seen += __popcll(eq);
  }
  for (int e = base + lane; e < kmax; e += kWave) out[e] = -1;
  if (lane == 0) cnt[row] = base;
}

// Query blocks per workgroup: as many as keep the score rows within 64 KB of
// LDS, and one when there are few query blocks (the workgroups are then few
// and their length, not the k̄ reads, sets the time).
inline int topk_qb(int nq, int nk) { return nq < 64 ? 1 : (nk <= 1024 ? (nk <= 512 ? 4 : 2) : 1); }

template <int D, bool OUT = false>
void launch_score_topk(const float* qm, const float* km, int B, int Hq, int Hkv, int Sq, int Sk, int bq, int bk,
                       int causal, int topk_count, int topk_bp, int32_t* idx, int32_t* cnt, int kmax,
                       hipStream_t stream, float* scores_out = nullptr) {
  const int nq = cdiv(Sq, bq), nk = cdiv(Sk, bk), qb = topk_qb(nq, nk);
  if (nq < 8) {  // few query blocks (decode): one query head per workgroup
    const dim3 grid(nq, B * Hkv, Hq / Hkv);
    score_topk_kernel<D, 1, OUT, 1><<<grid, kTopkThreads, (size_t)nk * sizeof(float), stream>>>(
        qm, km, Hq, Hkv, Sq, Sk, bq, bk, causal, topk_count, topk_bp, idx, cnt, kmax, scores_out);
    return;
  }
  const size_t lds = (size_t)qb * kHeadChunk * nk * sizeof(float);
  const dim3 grid(cdiv(nq, qb), B * Hkv);
  if (qb == 4)
    score_topk_kernel<D, 4, OUT><<<grid, kTopkThreads, lds, stream>>>(
        qm, km, Hq, Hkv, Sq, Sk, bq, bk, causal, topk_count, topk_bp, idx, cnt, kmax, scores_out);
  else if (qb == 2)
    score_topk_kernel<D, 2, OUT><<<grid, kTopkThreads, lds, stream>>>(
        qm, km, Hq, Hkv, Sq, Sk, bq, bk, causal, topk_count, topk_bp, idx, cnt, kmax, scores_out);
  else
    score_topk_kernel<D, 1, OUT><<<grid, kTopkThreads, lds, stream>>>(
        qm, km, Hq, Hkv, Sq, Sk, bq, bk, causal, topk_count, topk_bp, idx, cnt, kmax, scores_out);
}

// Raise the dynamic LDS limit of every score kernel once per device (long sequences).
static thrift_status configure_score_kernels() {
  static std::atomic<uint64_t> configured{0};
  return once_per_device(configured, [] {
    const void* kernels[] = {
        (const void*)score_topk_kernel<128, 1>,       (const void*)score_topk_kernel<128, 2>,
        (const void*)score_topk_kernel<128, 4>,       (const void*)score_topk_kernel<64, 1>,
        (const void*)score_topk_kernel<64, 2>,        (const void*)score_topk_kernel<64, 4>,
        (const void*)score_topk_kernel<128, 1, true>, (const void*)score_topk_kernel<128, 2, true>,
        (const void*)score_topk_kernel<128, 4, true>, (const void*)score_topk_kernel<64, 1, true>,
        (const void*)score_topk_kernel<64, 2, true>,  (const void*)score_topk_kernel<64, 4, true>,
        (const void*)score_topk_kernel<128, 1, false, 1>, (const void*)score_topk_kernel<64, 1, false, 1>,
        (const void*)score_topk_kernel<128, 1, true, 1>,  (const void*)score_topk_kernel<64, 1, true, 1>};
    for (const void* kf : kernels)
      if (hipFuncSetAttribute(kf, hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024) != hipSuccess)
        return THRIFT_EHIP;
    return THRIFT_OK;
  });
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

// Selection from fp16 queries and keys (q16, k16: means computed here into
// the workspace) or from means the caller computed (qbar, kbar).
static thrift_status select_common(const void* q16, const float* qbar, const void* k16, const float* kbar,
                                   int B, int Hq, int Hkv, int Sq, int Sk, int D, int block_q,
                                   int block_k, int causal, int topk_count, int topk_bp, int32_t* idx,
                                   int32_t* cnt, int kmax, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  if ((!q16 && !qbar) || (!k16 && !kbar) || !idx || !cnt) return THRIFT_EINVAL;
  if (!qbar && !workspace) return THRIFT_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < Sq || (causal != 0 && causal != 1)) return THRIFT_EINVAL;
  if (Hq % Hkv != 0) return THRIFT_EINVAL;
  if (topk_count < 0 && (topk_bp < 0 || topk_bp > 10000)) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if ((block_q != 64 && block_q != 128) || block_k != 64) return THRIFT_EUNSUPPORTED;
  if (Sk > 262144) return THRIFT_EUNSUPPORTED;
  int need = thrift_select_kmax_kv(Sq, Sk, block_q, block_k, causal, topk_count, topk_bp);
  if (kmax < need || kmax < 1) return THRIFT_EINVAL;
  if ((q16 && !aligned16(q16)) || (qbar && !aligned16(qbar)) || (k16 && !aligned16(k16)) ||
      (kbar && !aligned16(kbar)) || (workspace && !aligned16(workspace)))
    return THRIFT_EALIGN;
  const int nq = cdiv(Sq, block_q), nk = cdiv(Sk, block_k);
  const size_t qbytes = (size_t)B * Hq * nq * D * sizeof(float);
  const size_t wneed = qbar ? 0 : (kbar ? qbytes : thrift_select_workspace_bytes_kv(B, Hq, Hkv, Sq, Sk, D, block_q, block_k));
  if (workspace_bytes < wneed) return THRIFT_EWORKSPACE;
  float* qm = qbar ? (float*)qbar : (float*)workspace;
  float* km = kbar ? (float*)kbar : (float*)((char*)workspace + ((qbytes + 255) / 256) * 256);
  auto q = qbar ? nullptr : (const _Float16*)q16;
  auto k = kbar ? nullptr : (const _Float16*)k16;
  if (configure_score_kernels() != THRIFT_OK) return THRIFT_EHIP;
  if (D == 128) {
    if (q) block_means_kernel<128><<<dim3(nq, B * Hq), kMeansThreads, 0, stream>>>(q, Sq, block_q, nq, 0, qm);
    if (k) block_means_kernel<128><<<dim3(nk, B * Hkv), kMeansThreads, 0, stream>>>(k, Sk, block_k, nk, 0, km);
    launch_score_topk<128>(qm, km, B, Hq, Hkv, Sq, Sk, block_q, block_k, causal, topk_count, topk_bp, idx, cnt,
                           kmax, stream);
  } else {
    if (q) block_means_kernel<64><<<dim3(nq, B * Hq), kMeansThreads, 0, stream>>>(q, Sq, block_q, nq, 0, qm);
    if (k) block_means_kernel<64><<<dim3(nk, B * Hkv), kMeansThreads, 0, stream>>>(k, Sk, block_k, nk, 0, km);
    launch_score_topk<64>(qm, km, B, Hq, Hkv, Sq, Sk, block_q, block_k, causal, topk_count, topk_bp, idx, cnt,
                          kmax, stream);
  }
  return launch_status();
}

extern "C" thrift_status thrift_select_blocks_kv(const void* q16, const void* k16, int B, int Hq,
                                                 int Hkv, int Sq, int Sk, int D, int block_q,
                                                 int block_k, int causal, int topk_count,
                                                 int topk_bp, int32_t* idx, int32_t* cnt, int kmax,
                                                 void* workspace, size_t workspace_bytes,
                                                 hipStream_t stream) {
  if (!q16 || !k16) return THRIFT_EINVAL;
  return select_common(q16, nullptr, k16, nullptr, B, Hq, Hkv, Sq, Sk, D, block_q, block_k, causal, topk_count,
                       topk_bp, idx, cnt, kmax, workspace, workspace_bytes, stream);
}

extern "C" thrift_status thrift_select_blocks_kbar(const void* q16, const float* kbar, int B, int Hq,
                                                   int Hkv, int Sq, int Sk, int D, int block_q,
                                                   int block_k, int causal, int topk_count,
                                                   int topk_bp, int32_t* idx, int32_t* cnt, int kmax,
                                                   void* workspace, size_t workspace_bytes,
                                                   hipStream_t stream) {
  if (!q16 || !kbar) return THRIFT_EINVAL;
  return select_common(q16, nullptr, nullptr, kbar, B, Hq, Hkv, Sq, Sk, D, block_q, block_k, causal, topk_count,
                       topk_bp, idx, cnt, kmax, workspace, workspace_bytes, stream);
}

extern "C" thrift_status thrift_select_blocks_means(const float* qbar, const float* kbar, int B, int Hq,
                                                    int Hkv, int Sq, int Sk, int D, int block_q,
                                                    int block_k, int causal, int topk_count,
                                                    int topk_bp, int32_t* idx, int32_t* cnt, int kmax,
                                                    hipStream_t stream) {
  if (!qbar || !kbar) return THRIFT_EINVAL;
  return select_common(nullptr, qbar, nullptr, kbar, B, Hq, Hkv, Sq, Sk, D, block_q, block_k, causal,
                       topk_count, topk_bp, idx, cnt, kmax, nullptr, 0, stream);
}

extern "C" thrift_status thrift_block_means(const void* x16, int B, int H, int S, int D, int blk, int j0,
                                            int j1, float* means, hipStream_t stream) {
  if (!x16 || !means || B < 1 || H < 1 || S < 1 || blk < 1) return THRIFT_EINVAL;
  const int nb = cdiv(S, blk);
  if (j0 < 0 || j1 > nb || j0 >= j1) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if (S > 262144 || B * H > 65535) return THRIFT_EUNSUPPORTED;
  if (!aligned16(x16)) return THRIFT_EALIGN;
  auto x = (const _Float16*)x16;
  if (D == 128)
    block_means_kernel<128><<<dim3(j1 - j0, B * H), kMeansThreads, 0, stream>>>(x, S, blk, nb, j0, means);
  else
    block_means_kernel<64><<<dim3(j1 - j0, B * H), kMeansThreads, 0, stream>>>(x, S, blk, nb, j0, means);
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

extern "C" int thrift_select_head_kmax(int Sq, int Sk, int block_q, int block_k, int causal) {
  if (Sq < 1 || Sk < Sq || block_q < 1 || block_k < 1) return -1;
  return valid_kv_blocks_kv(cdiv(Sq, block_q) - 1, Sq, Sk, block_q, block_k, causal);  // the largest n_i
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

extern "C" size_t thrift_select_head_workspace_bytes(int B, int Hq, int Sq, int Sk, int block_q, int block_k) {
  if (B < 1 || Hq < 1 || Sq < 1 || Sk < 1 || block_q < 1 || block_k < 1) return 0;
  const size_t rows = (size_t)B * Hq * cdiv(Sq, block_q);
  return align256(rows * cdiv(Sk, block_k) * sizeof(float)) + align256((size_t)B * Hq * 4 * sizeof(uint32_t)) +
         align256((size_t)B * Hq * 256 * sizeof(uint32_t)) + align256(rows * sizeof(int32_t));
}

extern "C" thrift_status thrift_select_blocks_head(const float* qbar, const float* kbar, int B, int Hq,
                                                   int Hkv, int Sq, int Sk, int D, int block_q,
                                                   int block_k, int causal, int topk_count, int topk_bp,
                                                   int32_t* idx, int32_t* cnt, int kmax, void* workspace,
                                                   size_t workspace_bytes, hipStream_t stream) {
  if (!qbar || !kbar || !idx || !cnt || !workspace) return THRIFT_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < Sq || (causal != 0 && causal != 1)) return THRIFT_EINVAL;
  if (Hq % Hkv != 0) return THRIFT_EINVAL;
  if (topk_count < 0 && (topk_bp < 0 || topk_bp > 10000)) return THRIFT_EINVAL;
  if (D != 64 && D != 128) return THRIFT_EUNSUPPORTED;
  if ((block_q != 64 && block_q != 128) || block_k != 64) return THRIFT_EUNSUPPORTED;
  if (Sk > 262144) return THRIFT_EUNSUPPORTED;
  if (kmax < thrift_select_head_kmax(Sq, Sk, block_q, block_k, causal)) return THRIFT_EINVAL;
  if (!aligned16(qbar) || !aligned16(kbar) || !aligned16(workspace)) return THRIFT_EALIGN;
  if (workspace_bytes < thrift_select_head_workspace_bytes(B, Hq, Sq, Sk, block_q, block_k))
    return THRIFT_EWORKSPACE;
  if (configure_score_kernels() != THRIFT_OK) return THRIFT_EHIP;
  const int nq = cdiv(Sq, block_q), nk = cdiv(Sk, block_k);
  const size_t rows = (size_t)B * Hq * nq;
  float* scores = (float*)workspace;
  uint32_t* hs = (uint32_t*)((char*)workspace + align256(rows * nk * sizeof(float)));
  uint32_t* ghist = (uint32_t*)((char*)hs + align256((size_t)B * Hq * 4 * sizeof(uint32_t)));
  int32_t* eqbase = (int32_t*)((char*)ghist + align256((size_t)B * Hq * 256 * sizeof(uint32_t)));
  if (D == 128)
    launch_score_topk<128, true>(qbar, kbar, B, Hq, Hkv, Sq, Sk, block_q, block_k, causal, topk_count, topk_bp,
                                 idx, cnt, kmax, stream, scores);
  else
    launch_score_topk<64, true>(qbar, kbar, B, Hq, Hkv, Sq, Sk, block_q, block_k, causal, topk_count, topk_bp,
                                idx, cnt, kmax, stream, scores);
  head_init_kernel<<<B * Hq, 256, 0, stream>>>(Sq, Sk, block_q, block_k, causal, topk_count, topk_bp, hs, ghist);
  const dim3 hgrid(cdiv(nq * nk, kHistChunk), B * Hq);
  for (int shift = 24; shift >= 0; shift -= 8) {
    head_hist_kernel<<<hgrid, 256, 0, stream>>>(scores, Sq, Sk, block_q, block_k, causal, shift, hs, ghist);
    head_pick_kernel<<<B * Hq, 256, 0, stream>>>(shift, hs, ghist);
  }
  const int rgrid = (int)((rows + 3) / 4);
  head_eqcount_kernel<<<rgrid, 256, 0, stream>>>(scores, (int)rows, nq, Sq, Sk, block_q, block_k, causal, hs,
                                                 eqbase);
  head_scan_kernel<<<B * Hq, 1024, 0, stream>>>(nq, eqbase);
  head_emit_kernel<<<rgrid, 256, 0, stream>>>(scores, (int)rows, nq, Sq, Sk, block_q, block_k, causal, hs, eqbase,
                                              idx, cnt, kmax);
  return launch_status();
}
