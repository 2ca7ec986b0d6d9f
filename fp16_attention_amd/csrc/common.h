// Shared device/host helpers of the gfx950 ThriftAttention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "thrift.h"

namespace thrift {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef short v2s_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Number of valid key blocks of query block i for Sq queries against Sk keys
// (Sq <= Sk; causal: the queries are the last Sq positions of the key
// sequence, so that for Sq = Sk the two are aligned at their starts; a block
// is valid when it holds a key not after the query block's last row).
__host__ __device__ inline int valid_kv_blocks_kv(int i, int Sq, int Sk, int bq, int bk, int causal) {
  if (!causal) return cdiv(Sk, bk);
  int last = (i + 1) * bq < Sq ? (i + 1) * bq - 1 : Sq - 1;
  return (Sk - Sq + last) / bk + 1;
}

__host__ __device__ inline int valid_kv_blocks(int i, int S, int bq, int bk, int causal) {
  return valid_kv_blocks_kv(i, S, S, bq, bk, causal);
}

// Promoted-block budget of a query block with n valid key blocks.
__host__ __device__ inline int topk_budget(int n, int topk_count, int topk_bp) {
  long long k = topk_count >= 0 ? (long long)topk_count : ((long long)n * topk_bp + 9999) / 10000;
  return (int)(k < n ? k : n);
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Runs set_up() once per device for the caller's flag word (kernel attributes
// such as the dynamic LDS limit are per device).  Concurrent first calls may
// both run set_up(), which only sets the same attributes twice.
template <class F>
inline thrift_status once_per_device(std::atomic<uint64_t>& done, F&& set_up) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return THRIFT_EHIP;
  const uint64_t bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return THRIFT_OK;
  if (set_up() != THRIFT_OK) return THRIFT_EHIP;
  done.fetch_or(bit, std::memory_order_release);
  return THRIFT_OK;
}

// ---- device helpers shared by the kernels ------------------------------------

// One 32x32x16 fp16 matrix product with fp32 accumulation.
__device__ inline v16f mfma_f16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum of this lane's value and that of lane +- 32 (the other half of a
// 32x32 product's column).
__device__ inline float pair_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// E4M3 byte -> value by the hardware conversion (OCP E4M3, exact; block
// scales are finite and non-negative).
__device__ inline float e4m3_to_float(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// 2688 / s2 for an NVFP4 level-2 block scale s2 (0 for s2 = 0), through the
// hardware reciprocal: within 2 u of the quotient (u = 2^-24) for every
// positive E4M3 value, which the arithmetic probes check exhaustively.
__device__ inline float nv_p_factor(float s2) { return s2 > 0.0f ? 2688.0f * __builtin_amdgcn_rcpf(s2) : 0.0f; }

// Key (within a 64-key tile) that A-operand row m of 32x32 S^T tile mt
// reads.  The MFMA output puts row (i/4)*8 + hi*4 + i%4 in register i of a
// lane of half hi, so register i of tile mt holds key hi*32 + mt*16 + i.
__device__ inline int krow(int mt, int m) { return ((m >> 2) & 1) * 32 + mt * 16 + (m >> 3) * 4 + (m & 3); }

inline thrift_status launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? THRIFT_OK : THRIFT_EHIP;
}

}  // namespace thrift
