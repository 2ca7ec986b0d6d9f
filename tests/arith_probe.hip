// Test infrastructure: probes of the device arithmetic that the parity
// bound's evaluation-error model rests on (the oracle's tho_eval_rel):
//  - the block-scaled FP4 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4
//    (E2M1 operands, E8M0 block scales, fp32 accumulator C);
//  - the fp16 matrix instruction v_mfma_f32_32x32x16_f16;
//  - the hardware exp2 (v_exp_f32);
//  - NVFP4's level-2 factor 2688 / s2 as the kernels form it, 2688 times the
//    hardware reciprocal (v_rcp_f32) of the E4M3 block scale s2.
// One wavefront per matrix launch; every access is within the buffers the
// caller sizes from ntest (64 lanes x ntest tests).  Built with the library
// (fp16_attention_amd/build.py) into tests/libarith_probe.so; not part of it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// a, b: per lane 16 bytes of E2M1 codes (lane (m, h): row/column m, channels
// 32h .. 32h+31 of the 64, low nibble first); sa, sb: per lane the E8M0
// scale of that 32-channel block (byte 0); c: per lane the 16 accumulator
// registers, replaced by the result.
__global__ void probe_fp4(const v4i* a, const v4i* b, const uint32_t* sa, const uint32_t* sb, float* c, int ntest) {
  const int lane = threadIdx.x;
  for (int t = 0; t < ntest; ++t) {
    const v4i x = a[t * 64 + lane], y = b[t * 64 + lane];
    const v8i xw = {x.x, x.y, x.z, x.w, 0, 0, 0, 0}, yw = {y.x, y.y, y.z, y.w, 0, 0, 0, 0};
    v16f acc;
    for (int i = 0; i < 16; ++i) acc[i] = c[(t * 64 + lane) * 16 + i];
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xw, yw, acc, 4, 4, 0, sa[t * 64 + lane], 0,
                                                          sb[t * 64 + lane]);
    for (int i = 0; i < 16; ++i) c[(t * 64 + lane) * 16 + i] = acc[i];
  }
}

// a, b: per lane 8 fp16 values (lane (m, h): row/column m, channels 8h .. 8h+7).
__global__ void probe_f16(const v8h* a, const v8h* b, float* c, int ntest) {
  const int lane = threadIdx.x;
  for (int t = 0; t < ntest; ++t) {
    v16f acc;
    for (int i = 0; i < 16; ++i) acc[i] = c[(t * 64 + lane) * 16 + i];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[t * 64 + lane], b[t * 64 + lane], acc, 0, 0, 0);
    for (int i = 0; i < 16; ++i) c[(t * 64 + lane) * 16 + i] = acc[i];
  }
}

__global__ void probe_exp2(const float* x, float* y, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = __builtin_amdgcn_exp2f(x[i]);
}

extern "C" int arith_probe_fp4(const void* a, const void* b, const void* sa, const void* sb, void* c, int ntest,
                               hipStream_t stream) {
  if (ntest < 1) return 1;
  probe_fp4<<<1, 64, 0, stream>>>((const v4i*)a, (const v4i*)b, (const uint32_t*)sa, (const uint32_t*)sb,
                                  (float*)c, ntest);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int arith_probe_f16(const void* a, const void* b, void* c, int ntest, hipStream_t stream) {
  if (ntest < 1) return 1;
  probe_f16<<<1, 64, 0, stream>>>((const v8h*)a, (const v8h*)b, (float*)c, ntest);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

__global__ void probe_nv_factor(const float* x, float* y, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 2688.0f * __builtin_amdgcn_rcpf(x[i]);
}

extern "C" int arith_probe_nv_factor(const void* x, void* y, int n, hipStream_t stream) {
  if (n < 1) return 1;
  probe_nv_factor<<<(n + 255) / 256, 256, 0, stream>>>((const float*)x, (float*)y, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int arith_probe_exp2(const void* x, void* y, int n, hipStream_t stream) {
  if (n < 1) return 1;
  probe_exp2<<<(n + 255) / 256, 256, 0, stream>>>((const float*)x, (float*)y, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
