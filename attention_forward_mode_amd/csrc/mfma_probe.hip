// mfma_probe.hip -- bf16 matrix-core throughput probe for gfx950 (declared in
// include/mfma_probe.h).  Each wave keeps four 32x32 fp32 accumulators and
// issues the 32x32x16 bf16 product on them in turn, so consecutive products
// never depend on each other and the matrix pipeline stays full.  The
// operands are pseudo-random (no constant folding, realistic bit switching);
// the accumulators are summed into `sink` at the end (no dead-code removal).
#include <hip/hip_runtime.h>

#include "mfma_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Operand element in [-1, 1) from an integer hash of (thread, slot): random
// bits like real data, so the products switch as many bits as real work does
// (a repeated constant operand would draw less power and run at a higher clock).
__device__ inline __bf16 operand(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (__bf16)((float)(x >> 8) * (2.0f / 16777216.0f) - 1.0f);
}

__global__ __launch_bounds__(MFMA_PROBE_THREADS) void mfma_probe_kernel(float* sink, int iters,
                                                                        uint32_t seed) {
  // four operand pairs, one per accumulator: consecutive products never share an operand
  bf16x8 a[4], b[4];
  const uint32_t t = (blockIdx.x * MFMA_PROBE_THREADS + threadIdx.x) * 64u + seed;
  for (int k = 0; k < 4; ++k)
    for (int i = 0; i < 8; ++i) {
      a[k][i] = operand(t + 16u * k + i);
      b[k][i] = operand(t + 16u * k + 8u + i);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * MFMA_PROBE_THREADS + threadIdx.x] = s;
}

}  // namespace

extern "C" int mfma_probe_launch(int workgroups, int iters, float* sink, void* stream) {
  if (sink == nullptr || workgroups < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(MFMA_PROBE_THREADS), 0,
                     static_cast<hipStream_t>(stream), sink, iters, 12345u);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
