// Measurement aid: a loop of dense bf16 matrix-core products with no memory
// traffic, the practical MFMA ceiling that the prefill kernels' throughput is
// set against (2.5 PFLOP/s is the part's specification at its peak engine
// clock; under sustained matrix load the clock is lower).  The instruction is
// the one the prefill tiles use, v_mfma_f32_32x32x16_bf16 (32 x 32 x 16, 32768
// flops), issued in four independent accumulator chains per wave so that a
// chain's latency never stalls the pipe; 256-thread workgroups, one wave per
// SIMD each.  The operands are small lane-dependent values of both signs, so
// the accumulators stay finite; they are reduced and stored only if the sum
// hits a fixed pattern, so the products cannot be dropped and nothing is
// written in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((float)(((lane + i) & 7) - 4) * 0.0078125f);
    b[i] = (__bf16)((float)(((lane * 3 + i) & 7) - 3) * 0.0078125f);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (s == 1234567.f) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_mfma_peak(void* sink, int workgroups, int iters, void* stream) {
  if (sink == nullptr || workgroups <= 0 || workgroups > 65535 || iters < 0) return PKV_EINVAL;
  if (iters == 0) return PKV_OK;
  hipLaunchKernelGGL(pkv::mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     (hipStream_t)stream, iters, (float*)sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}
