// Measurement aid: a loop of dense bf16 matrix-core products with no memory
// traffic, the practical MFMA ceiling that the prefill kernels' throughput is
// set against (2.5 PFLOP/s is the part's specification at its peak engine
// clock; under sustained matrix load the clock is lower).  The instruction is
// the one the prefill tiles use, v_mfma_f32_32x32x16_bf16 (32 x 32 x 16, 32768
// flops), issued in four independent accumulator chains per wave so that a
// chain's latency never stalls the pipe; 256-thread workgroups, one wave per
// SIMD each.  The operands are bf16 values with hashed signs and mantissas
// (every bit pattern of a random matrix, so the datapath toggles as much as
// on real data; the clock the part holds depends on it) and a fixed small
// exponent, so the accumulators stay finite; they are reduced and stored
// only if the sum hits a fixed pattern, so the products cannot be dropped
// and nothing is written in practice.
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
  // a different operand pair for each chain, so that consecutive products
  // never see the same inputs
  bf16x8 a[kChains], b[kChains];
  uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 0x9E3779B9u + 0x7F4A7C15u;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // sign and 7 mantissa bits from a xorshift stream; exponent of 2^-7
      h ^= h << 13;
      h ^= h >> 17;
      h ^= h << 5;
      a[c][i] = __builtin_bit_cast(__bf16, (unsigned short)((h & 0x807Fu) | 0x3C00u));
      b[c][i] = __builtin_bit_cast(__bf16, (unsigned short)(((h >> 16) & 0x807Fu) | 0x3C00u));
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[c], acc[c], 0, 0, 0);
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
