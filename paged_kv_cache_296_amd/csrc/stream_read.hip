// Measurement aids: a plain streaming read of one device buffer, the
// practical HBM read ceiling that the decode kernels' K/V bandwidth is set
// against, and a plain copy (further down), the ceiling for the cache write (the 8 TB/s figure is the part's specification; no kernel reaches
// it).  Every lane reads 16-byte words, four in flight, grid-stride over
// windows of at most 1 GiB (one buffer descriptor each), with the same
// non-temporal cache hint the decode kernels put on their K/V loads, or
// none.  The words are XOR-folded and stored only if the fold hits a fixed
// pattern, so the loads cannot be dropped and nothing is written in
// practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr long long kWindow = 1LL << 30;

template <int CPOL>
__global__ __launch_bounds__(256) void stream_read_kernel(const char* __restrict__ p,
                                                          long long bytes, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const int stride = gridDim.x * 256;
  for (long long base = 0; base < bytes; base += kWindow) {
    const long long wb = bytes - base < kWindow ? bytes - base : kWindow;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p + base), (short)0, (int)wb, 0x00020000);
    const int n = (int)(wb / 16);
    int i = blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n; i += 4 * stride) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * i, 0, CPOL);
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (i + stride), 0, CPOL);
      const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (i + 2 * stride), 0, CPOL);
      const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (i + 3 * stride), 0, CPOL);
      acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n; i += stride) acc ^= __builtin_amdgcn_raw_buffer_load_b128(r, 16 * i, 0, CPOL);
  }
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == 0x85ebca6bu && acc.w == 0xc2b2ae35u)
    sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Plain device copy of `bytes` bytes (< 2 GiB), the same loads plus 16-byte
// stores, eight words in flight per lane: the practical ceiling for kernels
// that move every byte they read (the paged cache write).
__global__ __launch_bounds__(256) void stream_copy_kernel(const char* __restrict__ src,
                                                          char* __restrict__ dst, int bytes) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc((void*)dst, (short)0, bytes, 0x00020000);
  const int n = bytes / 16, stride = gridDim.x * 256;
  int i = blockIdx.x * 256 + threadIdx.x;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (i + u * stride), 0, 2);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, 16 * (i + u * stride), 0, 0);
  }
  for (; i < n; i += stride)
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_amdgcn_raw_buffer_load_b128(rs, 16 * i, 0, 2),
                                           rd, 16 * i, 0, 0);
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_stream_read(const void* buf, size_t bytes, void* sink, int workgroups,
                               int nontemporal, void* stream) {
  if (buf == nullptr || sink == nullptr || workgroups <= 0 || workgroups > 65535 ||
      bytes % 16 != 0 || (nontemporal != 0 && nontemporal != 1))
    return PKV_EINVAL;
  if (bytes == 0) return PKV_OK;
  const dim3 grid((unsigned)workgroups), block(256);
  if (nontemporal)
    hipLaunchKernelGGL(pkv::stream_read_kernel<2>, grid, block, 0, (hipStream_t)stream,
                       (const char*)buf, (long long)bytes, (pkv::u32x4*)sink);
  else
    hipLaunchKernelGGL(pkv::stream_read_kernel<0>, grid, block, 0, (hipStream_t)stream,
                       (const char*)buf, (long long)bytes, (pkv::u32x4*)sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

extern "C" int pkv_stream_copy(const void* src, void* dst, size_t bytes, int workgroups,
                               void* stream) {
  if (src == nullptr || dst == nullptr || workgroups <= 0 || workgroups > 65535 ||
      bytes % 16 != 0 || bytes >= ((size_t)1 << 31))
    return PKV_EINVAL;
  if (bytes == 0) return PKV_OK;
  hipLaunchKernelGGL(pkv::stream_copy_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     (hipStream_t)stream, (const char*)src, (char*)dst, (int)bytes);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}
