// Measurement aids: a plain streaming read of one device buffer, the
// practical HBM read ceiling that the decode kernels' K/V bandwidth is set
// against, and a plain copy (further down), the ceiling for the cache write
// (the 8 TB/s figure is the part's specification; no kernel reaches it).
// In the read each wave streams one contiguous chunk of the buffer (the
// chunks tile it in wave order) in bursts of four 16-byte loads per lane,
// with the same non-temporal cache hint the decode kernels put on their K/V
// loads, or none.  Against the previous form (every lane grid-stride over
// the whole buffer, four loads in flight), on one box: 8 GiB read 6.50 ->
// 7.14 TB/s (2048 workgroups, which at this kernel's register use are all
// resident at once, 1 MB per wave; the grid-stride form peaked at 6.75 with
// 8192).  The grid-stride sweep keeps
// every workgroup's requests inside one narrow window of the buffer at a
// time.  The copy keeps the grid-stride form, which stays the faster one at
// the cache write's size (83 MB, each call after a 1 GiB buffer was
// overwritten: 5.1-5.2 against at most 4.98 TB/s for one chunk per wave).
// The read's words are XOR-folded and stored only if the fold hits a fixed
// pattern, so the loads cannot be dropped and nothing is written in
// practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrc = 0x00020000;  // gfx9-family buffer descriptor word 3

// This wave's chunk [b0, b0 + n) of a `bytes`-byte buffer cut into `chunk`-
// byte pieces (chunk a multiple of 1 KiB, at most 1 GiB); n = 0 past the end.
__device__ __forceinline__ int wave_chunk(long long bytes, long long chunk, long long& b0) {
  const long long w = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  b0 = w * chunk;
  if (b0 >= bytes) return 0;
  return (int)(bytes - b0 < chunk ? bytes - b0 : chunk);
}

template <int CPOL>
__global__ __launch_bounds__(256) void stream_read_kernel(const char* __restrict__ p, long long bytes, long long chunk,
                        u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  long long b0;
  const int n = wave_chunk(bytes, chunk, b0);
  if (n > 0) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p + b0), (short)0, n, kRsrc);
    int o = 16 * (threadIdx.x & 63);
    for (; o + 3 * 1024 < n; o += 4 * 1024) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, CPOL);
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, o + 1024, 0, CPOL);
      const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(r, o + 2048, 0, CPOL);
      const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, o + 3072, 0, CPOL);
      acc ^= a ^ b ^ c ^ d;
    }
    for (; o < n; o += 1024) acc ^= __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, CPOL);
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

// Chunk per wave for `bytes` over 4 * workgroups waves, rounded up to 1 KiB;
// 0 if it would exceed 1 GiB.
long long chunk_of(size_t bytes, int workgroups) {
  const long long waves = 4LL * workgroups;
  long long c = ((long long)bytes + waves - 1) / waves;
  c = (c + 1023) / 1024 * 1024;
  return c > (1LL << 30) ? 0 : c;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_stream_read(const void* buf, size_t bytes, void* sink, int workgroups,
                               int nontemporal, void* stream) {
  if (buf == nullptr || sink == nullptr || workgroups <= 0 || workgroups > 65535 ||
      bytes % 16 != 0 || (nontemporal != 0 && nontemporal != 1))
    return PKV_EINVAL;
  if (bytes == 0) return PKV_OK;
  const long long chunk = pkv::chunk_of(bytes, workgroups);
  if (chunk == 0) return PKV_EINVAL;
  const dim3 grid((unsigned)workgroups), block(256);
  if (nontemporal)
    hipLaunchKernelGGL(pkv::stream_read_kernel<2>, grid, block, 0, (hipStream_t)stream,
                       (const char*)buf, (long long)bytes, chunk, (pkv::u32x4*)sink);
  else
    hipLaunchKernelGGL(pkv::stream_read_kernel<0>, grid, block, 0, (hipStream_t)stream,
                       (const char*)buf, (long long)bytes, chunk, (pkv::u32x4*)sink);
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
