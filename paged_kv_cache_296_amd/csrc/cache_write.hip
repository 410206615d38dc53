// Cache write of packed K/V rows for gfx950.
//
// What is computed (HF Transformers "paged attention" page, section "Jalur
// Varlen", cache behaviour: the varlen kernel cannot reach the paged cache,
// so new rows are written into it by a separate update; slot rule of section
// "Jalur decode"): row cu[b] + i of request b is token p = start[b] + i of
// sequence b and is copied, bit for bit, to slot p mod block_size of
// physical block block_table[b][p / block_size], for K and for V.
//
// How: one wave per packed row.  Everything that locates the row -- its
// request (a binary search of cu), its token position, its table entry --
// is wave-uniform, so it runs on the scalar unit from the scalar cache; the
// 64 lanes then move the row's Hkv * D elements (2 KB per row of K at 8 kv
// heads x 128 bf16) in 16-byte pieces, K and V interleaved so that each lane
// has four loads in flight.  The row is contiguous at both ends (a token row
// of the cache is [Hkv][D] like a packed row), so both sides are coalesced.
// HBM bound: 2 reads + 2 writes of the row per packed row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWavesPerGroup = 4;
constexpr unsigned kErrBlock = 1u, kErrSpan = 2u, kErrCu = 4u;

__global__ __launch_bounds__(kWavesPerGroup * 64) void cache_write_kernel(CacheWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long gw = (long long)blockIdx.x * kWavesPerGroup + wave;

  // every entry pair of cu is checked by some lane of some wave
  bool bad_cu = false;
  for (long long i = gw * 64 + lane; i < a.batch; i += (long long)gridDim.x * kWavesPerGroup * 64)
    bad_cu |= a.cu[i + 1] < a.cu[i];
  if (gw == 0 && lane == 0) bad_cu |= a.cu[0] != 0 || a.cu[a.batch] != a.total;
  if (bad_cu && a.err_flag) atomicOr(a.err_flag, (int)kErrCu);
  if (gw >= a.total || a.batch <= 0) return;

  // the request of row r: the last b with cu[b] <= r (uniform, scalar loads)
  const int r = (int)gw;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int b = lo;
  const int c0 = a.cu[b], c1 = a.cu[b + 1];
  unsigned err = 0;
  if (!(c0 <= r && r < c1)) err = kErrCu;
  const int st = a.start[b];
  const long long p = (long long)st + (r - c0);
  if (!err && (st < 0 || p >= (long long)a.max_blocks_per_seq * a.block_size)) err = kErrSpan;
  int pb = 0;
  if (!err) {
    pb = a.block_table[(long long)b * a.max_blocks_per_seq + p / a.block_size];
    if (pb < 0 || pb >= a.num_blocks) err = kErrBlock;
  }
  if (err) {
    if (a.err_flag && lane == 0) atomicOr(a.err_flag, (int)err);
    return;
  }
  const long long src = (long long)r * a.row_bytes;
  const long long dst = ((long long)pb * a.block_size + p % a.block_size) * a.row_bytes;
  const char* ks = (const char*)a.k + src;
  const char* vs = (const char*)a.v + src;
  char* kd = (char*)a.k_cache + dst;
  char* vd = (char*)a.v_cache + dst;
  const int n16 = a.row_bytes / 16;
  int c = lane;
  for (; c + 64 < n16; c += 128) {
    const u32x4 k0 = *reinterpret_cast<const u32x4*>(ks + 16 * c);
    const u32x4 k1 = *reinterpret_cast<const u32x4*>(ks + 16 * (c + 64));
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(vs + 16 * c);
    const u32x4 v1 = *reinterpret_cast<const u32x4*>(vs + 16 * (c + 64));
    *reinterpret_cast<u32x4*>(kd + 16 * c) = k0;
    *reinterpret_cast<u32x4*>(kd + 16 * (c + 64)) = k1;
    *reinterpret_cast<u32x4*>(vd + 16 * c) = v0;
    *reinterpret_cast<u32x4*>(vd + 16 * (c + 64)) = v1;
  }
  if (c < n16) {
    const u32x4 k0 = *reinterpret_cast<const u32x4*>(ks + 16 * c);
    const u32x4 v0 = *reinterpret_cast<const u32x4*>(vs + 16 * c);
    *reinterpret_cast<u32x4*>(kd + 16 * c) = k0;
    *reinterpret_cast<u32x4*>(vd + 16 * c) = v0;
  }
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
  if (a.total == 0 && a.batch == 0) return hipSuccess;
  // at least one group so that cu is always checked
  const long long groups = a.total > 0 ? (a.total + kWavesPerGroup - 1) / kWavesPerGroup : 1;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)groups), dim3(kWavesPerGroup * 64), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pkv
