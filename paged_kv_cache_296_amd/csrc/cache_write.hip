// Cache write of packed K/V rows for gfx950.
//
// What is computed (HF Transformers "paged attention" page, section "Jalur
// Varlen", cache behaviour: the varlen kernel cannot reach the paged cache,
// so new rows are written into it by a separate update; slot rule of section
// "Jalur decode"): row cu[b] + i of request b is token p = start[b] + i of
// sequence b and is copied, bit for bit, to slot p mod block_size of
// physical block block_table[b][p / block_size], for K and for V.
//
// How: one wave per 2 consecutive packed rows.  The 64 lanes move the rows'
// Hkv * D elements (2 KB per row of K at 8 kv heads x 128 bf16) in 16-byte
// pieces, issuing the loads of both rows of K and V first -- each lane has 8
// loads in flight -- and only then locating the rows' slots: everything
// that locates a row -- its request (one load of cu per lane and a ballot,
// or a binary search for large batches), its token position, its table
// entry -- is wave-uniform and runs on the scalar unit, three dependent
// round trips that the loads now overlap (39.0-39.7 -> 36.2-36.4 us on the
// 16-request prefill batch; 1 and 4 rows per wave 39.6 and 37.5 us).  A row is contiguous at both ends (a
// token row of the cache is [Hkv][D] like a packed row), so both sides are
// coalesced.  The packed rows are read once, with the non-temporal hint
// (measured 28 % faster than plain loads on the 16-request prefill batch:
// 55.5 -> 40.0 us with the last-level cache flushed before each call; the
// same hint on the stores changed nothing).  HBM bound: 2 reads + 2 writes
// of the row per packed row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWavesPerGroup = 4;
constexpr int kRowsPerWave = 2;   // rows one wave copies, all loads in flight together
constexpr int kMaxPieces = 4;     // 16-byte pieces per lane per row (row_bytes <= 4 KB)
constexpr unsigned kErrBlock = 1u, kErrSpan = 2u, kErrCu = 4u;

// 16 bytes read once: non-temporal load (global_load_dwordx4 ... nt)
__device__ __forceinline__ u32x4 load_once(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// The request of packed row r: the last b with cu[b] <= r.  Up to 63
// requests: one load of cu per lane and a ballot; more: a binary search on
// the scalar unit.
__device__ __forceinline__ int request_of(const int32_t* cu, int batch, int r, int lane) {
  if (batch < 64) {
    const bool le = lane <= batch && cu[min(lane, batch)] <= r;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(le);
    const int cnt = __builtin_popcountll(m);  // cu[0..cnt-1] <= r for a non-decreasing cu
    return min(max(cnt - 1, 0), batch - 1);
  }
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

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
  const long long r0 = gw * kRowsPerWave;
  if (r0 >= a.total || a.batch <= 0) return;

  // the rows' loads go out first: their source depends only on the row
  // number, and the lookups below (cu, then start, then the table entry)
  // are three dependent round trips that now overlap them
  const int n16 = a.row_bytes / 16;
  const int nrows = (int)min((long long)kRowsPerWave, a.total - r0);
  u32x4 kx[kRowsPerWave][kMaxPieces], vx[kRowsPerWave][kMaxPieces];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
    for (int j = 0; j < kMaxPieces; ++j) {
      const int c = lane + 64 * j;
      if (i < nrows && c < n16) {
        const long long off = (r0 + i) * a.row_bytes + 16 * c;
        kx[i][j] = load_once((const char*)a.k + off);
        vx[i][j] = load_once((const char*)a.v + off);
      }
    }

  // locate this wave's rows (uniform: scalar registers)
  long long src[kRowsPerWave], dst[kRowsPerWave];
  bool ok[kRowsPerWave];
  int b = __builtin_amdgcn_readfirstlane(request_of(a.cu, a.batch, (int)r0, lane));
  unsigned err = 0;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    ok[i] = false;
    src[i] = dst[i] = 0;
    if (i >= nrows) continue;
    const int r = (int)r0 + i;
    while (b + 1 < a.batch && a.cu[b + 1] <= r) ++b;  // rows are consecutive
    const int c0 = a.cu[b], c1 = a.cu[b + 1];
    if (!(c0 <= r && r < c1)) {
      err |= kErrCu;
      continue;
    }
    const int st = a.start[b];
    const long long p = (long long)st + (r - c0);
    if (st < 0 || p >= (long long)a.max_blocks_per_seq * a.block_size) {
      err |= kErrSpan;
      continue;
    }
    const int pb = a.block_table[(long long)b * a.max_blocks_per_seq + p / a.block_size];
    if (pb < 0 || pb >= a.num_blocks) {
      err |= kErrBlock;
      continue;
    }
    ok[i] = true;
    src[i] = (long long)r * a.row_bytes;
    dst[i] = ((long long)pb * a.block_size + p % a.block_size) * a.row_bytes;
  }
  if (err && a.err_flag && lane == 0) atomicOr(a.err_flag, (int)err);

  // then the stores of the rows that have a slot
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
    for (int j = 0; j < kMaxPieces; ++j) {
      const int c = lane + 64 * j;
      if (ok[i] && c < n16) {
        *reinterpret_cast<u32x4*>((char*)a.k_cache + dst[i] + 16 * c) = kx[i][j];
        *reinterpret_cast<u32x4*>((char*)a.v_cache + dst[i] + 16 * c) = vx[i][j];
      }
    }
  // rows longer than 4 KB: the rest piece by piece
  for (int i = 0; i < kRowsPerWave; ++i) {
    if (!ok[i]) continue;
    for (int c = lane + 64 * kMaxPieces; c < n16; c += 64) {
      const u32x4 kv = load_once((const char*)a.k + src[i] + 16 * c);
      const u32x4 vv = load_once((const char*)a.v + src[i] + 16 * c);
      *reinterpret_cast<u32x4*>((char*)a.k_cache + dst[i] + 16 * c) = kv;
      *reinterpret_cast<u32x4*>((char*)a.v_cache + dst[i] + 16 * c) = vv;
    }
  }
}

// Whole-block copies (the copy-on-write step of the block manager): pair
// blockIdx.y copies block src -> dst of both pools; the workgroups along x
// split the block into 4 KB pieces per pass of 256 lanes x 16 bytes.  The
// source blocks are read with the non-temporal hint (4096 pairs of 32 KB
// bf16 blocks, cache flushed: 3.84-3.94 -> 4.83 TB/s moved).
constexpr int kCopyPieces = 4;  // 16-byte pieces per lane per workgroup
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int i = blockIdx.y;
  const int s = a.src[i], d = a.dst[i];
  if (s < 0 || s >= a.num_blocks || d < 0 || d >= a.num_blocks) {
    if (a.err_flag && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.err_flag, (int)kErrBlock);
    return;
  }
  const long long n16 = a.block_bytes / 16;
  const long long base = (long long)blockIdx.x * 256 * kCopyPieces + threadIdx.x;
  const char* ks = (const char*)a.k_cache + (long long)s * a.block_bytes;
  const char* vs = (const char*)a.v_cache + (long long)s * a.block_bytes;
  char* kd = (char*)a.k_cache + (long long)d * a.block_bytes;
  char* vd = (char*)a.v_cache + (long long)d * a.block_bytes;
  u32x4 kx[kCopyPieces], vx[kCopyPieces];
#pragma unroll
  for (int j = 0; j < kCopyPieces; ++j) {
    const long long c = base + 256 * j;
    if (c < n16) {
      kx[j] = load_once(ks + 16 * c);
      vx[j] = load_once(vs + 16 * c);
    }
  }
#pragma unroll
  for (int j = 0; j < kCopyPieces; ++j) {
    const long long c = base + 256 * j;
    if (c < n16) {
      *reinterpret_cast<u32x4*>(kd + 16 * c) = kx[j];
      *reinterpret_cast<u32x4*>(vd + 16 * c) = vx[j];
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const long long per_wg = 256LL * 16 * kCopyPieces;
  const long long gx = (a.block_bytes + per_wg - 1) / per_wg;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)a.n), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
  if (a.total == 0 && a.batch == 0) return hipSuccess;
  // at least one group so that cu is always checked
  const long long per_group = (long long)kWavesPerGroup * kRowsPerWave;
  const long long groups = a.total > 0 ? (a.total + per_group - 1) / per_group : 1;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)groups), dim3(kWavesPerGroup * 64), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pkv
