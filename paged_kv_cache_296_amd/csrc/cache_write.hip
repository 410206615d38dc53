// Cache write of packed K/V rows for gfx950.
//
// What is computed (HF Transformers "paged attention" page, section "Jalur
// Varlen", cache behaviour: the varlen kernel cannot reach the paged cache,
// so new rows are written into it by a separate update; slot rule of section
// "Jalur decode"): row cu[b] + i of request b is token p = start[b] + i of
// sequence b and is copied, bit for bit, to slot p mod block_size of
// physical block block_table[b][p / block_size], for K and for V.
//
// How: one wave per 2 consecutive packed rows; the 64 lanes move a row's
// Hkv * D elements (2 KB per row of K at 8 kv heads x 128 bf16) in 16-byte
// pieces, P pieces per lane (P = row bytes / 1 KB rounded up, at most 4; a
// template parameter).  A row is contiguous at both ends (a token row of the
// cache is [Hkv][D] like a packed row), so both sides are coalesced.  The
// order of a wave's memory traffic is what sets the time: on gfx9 the
// vector-memory counter retires loads in issue order, so any vector load
// issued after the rows' loads and waited on waits for all of them.  So:
//   1. each lane loads cu[lane] and start[lane] (requests up to 63): with
//      the first waves' check of cu at the kernel's start, the only vector
//      loads besides the rows', and issued before them;
//   2. the rows' loads go out, all of them unconditionally, through buffer
//      descriptors that bound them to the wave's rows (a lane past the row
//      end gets an out-of-range offset: no memory access);
//   3. waiting only for step 1, a ballot on cu gives each row's request,
//      lane reads give its cu and start, and the table entry comes through
//      the scalar cache (more than 63 requests: a binary search there too),
//      all while the rows are in flight;
//   4. the stores, through one descriptor per destination row whose range
//      is empty when the row has no valid slot.
// Against the previous form (conditional global loads, and lookups issued as
// vector loads after the rows: four dependent round trips that each waited
// for every row load), on the 16-request prefill batch (167 MB moved) with
// the last-level cache cold, same box: 33.6-33.7 -> 31.0-31.1 us by events
// (5.37 TB/s; a plain copy of the same bytes 29.7-30.0 us).  The packed rows
// are read once, with the non-temporal hint (measured 28 % faster than plain
// loads on that batch); the same hint on the stores measured 8 % slower.
// One or four rows per wave: 31.2 and 32.1 us.  HBM bound: 2 reads + 2
// writes of the row per packed row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const int32_t __attribute__((address_space(4))) cint32;
constexpr int kWavesPerGroup = 4;
constexpr int kRowsPerWave = 2;   // rows one wave copies, all loads in flight together
constexpr int kMaxPieces = 4;     // 16-byte pieces per lane per row in the unrolled part
constexpr int kRsrc = 0x00020000;  // gfx9-family buffer descriptor word 3
constexpr int kLoadNT = 2;         // cache policy bits of a buffer op: non-temporal
constexpr unsigned kOutOfRange = 0x80000000u;  // above every range used here (< 2^31)
constexpr unsigned kErrBlock = 1u, kErrSpan = 2u, kErrCu = 4u;

// 16 bytes read once: non-temporal load (global_load_dwordx4 ... nt)
__device__ __forceinline__ u32x4 load_once(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrc);
}

// p[i] through the scalar cache (p and i wave-uniform; p is read-only here)
__device__ __forceinline__ int sload(const int32_t* p, long long i) {
  return reinterpret_cast<cint32*>(reinterpret_cast<uintptr_t>(p))[i];
}

// The request of packed row r: the last b with cu[b] <= r, clamped to
// [0, batch - 1].  cu_l: lane l holds cu[min(l, batch)] (used for batch < 64).
__device__ __forceinline__ int request_of(const int32_t* cu, int batch, int r, int lane,
                                          int cu_l) {
  if (batch < 64) {
    const bool le = lane <= batch && cu_l <= r;
    const int cnt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
    return min(max(cnt - 1, 0), batch - 1);  // cu[0..cnt-1] <= r for a non-decreasing cu
  }
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sload(cu, mid) <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int P>
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

  // 1. the lookup tables' first 64 entries, one per lane
  const int cu_l = a.cu[min(lane, a.batch)];
  const int st_l = a.start[min(lane, a.batch - 1)];
  __builtin_amdgcn_sched_barrier(0);

  // 2. the rows' loads
  const int rb = a.row_bytes;
  const int nrows = (int)min((long long)kRowsPerWave, a.total - r0);
  const __amdgpu_buffer_rsrc_t ks = rsrc((const char*)a.k + r0 * rb, nrows * rb);
  const __amdgpu_buffer_rsrc_t vs = rsrc((const char*)a.v + r0 * rb, nrows * rb);
  unsigned piece[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int o = 16 * (lane + 64 * j);
    piece[j] = o < rb ? (unsigned)o : kOutOfRange;
  }
  u32x4 kx[kRowsPerWave][P], vx[kRowsPerWave][P];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const unsigned o = piece[j] == kOutOfRange ? kOutOfRange : piece[j] + i * rb;
      kx[i][j] = __builtin_amdgcn_raw_buffer_load_b128(ks, o, 0, kLoadNT);
      vx[i][j] = __builtin_amdgcn_raw_buffer_load_b128(vs, o, 0, kLoadNT);
    }
  __builtin_amdgcn_sched_barrier(0);

  // 3. locate this wave's rows (uniform: scalar registers)
  long long dst[kRowsPerWave];
  bool ok[kRowsPerWave];
  unsigned err = 0;
  const bool small = a.batch < 64;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    ok[i] = false;
    dst[i] = 0;
    if (i >= nrows) continue;
    const int r = (int)r0 + i;
    const int b = __builtin_amdgcn_readfirstlane(request_of(a.cu, a.batch, r, lane, cu_l));
    const int c0 = small ? __builtin_amdgcn_readlane(cu_l, b) : sload(a.cu, b);
    const int c1 = small ? __builtin_amdgcn_readlane(cu_l, b + 1) : sload(a.cu, b + 1);
    if (!(c0 <= r && r < c1)) {
      err |= kErrCu;
      continue;
    }
    const int st = small ? __builtin_amdgcn_readlane(st_l, b) : sload(a.start, b);
    const long long p = (long long)st + (r - c0);
    if (st < 0 || p >= (long long)a.max_blocks_per_seq * a.block_size) {
      err |= kErrSpan;
      continue;
    }
    const int pb = sload(a.block_table, (long long)b * a.max_blocks_per_seq + p / a.block_size);
    if (pb < 0 || pb >= a.num_blocks) {
      err |= kErrBlock;
      continue;
    }
    ok[i] = true;
    dst[i] = ((long long)pb * a.block_size + p % a.block_size) * rb;
  }
  if (err && a.err_flag && lane == 0) atomicOr(a.err_flag, (int)err);

  // 4. the stores; a row without a slot has an empty range
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const __amdgpu_buffer_rsrc_t kd = rsrc((char*)a.k_cache + dst[i], ok[i] ? rb : 0);
    const __amdgpu_buffer_rsrc_t vd = rsrc((char*)a.v_cache + dst[i], ok[i] ? rb : 0);
#pragma unroll
    for (int j = 0; j < P; ++j) {
      __builtin_amdgcn_raw_buffer_store_b128(kx[i][j], kd, piece[j], 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(vx[i][j], vd, piece[j], 0, 0);
    }
  }
  // rows longer than 4 KB: the rest piece by piece
  if (P == kMaxPieces) {
    for (int i = 0; i < kRowsPerWave; ++i) {
      if (!ok[i]) continue;
      const long long src = (r0 + i) * rb;
      for (int c = lane + 64 * kMaxPieces; c < rb / 16; c += 64) {
        const u32x4 kv = load_once((const char*)a.k + src + 16 * c);
        const u32x4 vv = load_once((const char*)a.v + src + 16 * c);
        *reinterpret_cast<u32x4*>((char*)a.k_cache + dst[i] + 16 * c) = kv;
        *reinterpret_cast<u32x4*>((char*)a.v_cache + dst[i] + 16 * c) = vv;
      }
    }
  }
}

// Whole-block copies (the copy-on-write step of the block manager): pair
// blockIdx.y copies block src -> dst of both pools; workgroup x of the pair
// moves bytes [16 KB x, 16 KB (x + 1)) of the block, four 4 KB passes of 256
// lanes x 16 bytes, all loads in flight before the first store.  The loads
// and stores are unconditional, through descriptors bounded to the
// workgroup's span (a lane past the block's end gets no access): loads
// issued under a per-lane condition are merged at the branch's join, and the
// merge waited for each pass's loads before the next pass was issued (4096
// pairs of 32 KB bf16 blocks, 537 MB moved, cache cold: 85.9-86.2 -> 84.1-84.2
// us, 6.38 TB/s).  The source blocks are read with the non-temporal hint
// (measured with the cache flushed by overwriting a 1 GiB buffer: 3.84-3.94
// -> 4.83 TB/s moved).
constexpr int kCopyPieces = 4;                     // 16-byte pieces per lane per workgroup
constexpr int kCopySpan = 256 * 16 * kCopyPieces;  // bytes per workgroup
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int i = blockIdx.y;
  const int s = a.src[i], d = a.dst[i];
  if (s < 0 || s >= a.num_blocks || d < 0 || d >= a.num_blocks) {
    if (a.err_flag && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(a.err_flag, (int)kErrBlock);
    return;
  }
  const long long off = (long long)blockIdx.x * kCopySpan;
  const int n = (int)min((long long)kCopySpan, a.block_bytes - off);
  const long long so = (long long)s * a.block_bytes + off, dof = (long long)d * a.block_bytes + off;
  const __amdgpu_buffer_rsrc_t ks = rsrc((const char*)a.k_cache + so, n);
  const __amdgpu_buffer_rsrc_t vs = rsrc((const char*)a.v_cache + so, n);
  const __amdgpu_buffer_rsrc_t kd = rsrc((char*)a.k_cache + dof, n);
  const __amdgpu_buffer_rsrc_t vd = rsrc((char*)a.v_cache + dof, n);
  u32x4 kx[kCopyPieces], vx[kCopyPieces];
#pragma unroll
  for (int j = 0; j < kCopyPieces; ++j) {
    const unsigned o = 16u * (threadIdx.x + 256u * j);
    kx[j] = __builtin_amdgcn_raw_buffer_load_b128(ks, o, 0, kLoadNT);
    vx[j] = __builtin_amdgcn_raw_buffer_load_b128(vs, o, 0, kLoadNT);
  }
#pragma unroll
  for (int j = 0; j < kCopyPieces; ++j) {
    const unsigned o = 16u * (threadIdx.x + 256u * j);
    __builtin_amdgcn_raw_buffer_store_b128(kx[j], kd, o, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(vx[j], vd, o, 0, 0);
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const long long gx = (a.block_bytes + kCopySpan - 1) / kCopySpan;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)a.n), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream) {
  if (a.total == 0 && a.batch == 0) return hipSuccess;
  // at least one group so that cu is always checked
  const long long per_group = (long long)kWavesPerGroup * kRowsPerWave;
  const long long groups = a.total > 0 ? (a.total + per_group - 1) / per_group : 1;
  const dim3 grid((unsigned)groups), block(kWavesPerGroup * 64);
  switch (min(kMaxPieces, (a.row_bytes + 1023) / 1024)) {
    case 1: hipLaunchKernelGGL(cache_write_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(cache_write_kernel<2>, grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(cache_write_kernel<3>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(cache_write_kernel<4>, grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
