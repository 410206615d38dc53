// Internal interface between the host entry points (pkv_api.hip) and the
// kernels (decode.hip, varlen.hip, cache_write.hip).  Not part of the public
// ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Everything one decode launch needs; passed by value as the kernel argument.
struct DecodeArgs {
  const void* q;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* cache_seqlens;
  const void* k_new;
  const void* v_new;
  void* out;
  float* ws_acc;      // [batch, num_kv_heads, n_parts, group * head_dim] unnormalised sums
  float2* ws_ml;      // [batch, num_kv_heads, n_parts, group] (running max, sum of exponentials)
  int* ctrl;          // [0] ticket counter, [1] number of work items (written by the plan kernel)
  int4* items;        // [batch * n_parts] work items (sequence, first partition << 8 | count, cached length, 0)
  int max_run;        // most partitions one work item may stream (slice bound, <= 255)
  int resident_waves; // waves of the persistent kernel resident at once
  int direct;         // 1: one wave per grid slot (small batches), 0: persistent + work list
  int32_t* err_flag;  // may be null
  int batch, num_heads, num_kv_heads, group;  // group = num_heads / num_kv_heads
  int head_chunks;    // ceil(group / 16): a wave covers at most 16 q heads
  int num_blocks, max_blocks_per_seq;
  int part_tokens;    // partition length in tokens (multiple of block_size)
  int n_parts;        // partitions per sequence slot in the workspace (1 = single pass)
  int has_new;
  float scale_log2;   // softmax_scale * log2(e): scores live in the exp2 domain
  long long total_units;  // upper bound: batch * n_parts * num_kv_heads * head_chunks
};

// Packed varlen (k, v packed, cu_k) or paged varlen (k, v are the caches,
// keys through block_table, lengths seqlens_k).
struct VarlenArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;         // packed only
  const int32_t* block_table;  // paged only: [batch, max_blocks_per_seq]
  const int32_t* seqlens_k;    // paged only: [batch]
  void* out;
  int32_t* err_flag;
  int batch, total_q, total_k, num_heads, num_kv_heads, group;
  int max_len_q, max_len_k;
  int num_blocks, block_size, max_blocks_per_seq;  // paged only
  int heads_per_wg;   // q heads of one kv group sharing a workgroup (1, 2 or 4)
  int q_tiles;        // ceil(max_len_q / rows per workgroup)
  float scale_log2;
};

struct CacheWriteArgs {
  const void* k;
  const void* v;
  const int32_t* cu;
  const int32_t* start;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  int32_t* err_flag;
  int batch, total;
  int row_bytes;      // num_kv_heads * head_dim * element size (a multiple of 16)
  int num_blocks, block_size, max_blocks_per_seq;
};

// Launchers return hipSuccess or the launch error.  dtype: 0 fp32, 1 bf16.
// phases: bit 0 = per-partition kernel (with the append), bit 1 = merge.
hipError_t launch_decode(int dtype, int head_dim, int block_size, const DecodeArgs& a,
                         int phases, hipStream_t stream);
hipError_t launch_varlen(int dtype, int head_dim, const VarlenArgs& a, hipStream_t stream);
hipError_t launch_varlen_paged(int dtype, int head_dim, const VarlenArgs& a, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t stream);

struct CopyBlocksArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* src;
  const int32_t* dst;
  int32_t* err_flag;
  int n;              // pairs
  int num_blocks;
  long long block_bytes;  // block_size * num_kv_heads * head_dim * element size
};
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);
// The library's own decode workspace for callers that cannot allocate: its
// size, and its device address on the current device (looked up once per
// device, then cached).
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(void** ptr);
// Table entries one paged-varlen workgroup stages in LDS (bounds max_length_k).
constexpr int kVarlenMaxTableEntries = 2048;
// Workgroup shape of the varlen kernel for a q-heads-per-kv-head ratio.
int varlen_heads_per_workgroup(int group);
int varlen_rows_per_workgroup(int group);

}  // namespace pkv
