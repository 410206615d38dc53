// Host entry points of libpkv.so: argument checks, the split-context launch
// plan, workspace sizing and the launches.  No allocation, no state, no
// synchronisation (see include/pkv.h for the contract).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_kernels.h"

namespace {

constexpr int kMaxPartitionBlocks = 256;  // LDS table slice per wave
constexpr int kAbiVersion = 3;

bool decode_shape_ok(int head_dim, int block_size) {
  return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32);
}

// Library choice of partition length: 512 tokens when the batch has enough
// units for that (each row assumed to average half its table span), else
// the length at which the expected units give each of the 2048 resident
// waves of the per-partition kernel about 1.75 of them, rounded up to a
// multiple of 64 tokens, at least 128; the whole row when it is shorter.
// Always a block multiple within the LDS slice.  Measured with the
// last-level cache flushed before each step, GQA-4 batches of 512..4096
// tokens, whole step: 32 sequences 83.2 (128-token partitions) / 77.0 (192)
// / 72.6 (384) us, 64 sequences 136.3 (256) / 130.5 (320) / 132.6 (384) /
// 137.0 (608) us, 128 sequences 235.8 (512) / 233.7 (640) us; the optimum
// moves in jumps with the drawn lengths (how the last round of units falls
// on the resident waves), which the host cannot see -- this rule picks 192 /
// 320 / 512 (the previous one, halving 512 while fewer than two units per
// wave were expected, picked 128 / 256 / 512).
int choose_partition(int batch, int num_kv_heads, int head_chunks, int block_size,
                     int max_blocks_per_seq) {
  const long long span = (long long)max_blocks_per_seq * block_size;
  const long long cap = (long long)kMaxPartitionBlocks * block_size;
  const long long base_units = (long long)batch * num_kv_heads * head_chunks;
  const double target = 1.75 * 2048;  // units
  const double half = (double)span / 2;
  long long p = 512;
  // expected units at partition p: base_units * (half / p + 0.5)
  if ((double)base_units * (half / 512 + 0.5) < target) {
    const double per_row = target / (double)base_units - 0.5;  // partitions per row
    const double want = half / per_row;
    p = ((long long)want + 63) / 64 * 64;
    if (p < 128) p = 128;
    if (p > 512) p = 512;
  }
  if (p > cap) p = cap;
  p -= p % block_size;
  if (p < block_size) p = block_size;
  if (span <= p) return (int)span;  // a single pass covers every row
  return (int)p;
}

struct DecodePlan {
  int part_tokens;
  int n_parts;
  int head_chunks;
};

int check_decode(int dtype, int has_new, int batch, int num_heads, int num_kv_heads, int head_dim,
                 int num_blocks, int block_size, int max_blocks_per_seq, int partition_tokens) {
  if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || partition_tokens < 0 || (has_new != 0 && has_new != 1))
    return PKV_EINVAL;
  if (dtype != PKV_FP32 && dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return PKV_EINVAL;
  if (!decode_shape_ok(head_dim, block_size)) return PKV_EUNSUPPORTED;
  if (partition_tokens != 0 &&
      (partition_tokens % block_size != 0 || partition_tokens / block_size > kMaxPartitionBlocks))
    return PKV_EUNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size > INT_MAX / 2) return PKV_EINVAL;
  if ((long long)num_blocks * block_size * num_kv_heads * head_dim > (1LL << 46)) return PKV_EINVAL;
  return PKV_OK;
}

DecodePlan plan_decode(int batch, int num_heads, int num_kv_heads, int block_size,
                       int max_blocks_per_seq, int partition_tokens) {
  DecodePlan p;
  const int group = num_heads / num_kv_heads;
  p.head_chunks = (group + 15) / 16;
  const long long span = (long long)max_blocks_per_seq * block_size;
  int pt = partition_tokens != 0
               ? partition_tokens
               : choose_partition(batch, num_kv_heads, p.head_chunks, block_size, max_blocks_per_seq);
  if (pt <= 0) pt = block_size;
  if (span <= pt) {
    // one pass; the partition spans the whole row (bounded by the LDS slice)
    if (span / block_size <= kMaxPartitionBlocks) {
      p.part_tokens = span > 0 ? (int)span : block_size;
      p.n_parts = 1;
      return p;
    }
  }
  p.part_tokens = pt;
  p.n_parts = (int)((span + pt - 1) / pt);
  if (p.n_parts < 1) p.n_parts = 1;
  return p;
}

// Workspace layout: [ctrl: 256 B][work items: batch * n_parts * 16 B]
// [partial sums: batch * heads * n_parts * head_dim * 4 B][(m, l) pairs], each
// part 256-byte aligned.
struct WorkspaceLayout {
  size_t items, acc, ml, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WorkspaceLayout layout_for(const DecodePlan& p, int batch, int num_heads, int head_dim) {
  WorkspaceLayout w;
  const size_t slots = (size_t)batch * num_heads * p.n_parts;
  w.items = 256;
  w.acc = w.items + align256((size_t)batch * p.n_parts * 16);
  w.ml = w.acc + (p.n_parts > 1 ? align256(slots * head_dim * sizeof(float)) : 0);
  w.total = w.ml + (p.n_parts > 1 ? align256(slots * 2 * sizeof(float)) : 0);
  return w;
}

size_t workspace_for(const DecodePlan& p, int batch, int num_heads, int head_dim) {
  return layout_for(p, batch, num_heads, head_dim).total;
}

}  // namespace

namespace pkv {

// Workgroup shape of the varlen kernels: 4 waves of 32 query rows share one
// kv head, taking up to 4 q heads of its group for the same rows (else
// several 32-row blocks of one head).
int varlen_heads_per_workgroup(int group) {
  return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
}

int varlen_rows_per_workgroup(int group) { return 32 * (4 / varlen_heads_per_workgroup(group)); }

}  // namespace pkv

extern "C" {

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape or dtype";
    case PKV_EWORKSPACE: return "workspace missing or too small";
    case PKV_EHIP: return "HIP launch failed";
    case PKV_ENOMEM: return "not enough free blocks";
    default: return "unknown status";
  }
}

int pkv_abi_version(void) { return kAbiVersion; }

int pkv_check_decode_args(int dtype, int has_new, int batch, int num_heads, int num_kv_heads,
                          int head_dim, int num_blocks, int block_size, int max_blocks_per_seq,
                          int partition_tokens) {
  return check_decode(dtype, has_new, batch, num_heads, num_kv_heads, head_dim, num_blocks,
                      block_size, max_blocks_per_seq, partition_tokens);
}

int pkv_decode_partition_tokens(int batch, int num_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_blocks_per_seq, int partition_tokens) {
  if (check_decode(PKV_BF16, 0, batch, num_heads, num_kv_heads, head_dim, 1, block_size,
                   max_blocks_per_seq, partition_tokens) != PKV_OK)
    return -1;
  return plan_decode(batch, num_heads, num_kv_heads, block_size, max_blocks_per_seq,
                     partition_tokens)
      .part_tokens;
}

size_t pkv_decode_workspace_bytes(int batch, int num_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_blocks_per_seq, int partition_tokens) {
  if (check_decode(PKV_BF16, 0, batch, num_heads, num_kv_heads, head_dim, 1, block_size,
                   max_blocks_per_seq, partition_tokens) != PKV_OK)
    return 0;
  DecodePlan p = plan_decode(batch, num_heads, num_kv_heads, block_size, max_blocks_per_seq,
                             partition_tokens);
  return workspace_for(p, batch, num_heads, head_dim);
}

}  // extern "C"

namespace {

// own_scratch: the library's static decode scratch replaces the caller's
// workspace (pkv_decode_noalloc).
int decode_impl(int phases, bool own_scratch, int dtype, const void* q, void* k_cache,
                void* v_cache,
                const int32_t* block_table, const int32_t* cache_seqlens,
                const void* k_new, const void* v_new, void* out,
                int batch, int num_heads, int num_kv_heads, int head_dim,
                int num_blocks, int block_size, int max_blocks_per_seq,
                float softmax_scale, int partition_tokens,
                void* workspace, size_t workspace_bytes,
                int32_t* err_flag, void* stream) {
  const int has_new = k_new != nullptr;
  if ((k_new == nullptr) != (v_new == nullptr)) return PKV_EINVAL;
  int rc = check_decode(dtype, has_new, batch, num_heads, num_kv_heads, head_dim, num_blocks,
                        block_size, max_blocks_per_seq, partition_tokens);
  if (rc != PKV_OK) return rc;
  if (!isfinite(softmax_scale)) return PKV_EINVAL;
  if (batch == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_table || !cache_seqlens || !out) return PKV_EINVAL;
  DecodePlan p = plan_decode(batch, num_heads, num_kv_heads, block_size, max_blocks_per_seq,
                             partition_tokens);
  const size_t need = workspace_for(p, batch, num_heads, head_dim);
  if (own_scratch) {
    if (need > pkv::kDecodeScratchBytes) return PKV_EWORKSPACE;
    // the scratch address is per device: the launch must go to the current one
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PKV_EHIP;
    if (stream != nullptr) {
      hipDevice_t sdev = -1;
      if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return PKV_EHIP;
      if (sdev != dev) return PKV_EINVAL;
    }
    if (pkv::decode_scratch(&workspace) != hipSuccess) return PKV_EHIP;
    workspace_bytes = pkv::kDecodeScratchBytes;
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PKV_EWORKSPACE;

  pkv::DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.cache_seqlens = cache_seqlens;
  a.k_new = k_new;
  a.v_new = v_new;
  a.out = out;
  const WorkspaceLayout wl = layout_for(p, batch, num_heads, head_dim);
  a.ctrl = (int*)workspace;
  a.items = (int4*)((char*)workspace + wl.items);
  a.ws_acc = p.n_parts > 1 ? (float*)((char*)workspace + wl.acc) : nullptr;
  a.ws_ml = p.n_parts > 1 ? (float2*)((char*)workspace + wl.ml) : nullptr;
  a.err_flag = err_flag;
  a.batch = batch;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.head_chunks = p.head_chunks;
  a.num_blocks = num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.part_tokens = p.part_tokens;
  a.n_parts = p.n_parts;
  a.has_new = has_new;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.total_units = (long long)batch * p.n_parts * num_kv_heads * p.head_chunks;
  // a work item may stream up to 8 consecutive partitions, within the table
  // slice one wave stages
  const int slice_runs = kMaxPartitionBlocks / (p.part_tokens / block_size);
  a.max_run = slice_runs < 1 ? 1 : (slice_runs > 8 ? 8 : slice_runs);
  a.resident_waves = 1;
  a.direct = 0;
  if (a.total_units >= (1LL << 31)) return PKV_EUNSUPPORTED;
  hipError_t e = pkv::launch_decode(dtype, head_dim, block_size, a, phases, (hipStream_t)stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // namespace

extern "C" {

#define PKV_DECODE_ARGS                                                                        \
  int dtype, const void *q, void *k_cache, void *v_cache, const int32_t *block_table,          \
      const int32_t *cache_seqlens, const void *k_new, const void *v_new, void *out,           \
      int batch, int num_heads, int num_kv_heads, int head_dim, int num_blocks, int block_size, \
      int max_blocks_per_seq, float softmax_scale, int partition_tokens, void *workspace,      \
      size_t workspace_bytes, int32_t *err_flag, void *stream
#define PKV_DECODE_FWD                                                                     \
  dtype, q, k_cache, v_cache, block_table, cache_seqlens, k_new, v_new, out, batch,        \
      num_heads, num_kv_heads, head_dim, num_blocks, block_size, max_blocks_per_seq,       \
      softmax_scale, partition_tokens, workspace, workspace_bytes, err_flag, stream

int pkv_decode(PKV_DECODE_ARGS) { return decode_impl(3, false, PKV_DECODE_FWD); }
int pkv_decode_partials(PKV_DECODE_ARGS) { return decode_impl(1, false, PKV_DECODE_FWD); }
int pkv_decode_merge(PKV_DECODE_ARGS) { return decode_impl(2, false, PKV_DECODE_FWD); }

int pkv_decode_noalloc(int dtype, const void* q, void* k_cache, void* v_cache,
                       const int32_t* block_table, const int32_t* cache_seqlens,
                       const void* k_new, const void* v_new, void* out, int batch,
                       int num_heads, int num_kv_heads, int head_dim, int num_blocks,
                       int block_size, int max_blocks_per_seq, float softmax_scale,
                       int partition_tokens, int32_t* err_flag, void* stream) {
  return decode_impl(3, true, dtype, q, k_cache, v_cache, block_table, cache_seqlens, k_new,
                     v_new, out, batch, num_heads, num_kv_heads, head_dim, num_blocks, block_size,
                     max_blocks_per_seq, softmax_scale, partition_tokens, nullptr, 0, err_flag,
                     stream);
}

int pkv_check_varlen_args(int dtype, int batch, int total_q, int total_k, int num_heads,
                          int num_kv_heads, int head_dim, int max_length_q, int max_length_k) {
  if (batch < 0 || total_q < 0 || total_k < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      max_length_q < 0 || max_length_k < 0)
    return PKV_EINVAL;
  if (dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if ((long long)total_q * num_heads * head_dim * 2 > (1LL << 31) * 64) return PKV_EINVAL;
  if ((long long)total_k * num_kv_heads * head_dim * 2 > (1LL << 31) * 64) return PKV_EINVAL;
  return PKV_OK;
}

int pkv_varlen(int dtype, const void* q, const void* k, const void* v,
               const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
               int max_length_q, int max_length_k, void* out,
               int batch, int total_q, int total_k, int num_heads, int num_kv_heads,
               int head_dim, float softmax_scale, int32_t* err_flag, void* stream) {
  int rc = pkv_check_varlen_args(dtype, batch, total_q, total_k, num_heads, num_kv_heads, head_dim,
                                 max_length_q, max_length_k);
  if (rc != PKV_OK) return rc;
  if (!isfinite(softmax_scale)) return PKV_EINVAL;
  if (batch == 0 || total_q == 0) return PKV_OK;
  if (!q || !out || !cu_seq_lens_q || !cu_seq_lens_k || (total_k > 0 && (!k || !v)))
    return PKV_EINVAL;
  const int rows = pkv::varlen_rows_per_workgroup(num_heads / num_kv_heads);
  const long long tiles = ((long long)max_length_q + rows - 1) / rows;
  if (tiles > 65535 || batch > 65535 || num_heads > 65535) return PKV_EUNSUPPORTED;
  pkv::VarlenArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_seq_lens_q;
  a.cu_k = cu_seq_lens_k;
  a.out = out;
  a.err_flag = err_flag;
  a.batch = batch;
  a.total_q = total_q;
  a.total_k = total_k;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.max_len_q = max_length_q;
  a.max_len_k = max_length_k;
  a.heads_per_wg = pkv::varlen_heads_per_workgroup(a.group);
  a.q_tiles = (int)tiles;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipError_t e = pkv::launch_varlen(dtype, head_dim, a, (hipStream_t)stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}


int pkv_check_cache_write_args(int dtype, int batch, int total, int num_kv_heads, int head_dim,
                               int num_blocks, int block_size, int max_blocks_per_seq) {
  if (batch < 0 || total < 0 || num_kv_heads <= 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return PKV_EINVAL;
  if (batch == 0 && total != 0) return PKV_EINVAL;
  if (dtype != PKV_FP32 && dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (block_size != 16 && block_size != 32) return PKV_EUNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size > INT32_MAX) return PKV_EINVAL;
  if ((long long)num_kv_heads * head_dim * (dtype == PKV_BF16 ? 2 : 4) > INT32_MAX / 2)
    return PKV_EINVAL;
  return PKV_OK;
}

int pkv_cache_write(int dtype, const void* k, const void* v, const int32_t* cu_seq_lens,
                    const int32_t* start, void* k_cache, void* v_cache,
                    const int32_t* block_table, int batch, int total, int num_kv_heads,
                    int head_dim, int num_blocks, int block_size, int max_blocks_per_seq,
                    int32_t* err_flag, void* stream) {
  int rc = pkv_check_cache_write_args(dtype, batch, total, num_kv_heads, head_dim, num_blocks,
                                      block_size, max_blocks_per_seq);
  if (rc != PKV_OK) return rc;
  if (batch == 0) return PKV_OK;
  if (!cu_seq_lens || !start || !block_table || !k_cache || !v_cache ||
      (total > 0 && (!k || !v)))
    return PKV_EINVAL;
  pkv::CacheWriteArgs a;
  a.k = k;
  a.v = v;
  a.cu = cu_seq_lens;
  a.start = start;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.err_flag = err_flag;
  a.batch = batch;
  a.total = total;
  a.row_bytes = num_kv_heads * head_dim * (dtype == PKV_BF16 ? 2 : 4);
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  hipError_t e = pkv::launch_cache_write(a, (hipStream_t)stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

int pkv_check_varlen_paged_args(int dtype, int batch, int total_q, int num_heads,
                                int num_kv_heads, int head_dim, int num_blocks, int block_size,
                                int max_blocks_per_seq, int max_length_q, int max_length_k) {
  if (batch < 0 || total_q < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks < 0 ||
      max_blocks_per_seq < 0 || max_length_q < 0 || max_length_k < 0)
    return PKV_EINVAL;
  if (dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  if (num_heads % num_kv_heads != 0) return PKV_EINVAL;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (block_size != 16 && block_size != 32) return PKV_EUNSUPPORTED;
  if ((long long)max_length_k > (long long)pkv::kVarlenMaxTableEntries * block_size)
    return PKV_EUNSUPPORTED;
  if ((long long)total_q * num_heads * head_dim * 2 > (1LL << 31) * 64) return PKV_EINVAL;
  // a block's bytes per kv head row set must stay a 32-bit buffer range
  if ((long long)block_size * num_kv_heads * head_dim * 2 > INT32_MAX) return PKV_EINVAL;
  return PKV_OK;
}

int pkv_varlen_paged(int dtype, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* cu_seq_lens_q,
                     const int32_t* seqlens_k, int max_length_q, int max_length_k, void* out,
                     int batch, int total_q, int num_heads, int num_kv_heads, int head_dim,
                     int num_blocks, int block_size, int max_blocks_per_seq,
                     float softmax_scale, int32_t* err_flag, void* stream) {
  int rc = pkv_check_varlen_paged_args(dtype, batch, total_q, num_heads, num_kv_heads, head_dim,
                                       num_blocks, block_size, max_blocks_per_seq, max_length_q,
                                       max_length_k);
  if (rc != PKV_OK) return rc;
  if (!isfinite(softmax_scale)) return PKV_EINVAL;
  if (batch == 0 || total_q == 0) return PKV_OK;
  if (!q || !out || !cu_seq_lens_q || !seqlens_k || !block_table ||
      (max_length_k > 0 && (!k_cache || !v_cache)))
    return PKV_EINVAL;
  const int group = num_heads / num_kv_heads;
  const int rows = pkv::varlen_rows_per_workgroup(group);
  const long long tiles = ((long long)max_length_q + rows - 1) / rows;
  if (tiles > 65535 || batch > 65535 || num_heads > 65535) return PKV_EUNSUPPORTED;
  pkv::VarlenArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.cu_q = cu_seq_lens_q;
  a.cu_k = nullptr;
  a.block_table = block_table;
  a.seqlens_k = seqlens_k;
  a.out = out;
  a.err_flag = err_flag;
  a.batch = batch;
  a.total_q = total_q;
  a.total_k = 0;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.max_len_q = max_length_q;
  a.max_len_k = max_length_k;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.heads_per_wg = pkv::varlen_heads_per_workgroup(group);
  a.q_tiles = (int)tiles;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipError_t e = pkv::launch_varlen_paged(dtype, head_dim, a, (hipStream_t)stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}


int pkv_copy_blocks(int dtype, void* k_cache, void* v_cache, const int32_t* src,
                    const int32_t* dst, int n, int num_blocks, int block_size, int num_kv_heads,
                    int head_dim, int32_t* err_flag, void* stream) {
  if (n < 0 || num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_EINVAL;
  if (dtype != PKV_FP32 && dtype != PKV_BF16) return PKV_EUNSUPPORTED;
  if (n == 0) return PKV_OK;
  if (n > 65535) return PKV_EUNSUPPORTED;
  if (!k_cache || !v_cache || !src || !dst) return PKV_EINVAL;
  const long long block_bytes =
      (long long)block_size * num_kv_heads * head_dim * (dtype == PKV_BF16 ? 2 : 4);
  if (block_bytes % 16 != 0) return PKV_EUNSUPPORTED;
  pkv::CopyBlocksArgs a;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.src = src;
  a.dst = dst;
  a.err_flag = err_flag;
  a.n = n;
  a.num_blocks = num_blocks;
  a.block_bytes = block_bytes;
  hipError_t e = pkv::launch_copy_blocks(a, (hipStream_t)stream);
  return e == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"
