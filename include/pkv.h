/*
 * pkv.h -- C ABI of libpkv.so: paged attention for one AMD MI355X (gfx950).
 *
 * Two calls compute attention; the rest are host-only helpers.
 *
 *   pkv_decode  one query token per sequence attends every cached token of
 *               its sequence, reading K and V through a block table, with the
 *               new token's K/V optionally written in place first.
 *               Defined by: HF Transformers "paged attention" page, section
 *               "Jalur decode" (block_table of shape (batch_size,
 *               max_blocks_per_seq), rows of physical block ids, -1 =
 *               unallocated, cache_seqlens, one token per sequence, in-place
 *               cache update); inference-notes "39 · PagedAttention",
 *               sections 1-3 (one softmax over all scores, exact, partial
 *               (m, l) results merged as m = max(m1, m2),
 *               l = l1 e^(m1-m) + l2 e^(m2-m)).
 *   pkv_varlen  packed variable-length sequences delimited by cumulative
 *               lengths, no mask: every query row attends every key row of
 *               its own sequence.  Defined by: HF "paged attention" page,
 *               section "Jalur Varlen" (cu_seq_lens_q/k, max_length_q/k,
 *               packed shapes [1, total, heads, head_dim]).
 *
 * Two more calls serve a prefill over a paged cache.  The same "Jalur
 * Varlen" section notes that the varlen kernel cannot reach the paged cache,
 * so the cache must be written (and read) around it by a separate update:
 *
 *   pkv_cache_write   scatters packed new K/V rows into their cache slots
 *                     through the block table (the "Jalur decode" address
 *                     rule applied to every row), bit for bit.
 *   pkv_varlen_paged  the varlen computation with each request's keys read
 *                     straight from the paged cache through its block-table
 *                     row, so no packed copy of a cached prefix is needed.
 *
 * Conventions shared by every call
 *  - Every tensor pointer is DEVICE memory owned by the caller, row-major,
 *    densely packed in the shape given.  The library allocates nothing,
 *    keeps no state between calls and never synchronises: work is enqueued
 *    on `stream` (a hipStream_t; NULL = the null stream) and results are
 *    valid once the caller has synchronised that stream.  Calls on different
 *    streams may run concurrently; `out` must not alias any input.
 *  - dtype: PKV_FP32 or PKV_BF16 for q, K, V, new K/V and out alike.
 *    Arithmetic is fp32 (bf16 products accumulate in fp32); the output is
 *    rounded to the input dtype (bf16: round to nearest even).
 *  - Grouped heads: q head h reads kv head h / (num_heads / num_kv_heads);
 *    num_heads must be a multiple of num_kv_heads.
 *  - Index tensors are int32.
 *  - Errors a host check can see (null pointer, bad size, unsupported shape,
 *    short workspace) return a status and enqueue nothing.  Errors in device
 *    data (a needed block_table entry that is -1 or >= num_blocks, a
 *    sequence longer than its table row, a bad cu_seq_lens array, a length
 *    above max_length_*) cannot be seen without a sync: the kernels never
 *    read or write out of bounds for them, OR a PKV_ERR_* bit into *err_flag
 *    (when err_flag is not NULL) and write NaN to that sequence's output.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* null pointer, negative or inconsistent size      */
  PKV_EUNSUPPORTED = 2,  /* shape or dtype this build has no kernel for       */
  PKV_EWORKSPACE = 3,    /* workspace NULL or smaller than required           */
  PKV_EHIP = 4,          /* the HIP runtime refused a launch                  */
  PKV_ENOMEM = 5         /* block manager: not enough free blocks (nothing changed) */
} pkv_status;

typedef enum { PKV_FP32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Bits OR-ed into *err_flag by the kernels (sticky: never cleared). */
#define PKV_ERR_BLOCK 1u   /* a needed block_table entry is -1 or >= num_blocks            */
#define PKV_ERR_SPAN 2u    /* cache_seqlens < 0, or cached (+ new) tokens exceed the row   */
#define PKV_ERR_CU 4u      /* cu_seq_lens not 0-based, decreasing, or not ending at total   */
#define PKV_ERR_MAXLEN 8u  /* a sequence longer than max_length_q / max_length_k            */

/* Text for a status code (static storage, never NULL). */
const char* pkv_status_string(int status);

/* ABI version of this library (bumped on any signature or layout change). */
int pkv_abi_version(void);

/*
 * Host-only validation of pkv_decode's scalar arguments (no device access,
 * usable without a GPU).  has_new is 1 when k_new/v_new are given.
 * Supported: head_dim 64 or 128; block_size 16 or 32; num_heads a multiple
 * of num_kv_heads; partition_tokens 0 (library choice) or a multiple of
 * block_size no larger than 256 blocks.
 */
int pkv_check_decode_args(int dtype, int has_new, int batch, int num_heads, int num_kv_heads,
                          int head_dim, int num_blocks, int block_size, int max_blocks_per_seq,
                          int partition_tokens);

/*
 * The split-context partition pkv_decode will use for these arguments, in
 * tokens: either the caller's non-zero partition_tokens, or the library's
 * choice for 0 (512 tokens, fewer -- down to 128 -- when the batch is too
 * small to give every SIMD a unit, the whole row when it is shorter; always
 * a block multiple).  A result >= max_blocks_per_seq * block_size means a single
 * pass (no partial results and no merge).  Returns -1 when
 * pkv_check_decode_args fails.
 */
int pkv_decode_partition_tokens(int batch, int num_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_blocks_per_seq, int partition_tokens);

/*
 * Bytes of device workspace pkv_decode needs: a work list of (sequence,
 * partition) items and a ticket counter, plus, with a split, fp32 partial
 * results (m, l, acc[head_dim]) for every (sequence, q head, partition).
 * Returns 0 for arguments pkv_check_decode_args rejects.
 */
size_t pkv_decode_workspace_bytes(int batch, int num_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_blocks_per_seq, int partition_tokens);

/*
 * Paged decode attention (HF page "Jalur decode"; inference-notes sections
 * 1-3).
 *
 *   q              [batch, 1, num_heads, head_dim]
 *   k_cache,       [num_blocks, block_size, num_kv_heads, head_dim]; token u of
 *   v_cache          physical block pb, kv head g is row (pb*block_size+u)*num_kv_heads+g.
 *                    Written ONLY at the new tokens' slots.
 *   block_table    [batch, max_blocks_per_seq] int32; logical block j of
 *                    sequence i is physical block block_table[i][j]; -1 =
 *                    unallocated.  Only entries j < ceil(L'_i / block_size)
 *                    are read (L'_i defined below).  Never modified.
 *   cache_seqlens  [batch] int32: L_i, tokens cached BEFORE this call.  Never
 *                    modified (the caller advances it).
 *   k_new, v_new   [batch, 1, num_kv_heads, head_dim], or both NULL.  When
 *                    given, sequence i's row is copied bit for bit into slot
 *                    L_i (logical block L_i / block_size, offset L_i mod
 *                    block_size; the caller must already have put that block
 *                    in the table) and is attended: L'_i = L_i + 1.  Without
 *                    them L'_i = L_i.
 *   out            [batch, 1, num_heads, head_dim]; L'_i = 0 gives zeros.
 *   softmax_scale  multiplies q.k before the softmax (1/sqrt(head_dim) usual).
 *   partition_tokens  split-context partition length in tokens (0 = library
 *                    choice, see pkv_decode_partition_tokens).  Partitions are
 *                    fixed logical token ranges; their partial (m, l, acc)
 *                    are merged by a second kernel.
 *   workspace      device buffer of at least pkv_decode_workspace_bytes(...)
 *                    bytes.  Scratch only: its contents need no
 *                    initialisation and are meaningless after the call.
 *   err_flag       device int32, optional (NULL = no reporting); PKV_ERR_* bits.
 *   stream         hipStream_t.
 *
 * Results depend only on logical positions: any placement of the same
 * logical blocks gives bit-identical output, and repeated calls agree
 * bitwise.  Two sequences must not append into the same slot.
 */
int pkv_decode(int dtype, const void* q, void* k_cache, void* v_cache,
               const int32_t* block_table, const int32_t* cache_seqlens,
               const void* k_new, const void* v_new, void* out,
               int batch, int num_heads, int num_kv_heads, int head_dim,
               int num_blocks, int block_size, int max_blocks_per_seq,
               float softmax_scale, int partition_tokens,
               void* workspace, size_t workspace_bytes,
               int32_t* err_flag, void* stream);

/*
 * The two phases of pkv_decode as separate calls, same arguments and same
 * checks.  pkv_decode_partials enqueues the per-partition kernel (and the
 * in-place append): with a split it writes fp32 partial results (m, l,
 * acc[head_dim]) of every (sequence, q head, partition) into the workspace,
 * without a split it writes `out` directly.  pkv_decode_merge enqueues the
 * merge of those partials into `out` (m = max m_k, l = sum l_k e^(m_k - m),
 * out = sum acc_k e^(m_k - m) / l; inference-notes section 3) and does
 * nothing without a split.  Calling partials then merge on one stream with
 * the same arguments and workspace is exactly pkv_decode.  The workspace
 * layout is private to this library version.
 */
int pkv_decode_partials(int dtype, const void* q, void* k_cache, void* v_cache,
                        const int32_t* block_table, const int32_t* cache_seqlens,
                        const void* k_new, const void* v_new, void* out,
                        int batch, int num_heads, int num_kv_heads, int head_dim,
                        int num_blocks, int block_size, int max_blocks_per_seq,
                        float softmax_scale, int partition_tokens,
                        void* workspace, size_t workspace_bytes,
                        int32_t* err_flag, void* stream);
int pkv_decode_merge(int dtype, const void* q, void* k_cache, void* v_cache,
                     const int32_t* block_table, const int32_t* cache_seqlens,
                     const void* k_new, const void* v_new, void* out,
                     int batch, int num_heads, int num_kv_heads, int head_dim,
                     int num_blocks, int block_size, int max_blocks_per_seq,
                     float softmax_scale, int partition_tokens,
                     void* workspace, size_t workspace_bytes,
                     int32_t* err_flag, void* stream);

/*
 * pkv_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments and results as pkv_decode without the workspace, which is
 * instead a static array of PKV_DECODE_NOALLOC_SCRATCH_BYTES per GPU inside
 * the library (reserved on every GPU the library runs on until the process
 * ends).  No hipMalloc, hipFree or other allocation happens in the call; the
 * first call on a device looks the array's address up once.
 *
 *  - Returns PKV_EWORKSPACE, enqueuing nothing, when pkv_decode_workspace_bytes
 *    for these arguments exceeds PKV_DECODE_NOALLOC_SCRATCH_BYTES (a longer
 *    partition_tokens needs less: e.g. 512 sequences x 32 heads x 8208 tokens
 *    fit with 2048-token partitions); PKV_EINVAL when `stream` belongs to a
 *    device other than the current one.
 *  - Every call on one GPU uses the same array: calls that may overlap in
 *    time on one GPU (different streams, different host threads) race and
 *    must be serialised by the caller.  Calls on one stream are ordered and
 *    safe.  The array needs no initialisation; each call's kernels write
 *    whatever they later read.
 */
#define PKV_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pkv_decode_noalloc(int dtype, const void* q, void* k_cache, void* v_cache,
                       const int32_t* block_table, const int32_t* cache_seqlens,
                       const void* k_new, const void* v_new, void* out,
                       int batch, int num_heads, int num_kv_heads, int head_dim,
                       int num_blocks, int block_size, int max_blocks_per_seq,
                       float softmax_scale, int partition_tokens,
                       int32_t* err_flag, void* stream);

/*
 * Host-only validation of pkv_varlen's scalar arguments.  Supported: bf16;
 * head_dim 64 or 128; num_heads a multiple of num_kv_heads.
 */
int pkv_check_varlen_args(int dtype, int batch, int total_q, int total_k, int num_heads,
                          int num_kv_heads, int head_dim, int max_length_q, int max_length_k);

/*
 * Variable-length attention over packed sequences, no mask (HF page
 * "Jalur Varlen").
 *
 *   q              [1, total_q, num_heads, head_dim]
 *   k, v           [1, total_k, num_kv_heads, head_dim]
 *   cu_seq_lens_q  [batch + 1] int32: query rows of sequence b are
 *                    cu_seq_lens_q[b] .. cu_seq_lens_q[b+1]-1 (cu[0] = 0,
 *                    non-decreasing, cu[batch] = total_q).
 *   cu_seq_lens_k  [batch + 1] int32, the same for key/value rows.
 *   max_length_q,  upper bounds on the per-sequence lengths; they size the
 *   max_length_k     launch.  A longer sequence is a data error.
 *   out            [1, total_q, num_heads, head_dim]; a sequence with no key
 *                    row outputs zeros.
 *   err_flag       device int32, optional.
 */
int pkv_varlen(int dtype, const void* q, const void* k, const void* v,
               const int32_t* cu_seq_lens_q, const int32_t* cu_seq_lens_k,
               int max_length_q, int max_length_k, void* out,
               int batch, int total_q, int total_k, int num_heads, int num_kv_heads,
               int head_dim, float softmax_scale, int32_t* err_flag, void* stream);

/*
 * Host-only validation of pkv_cache_write's scalar arguments.  Supported:
 * fp32 or bf16; head_dim 64 or 128; block_size 16 or 32.
 */
int pkv_check_cache_write_args(int dtype, int batch, int total, int num_kv_heads, int head_dim,
                               int num_blocks, int block_size, int max_blocks_per_seq);

/*
 * Writes packed K/V rows into the paged cache (HF page, "Jalur Varlen",
 * cache behaviour; slot rule of "Jalur decode").
 *
 *   k, v           [1, total, num_kv_heads, head_dim]: new rows, request b's
 *                    rows are cu_seq_lens[b] .. cu_seq_lens[b+1]-1.
 *   cu_seq_lens    [batch + 1] int32 (cu[0] = 0, non-decreasing, cu[batch] =
 *                    total).
 *   start          [batch] int32: tokens of sequence b already cached; row
 *                    cu[b] + i becomes token p = start[b] + i, stored at slot
 *                    p mod block_size of physical block block_table[b][p /
 *                    block_size].  Never modified (the caller advances it).
 *   k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim]; only
 *                    the target slots are written, each with a bit-for-bit
 *                    copy of its row.
 *   block_table    [batch, max_blocks_per_seq] int32; the caller has put every
 *                    needed block in the table.
 *   err_flag       device int32, optional.
 *
 * A row whose slot cannot be resolved (cu not a valid cumulative array:
 * PKV_ERR_CU; start < 0 or p past the table row: PKV_ERR_SPAN; entry -1 or
 * >= num_blocks: PKV_ERR_BLOCK) is not written and sets the bit; the other
 * rows are written.  Two rows must not target the same slot.
 */
int pkv_cache_write(int dtype, const void* k, const void* v, const int32_t* cu_seq_lens,
                    const int32_t* start, void* k_cache, void* v_cache,
                    const int32_t* block_table, int batch, int total, int num_kv_heads,
                    int head_dim, int num_blocks, int block_size, int max_blocks_per_seq,
                    int32_t* err_flag, void* stream);

/*
 * Host-only validation of pkv_varlen_paged's scalar arguments.  Supported:
 * bf16; head_dim 64 or 128; block_size 16 or 32; num_heads a multiple of
 * num_kv_heads; max_length_k at most 2048 table entries (32768 tokens at
 * block_size 16).
 */
int pkv_check_varlen_paged_args(int dtype, int batch, int total_q, int num_heads,
                                int num_kv_heads, int head_dim, int num_blocks, int block_size,
                                int max_blocks_per_seq, int max_length_q, int max_length_k);

/*
 * Varlen attention (no mask) whose keys come from the paged cache: query rows
 * cu_seq_lens_q[b] .. cu_seq_lens_q[b+1]-1 attend the first seqlens_k[b]
 * tokens of sequence b, read through block_table[b] (HF page "Jalur Varlen"
 * computation, "Jalur decode" addressing).
 *
 *   q              [1, total_q, num_heads, head_dim]
 *   k_cache, v_cache  [num_blocks, block_size, num_kv_heads, head_dim]; read only.
 *   block_table    [batch, max_blocks_per_seq] int32; entries j <
 *                    ceil(seqlens_k[b] / block_size) are read.
 *   cu_seq_lens_q  [batch + 1] int32.
 *   seqlens_k      [batch] int32: keys of request b (0 gives zeros).
 *   max_length_q,  upper bounds on the per-request lengths; they size the
 *   max_length_k     launch.  A longer request is a data error.
 *   out            [1, total_q, num_heads, head_dim].
 *   err_flag       device int32, optional: PKV_ERR_CU, PKV_ERR_MAXLEN,
 *                    PKV_ERR_SPAN (seqlens_k < 0 or past the table row),
 *                    PKV_ERR_BLOCK; the request's rows get NaN.
 *
 * Given the same keys, the output equals pkv_varlen's bit for bit: the
 * kernels share their arithmetic and differ only in where a key tile is
 * fetched from.
 */
int pkv_varlen_paged(int dtype, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* cu_seq_lens_q,
                     const int32_t* seqlens_k, int max_length_q, int max_length_k, void* out,
                     int batch, int total_q, int num_heads, int num_kv_heads, int head_dim,
                     int num_blocks, int block_size, int max_blocks_per_seq,
                     float softmax_scale, int32_t* err_flag, void* stream);

/* ------------------------------------------------------------ block manager
 *
 * Host-side bookkeeping of the physical blocks of one K/V pool (e2hang
 * notes "Paged Attention", section "物理块管理" (physical block management,
 * block allocation strategy), the logical-page mapping section before it,
 * and its closing "注意事项" (block reclamation, shared-block reference
 * counts); paweldubiel notes "PagedAttention", section "Mechanizm i
 * szczegóły": blocks are added only as a sequence grows, unchanged blocks
 * may be shared):
 *  - a free list handed out from its end (pop) and refilled at its end
 *    (push); initially blocks 0 .. num_blocks-1, so block num_blocks-1 goes
 *    first;
 *  - a sequence of L tokens owns ceil(L / block_size) blocks in logical
 *    order; growing it by n tokens takes ceil((L+n) / block_size) minus the
 *    blocks it has;
 *  - too few free blocks is PKV_ENOMEM and changes nothing (no partial
 *    allocation);
 *  - blocks carry reference counts: a fork shares every block of the parent
 *    with the child; a block returns to the free list when its count drops
 *    to 0;
 *  - copy-on-write: before an append writes into a partially filled last
 *    block that another sequence also holds, that block is replaced in the
 *    appending sequence by a fresh copy.  The manager only decides; the
 *    caller copies the block contents on the GPU (pkv_copy_blocks) before
 *    writing into it.  Full shared blocks are never written, so never copied.
 * Host memory only; no device access.  Calls on one manager are serialised
 * by a mutex inside it.  Sequence ids are caller-chosen int64 keys.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* New manager over blocks 0 .. num_blocks-1, all free.  *out = NULL on error. */
int pkv_bm_create(int num_blocks, int block_size, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);

/* Free blocks now (-1 for a NULL manager). */
int pkv_bm_num_free(const pkv_block_manager* bm);

/* Reference count of a block (0 = free; -1 = bad block id or manager). */
int pkv_bm_ref_count(const pkv_block_manager* bm, int block);

/* New sequence `seq` of num_tokens tokens (its KV rows are written by the
 * caller): takes ceil(num_tokens / block_size) blocks.  EINVAL if seq
 * exists or num_tokens < 0; ENOMEM if too few blocks are free. */
int pkv_bm_allocate(pkv_block_manager* bm, int64_t seq, int num_tokens);

/* New sequence `child` sharing every block and the length of `parent`
 * (each shared block's count + 1).  EINVAL if parent is unknown or child
 * exists. */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);

/* Grows `seq` by num_tokens tokens, to be written at positions L ..
 * L+num_tokens-1.  If L is not a multiple of block_size, num_tokens > 0 and
 * the last block is shared, that block is copied on write: a fresh block
 * replaces it in this sequence, and (old, new) is written to
 * cow_src[0] / cow_dst[0] with *n_cow = 1 (else *n_cow = 0).  Then any
 * further blocks are taken.  On ENOMEM or EINVAL nothing changes.
 * cow_src / cow_dst: host arrays of at least one entry. */
int pkv_bm_append(pkv_block_manager* bm, int64_t seq, int num_tokens, int32_t* cow_src,
                  int32_t* cow_dst, int* n_cow);

/* Ends `seq`: each of its blocks loses one reference, and blocks reaching 0
 * are pushed on the free list in logical order.  EINVAL if unknown. */
int pkv_bm_release(pkv_block_manager* bm, int64_t seq);

/* Tokens of `seq` (-1 if unknown). */
int64_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq);

/* Exports rows of the block table for seqs[0..n): table [n,
 * max_blocks_per_seq] int32 (host), row i = the physical blocks of seqs[i]
 * in logical order, -1 padded; seqlens [n] int32 (host).  EINVAL if a
 * sequence is unknown or has more blocks than max_blocks_per_seq. */
int pkv_bm_table(const pkv_block_manager* bm, const int64_t* seqs, int n,
                 int max_blocks_per_seq, int32_t* table, int32_t* seqlens);

/*
 * Copies whole blocks of both pools on the GPU: for i < n, block src[i] of
 * k_cache and of v_cache ([num_blocks, block_size, num_kv_heads, head_dim])
 * is copied bit for bit onto block dst[i] (the copy-on-write step above).
 * src, dst: device int32 arrays; every dst must differ from every src and
 * from the other dsts.  An id outside [0, num_blocks) sets PKV_ERR_BLOCK and
 * its pair is skipped.
 */
int pkv_copy_blocks(int dtype, void* k_cache, void* v_cache, const int32_t* src,
                    const int32_t* dst, int n, int num_blocks, int block_size, int num_kv_heads,
                    int head_dim, int32_t* err_flag, void* stream);

/* ------------------------------------------------------ measurement aid
 *
 * Reads `bytes` bytes of the device buffer `buf` once, as a plain stream
 * (`workgroups` workgroups of four waves; each wave reads one contiguous
 * chunk of bytes / (4 * workgroups) bytes, rounded up to 1 KiB, in 16-byte
 * loads), with the non-temporal cache hint the
 * decode kernels put on their K/V loads (nontemporal = 1) or none (0).  It
 * computes nothing; timing it gives the practical HBM read ceiling the decode
 * bandwidth is compared with.  `sink` is device memory of workgroups * 4096
 * bytes that the kernel may write (in practice it writes nothing).  bytes
 * must be a multiple of 16; workgroups in 1 .. 65535; a wave's chunk may not
 * exceed 1 GiB.  PKV_EINVAL on bad arguments.
 */
int pkv_stream_read(const void* buf, size_t bytes, void* sink, int workgroups, int nontemporal,
                    void* stream);

/* Copies `bytes` bytes (a multiple of 16, below 2 GiB) from device buffer
 * `src` to device buffer `dst` (not overlapping) with `workgroups`
 * workgroups of 256 lanes: 16-byte loads with the non-temporal hint, eight
 * in flight per lane, and 16-byte stores.  Timing it gives the practical
 * ceiling for kernels that write every byte they read, which the paged
 * cache write is compared with.  PKV_EINVAL on bad arguments.
 */
int pkv_stream_copy(const void* src, void* dst, size_t bytes, int workgroups, void* stream);

/* Runs `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 products
 * (32768 flops each) in every wave of `workgroups` workgroups of 256 lanes,
 * with operands held in registers and no memory traffic: timing it gives the
 * practical dense bf16 matrix-core ceiling (at the clock the part sustains
 * under that load) that the prefill throughput is compared with.  Flops per
 * call: workgroups * 4 waves * iters * 4 * 32768.  `sink` is device memory of
 * workgroups * 1024 bytes that the kernel may write (in practice it writes
 * nothing).  workgroups in 1 .. 65535, iters >= 0.  PKV_EINVAL on bad
 * arguments.
 */
int pkv_mfma_peak(void* sink, int workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
