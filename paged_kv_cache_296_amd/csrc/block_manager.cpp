// Host block manager of one paged K/V pool: free list, per-block reference
// counts, per-sequence logical -> physical block lists, copy-on-write
// decisions.
//
// Rules (e2hang notes "Paged Attention": section "物理块管理", the
// allocator hands out blocks from the end of its free list and puts freed
// blocks back at the end, and refuses an allocation it cannot serve in
// full; the logical-page mapping section: a sequence of L tokens holds
// ceil(L / block_size) blocks; "注意事项": blocks of finished sequences go
// back, shared blocks keep reference counts.  paweldubiel notes
// "PagedAttention", "Mechanizm i szczegóły": a new block is taken only when
// the last one is full -- 4 tokens fit one 4-slot block, the 5th opens the
// second -- and unchanged blocks may be shared.)  Copy-on-write follows from
// sharing: a block two sequences hold must not be written, so the partially
// filled last block is duplicated before an append writes into it.
#include <stdint.h>

#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"

struct pkv_block_manager {
  int num_blocks = 0, block_size = 0;
  std::vector<int32_t> free_list;  // next block handed out = back()
  std::vector<int32_t> ref;        // per block; 0 = free
  struct Seq {
    std::vector<int32_t> blocks;   // logical order
    int64_t len = 0;
  };
  std::unordered_map<int64_t, Seq> seqs;
  mutable std::mutex mu;

  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_list.push_back(b);
  }
};

extern "C" {

int pkv_bm_create(int num_blocks, int block_size, pkv_block_manager** out) {
  if (!out) return PKV_EINVAL;
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0) return PKV_EINVAL;
  auto* bm = new (std::nothrow) pkv_block_manager;
  if (!bm) return PKV_ENOMEM;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->free_list.resize(num_blocks);
  for (int i = 0; i < num_blocks; ++i) bm->free_list[i] = i;
  bm->ref.assign(num_blocks, 0);
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_num_free(const pkv_block_manager* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  return (int)bm->free_list.size();
}

int pkv_bm_ref_count(const pkv_block_manager* bm, int block) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  if (block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int pkv_bm_allocate(pkv_block_manager* bm, int64_t seq, int num_tokens) {
  if (!bm || num_tokens < 0) return PKV_EINVAL;
  std::lock_guard<std::mutex> g(bm->mu);
  if (bm->seqs.count(seq)) return PKV_EINVAL;
  const int64_t need = bm->blocks_for(num_tokens);
  if ((int64_t)bm->free_list.size() < need) return PKV_ENOMEM;
  pkv_block_manager::Seq s;
  s.len = num_tokens;
  s.blocks.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
  bm->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm) return PKV_EINVAL;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end() || bm->seqs.count(child)) return PKV_EINVAL;
  pkv_block_manager::Seq s = it->second;
  for (int32_t b : s.blocks) ++bm->ref[b];
  bm->seqs.emplace(child, std::move(s));
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* bm, int64_t seq, int num_tokens, int32_t* cow_src,
                  int32_t* cow_dst, int* n_cow) {
  if (!bm || num_tokens < 0 || !cow_src || !cow_dst || !n_cow) return PKV_EINVAL;
  *n_cow = 0;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_EINVAL;
  auto& s = it->second;
  if (num_tokens == 0) return PKV_OK;
  // the append writes into the last block when it is partially filled
  const bool writes_last = s.len % bm->block_size != 0;
  const bool cow = writes_last && bm->ref[s.blocks.back()] > 1;
  const int64_t grow = bm->blocks_for(s.len + num_tokens) - (int64_t)s.blocks.size();
  if ((int64_t)bm->free_list.size() < grow + (cow ? 1 : 0)) return PKV_ENOMEM;
  if (cow) {
    const int32_t old = s.blocks.back();
    const int32_t fresh = bm->take();
    --bm->ref[old];  // still held by the other sequence(s): never reaches 0 here
    s.blocks.back() = fresh;
    cow_src[0] = old;
    cow_dst[0] = fresh;
    *n_cow = 1;
  }
  for (int64_t i = 0; i < grow; ++i) s.blocks.push_back(bm->take());
  s.len += num_tokens;
  return PKV_OK;
}

int pkv_bm_release(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return PKV_EINVAL;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PKV_EINVAL;
  for (int32_t b : it->second.blocks) bm->drop(b);
  bm->seqs.erase(it);
  return PKV_OK;
}

int64_t pkv_bm_seq_len(const pkv_block_manager* bm, int64_t seq) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> g(bm->mu);
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int pkv_bm_table(const pkv_block_manager* bm, const int64_t* seqs, int n,
                 int max_blocks_per_seq, int32_t* table, int32_t* seqlens) {
  if (!bm || n < 0 || max_blocks_per_seq < 0 || (n > 0 && (!seqs || !table || !seqlens)))
    return PKV_EINVAL;
  std::lock_guard<std::mutex> g(bm->mu);
  for (int i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || (int64_t)it->second.blocks.size() > max_blocks_per_seq ||
        it->second.len > INT32_MAX)
      return PKV_EINVAL;
  }
  for (int i = 0; i < n; ++i) {
    const auto& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = table + (int64_t)i * max_blocks_per_seq;
    for (int j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int)s.blocks.size() ? s.blocks[j] : -1;
    seqlens[i] = (int32_t)s.len;
  }
  return PKV_OK;
}

}  // extern "C"
