// Drives the host side of libpkv -- the argument checks, partition choice,
// workspace sizing and launch planning of pkv_api.hip, and the block manager
// of block_manager.cpp -- under AddressSanitizer and UndefinedBehaviorSanitizer,
// with the kernel launchers replaced by stubs (no GPU is touched).  The stubs
// check that every region the launch plan carves out of the workspace lies
// inside the bytes the caller passed.  The block manager runs a scripted
// scenario (fork, copy-on-write, out of blocks, release) and a random
// sequence of operations with its invariants checked after each one, from
// several threads on one manager.  Exits non-zero on the first failed
// expectation; the sanitizers abort on any memory or arithmetic error.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include <random>
#include <set>
#include <thread>
#include <vector>

#include "pkv.h"
#include "pkv_kernels.h"

static int failures = 0;
#define EXPECT(cond)                                                                   \
  do {                                                                                 \
    if (!(cond)) {                                                                     \
      if (failures < 20)                                                               \
        fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

// ------------------------------------------------------------ launch stubs
// the workspace of the current call: a stand-in address (never dereferenced
// by host code) and its size
static const uintptr_t kWs = 0x10000000;
static size_t g_ws_bytes = 0;
static int g_launches = 0;

static bool inside(const void* p, size_t bytes) {
  const uintptr_t c = (uintptr_t)p;
  return c >= kWs && bytes <= g_ws_bytes && c - kWs <= g_ws_bytes - bytes;
}

namespace pkv {
hipError_t launch_decode(int, int head_dim, int block_size, const DecodeArgs& a, int,
                         hipStream_t) {
  ++g_launches;
  EXPECT(a.group * a.num_kv_heads == a.num_heads);
  EXPECT(a.n_parts >= 1 && a.part_tokens >= 1 && a.part_tokens % block_size == 0);
  // the partitions cover the whole table row
  EXPECT((long long)a.n_parts * a.part_tokens >= (long long)a.max_blocks_per_seq * block_size);
  EXPECT(inside(a.ctrl, 3 * sizeof(int)));
  EXPECT(inside(a.items, (size_t)a.batch * a.n_parts * sizeof(int4)));
  if (a.n_parts > 1) {
    const size_t slots = (size_t)a.batch * a.num_heads * a.n_parts;
    EXPECT(inside(a.ws_acc, slots * head_dim * sizeof(float)));
    EXPECT(inside(a.ws_ml, slots * sizeof(float2)));
  }
  EXPECT(a.max_run >= 1 && a.max_run <= 8);
  return hipSuccess;
}
hipError_t launch_varlen(int, int, const VarlenArgs& a, hipStream_t) {
  ++g_launches;
  EXPECT(a.heads_per_wg >= 1 && a.group % a.heads_per_wg == 0 && a.q_tiles >= 0);
  return hipSuccess;
}
hipError_t launch_varlen_paged(int, int, const VarlenArgs& a, hipStream_t) {
  ++g_launches;
  EXPECT(a.block_size % 16 == 0 && a.q_tiles >= 0);
  return hipSuccess;
}
hipError_t launch_cache_write(const CacheWriteArgs& a, hipStream_t) {
  ++g_launches;
  EXPECT(a.row_bytes % 16 == 0 && a.row_bytes > 0);
  return hipSuccess;
}
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t) {
  ++g_launches;
  EXPECT(a.block_bytes % 16 == 0 && a.n > 0);
  return hipSuccess;
}
// the static scratch of pkv_decode_noalloc: the same stand-in address
hipError_t decode_scratch(void** ptr) {
  *ptr = (void*)kWs;
  return hipSuccess;
}
}  // namespace pkv

// the two runtime queries pkv_decode_noalloc makes: device 0 for everything
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* dev) {
  *dev = 0;
  return hipSuccess;
}

// a stand-in for device pointers: the host code never dereferences them
static void* const kFake = (void*)(uintptr_t)0x100000;

static void decode_plans() {
  const int batches[] = {0, 1, 3, 64, 256, 1500, 70000, INT_MAX};
  const int heads[][2] = {{4, 4}, {32, 8}, {64, 8}, {20, 1}, {7, 3}, {1 << 20, 1}, {0, 1}};
  const int dims[] = {64, 128, 96, -1};
  const int bss[] = {16, 32, 8, 0};
  const int maxbs[] = {0, 1, 4, 2048, 513, 1 << 26, -3};
  const int parts[] = {0, 16, 48, 512, 4096, 8192, 17, -16};
  for (int B : batches)
    for (auto& h : heads)
      for (int D : dims)
        for (int bs : bss)
          for (int mb : maxbs)
            for (int pt : parts) {
              const int rc = pkv_check_decode_args(PKV_BF16, 1, B, h[0], h[1], D, 1000, bs, mb, pt);
              const int ptok = pkv_decode_partition_tokens(B, h[0], h[1], D, bs, mb, pt);
              const size_t need = pkv_decode_workspace_bytes(B, h[0], h[1], D, bs, mb, pt);
              EXPECT((rc == PKV_OK) == (ptok > 0));
              EXPECT((rc == PKV_OK) == (need > 0));
              if (rc != PKV_OK) continue;
              EXPECT(pt == 0 || ptok == pt || ptok >= (long long)mb * bs);
              g_ws_bytes = need;
              const int before = g_launches;
              const int r = pkv_decode(PKV_BF16, kFake, kFake, kFake, (const int32_t*)kFake,
                                       (const int32_t*)kFake, kFake, kFake, kFake, B, h[0], h[1],
                                       D, 1000, bs, mb, 0.1f, pt, (void*)kWs, need, nullptr,
                                       nullptr);
              EXPECT(r == PKV_OK || r == PKV_EUNSUPPORTED);
              EXPECT(B == 0 || r != PKV_OK || g_launches == before + 1);
              // the no-alloc form: the library's scratch, or a refusal when the
              // workspace would not fit in it
              g_ws_bytes = pkv::kDecodeScratchBytes;
              const int before_na = g_launches;
              const int rn = pkv_decode_noalloc(PKV_BF16, kFake, kFake, kFake,
                                                (const int32_t*)kFake, (const int32_t*)kFake,
                                                kFake, kFake, kFake, B, h[0], h[1], D, 1000, bs,
                                                mb, 0.1f, pt, nullptr, nullptr);
              if (need > pkv::kDecodeScratchBytes)
                EXPECT(B == 0 ? rn == PKV_OK : (rn == PKV_EWORKSPACE && g_launches == before_na));
              else
                EXPECT(rn == r && (B == 0 || r != PKV_OK || g_launches == before_na + 1));
              g_ws_bytes = need;
              // one byte short of the workspace is refused before any launch
              if (need > 1) {
                const int r2 = pkv_decode_partials(PKV_BF16, kFake, kFake, kFake,
                                                   (const int32_t*)kFake, (const int32_t*)kFake,
                                                   nullptr, nullptr, kFake, B, h[0], h[1], D,
                                                   1000, bs, mb, 0.1f, pt, (void*)kWs, need - 1,
                                                   nullptr, nullptr);
                EXPECT(B == 0 || r2 == PKV_EWORKSPACE);
              }
            }
  // argument errors that return before the plan
  EXPECT(pkv_decode(PKV_BF16, nullptr, kFake, kFake, (const int32_t*)kFake, (const int32_t*)kFake,
                    nullptr, nullptr, kFake, 2, 8, 2, 128, 10, 16, 4, 0.1f, 0, nullptr, 0,
                    nullptr, nullptr) == PKV_EINVAL);
  EXPECT(pkv_decode(PKV_BF16, kFake, kFake, kFake, (const int32_t*)kFake, (const int32_t*)kFake,
                    kFake, nullptr, kFake, 2, 8, 2, 128, 10, 16, 4, 0.1f, 0, nullptr, 0, nullptr,
                    nullptr) == PKV_EINVAL);
  EXPECT(pkv_decode(5, kFake, kFake, kFake, (const int32_t*)kFake, (const int32_t*)kFake, nullptr,
                    nullptr, kFake, 2, 8, 2, 128, 10, 16, 4, 0.1f, 0, nullptr, 0, nullptr,
                    nullptr) == PKV_EUNSUPPORTED);
  EXPECT(pkv_decode(PKV_BF16, kFake, kFake, kFake, (const int32_t*)kFake, (const int32_t*)kFake,
                    nullptr, nullptr, kFake, 2, 8, 2, 128, 10, 16, 4, __builtin_inff(), 0,
                    nullptr, 0, nullptr, nullptr) == PKV_EINVAL);
}

static void varlen_plans() {
  const int vals[] = {0, 1, 7, 2048, 65536 * 32, INT_MAX, -1};
  const int heads[][2] = {{32, 8}, {8, 8}, {6, 2}, {3, 2}, {0, 1}, {65536, 1}};
  for (int B : vals)
    for (int T : vals)
      for (auto& h : heads)
        for (int D : {64, 128, 80})
          for (int ml : vals) {
            const int rc = pkv_check_varlen_args(PKV_BF16, B, T, T, h[0], h[1], D, ml, ml);
            const int r = pkv_varlen(PKV_BF16, kFake, kFake, kFake, (const int32_t*)kFake,
                                     (const int32_t*)kFake, ml, ml, kFake, B, T, T, h[0], h[1], D,
                                     0.1f, nullptr, nullptr);
            EXPECT(rc != PKV_OK ? r == rc : (r == PKV_OK || r == PKV_EUNSUPPORTED));
            for (int bs : {16, 32, 8}) {
              const int rcp = pkv_check_varlen_paged_args(PKV_BF16, B, T, h[0], h[1], D, 100, bs,
                                                          ml, ml, ml);
              const int rp = pkv_varlen_paged(PKV_BF16, kFake, kFake, kFake,
                                              (const int32_t*)kFake, (const int32_t*)kFake,
                                              (const int32_t*)kFake, ml, ml, kFake, B, T, h[0],
                                              h[1], D, 100, bs, ml, 0.1f, nullptr, nullptr);
              EXPECT(rcp != PKV_OK ? rp == rcp : (rp == PKV_OK || rp == PKV_EUNSUPPORTED));
              const int rcw = pkv_check_cache_write_args(PKV_FP32, B, T, h[1], D, 100, bs, ml);
              const int rw = pkv_cache_write(PKV_FP32, kFake, kFake, (const int32_t*)kFake,
                                             (const int32_t*)kFake, kFake, kFake,
                                             (const int32_t*)kFake, B, T, h[1], D, 100, bs, ml,
                                             nullptr, nullptr);
              EXPECT(rcw != PKV_OK ? rw == rcw : rw == PKV_OK);
            }
          }
  for (int n : {0, 1, 65535, 65536, -1})
    for (int D : {64, 128, 1})
      (void)pkv_copy_blocks(PKV_BF16, kFake, kFake, (const int32_t*)kFake, (const int32_t*)kFake,
                            n, 100, 16, 8, D, nullptr, nullptr);
  for (int s = -2; s < 8; ++s) EXPECT(pkv_status_string(s) != nullptr);
}

// ----------------------------------------------------------- block manager
static void bm_scenario() {
  pkv_block_manager* bm = nullptr;
  EXPECT(pkv_bm_create(-1, 4, &bm) != PKV_OK && bm == nullptr);
  EXPECT(pkv_bm_create(8, 4, &bm) == PKV_OK && bm);
  EXPECT(pkv_bm_allocate(bm, 1, 6) == PKV_OK);          // blocks 7, 6
  EXPECT(pkv_bm_num_free(bm) == 6);
  EXPECT(pkv_bm_allocate(bm, 1, 1) == PKV_EINVAL);      // exists
  EXPECT(pkv_bm_fork(bm, 1, 2) == PKV_OK);
  EXPECT(pkv_bm_ref_count(bm, 7) == 2 && pkv_bm_ref_count(bm, 6) == 2);
  int32_t src = -1, dst = -1;
  int n = -1;
  EXPECT(pkv_bm_append(bm, 2, 1, &src, &dst, &n) == PKV_OK && n == 1 && src == 6 && dst == 5);
  EXPECT(pkv_bm_append(bm, 2, 100, &src, &dst, &n) == PKV_ENOMEM);
  EXPECT(pkv_bm_seq_len(bm, 2) == 7);
  int64_t seqs[2] = {1, 2};
  int32_t table[2 * 3], lens[2];
  EXPECT(pkv_bm_table(bm, seqs, 2, 3, table, lens) == PKV_OK);
  EXPECT(table[0] == 7 && table[1] == 6 && table[2] == -1 && table[4] == 5 && lens[1] == 7);
  EXPECT(pkv_bm_table(bm, seqs, 2, 1, table, lens) == PKV_EINVAL);
  EXPECT(pkv_bm_release(bm, 1) == PKV_OK && pkv_bm_release(bm, 1) == PKV_EINVAL);
  EXPECT(pkv_bm_release(bm, 2) == PKV_OK && pkv_bm_num_free(bm) == 8);
  EXPECT(pkv_bm_ref_count(bm, 8) == -1 && pkv_bm_ref_count(bm, -1) == -1);
  pkv_bm_destroy(bm);
  EXPECT(pkv_bm_num_free(nullptr) == -1);
}

// random operations on one manager; the invariant: every block is either on
// the free list or referenced, and its count equals the number of sequences
// holding it
static void bm_random(pkv_block_manager* bm, int num_blocks, int seed, int64_t id_base,
                      bool check_global) {
  std::mt19937 rng(seed);
  std::set<int64_t> live;
  for (int step = 0; step < 4000; ++step) {
    const int op = (int)(rng() % 5);
    const int64_t id = id_base + (int64_t)(rng() % 24);
    int32_t src, dst;
    int n;
    switch (op) {
      case 0:
        if (pkv_bm_allocate(bm, id, (int)(rng() % 40)) == PKV_OK) live.insert(id);
        break;
      case 1:
        if (!live.empty()) {
          const int64_t p = *std::next(live.begin(), rng() % live.size());
          if (pkv_bm_fork(bm, p, id) == PKV_OK) live.insert(id);
        }
        break;
      case 2:
        if (live.count(id)) (void)pkv_bm_append(bm, id, (int)(rng() % 9), &src, &dst, &n);
        break;
      case 3:
        if (live.count(id)) {
          EXPECT(pkv_bm_release(bm, id) == PKV_OK);
          live.erase(id);
        }
        break;
      default:
        if (!live.empty()) {
          std::vector<int64_t> ids(live.begin(), live.end());
          std::vector<int32_t> t(ids.size() * num_blocks), l(ids.size());
          EXPECT(pkv_bm_table(bm, ids.data(), (int)ids.size(), num_blocks, t.data(),
                              l.data()) == PKV_OK);
          if (check_global) {
            std::vector<int> held(num_blocks, 0);
            for (int32_t b : t)
              if (b >= 0) ++held[b];
            int in_use = 0;
            for (int b = 0; b < num_blocks; ++b) {
              EXPECT(pkv_bm_ref_count(bm, b) == held[b]);
              in_use += held[b] > 0;
            }
            EXPECT(in_use + pkv_bm_num_free(bm) == num_blocks);
          }
        }
    }
  }
  for (int64_t id : live) EXPECT(pkv_bm_release(bm, id) == PKV_OK);
}

static void bm_checks() {
  bm_scenario();
  pkv_block_manager* bm = nullptr;
  EXPECT(pkv_bm_create(96, 4, &bm) == PKV_OK);
  bm_random(bm, 96, 1, 0, true);
  EXPECT(pkv_bm_num_free(bm) == 96);
  // several threads on one manager, disjoint sequence ids
  std::vector<std::thread> th;
  for (int t = 0; t < 4; ++t) th.emplace_back(bm_random, bm, 96, 10 + t, 1000 * (t + 1), false);
  for (auto& x : th) x.join();
  EXPECT(pkv_bm_num_free(bm) == 96);
  pkv_bm_destroy(bm);
}

int main() {
  decode_plans();
  varlen_plans();
  bm_checks();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host driver ok (%d stub launches)\n", g_launches);
  return 0;
}
