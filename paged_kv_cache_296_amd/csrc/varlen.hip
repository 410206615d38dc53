// Variable-length (packed) attention for gfx950, no mask.
//
// What is computed (HF Transformers "paged attention" page, section "Jalur
// Varlen"): sequences are packed along one token axis; the cumulative
// lengths cu_seq_lens_q / cu_seq_lens_k say which query rows and which
// key/value rows belong to request b.  Every query row attends every key row
// of its own request; a request with no key row outputs zeros.
//
// How:
//  * A workgroup is 4 waves; each wave owns 32 query rows of one q head.  The
//    waves of a workgroup share one kv head: with grouped heads they take up
//    to 4 q heads of the group (same 32 rows), otherwise 4 consecutive row
//    blocks of one head, so every K/V tile fetched is used by all 4 waves.
//  * Up to 256 requests run in a persistent grid (two workgroups per CU) that
//    walks a list of the work items every workgroup builds in LDS, requests
//    ranked longest first; larger batches get one workgroup per item.
//  * K and V stream through LDS in 64-key tiles, double buffered, moved from
//    HBM straight into LDS by buffer loads with the LDS-destination bit (no
//    register staging).  Both tiles are stored row-major, one 2*D-byte row
//    per key, with the 16-byte chunks of a row permuted by an XOR of the row
//    index so that the MFMA operand reads below hit distinct LDS banks.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows are the A operand
//    (16-byte LDS reads), the query rows sit on the lane axis (B operand held
//    in registers), so a row's max and sum are in-lane reductions plus one
//    exchange between the two 32-lane halves.
//  * O^T = V^T P^T with the same MFMA: the A operand V^T is read from the
//    row-major V tile by ds_read_b64_tr_b16 (a transposing LDS read), and the
//    key order of each 8-key half matches the order of the S^T accumulator,
//    so P^T is the S^T accumulator rounded to bf16, with no data movement.
//    O^T keeps one query row per lane, so the softmax rescale is lane-local.
//  * Online softmax in the exp2 domain with a lazy reference: a row's
//    exponentials are taken against its running reference before the tile's
//    max is known, and the reference only moves (the accumulators rescaled,
//    the tile's exponentials taken again) when the lane's sum of them shows
//    that the tile's max has run more than 2^8 past it; so exponentials stay
//    below 2^13 and the row max is taken only on the first and last tile of
//    an item and on the rare tile that moves the reference.  The final
//    division by the row sum happens once in the epilogue; bf16 output
//    rounds to nearest even.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "pkv_kernels.h"

namespace pkv {
namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

constexpr int kWaves = 4;        // waves per workgroup
constexpr int kWaveRows = 32;    // query rows per wave
constexpr int kKeys = 64;        // keys per LDS tile
constexpr float kLazy = 8.f;     // log2 of the largest exponential kept before a rescale
constexpr float kLazySum = 8192.f;  // 32 exponentials of at most 2^8 each
constexpr unsigned kErrBlock = 1u, kErrSpan = 2u, kErrCu = 4u, kErrMaxLen = 8u;

template <int D>
struct Geo {
  static constexpr int ROWB = 2 * D;                     // bytes of one key row
  static constexpr int CH = D / 8;                       // 16-byte chunks per row
  static constexpr int TILEB = kKeys * ROWB;             // one K (or V) tile
  static constexpr int NLOAD = TILEB / (1024 * kWaves);  // 1 KB loads per wave per tile
  static constexpr int KS = D / 16;                      // 16-dim k-steps of S^T
  static constexpr int DT = D / 32;                      // 32-dim row tiles of O^T
};

// Physical 16-byte chunk = logical chunk XOR swz(row).  For D = 128 (16
// chunks per row) the 16 rows read together by a K operand load land on 16
// different chunks, any 8 aligned rows on 8 different chunks modulo 8, and
// the 4 rows x 4 chunks of one transposing V read on 16 different chunks.
// For D = 64 (8 chunks) the K reads of 8 aligned rows and the 4 x 2 chunks of
// a 16-lane V read are conflict free.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128)
    return ((0xCA60 >> (4 * (row & 3))) & 15) ^ ((row >> 2) & 1) ^ (row & 8);
  else
    return ((row & 3) << 1) | ((row >> 2) & 1);
}

// x of lane l and of lane l ^ 32 (in either order) by one v_permlane32_swap;
// max and + of the pair are then the same in both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// two floats to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(u32, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Buffer resource of `bytes` bytes at `base` (raw, stride 0; reads past the
// end return zeros).  base must be wave-uniform.
__device__ __forceinline__ u32x4 vsharp(const char* base, int bytes) {
  const unsigned long long p = (unsigned long long)base;
  return u32x4{(u32)p, (u32)(p >> 32) & 0xffffu, (u32)bytes, 0x00020000u};
}

// 16 bytes per lane from buffer offset `voff` into LDS at lds_addr + 16*lane.
// Written as inline asm so that the compiler does not see an LDS write in
// flight: it would otherwise wait for every such load before each
// transposing LDS read.  The loop waits for these loads itself (vmcnt(0) and
// a barrier before a stage is read).  One wait state is needed between the
// M0 write and the load.  The compiler treats m0 as reserved and warns that
// it may not honour the clobber; nothing else in these kernels uses m0 (the
// generated code has no other m0 access), so the value left there is dead.
__device__ __forceinline__ void load_to_lds(u32x4 rs, int voff, u32 lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(lds_addr)
               : "memory", "m0");
}

// This wave's byte offset inside an LDS tile (its share of the tile's 1 KB
// loads).  Recomputed at each use: the value is hidden from the optimiser, so
// the tile addresses built on it are not all hoisted out of the tile loop,
// where each would hold a scalar register of its own (and push others into
// spill slots).
template <int D>
__device__ __forceinline__ u32 wave_lds_offset(int wave) {
  u32 w = (u32)wave;
  asm volatile("" : "+s"(w));
  return w * (u32)(Geo<D>::NLOAD * 1024);
}

// Moves rows t0 .. t0+valid-1 (valid <= 64) of K or V into one LDS tile.
// Lane offsets `off` address the full tile; rows past `valid` are clamped to
// the last valid row (their scores are masked, so any finite copy will do).
template <int D, bool PARTIAL>
__device__ __forceinline__ void issue_tile(const char* g, long long t0, int valid, int tok,
                                           lds_char* tile, int wave, int lane, const int* off) {
  using G = Geo<D>;
  const u32x4 rs = vsharp(g + t0 * tok, valid * tok);
  const u32 t = (u32)(uintptr_t)tile + wave_lds_offset<D>(wave);
#pragma unroll
  for (int i = 0; i < G::NLOAD; ++i) {
    int o = off[i];
    if (PARTIAL) o -= max(((wave * G::NLOAD + i) * 64 + lane) / G::CH - (valid - 1), 0) * tok;
    load_to_lds(rs, o, t + i * 1024);
  }
}

// Paged keys: tile rows t0 .. t0+63 of the request are tokens of the
// table-listed blocks.  A wave's share of a tile (16 consecutive rows, 16 or
// 32 per block, tiles starting on a 64-token boundary) lies in ONE block, so
// the block id is one LDS read per wave and tile, and the buffer descriptor is
// bounded to that block.  Rows past len_k are clamped to the last key (same
// block: the clamp never leaves the wave's 16-row group unless every row of
// the wave is clamped).  coff: the lane's swizzled chunk offset per load.
template <int D, bool PARTIAL>
__device__ __forceinline__ void issue_tile_paged(const char* cache, const int* slice, int t0,
                                                 int len_k, int bs, int tok, lds_char* tile,
                                                 int wave, int lane, const int* coff) {
  using G = Geo<D>;
  constexpr int RPI = 1024 / G::ROWB;     // rows per 1 KB load
  constexpr int RPW = G::NLOAD * RPI;     // rows per wave per tile
  const int tw = t0 + RPW * wave;
  const int tf = PARTIAL ? min(tw, len_k - 1) : tw;
  const int j = tf / bs;
  const int pb = __builtin_amdgcn_readfirstlane(slice[j]);
  const u32x4 rs = vsharp(cache + (long long)pb * bs * tok, bs * tok);
  const u32 t = (u32)(uintptr_t)tile + wave_lds_offset<D>(wave);
#pragma unroll
  for (int i = 0; i < G::NLOAD; ++i) {
    int tl = tw + i * RPI + lane / G::CH;
    if (PARTIAL) tl = min(tl, len_k - 1);
    load_to_lds(rs, (tl - j * bs) * tok + coff[i], t + i * 1024);
  }
}

// LDS byte address -> typed LDS pointer.  The operand offsets hold absolute
// LDS addresses (the dynamic LDS base added once, up front), and the tile
// offsets are compile-time constants, so every operand read is one register
// plus an immediate offset.
template <class T>
__device__ __forceinline__ T* lds_at(u32 addr) {
  return (T*)(size_t)addr;
}

// Reads the K operand of step i of S^T = K Q^T: k-step i / 2, key block i % 2
// (kt: the tile's byte offset in LDS; koff: the lane's absolute addresses).
template <int D>
__device__ __forceinline__ u32x4 k_operand(u32 kt, const u32* koff, int i) {
  return *lds_at<lds_u32x4>(kt + koff[i >> 1] + 32 * (i & 1) * Geo<D>::ROWB);
}

// Masks keys past `valid` (MASK), takes the row max of the tile's scores and
// moves the lazy softmax reference when the max has run more than 2^8 past
// it (rescaling l and the O^T accumulators).  Returns -reference.
template <int D, bool MASK>
__device__ __forceinline__ float softmax_head(f32x16 (&s)[2], f32x16* acc, float& m_ref,
                                              float& l_run, float c, int valid, int hh) {
  using G = Geo<D>;
  // key of accumulator element r of block mt: 32 mt + 8 (r / 4) + 4 hh + r % 4;
  // keys past the end score -inf (c > 0, so they give exp2(-inf) = 0)
  if (MASK) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3) >= valid) s[mt][r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
  mx = pair_max(mx);
  const float ms = mx * c;
  if (__builtin_amdgcn_ballot_w64(ms > m_ref + kLazy) != 0) {
    const float mn = fmaxf(m_ref, ms);
    const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m_ref - mn);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < G::DT; ++d) acc[d] *= alpha;
    m_ref = mn;
  }
  return -m_ref;
}

// Exponentials of elements 2e, 2e+1 of the flattened scores, packed to bf16.
// The row sum takes the packed pair (one v_dot2 against (1, 1) instead of two
// adds), so the normaliser sums exactly the bf16 probabilities that P.V
// multiplies.
__device__ __forceinline__ void exp_pair(const f32x16 (&s)[2], int e, float c, float neg_m,
                                         float& psum, u32 (&pw)[2][8]) {
  const int mt = e >> 3, r = 2 * (e & 7);
  const float p0 = fast_exp2(fmaf(s[mt][r], c, neg_m));
  const float p1 = fast_exp2(fmaf(s[mt][r + 1], c, neg_m));
  const u32 w = pack_bf16x2(p0, p1);
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, psum, false);
  pw[mt][r >> 1] = w;
}

// exp_pair in two halves, for a software pipeline: the exponentials of a
// pair, then (one MFMA later) their bf16 packing and row sum, so that no
// instruction waits on a transcendental result issued just before it.
__device__ __forceinline__ void exp_pair_start(const f32x16 (&s)[2], int e, float c, float neg_m,
                                               float& p0, float& p1) {
  const int mt = e >> 3, r = 2 * (e & 7);
  p0 = fast_exp2(fmaf(s[mt][r], c, neg_m));
  p1 = fast_exp2(fmaf(s[mt][r + 1], c, neg_m));
}
__device__ __forceinline__ void exp_pair_finish(float p0, float p1, int e, float& psum,
                                                u32 (&pw)[2][8]) {
  const int mt = e >> 3, r = 2 * (e & 7);
  const u32 w = pack_bf16x2(p0, p1);
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, psum, false);
  pw[mt][r >> 1] = w;
}

// S^T of the next tile (16 MFMAs, K operand read four steps ahead) with the
// exponentials of the current tile spread between them, so that the matrix
// core and the vector ALU of one wave work at the same time; each slot
// packs and sums the pairs whose exponentials the slot before started.  The
// scheduling fences keep this interleaving and keep the K reads from all
// being hoisted.
template <int D>
__device__ __forceinline__ void qk_and_exp(u32 kt, const u32x4* qr, const u32* koff,
                                           f32x16 (&sn)[2], const f32x16 (&sc)[2], float c,
                                           float neg_m, float& psum, u32 (&pw)[2][8]) {
  using G = Geo<D>;
  constexpr int NQK = 2 * G::KS;
  constexpr int EPS = 16 / NQK;  // exponential pairs per MFMA
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[mt][r] = 0.f;
  u32x4 kf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kf[i] = k_operand<D>(kt, koff, i);
  float p0[EPS], p1[EPS];
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[i & 3]),
                                                        __builtin_bit_cast(bf16x8, qr[i >> 1]),
                                                        sn[i & 1], 0, 0, 0);
    if (i + 4 < NQK) kf[i & 3] = k_operand<D>(kt, koff, i + 4);
    if (i > 0) {
#pragma unroll
      for (int e = 0; e < EPS; ++e) exp_pair_finish(p0[e], p1[e], EPS * (i - 1) + e, psum, pw);
    }
#pragma unroll
    for (int e = 0; e < EPS; ++e) exp_pair_start(sc, EPS * i + e, c, neg_m, p0[e], p1[e]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int e = 0; e < EPS; ++e) exp_pair_finish(p0[e], p1[e], EPS * (NQK - 1) + e, psum, pw);
}

// S^T of one tile alone (the first tile).
template <int D>
__device__ __forceinline__ void qk_only(u32 kt, const u32x4* qr, const u32* koff,
                                        f32x16 (&sn)[2]) {
  using G = Geo<D>;
  constexpr int NQK = 2 * G::KS;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[mt][r] = 0.f;
  u32x4 kf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kf[i] = k_operand<D>(kt, koff, i);
#pragma unroll
  for (int i = 0; i < NQK; ++i) {
    sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[i & 3]),
                                                        __builtin_bit_cast(bf16x8, qr[i >> 1]),
                                                        sn[i & 1], 0, 0, 0);
    if (i + 4 < NQK) kf[i & 3] = k_operand<D>(kt, koff, i + 4);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// V^T operand i of the tile's P.V product: keys 16 kc .. 16 kc + 15 (kc =
// i / DT) of dims 32 d .. 32 d + 31 (d = i % DT).  This lane's P^T operand
// holds keys 16 kc + 4 hh + {0..3} and 16 kc + 8 + 4 hh + {0..3}, and the two
// transposing reads fetch V^T for exactly those keys.
template <int D>
__device__ __forceinline__ i16x8 v_operand(u32 vt, const u32* voff, int i) {
  using G = Geo<D>;
  const int kc = i / G::DT, d = i % G::DT;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      lds_at<lds_i16x4>(vt + voff[2 * d] + 16 * kc * G::ROWB));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      lds_at<lds_i16x4>(vt + voff[2 * d + 1] + 16 * kc * G::ROWB));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// O^T += V^T P^T over the tile's 64 keys, 16 keys per step.  vf: operands 0
// and 1, read by the caller (in the tile loop before the overflow check, so
// that their latency runs under the last QK^T MFMAs); the reads run two
// MFMAs ahead.
template <int D>
__device__ __forceinline__ void pv(u32 vt, const u32* voff, const u32 (&pw)[2][8],
                                   f32x16* acc, i16x8 (&vf)[2]) {
  using G = Geo<D>;
  constexpr int NPV = 4 * G::DT;
#pragma unroll
  for (int i = 0; i < NPV; ++i) {
    const int kc = i / G::DT, d = i % G::DT;
    const int mt = kc >> 1, ap = kc & 1;
    const u32x4 pf = {pw[mt][4 * ap], pw[mt][4 * ap + 1], pw[mt][4 * ap + 2], pw[mt][4 * ap + 3]};
    acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf[i & 1]),
                                                     __builtin_bit_cast(bf16x8, pf), acc[d],
                                                     0, 0, 0);
    if (i + 2 < NPV) vf[i & 1] = v_operand<D>(vt, voff, i + 2);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One work item: q-row tile qt of request b, q heads hy * heads_per_wg ..
// (+ heads_per_wg - 1).  PAGED = false: keys packed like the queries (cu_k);
// true: keys are the first seqlens_k[b] tokens of sequence b in the paged
// cache (block_table).  Every exit is uniform over the workgroup.
template <int D, bool PAGED>
// cq = (cu_q[b], cu_q[b + 1]); ck = (cu_k[b], cu_k[b + 1]) (packed) or
// (0, seqlens_k[b]) (paged), read by the caller.
__device__ __forceinline__ void varlen_item(const VarlenArgs& a, int qt, int hy, int b,
                                            int2 cq, int2 ck) {
  using G = Geo<D>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps row math scalar
  const int n = lane & 31, hh = lane >> 5;
  const int hpw = a.heads_per_wg, rb = kWaves / hpw;
  const int hw = wave % hpw, rbi = wave / hpw;
  const int h0 = hy * hpw;
  const int wg_rows = kWaveRows * rb;

  const int q0 = cq.x, q1 = cq.y;
  const int len_q = q1 - q0;
  const bool q_ok = q0 >= 0 && q1 >= q0 && q1 <= a.total_q && (b != 0 || q0 == 0) &&
                    (b != a.batch - 1 || q1 == a.total_q);
  int k0s = 0, len_k;
  unsigned err = 0;
  if constexpr (PAGED) {
    len_k = ck.y;
    if (!q_ok) err = kErrCu;
    else if (len_k < 0 || (long long)len_k > (long long)a.max_blocks_per_seq * a.block_size)
      err = kErrSpan;
    else if (len_q > a.max_len_q || len_k > a.max_len_k) err = kErrMaxLen;
  } else {
    k0s = ck.x;
    const int k1s = ck.y;
    len_k = k1s - k0s;
    const bool cu_ok = q_ok && k0s >= 0 && k1s >= k0s && k1s <= a.total_k &&
                       (b != 0 || k0s == 0) && (b != a.batch - 1 || k1s == a.total_k);
    if (!cu_ok) err = kErrCu;
    else if (len_q > a.max_len_q || len_k > a.max_len_k) err = kErrMaxLen;
  }
  // A request the kernel cannot run: flag it and write NaN to its rows (when
  // the rows themselves can be located).
  auto fail = [&](unsigned bit) {
    if (a.err_flag && tid == 0 && qt == 0 && hy == 0) atomicOr(a.err_flag, (int)bit);
    if (!(q0 >= 0 && q1 >= q0 && q1 <= a.total_q)) return;  // nowhere safe to write
    const int r0 = qt * wg_rows, r1 = min(len_q, r0 + wg_rows);
    for (int i = tid; i < (r1 > r0 ? (r1 - r0) * hpw : 0); i += 256) {
      const int r = r0 + i / hpw, hq = h0 + i % hpw;
      __bf16* o = (__bf16*)a.out + ((long long)(q0 + r) * a.num_heads + hq) * D;
      for (int d = 0; d < D; ++d) o[d] = (__bf16)__builtin_nanf("");
    }
  };
  if (err) {
    fail(err);
    return;
  }
  if (qt * wg_rows >= len_q) return;

  const int h = h0 + hw;
  const int kvh = h0 / a.group;
  const int tok_q = a.num_heads * D * 2;     // bytes between query rows
  const int tok_k = a.num_kv_heads * D * 2;  // bytes between key rows
  const char* kg = (const char*)a.k + (long long)k0s * tok_k + (long long)kvh * D * 2;
  const char* vg = (const char*)a.v + (long long)k0s * tok_k + (long long)kvh * D * 2;
  lds_char* lds = (lds_char*)smem;
  // paged: the request's table entries, validated and staged in LDS after
  // the four tiles
  int* slice = reinterpret_cast<int*>(smem + 4 * G::TILEB);
  if constexpr (PAGED) {
    const int nblk = (len_k + a.block_size - 1) / a.block_size;
    const int32_t* trow = a.block_table + (long long)b * a.max_blocks_per_seq;
    bool bad = false;
    for (int e = tid; e < nblk; e += 256) {
      const int pb = trow[e];
      bad |= pb < 0 || pb >= a.num_blocks;
      slice[e] = pb;
    }
    if (__syncthreads_or(bad)) {
      fail(kErrBlock);
      return;
    }
  }

  // this lane's query row as the B operand: dims 16 s + 8 hh + 0..7; a
  // negative scale is folded into q (a sign flip is exact in bf16)
  const int row = qt * wg_rows + rbi * kWaveRows + n;
  const bool row_ok = row < len_q;
  const bool wave_active = qt * wg_rows + rbi * kWaveRows < len_q;
  // c > 0 always: a zero scale zeroes q instead (every score is then 0)
  const u32 sign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const float c = a.scale_log2 == 0.f ? 1.f : fabsf(a.scale_log2);
  u32x4 qr[G::KS];
  {
    const char* qp = (const char*)a.q + (long long)(q0 + (row_ok ? row : 0)) * tok_q +
                     (long long)h * D * 2 + 16 * hh;
    // rows past the end read row 0, then zero
    const u32 keep = row_ok && a.scale_log2 != 0.f ? ~0u : 0u;
#pragma unroll
    for (int s = 0; s < G::KS; ++s)
      qr[s] = (*reinterpret_cast<const u32x4*>(qp + 32 * s) ^ sign) & keep;
  }

  // lane offsets: tile loads (same for K and V), K operand reads, V^T reads
  // (packed: row offset + swizzled chunk; paged: the swizzled chunk only, the
  // row offset depends on the block)
  int loff[G::NLOAD];
#pragma unroll
  for (int i = 0; i < G::NLOAD; ++i) {
    const int cl = (wave * G::NLOAD + i) * 64 + lane;
    const int r = cl / G::CH, ps = cl % G::CH;
    loff[i] = (PAGED ? 0 : r * tok_k) + 16 * (ps ^ swz<D>(r));
  }
  const u32 lbase = (u32)(uintptr_t)lds;
  u32 koff[G::KS];
#pragma unroll
  for (int ks = 0; ks < G::KS; ++ks) {
    koff[ks] = lbase + n * G::ROWB + 16 * ((2 * ks + hh) ^ swz<D>(n));
    asm volatile("" : "+v"(koff[ks]));  // keep the sum: not re-split into base + offset per read
  }
  u32 voff[2 * G::DT];
  {
    const int q16 = lane & 15, grp = (lane >> 4) & 1;
#pragma unroll
    for (int d = 0; d < G::DT; ++d)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int vr = 8 * r + 4 * hh + (q16 >> 2);
        const int lc = 4 * d + 2 * grp + ((q16 >> 1) & 1);
        voff[2 * d + r] = lbase + vr * G::ROWB + 16 * (lc ^ swz<D>(vr)) + 8 * (q16 & 1);
      }
  }

  f32x16 acc[G::DT];
#pragma unroll
  for (int d = 0; d < G::DT; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m_ref = -INFINITY, l_run = 0.f;

  // LDS: K tiles at [0, 2 TILEB) and V tiles at [2 TILEB, 4 TILEB), double
  // buffered by tile parity.  Iteration j reads K of tile j+1 (the next
  // S^T) and V of tile j, and meanwhile loads K of tile j+2 and V of tile
  // j+1 into the buffers that iteration j-1 finished with.
  const int nk = (len_k + kKeys - 1) / kKeys;
  const int last_valid = len_k - (nk - 1) * kKeys;  // keys in the last tile
  const bool partial = last_valid < kKeys;
  auto kbuf = [&](int j) { return lds + (j & 1) * G::TILEB; };
  auto vbuf = [&](int j) { return lds + (2 + (j & 1)) * G::TILEB; };
  auto kofs = [&](int j) { return (u32)((j & 1) * G::TILEB); };        // byte offsets of the
  auto vofs = [&](int j) { return (u32)((2 + (j & 1)) * G::TILEB); };  // same tiles
  auto issue = [&](const char* g, int j, lds_char* tile) {
    if constexpr (PAGED) {
      if (j + 1 < nk || !partial)
        issue_tile_paged<D, false>(g, slice, j * kKeys, len_k, a.block_size, tok_k, tile, wave,
                                   lane, loff);
      else
        issue_tile_paged<D, true>(g, slice, j * kKeys, len_k, a.block_size, tok_k, tile, wave,
                                  lane, loff);
    } else {
      if (j + 1 < nk || !partial)
        issue_tile<D, false>(g, (long long)j * kKeys, kKeys, tok_k, tile, wave, lane, loff);
      else
        issue_tile<D, true>(g, (long long)j * kKeys, last_valid, tok_k, tile, wave, lane, loff);
    }
  };
  auto wait_all = [&]() {
    // own loads done, then everyone's; this also retires every wave's reads
    // of the buffers the following issues overwrite
    __builtin_amdgcn_s_waitcnt(0x3f70);  // vmcnt(0)
    __syncthreads();
  };
  f32x16 sa[2], sb[2];
  auto step = [&](int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) {  // tile j, with a next tile
    wait_all();
    if (j + 2 < nk) issue(kg, j + 2, kbuf(j));
    issue(vg, j + 1, vbuf(j + 1));
    if (!wave_active) return;
    float psum = 0.f;
    u32 pw[2][8];
    // the interleaved phase runs at raised wave priority, so that the other
    // wave on this SIMD fills in around it rather than competing for issue
    // (without it, or with P.V raised instead: 7 % slower at head_dim 64,
    // 2-3 % on short items at head_dim 128, the 16-request batch even)
    __builtin_amdgcn_s_setprio(1);
    qk_and_exp<D>(kofs(j + 1), qr, koff, sn, sc, c, -m_ref, psum, pw);
    // P.V's first two V^T operands go out here, before the overflow check,
    // rather than at the start of P.V: their LDS latency then runs under the
    // last QK^T MFMAs (+1.4 to +1.9 % on the 16-request batch, uniform
    // batches and head_dim 64, +0.6 to +1 % on the mixed-step prefill; two
    // boxes, two rounds each)
    i16x8 vf[2] = {v_operand<D>(vofs(j), voff, 0), v_operand<D>(vofs(j), voff, 1)};
    __builtin_amdgcn_s_setprio(0);
    // the exponentials were taken against the current reference before the
    // tile's max is known; the lane's sum of its 32 of them bounds each, so
    // only a sum past 32 * 2^8 (or inf / NaN) asks for the max, which then
    // lies more than 2^8 above the reference: the reference moves and the
    // exponentials are taken again
    if (__builtin_amdgcn_ballot_w64(!(psum <= kLazySum)) != 0) {
      const float neg_m = softmax_head<D, false>(sc, acc, m_ref, l_run, c, kKeys, hh);
      psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) exp_pair(sc, e, c, neg_m, psum, pw);
    }
    l_run += psum;
    pv<D>(vofs(j), voff, pw, acc, vf);
  };
  if (nk > 0) {
    issue(kg, 0, kbuf(0));
    issue(vg, 0, vbuf(0));
    if (nk > 1) issue(kg, 1, kbuf(1));
    wait_all();
    if (wave_active) {
      qk_only<D>(kofs(0), qr, koff, sa);
      // a full first tile sets the reference (the last tile, also when it
      // is the first, takes its own max below)
      if (nk > 1) softmax_head<D, false>(sa, acc, m_ref, l_run, c, kKeys, hh);
    }
    int j = 0;
    for (; j + 2 < nk; j += 2) {
      step(j, sa, sb);
      step(j + 1, sb, sa);
    }
    if (j + 1 < nk) {
      step(j, sa, sb);
      ++j;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) sa[mt] = sb[mt];
    }
    // last tile (j = nk - 1): scores in sa, V in vbuf(j)
    wait_all();
    if (wave_active) {
      const float neg_m = partial
          ? softmax_head<D, true>(sa, acc, m_ref, l_run, c, last_valid, hh)
          : softmax_head<D, false>(sa, acc, m_ref, l_run, c, kKeys, hh);
      float psum = 0.f;
      u32 pw[2][8];
#pragma unroll
      for (int e = 0; e < 16; ++e) exp_pair(sa, e, c, neg_m, psum, pw);
      l_run += psum;
      i16x8 vf[2] = {v_operand<D>(vofs(j), voff, 0), v_operand<D>(vofs(j), voff, 1)};
      pv<D>(vofs(j), voff, pw, acc, vf);
    }
  }

  // Output: the wave's 32 rows x D go through LDS -- the two K tile
  // buffers, idle since the last QK^T and the barrier after it -- so that
  // the global stores write whole contiguous head rows (16 lanes x 16 bytes
  // per row, 64 / CH rows per instruction) instead of 8-byte pieces spread
  // over 32 rows 8 KB apart.  Chunk c (16 bytes) of staged row n sits at
  // chunk position c ^ (n % CH).  Timing-only runs without any output store
  // were 4-11 % faster than the scattered stores; the LDS round trip gets
  // 1-5 % of it back (most on short items).
  if (!wave_active) return;
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // lane-dependent staging addresses are rebuilt here on every item rather
  // than hoisted out of the persistent loop, where they would be live
  // through the tile loop
  u32 srow = lbase + wave * (kWaveRows * G::ROWB) + n * G::ROWB;
  int sx = n % G::CH, ln = lane;
  asm volatile("" : "+v"(srow), "+v"(sx), "+v"(ln));
  const u32 stage = lbase + wave * (kWaveRows * G::ROWB);
  // O^T element r of row tile d is dim 32 d + 8 (r / 4) + 4 hh + r % 4: the
  // 8 bytes of dims 32 d + 8 g + 4 hh .. + 3 are half hh of chunk 4 d + g
#pragma unroll
  for (int d = 0; d < G::DT; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = {pack_bf16x2(acc[d][4 * g] * inv, acc[d][4 * g + 1] * inv),
                       pack_bf16x2(acc[d][4 * g + 2] * inv, acc[d][4 * g + 3] * inv)};
      *lds_at<lds_u32x2>(srow + 16 * ((4 * d + g) ^ sx) + 8 * hh) = w;
      __builtin_amdgcn_sched_barrier(0);  // one piece live at a time: no spills
    }
  const int wrow0 = qt * wg_rows + rbi * kWaveRows;  // the wave's first row in the request
  char* ob = (char*)a.out + (long long)(q0 + wrow0) * tok_q + (long long)h * D * 2;
#pragma unroll
  for (int i = 0; i < kWaveRows * G::CH / 64; ++i) {
    const int pc = 64 * i + ln, rr = pc / G::CH, ch = pc % G::CH;
    const u32x4 v = *lds_at<lds_u32x4>(stage + rr * G::ROWB + 16 * (ch ^ (rr % G::CH)));
    if (wrow0 + rr < len_q) *reinterpret_cast<u32x4*>(ob + (long long)rr * tok_q + 16 * ch) = v;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One workgroup per item of the full (q tile, head group, request) grid;
// items past a request's rows exit at once.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void varlen_kernel(VarlenArgs a) {
  const int b = blockIdx.z;
  const int2 cq = make_int2(a.cu_q[b], a.cu_q[b + 1]);
  const int2 ck = PAGED ? make_int2(0, a.seqlens_k[b]) : make_int2(a.cu_k[b], a.cu_k[b + 1]);
  varlen_item<D, PAGED>(a, blockIdx.x, blockIdx.y, b, cq, ck);
}

// Persistent form for batches of up to kPersistMaxPacked (packed keys) or
// kPersistMaxPaged (paged keys) requests: as many workgroups as fit on the
// device, each building the same item list in LDS -- only the q tiles a
// request has; up to kRankMaxBatch requests ranked by key-tile count,
// longest first, larger batches in request order -- and taking items
// k * G + w (k even) or k * G + G - 1 - w (k odd) of it, w being the
// workgroup's slot in XCD-major order, so that every workgroup gets a
// similar mix of long and short items and a ranked list ends on the
// shortest ones.  Saves the launch and request lookups of the empty and the
// per-tile workgroups and drains the tail in order.
constexpr int kRankMaxBatch = 256;
constexpr int kPersistMaxPacked = 960;
constexpr int kPersistMaxPaged = 480;
template <int D>
constexpr int persist_list_offset(bool paged) {
  return 4 * Geo<D>::TILEB + (paged ? kVarlenMaxTableEntries * (int)sizeof(int) : 0);
}
// pre[B + 1], nqt[B], copies of cu_q[B + 1] and of cu_k (or seqlens_k)
// [B + 1], and ord[B] for a ranked batch; at most 80 KB per workgroup in all
// (two per CU) at the batch limits
constexpr int persist_list_bytes(int B) {
  return (4 * B + 3 + (B <= kRankMaxBatch ? B : 0)) * (int)sizeof(int);
}

template <int D, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void varlen_persistent_kernel(VarlenArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int B = a.batch;
  const bool ranked = B <= kRankMaxBatch;
  int* pre = reinterpret_cast<int*>(smem + persist_list_offset<D>(PAGED));  // [B + 1] items before rank r
  int* nqt = pre + B + 1;                   // q tiles of request b
  int* lcq = nqt + B;                       // [B + 1] copy of cu_q
  int* lck = lcq + B + 1;                   // [B + 1] copy of cu_k, or seqlens_k
  int* ord = lck + B + 1;                   // rank -> request (ranked batches)
  // scratch while the list is built: the tile buffers, idle until the
  // first item (key tiles of up to kRankMaxBatch requests, then 256 partial
  // sums of the scan)
  int* key = reinterpret_cast<int*>(smem);
  int* part = key + kRankMaxBatch;
  const int hpw = a.heads_per_wg, hg = a.num_heads / hpw;
  const int wg_rows = kWaveRows * (kWaves / hpw);
  for (int i = tid; i <= B; i += 256) {
    lcq[i] = a.cu_q[i];
    lck[i] = PAGED ? (i < B ? a.seqlens_k[i] : 0) : a.cu_k[i];
  }
  for (int i = tid; i < B; i += 256) {
    // the q tiles the full grid would give this request (at least one, so
    // that its lengths are checked); key tiles for the ranking only
    long long lq = (long long)a.cu_q[i + 1] - a.cu_q[i];
    lq = lq < 0 ? 0 : (lq > (long long)a.q_tiles * wg_rows ? (long long)a.q_tiles * wg_rows : lq);
    const int t = (int)((lq + wg_rows - 1) / wg_rows);
    nqt[i] = t > 0 ? t : 1;
    if (ranked) {
      long long lk = PAGED ? (long long)a.seqlens_k[i] : (long long)a.cu_k[i + 1] - a.cu_k[i];
      lk = lk < 0 ? 0 : (lk > a.max_len_k ? a.max_len_k : lk);
      key[i] = (int)((lk + kKeys - 1) / kKeys);
    }
  }
  __syncthreads();
  if (ranked && tid < B) {
    const int kb = key[tid];
    int r = 0;
    for (int j = 0; j < B; ++j) {
      const int kj = key[j];
      r += (kj > kb) || (kj == kb && j < tid);
    }
    ord[r] = tid;
  }
  __syncthreads();
  // prefix sums of the items in rank order: thread t takes ranks 4t .. 4t+3
  // (B <= 1024), then a scan of the 256 partial sums
  int run[4], acc_items = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 4 * tid + k;
    acc_items += r < B ? nqt[ranked ? ord[r] : r] * hg : 0;
    run[k] = acc_items;
  }
  part[tid] = acc_items;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  const int base_items = tid > 0 ? part[tid - 1] : 0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (4 * tid + k < B) pre[4 * tid + k + 1] = base_items + run[k];
  if (tid == 0) pre[0] = 0;
  __syncthreads();
  const int total = pre[B];
  // slot of this workgroup in XCD-major order: workgroups are dealt to the
  // 8 XCDs round robin (w % 8), so neighbouring slots -- consecutive items
  // of one request and head group, which read the same K/V tiles -- run on
  // the same XCD and share its L2
  const int G = gridDim.x;
  const int w = G % 8 == 0 ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : blockIdx.x;
  for (int k = 0;; ++k) {
    const long long item = (long long)k * G + ((k & 1) ? G - 1 - w : w);
    if (item >= total) break;
    int lo = 0, hi = B;  // pre[lo] <= item < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= item) lo = mid;
      else hi = mid;
    }
    const int b = __builtin_amdgcn_readfirstlane(ranked ? ord[lo] : lo);
    const int rem = (int)item - pre[lo];
    const int t = nqt[b];
    const int hy = __builtin_amdgcn_readfirstlane(rem / t);
    const int qt = __builtin_amdgcn_readfirstlane(rem - (rem / t) * t);
    __syncthreads();  // every wave is done with the previous item's tiles
    const int2 cq = make_int2(__builtin_amdgcn_readfirstlane(lcq[b]),
                              __builtin_amdgcn_readfirstlane(lcq[b + 1]));
    const int2 ck = PAGED ? make_int2(0, __builtin_amdgcn_readfirstlane(lck[b]))
                          : make_int2(__builtin_amdgcn_readfirstlane(lck[b]),
                                      __builtin_amdgcn_readfirstlane(lck[b + 1]));
    varlen_item<D, PAGED>(a, qt, hy, b, cq, ck);
  }
}

// Dynamic LDS above 64 KB must be allowed per kernel.  Each instantiation
// allows, once per device, the most it can ever request (the persistent form
// at its batch limit), so later launches with larger lists are covered too.
// Keyed by the template arguments: all four kernels of a form share one
// function type.
template <int D, bool PAGED, bool PERSIST>
hipError_t allow_lds() {
  static std::atomic<bool> done[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64 && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  size_t lds;
  const void* kernel;
  if constexpr (PERSIST) {
    lds = persist_list_offset<D>(PAGED) +
          persist_list_bytes(PAGED ? kPersistMaxPaged : kPersistMaxPacked);
    kernel = (const void*)varlen_persistent_kernel<D, PAGED>;
  } else {
    lds = 4 * Geo<D>::TILEB + (PAGED ? kVarlenMaxTableEntries * sizeof(int) : 0);
    kernel = (const void*)varlen_kernel<D, PAGED>;
  }
  const hipError_t e =
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess && dev >= 0 && dev < 64) done[dev].store(true, std::memory_order_release);
  return e;
}

// Workgroups of varlen_persistent_kernel<D, PAGED> that fit on the device at
// once (launch geometry only), per device and instantiation; the dynamic LDS
// size varies with the batch, so the cached value is kept with the size it
// was taken for.
template <int D, bool PAGED>
int persistent_workgroups(size_t lds) {
  static std::atomic<unsigned long long> cache[64];  // lds << 32 | workgroups
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const unsigned long long c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0 && (c >> 32) == lds) return (int)(c & 0xffffffffu);
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, varlen_persistent_kernel<D, PAGED>,
                                                   256, lds) != hipSuccess)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const int v = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 256);
  if (dev >= 0 && dev < 64)
    cache[dev].store(((unsigned long long)lds << 32) | (unsigned)v, std::memory_order_relaxed);
  return v;
}

template <int D, bool PAGED>
hipError_t launch_v(const VarlenArgs& a, hipStream_t stream) {
  const long long hg = a.num_heads / a.heads_per_wg;
  const long long items = (long long)a.batch * a.q_tiles * hg;  // the full grid
  if (a.batch <= (PAGED ? kPersistMaxPaged : kPersistMaxPacked) && items < (1LL << 31)) {
    const size_t lds = persist_list_offset<D>(PAGED) + persist_list_bytes(a.batch);
    hipError_t e = allow_lds<D, PAGED, true>();
    if (e != hipSuccess) return e;
    long long grid = persistent_workgroups<D, PAGED>(lds);
    if (grid > items) grid = items;
    hipLaunchKernelGGL((varlen_persistent_kernel<D, PAGED>), dim3((unsigned)grid), dim3(256), lds,
                       stream, a);
    return hipGetLastError();
  }
  const size_t lds = 4 * Geo<D>::TILEB + (PAGED ? kVarlenMaxTableEntries * sizeof(int) : 0);
  hipError_t e = allow_lds<D, PAGED, false>();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((varlen_kernel<D, PAGED>), dim3(a.q_tiles, (unsigned)hg, a.batch), dim3(256),
                     lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_varlen(int dtype, int head_dim, const VarlenArgs& a, hipStream_t stream) {
  if (dtype != 1) return hipErrorInvalidValue;
  if (a.q_tiles == 0 || a.batch == 0) return hipSuccess;
  if (head_dim == 128) return launch_v<128, false>(a, stream);
  if (head_dim == 64) return launch_v<64, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_varlen_paged(int dtype, int head_dim, const VarlenArgs& a,
                               hipStream_t stream) {
  if (dtype != 1) return hipErrorInvalidValue;
  if (a.q_tiles == 0 || a.batch == 0) return hipSuccess;
  if (a.block_size % 16 != 0) return hipErrorInvalidValue;  // a wave's 16 rows in one block
  if (head_dim == 128) return launch_v<128, true>(a, stream);
  if (head_dim == 64) return launch_v<64, true>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
