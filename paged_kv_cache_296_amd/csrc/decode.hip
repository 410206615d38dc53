// Paged decode attention for gfx950.
//
// What is computed (HF Transformers "paged attention" page, section "Jalur
// decode"; inference-notes "39 · PagedAttention", sections 1-3): one query
// token per sequence attends every cached token of its sequence, whose K and
// V rows sit in scattered physical blocks named by the sequence's row of the
// block table; one softmax over all scores; the output is the softmax-weighted
// sum of the values.  The new token's K/V (optional) is written into its slot
// in place and attended too.
//
// How (MI355X-first, not the pages' warp-per-block layout):
//  * One wave64 owns one unit (sequence, partition, kv head, chunk of <= 16 q
//    heads).  Every q head of a GQA group shares the unit's K/V bytes, so each
//    KV byte crosses HBM once per kv head.
//  * A 16-token tile of K is loaded straight from HBM into the A operand of
//    v_mfma_f32_16x16x32_bf16 (lane = token, 16-byte runs of the head row);
//    the q heads are the B operand (zero-padded to 16).  The product is S^T:
//    each lane ends up with 4 tokens' scores for ONE q head.
//  * P.V is computed as O^T = V^T P^T with v_mfma_f32_16x16x16_bf16: the P^T
//    operand is exactly the S^T accumulator layout, so scores never move
//    between lanes, and the O^T accumulator of a lane also belongs to that
//    lane's q head: the online-softmax rescale is lane-local.  V needs a
//    4-token transpose inside each lane (one byte permute per packed pair),
//    nothing through LDS.
//  * fp32 inputs take the same structure with v_mfma_f32_16x16x4f32.
//  * Online softmax in the exp2 domain; max/sum across the 4 token groups of a
//    head use ds_swizzle (swap 16) and a 32-lane exchange.
//  * Split-context: fixed logical partitions write fp32 partials (m, l, acc)
//    and a second kernel merges them with m = max m_k, l = sum l_k 2^(m_k-m)
//    (inference-notes section 3; the value sums take the same factor).
//  * The partition's block-table slice is validated and staged in LDS once;
//    each tile's physical block id comes back as a scalar, so the 64-bit block
//    base is scalar arithmetic and the per-lane offsets stay 32-bit.
//  * Loads of tile t+1 are issued before tile t is computed (double buffer in
//    registers); the last tile of the last partition is the only one that
//    masks tokens or substitutes the new token's K/V.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "pkv_kernels.h"

namespace pkv {
namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 2;        // waves per workgroup (independent units)
constexpr int kMaxSlice = 256;   // table entries one partition may span
constexpr unsigned kErrBlock = 1u, kErrSpan = 2u;

template <bool BF16, int D>
struct Shape {
  static constexpr int ESZ = BF16 ? 2 : 4;
  static constexpr int ROW = D * ESZ;     // bytes of one token's row for one kv head
  static constexpr int NKL = ROW / 64;    // 16-byte K (and Q) pieces per lane
  static constexpr int E = D / 16;        // value elements per lane per token
  static constexpr int VW = E * ESZ / 4;  // ... in 32-bit words
  static constexpr int NACC = E;          // f32x4 accumulators per lane
  static_assert(NKL >= 1 && VW >= 2, "unsupported head_dim");
};

// fp32 operands of v_mfma_f32_16x16x4f32 are kept as float from the load
// on: this compiler mis-lowers a u32 -> float bit-cast feeding that MFMA
// (all four extracted elements collapse onto one register).  bf16 data is
// carried as raw 32-bit words and bit-cast to bf16 vectors, which is sound.
template <bool BF16>
struct Words {
  using vec = u32x4;   // 16 bytes
  using vec2 = u32x2;  // 8 bytes
  using word = u32;
};
template <>
struct Words<false> {
  using vec = f32x4;
  using vec2 = float __attribute__((ext_vector_type(2)));
  using word = float;
};

template <bool BF16, class S>
struct Tile {
  using W = Words<BF16>;
  typename W::vec k[S::NKL];      // K: token (lane & 15), bytes [64t + 16(lane>>4), +16)
  typename W::word v[4][S::VW];   // V: tokens 4(lane>>4)+i, elements [E(lane&15), +E)
};

// Exchange with lane ^ 16 inside each 32-lane half.
__device__ __forceinline__ float swap16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x),
                                                               (0x10 << 10) | 0x1f));
}
__device__ __forceinline__ float swap32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (u32)__builtin_bit_cast(unsigned short, a) |
         ((u32)__builtin_bit_cast(unsigned short, b) << 16);
}

constexpr int kRsrcFlags = 0x00020000;  // gfx9-family buffer descriptor word 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kRsrcFlags);
}

// V words of one token for this lane: E elements at byte voff + soff.
template <bool BF16, class S>
__device__ __forceinline__ void load_v(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                       typename Words<BF16>::word* w) {
  using W = Words<BF16>;
  if constexpr (S::VW == 2) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    const typename W::vec2 y = __builtin_bit_cast(typename W::vec2, x);
    w[0] = y[0];
    w[1] = y[1];
  } else {
#pragma unroll
    for (int j = 0; j < S::VW / 4; ++j) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * j, soff, 0);
      const typename W::vec y = __builtin_bit_cast(typename W::vec, x);
      w[4 * j] = y[0];
      w[4 * j + 1] = y[1];
      w[4 * j + 2] = y[2];
      w[4 * j + 3] = y[3];
    }
  }
}

// Issue the loads of one 16-token tile.  tk/tv point at the tile's first
// token row of this kv head (uniform, 64-bit scalar); `bytes` is what is left
// of the physical block from there, so the buffer descriptors bound every
// access to the block.  koff/voff are the lane's loop-invariant offsets.
template <bool BF16, class S>
__device__ __forceinline__ void load_tile(Tile<BF16, S>& r, const char* tk, const char* tv,
                                          int bytes, int koff, int voff, int tok) {
  using W = Words<BF16>;
  const __amdgpu_buffer_rsrc_t rk = rsrc(tk, bytes), rv = rsrc(tv, bytes);
#pragma unroll
  for (int t = 0; t < S::NKL; ++t)
    r.k[t] = __builtin_bit_cast(typename W::vec,
                                __builtin_amdgcn_raw_buffer_load_b128(rk, koff + 64 * t, 0, 0));
#pragma unroll
  for (int i = 0; i < 4; ++i) load_v<BF16, S>(rv, voff, i * tok, r.v[i]);
}

// A one-token tile holding the new token (token 0; every other slot zero),
// read from k_new/v_new: the cache slot is being written by this call and is
// never read back.
template <bool BF16, class S>
__device__ __forceinline__ void new_token_tile(Tile<BF16, S>& r, int lane, const char* knew,
                                               const char* vnew) {
  using W = Words<BF16>;
  const int r16 = lane & 15, q4 = lane >> 4;
  const typename W::vec z = {0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < S::NKL; ++t)
    r.k[t] = r16 == 0 ? *reinterpret_cast<const typename W::vec*>(knew + 16 * q4 + 64 * t) : z;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < S::VW; ++w) r.v[i][w] = 0;
  if (q4 == 0) {
    const char* p = vnew + r16 * (S::E * S::ESZ);
    if constexpr (S::VW == 2) {
      const typename W::vec2 x = *reinterpret_cast<const typename W::vec2*>(p);
      r.v[0][0] = x[0];
      r.v[0][1] = x[1];
    } else {
#pragma unroll
      for (int j = 0; j < S::VW / 4; ++j) {
        const typename W::vec x = *reinterpret_cast<const typename W::vec*>(p + 16 * j);
        r.v[0][4 * j] = x[0];
        r.v[0][4 * j + 1] = x[1];
        r.v[0][4 * j + 2] = x[2];
        r.v[0][4 * j + 3] = x[3];
      }
    }
  }
}

// Scores S^T of one tile: lane holds tokens 4(lane>>4)+i, q head (lane&15).
template <bool BF16, class S>
__device__ __forceinline__ f32x4 tile_scores(const Tile<BF16, S>& r,
                                             const typename Words<BF16>::vec* qr) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < S::NKL; ++t) {
    if constexpr (BF16) {
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r.k[t]),
                                                  __builtin_bit_cast(bf16x8, qr[t]), s, 0, 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(r.k[t][e], qr[t][e], s, 0, 0, 0);
    }
  }
  return s;
}

// Online-softmax update and P.V for one tile.  nvalid < 16 masks the tail.
template <bool BF16, class S, bool MASK>
__device__ __forceinline__ void tile_update(Tile<BF16, S>& r, f32x4 s, int nvalid, int lane,
                                            float scale_log2, float& m_run, float& l_run,
                                            f32x4* acc) {
  const int q4 = lane >> 4;
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s[i] * scale_log2;
    if (MASK && 4 * q4 + i >= nvalid) x[i] = -INFINITY;
  }
  if (MASK) {
    // tokens past the end may hold anything (NaN included): zero their V
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * q4 + i >= nvalid)
#pragma unroll
        for (int w = 0; w < S::VW; ++w) r.v[i][w] = 0;
  }
  float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mt = fmaxf(mt, swap16(mt));
  mt = fmaxf(mt, swap32(mt));
  const float m_new = fmaxf(m_run, mt);
  const float alpha = fast_exp2(m_run - m_new);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] - m_new);
  l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  m_run = m_new;
#pragma unroll
  for (int c = 0; c < S::NACC; ++c) acc[c] *= alpha;

  if constexpr (BF16) {
    const u32x2 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    const i16x4 pb = __builtin_bit_cast(i16x4, pw);
#pragma unroll
    for (int c = 0; c < S::E; ++c) {
      const int w = c >> 1;
      u32 t01, t23;
      if (c & 1) {
        t01 = (r.v[0][w] >> 16) | (r.v[1][w] & 0xffff0000u);
        t23 = (r.v[2][w] >> 16) | (r.v[3][w] & 0xffff0000u);
      } else {
        t01 = (r.v[0][w] & 0xffffu) | (r.v[1][w] << 16);
        t23 = (r.v[2][w] & 0xffffu) | (r.v[3][w] << 16);
      }
      const u32x2 aw = {t01, t23};
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, aw), pb,
                                                         acc[c], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < S::E; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(r.v[i][c], p[i], acc[c], 0, 0, 0);
  }
}

// Store a lane's D/4 contiguous output dims (already scaled) as dtype.
template <bool BF16, class S>
__device__ __forceinline__ void store_out(char* dst, const float* o) {
  constexpr int N = 4 * S::E;  // floats per lane
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < N / 8; ++j) {
      u32x4 w = {pack_bf16x2(o[8 * j], o[8 * j + 1]), pack_bf16x2(o[8 * j + 2], o[8 * j + 3]),
                 pack_bf16x2(o[8 * j + 4], o[8 * j + 5]), pack_bf16x2(o[8 * j + 6], o[8 * j + 7])};
      *reinterpret_cast<u32x4*>(dst + 16 * j) = w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < N / 4; ++j) {
      f32x4 w = {o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
      *reinterpret_cast<f32x4*>(dst + 16 * j) = w;
    }
  }
}

// One unit of work: (sequence, partition, kv head, chunk of <= 16 q heads).
template <bool BF16, int D, int BS>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a, int* slice_w, int lane, int seq,
                                            int part, int L, int kvh, int hc) {
  using S = Shape<BF16, D>;
  const int r16 = lane & 15, q4 = lane >> 4;

  const int Lp = L + a.has_new;
  const int tb = part * a.part_tokens;

  // q head held by this lane (padding lanes: hq < 0)
  const int hin = hc * 16 + r16;
  const int hq = hin < a.group ? kvh * a.group + hin : -1;
  const bool split = a.n_parts > 1;

  auto write_result = [&](float m, float l, const float* o /*4E values*/) {
    if (hq < 0) return;
    if (split) {
      const long long slot = ((long long)seq * a.num_heads + hq) * a.n_parts + part;
      float* dst = a.ws_acc + slot * D + 4 * S::E * q4;
#pragma unroll
      for (int j = 0; j < S::E; ++j) {
        f32x4 w = {o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
        *reinterpret_cast<f32x4*>(dst + 4 * j) = w;
      }
      if (q4 == 0) a.ws_ml[slot] = make_float2(m, l);
    } else {
      char* dst = (char*)a.out + (((long long)seq * a.num_heads + hq) * D + 4 * S::E * q4) * S::ESZ;
      store_out<BF16, S>(dst, o);
    }
  };
  auto fail = [&](unsigned bit) {
    if (a.err_flag && lane == 0) atomicOr(a.err_flag, (int)bit);
    float o[4 * S::E];
#pragma unroll
    for (int j = 0; j < 4 * S::E; ++j) o[j] = __builtin_nanf("");
    write_result(__builtin_nanf(""), __builtin_nanf(""), o);
  };

  if (L < 0 || (long long)Lp > (long long)a.max_blocks_per_seq * BS) {
    if (part == 0) fail(kErrSpan);
    return;
  }
  if (tb >= Lp && part > 0) return;  // partition past the end of this sequence
  const int te = min(tb + a.part_tokens, Lp);
  const int nblk = te > tb ? (te - tb + BS - 1) / BS : 0;
  const int jb0 = tb / BS;

  // stage and validate the table slice
  bool bad = false;
  const int32_t* row = a.block_table + (long long)seq * a.max_blocks_per_seq + jb0;
  for (int e = lane; e < nblk; e += 64) {
    const int pb = row[e];
    bad |= (pb < 0) | (pb >= a.num_blocks);
    slice_w[e] = pb;
  }
  if (__any(bad)) {
    fail(kErrBlock);
    return;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int tok = a.num_kv_heads * S::ROW;                   // bytes between token rows
  const long long blk = (long long)BS * tok;                 // bytes per physical block
  const char* kbase = (const char*)a.k_cache + (long long)kvh * S::ROW;
  const char* vbase = (const char*)a.v_cache + (long long)kvh * S::ROW;
  const char* knew = a.has_new ? (const char*)a.k_new + ((long long)seq * a.num_kv_heads + kvh) * S::ROW : nullptr;
  const char* vnew = a.has_new ? (const char*)a.v_new + ((long long)seq * a.num_kv_heads + kvh) * S::ROW : nullptr;

  // in-place append of the new token: one wave per (sequence, kv head)
  const bool owns_new = a.has_new && L >= tb && L < te;
  if (owns_new && hc == 0) {
    const int pb = slice_w[(L - tb) / BS];
    const long long off = (long long)pb * blk + (long long)(L % BS) * tok + (long long)kvh * S::ROW;
    for (int c = lane; c < S::ROW / 16; c += 64) {
      *reinterpret_cast<u32x4*>((char*)a.k_cache + off + 16 * c) =
          *reinterpret_cast<const u32x4*>(knew + 16 * c);
      *reinterpret_cast<u32x4*>((char*)a.v_cache + off + 16 * c) =
          *reinterpret_cast<const u32x4*>(vnew + 16 * c);
    }
  }

  // this lane's q head as the B operand (same byte runs as K's A operand)
  using QV = typename Words<BF16>::vec;
  QV qr[S::NKL];
  {
    const char* qp = (const char*)a.q + ((long long)seq * a.num_heads + (hq < 0 ? 0 : hq)) * S::ROW + 16 * q4;
#pragma unroll
    for (int t = 0; t < S::NKL; ++t) {
      QV z = {0, 0, 0, 0};
      qr[t] = hq < 0 ? z : *reinterpret_cast<const QV*>(qp + 64 * t);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[S::NACC];
#pragma unroll
  for (int c = 0; c < S::NACC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // cached tokens of this partition are tiled; the new token (if this
  // partition owns it) is folded in last as its own one-token tile
  const int tend = owns_new ? L : te;
  const int ntiles = (tend - tb + 15) / 16;
  const int last = ntiles - 1;
  const int nvalid_last = tend - (tb + 16 * last);
  const int koff = r16 * tok + 16 * q4;
  const int voff = 4 * q4 * tok + r16 * (S::E * S::ESZ);

  auto issue = [&](int t, Tile<BF16, S>& r) __attribute__((always_inline)) {
    const int pb = __builtin_amdgcn_readfirstlane(slice_w[(16 * t) / BS]);
    const int inblk = (16 * t) % BS;
    const long long off = (long long)pb * blk + (long long)inblk * tok;
    load_tile<BF16, S>(r, kbase + off, vbase + off, (BS - inblk) * tok, koff, voff, tok);
  };
  auto compute_full = [&](Tile<BF16, S>& r) __attribute__((always_inline)) {
    tile_update<BF16, S, false>(r, tile_scores<BF16, S>(r, qr), 16, lane, a.scale_log2, m_run,
                                l_run, acc);
  };
  auto compute = [&](int t, Tile<BF16, S>& r) __attribute__((always_inline)) {
    if (t == last)
      tile_update<BF16, S, true>(r, tile_scores<BF16, S>(r, qr), nvalid_last, lane, a.scale_log2,
                                 m_run, l_run, acc);
    else
      compute_full(r);
  };

  {
    // three-tile register ring: while one tile is computed, the next two are
    // in flight.  The steady-state trip is branch free so the wait counts
    // stay exact; the last 2..4 tiles are finished after it.
    Tile<BF16, S> b0, b1, b2;
    if (ntiles > 0) {
      // straight-line prologue (a single-tile partition loads its tile
      // twice): a conditional issue on the way into the loop would make
      // every wait in it conservative
      issue(0, b0);
      issue(min(1, last), b1);
      int t = 0;
      // sched_barrier keeps the compiler from hoisting work on a tile whose
      // loads were just issued above the compute of the tile before it
      // (that would turn the ring back into a wait for every load in flight)
      for (; t + 5 <= ntiles; t += 3) {
        issue(t + 2, b2);
        __builtin_amdgcn_sched_barrier(0);
        compute_full(b0);
        __builtin_amdgcn_sched_barrier(0);
        issue(t + 3, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute_full(b1);
        __builtin_amdgcn_sched_barrier(0);
        issue(t + 4, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute_full(b2);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int rem = ntiles - t;  // 1..4 tiles left; t, t+1 already issued
      if (rem >= 3) issue(t + 2, b2);
      compute(t, b0);
      if (rem >= 4) issue(t + 3, b0);
      if (rem >= 2) compute(t + 1, b1);
      if (rem >= 3) compute(t + 2, b2);
      if (rem >= 4) compute(t + 3, b0);
    }
    if (owns_new) {
      new_token_tile<BF16, S>(b1, lane, knew, vnew);
      tile_update<BF16, S, true>(b1, tile_scores<BF16, S>(b1, qr), 1, lane, a.scale_log2, m_run,
                                 l_run, acc);
    }
  }

  // total of the 4 token groups of this head
  float l_tot = l_run + swap16(l_run);
  l_tot += swap32(l_tot);

  float o[4 * S::E];
  const float inv = split ? 1.f : (l_tot > 0.f ? 1.f / l_tot : 0.f);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < S::E; ++c) o[S::E * i + c] = acc[c][i] * inv;
  write_result(m_run, l_tot, o);
}

// Persistent per-partition kernel: each wave takes units by ticket from the
// work list the plan kernel built (full partitions first, the shorter last
// partitions after them), prefetching its next ticket while it works, until
// the list is exhausted.  No workgroup is launched for an empty partition and
// the tail drains on the shortest units.
template <bool BF16, int D, int BS>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(BF16 ? 2 : 1)))
void decode_partial_kernel(DecodeArgs a) {
  __shared__ int slice[kWaves][kMaxSlice];
  const int lane = threadIdx.x & 63;
  // the wave index is uniform; saying so keeps everything derived from it
  // (unit, kv head, block bases, buffer descriptors) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int per_item = a.num_kv_heads * a.head_chunks;
  const unsigned total = (unsigned)a.ctrl[1] * (unsigned)per_item;
  int ticket = lane == 0 ? atomicAdd(&a.ctrl[0], 1) : 0;
  for (;;) {
    const unsigned u = (unsigned)__builtin_amdgcn_readfirstlane(ticket);
    if (u >= total) break;
    ticket = lane == 0 ? atomicAdd(&a.ctrl[0], 1) : 0;
    const int4 item = a.items[u / (unsigned)per_item];
    const int r = (int)(u % (unsigned)per_item);
    decode_unit<BF16, D, BS>(a, slice[wave], lane, __builtin_amdgcn_readfirstlane(item.x),
                             __builtin_amdgcn_readfirstlane(item.y),
                             __builtin_amdgcn_readfirstlane(item.z), r / a.head_chunks,
                             r % a.head_chunks);
  }
}

// Work list for the persistent kernel, one workgroup: for every sequence its
// full partitions, then (after all full partitions of all sequences) its
// last partial one, each item carrying (sequence, partition, cached length); a sequence with nothing to attend or a bad length gets
// one unit so that its output is written.  Also resets the ticket counter.
__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a, int block_size) {
  __shared__ int s_full[1024], s_part[1024];
  __shared__ int carry_full, carry_part, total_full;
  const int tid = threadIdx.x;
  const long long span = (long long)a.max_blocks_per_seq * block_size;
  auto counts = [&](int i, int& nf, int& np) {
    const int L = a.cache_seqlens[i];
    const int Lp = L + a.has_new;
    if (L < 0 || (long long)Lp > span) {
      nf = 0;
      np = 1;
      return;
    }
    nf = Lp / a.part_tokens;
    np = (Lp % a.part_tokens != 0 || Lp == 0) ? 1 : 0;
  };
  // pass 1: number of full partitions over the batch
  int my = 0;
  for (int i = tid; i < a.batch; i += 1024) {
    int nf, np;
    counts(i, nf, np);
    my += nf;
  }
  s_full[tid] = my;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) s_full[tid] += s_full[tid + off];
    __syncthreads();
  }
  if (tid == 0) {
    total_full = s_full[0];
    carry_full = 0;
    carry_part = 0;
    a.ctrl[0] = 0;
  }
  __syncthreads();
  // pass 2: exclusive scans in chunks of 1024 sequences, then write items
  for (int base = 0; base < a.batch; base += 1024) {
    const int i = base + tid;
    int nf = 0, np = 0;
    if (i < a.batch) counts(i, nf, np);
    s_full[tid] = nf;
    s_part[tid] = np;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int vf = tid >= off ? s_full[tid - off] : 0;
      const int vp = tid >= off ? s_part[tid - off] : 0;
      __syncthreads();
      s_full[tid] += vf;
      s_part[tid] += vp;
      __syncthreads();
    }
    const int ef = carry_full + s_full[tid] - nf;  // exclusive offsets
    const int ep = carry_part + s_part[tid] - np;
    const int L = i < a.batch ? a.cache_seqlens[i] : 0;
    for (int p = 0; p < nf; ++p) a.items[ef + p] = make_int4(i, p, L, 0);
    if (np) a.items[total_full + ep] = make_int4(i, nf, L, 0);
    __syncthreads();
    if (tid == 1023) {
      carry_full += s_full[1023];
      carry_part += s_part[1023];
    }
    __syncthreads();
  }
  if (tid == 0) a.ctrl[1] = total_full + carry_part;
}


// Merge of the partitions of one (sequence, q head): m = max m_k,
// l = sum l_k 2^(m_k - m), out = sum acc_k 2^(m_k - m) / l, in fixed order.
template <bool BF16, int D, int BS>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  using S = Shape<BF16, D>;
  constexpr int PER = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const long long idx = (long long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (idx >= (long long)a.batch * a.num_heads) return;
  const int seq = (int)(idx / a.num_heads);
  const int L = __builtin_amdgcn_readfirstlane(a.cache_seqlens[seq]);
  const int Lp = L + a.has_new;
  char* dst = (char*)a.out + (idx * D + PER * lane) * S::ESZ;
  float o[PER];
  auto store = [&]() {
    if constexpr (BF16) {
      if constexpr (PER == 2) {
        *reinterpret_cast<u32*>(dst) = pack_bf16x2(o[0], o[1]);
      } else {
        __bf16 h = (__bf16)o[0];
        *reinterpret_cast<__bf16*>(dst) = h;
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) reinterpret_cast<float*>(dst)[j] = o[j];
    }
  };
  if (L < 0 || (long long)Lp > (long long)a.max_blocks_per_seq * BS) {
#pragma unroll
    for (int j = 0; j < PER; ++j) o[j] = __builtin_nanf("");
    store();
    return;
  }
  const int np = Lp > 0 ? (Lp + a.part_tokens - 1) / a.part_tokens : 1;
  const float2* ml = a.ws_ml + idx * a.n_parts;
  const float* acc = a.ws_acc + idx * a.n_parts * D + PER * lane;
  float M = -INFINITY;
  bool nan = false;
  for (int k = lane; k < np; k += 64) {
    const float m = ml[k].x;
    nan |= m != m;
    M = fmaxf(M, m);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (__any(nan)) {
#pragma unroll
    for (int j = 0; j < PER; ++j) o[j] = __builtin_nanf("");
    store();
    return;
  }
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[j] = 0.f;
  if (M != -INFINITY) {
    for (int k = 0; k < np; ++k) {
      const float2 mk = ml[k];
      const float w = fast_exp2(mk.x - M);
      ls += mk.y * w;
#pragma unroll
      for (int j = 0; j < PER; ++j) o[j] += acc[(long long)k * D + j] * w;
    }
  }
  const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[j] *= inv;
  store();
}

// Workgroups of the persistent kernel that fit on the device at once; queried
// once per device and kernel (launch geometry only, no other state).
template <class Kernel>
int resident_workgroups(Kernel kernel, int threads) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  const int v = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 256);
  if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <bool BF16, int D, int BS>
hipError_t launch_one(const DecodeArgs& a, int phases, hipStream_t stream) {
  if (phases & 1) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, a, BS);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const auto kernel = decode_partial_kernel<BF16, D, BS>;
    long long wgs = resident_workgroups(kernel, kWaves * 64);
    const long long need = (a.total_units + kWaves - 1) / kWaves;
    if (wgs > need) wgs = need;
    if (wgs > 0) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(kWaves * 64), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if ((phases & 2) && a.n_parts > 1) {
    const long long heads = (long long)a.batch * a.num_heads;
    hipLaunchKernelGGL((decode_merge_kernel<BF16, D, BS>), dim3((unsigned)((heads + 3) / 4)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, int block_size, const DecodeArgs& a,
                         int phases, hipStream_t stream) {
  const bool bf = dtype == 1;
#define PKV_CASE(B, Dm, BSz)                                           \
  if (bf == B && head_dim == Dm && block_size == BSz)                  \
    return launch_one<B, Dm, BSz>(a, phases, stream);
  PKV_CASE(true, 128, 16)
  PKV_CASE(true, 128, 32)
  PKV_CASE(true, 64, 16)
  PKV_CASE(true, 64, 32)
  PKV_CASE(false, 128, 16)
  PKV_CASE(false, 128, 32)
  PKV_CASE(false, 64, 16)
  PKV_CASE(false, 64, 32)
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
