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
//  * A 16-token tile of K is the A operand of v_mfma_f32_16x16x32_bf16 (lane =
//    token, 16-byte runs of the head row); the q heads are the B operand
//    (zero-padded to 16).  The product is S^T: each lane ends up with 4
//    tokens' scores for ONE q head.  bf16 K is loaded as whole head rows
//    (one load instruction: 4 rows x 256 B at head_dim 128, instead of 16
//    rows x 64 B in the operand layout) and re-laid into the operand layout
//    through a small per-wave LDS stage right before its scores: the
//    long-context batch 1510 -> 1480 us per step, the mixed step's decode
//    half 1347 -> 1327 us (same box, two rounds).
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

constexpr int kWaves = 4;        // waves per workgroup (units of neighbouring kv heads)
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

// Cache policy of the K/V tile loads (the buffer instructions' aux bits:
// 1 = sc0, 2 = nt, 16 = sc1).  Each K/V byte is read once per call, and
// with the last-level cache flushed before every step the non-temporal hint
// is the faster policy for both launch forms: the persistent kernel on the
// long-context batch 5.93 -> 6.16 TB/s (the mixed step's decode half 5.96 ->
// 6.39); the direct grid on 1 / 2 / 4 long GQA-4 sequences 54.5 -> 41.1,
// 71.5 -> 49.2, 116 -> 73 us.  (Without the flush, repeated steps over a
// small batch find part of it cached, and the hint then cost the direct
// grid 6 % at 64 sequences, a batch the persistent kernel serves now.)
constexpr int kCpolStream = 2;
constexpr int kRsrcFlags = 0x00020000;  // gfx9-family buffer descriptor word 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kRsrcFlags);
}

// V words of one token for this lane: E elements at byte voff + soff.
template <bool BF16, class S, int CPOL>
__device__ __forceinline__ void load_v(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                       typename Words<BF16>::word* w) {
  using W = Words<BF16>;
  if constexpr (S::VW == 2) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, CPOL);
    const typename W::vec2 y = __builtin_bit_cast(typename W::vec2, x);
    w[0] = y[0];
    w[1] = y[1];
  } else {
#pragma unroll
    for (int j = 0; j < S::VW / 4; ++j) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16 * j, soff, CPOL);
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
template <bool BF16, class S, int CPOL>
__device__ __forceinline__ void load_tile(Tile<BF16, S>& r, const char* tk, const char* tv,
                                          int bytes, int koff, int kstep, int voff, int tok) {
  using W = Words<BF16>;
  const __amdgpu_buffer_rsrc_t rk = rsrc(tk, bytes), rv = rsrc(tv, bytes);
#pragma unroll
  for (int t = 0; t < S::NKL; ++t)
    r.k[t] = __builtin_bit_cast(typename W::vec,
                                __builtin_amdgcn_raw_buffer_load_b128(rk, koff + kstep * t, 0, CPOL));
#pragma unroll
  for (int i = 0; i < 4; ++i) load_v<BF16, S, CPOL>(rv, voff, i * tok, r.v[i]);
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

// One unit of work: a run of `nparts` consecutive partitions of one
// sequence, starting at partition `p0`, for one kv head and one chunk of <= 16
// of its q heads.  The run is streamed as one tile sequence (the register ring
// never drains inside it).  Each partition starts from a fresh (m, l, acc);
// at its end the partial is folded into the run's state in LDS with the
// (m, l) merge, and the run's merged partial is written once, at the end, to
// the slot of its first partition.  (A global store in mid-stream would make
// every later tile wait also wait for the store's acknowledgement: the
// vector-memory counter retires loads and stores in order.)
// `started` runs once per unit, right after the unit's last tile loads are
// issued (or where it gives up early): the persistent kernel takes its next
// ticket there, so that the ticket atomic -- slow on its one contended
// counter -- sits behind every load of the unit in the in-order
// vector-memory counter, where no wait of the unit waits for it; it has the
// unit's last tiles to complete before the next ticket exchange needs it.
template <bool BF16, int D, int BS, int CPOL, class Started>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a, int* slice_w, float* run_w,
                                            char* kst, int lane, int seq, int p0, int nparts,
                                            int L, int kvh, int hc, Started&& started) {
  using S = Shape<BF16, D>;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int P = a.part_tokens;
  const int Lp = L + a.has_new;
  const int tb = p0 * P;

  // q head held by this lane (padding lanes: hq < 0)
  const int hin = hc * 16 + r16;
  const int hq = hin < a.group ? kvh * a.group + hin : -1;
  const bool split = a.n_parts > 1;

  // Partials of one (sequence, kv head, partition) are one block of
  // group * D floats; this chunk's heads occupy [16 hc D, (16 hc + gc) D) of
  // it, laid out as [j][q4][head][4] so that each store instruction writes one
  // contiguous run of 64 gc bytes (not 16-byte pieces a cache line apart).
  const int gc = min(16, a.group - 16 * hc);
  auto write_result = [&](int part, float m, float l, const float* o /*4E values*/) {
    if (hq < 0) return;
    if (split) {
      const long long blk_id = ((long long)seq * a.num_kv_heads + kvh) * a.n_parts + part;
      float* dst = a.ws_acc + blk_id * a.group * D + 16 * hc * D;
#pragma unroll
      for (int j = 0; j < S::E; ++j) {
        f32x4 w = {o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
        *reinterpret_cast<f32x4*>(dst + 4 * ((j * 4 + q4) * gc + r16)) = w;
      }
      if (q4 == 0) a.ws_ml[blk_id * a.group + 16 * hc + r16] = make_float2(m, l);
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
    write_result(p0, __builtin_nanf(""), __builtin_nanf(""), o);
  };

  if (L < 0 || (long long)Lp > (long long)a.max_blocks_per_seq * BS) {
    fail(kErrSpan);
    started();
    return;
  }
  const int te = min(tb + nparts * P, Lp);
  const int nblk = te > tb ? (te - tb + BS - 1) / BS : 0;
  const int jb0 = tb / BS;

  // stage and validate the table slice of the run
  bool bad = false;
  const int32_t* row = a.block_table + (long long)seq * a.max_blocks_per_seq + jb0;
  for (int e = lane; e < nblk; e += 64) {
    const int pb = row[e];
    bad |= (pb < 0) | (pb >= a.num_blocks);
    slice_w[e] = pb;
  }
  if (__any(bad)) {
    fail(kErrBlock);
    started();
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

  // End of partition `part`: fold its (m, l, acc) into the run state, then
  // start the next partition afresh.  The run state lives in LDS, lane-major
  // ([value][lane]); the last partition of the run writes the merged partial
  // (or, without a split, the normalised output).  Values are handled E at a
  // time (one row i of the accumulators: dims E (4 q4 + i) + c) to keep the
  // register footprint small.
  auto flush = [&](int part) __attribute__((always_inline)) {
    float l_tot = l_run + swap16(l_run);  // total of the 4 token groups of this head
    l_tot += swap32(l_tot);
    const bool first = part == p0, final = part == p0 + nparts - 1;
    float m = m_run, l = l_tot, fa = 0.f, fb = 1.f;
    if (!first) {
      // merge with the run so far: m' = max(M, m), l' = L 2^(M-m') + l 2^(m-m')
      const float M = run_w[4 * S::E * 64 + lane], Lr = run_w[(4 * S::E + 1) * 64 + lane];
      const float mn = fmaxf(M, m);
      fa = fast_exp2(M - mn);
      fb = fast_exp2(m - mn);
      l = Lr * fa + l * fb;
      m = mn;
    }
    const float inv = (final && !split) ? (l > 0.f ? 1.f / l : 0.f) : 1.f;
    const long long blk_id = ((long long)seq * a.num_kv_heads + kvh) * a.n_parts + p0;
    float* wsd = split ? a.ws_acc + blk_id * a.group * D + 16 * hc * D : nullptr;
    char* outd = (char*)a.out + (((long long)seq * a.num_heads + (hq < 0 ? 0 : hq)) * D +
                                 4 * S::E * q4) * S::ESZ;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v[S::E];
#pragma unroll
      for (int c = 0; c < S::E; ++c) {
        const int j = S::E * i + c;
        v[c] = first ? acc[c][i] : run_w[j * 64 + lane] * fa + acc[c][i] * fb;
      }
      if (!final) {
#pragma unroll
        for (int c = 0; c < S::E; ++c) run_w[(S::E * i + c) * 64 + lane] = v[c];
      } else if (hq >= 0) {
        if (split) {
#pragma unroll
          for (int c = 0; c < S::E; c += 4) {
            const int j4 = (S::E * i + c) / 4;
            *reinterpret_cast<f32x4*>(wsd + 4 * ((j4 * 4 + q4) * gc + r16)) =
                f32x4{v[c], v[c + 1], v[c + 2], v[c + 3]};
          }
        } else if constexpr (BF16) {
          if constexpr (S::E == 8) {
            *reinterpret_cast<u32x4*>(outd + 16 * i) =
                u32x4{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv),
                      pack_bf16x2(v[4] * inv, v[5] * inv), pack_bf16x2(v[6] * inv, v[7] * inv)};
          } else {
            *reinterpret_cast<u32x2*>(outd + 8 * i) =
                u32x2{pack_bf16x2(v[0] * inv, v[1] * inv), pack_bf16x2(v[2] * inv, v[3] * inv)};
          }
        } else {
#pragma unroll
          for (int c = 0; c < S::E; c += 4)
            *reinterpret_cast<f32x4*>(outd + 4 * (S::E * i + c)) =
                f32x4{v[c] * inv, v[c + 1] * inv, v[c + 2] * inv, v[c + 3] * inv};
        }
      }
    }
    if (!final) {
      run_w[4 * S::E * 64 + lane] = m;
      run_w[(4 * S::E + 1) * 64 + lane] = l;
    } else if (split && hq >= 0 && q4 == 0) {
      a.ws_ml[blk_id * a.group + 16 * hc + r16] = make_float2(m, l);
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int c = 0; c < S::NACC; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // cached tokens of the run are tiled; the new token (if the run owns it)
  // is folded in last as its own one-token tile
  const int tend = owns_new ? L : te;
  const int ntiles = (tend - tb + 15) / 16;
  const int last = ntiles - 1;
  const int nvalid_last = tend - (tb + 16 * last);
  const int tpp = P / 16;  // tiles per partition (P is a multiple of 16)
  // K: bf16 tiles are loaded as whole token rows (each load instruction
  // covers 64 / LPR rows of LPR 16-byte pieces: 4 rows of 256 B at head_dim
  // 128) and re-laid into the MFMA operand layout (lane = token, 64-byte
  // steps along the row) through the wave's LDS stage just before their
  // scores are taken; fp32 tiles are loaded in the operand layout directly
  constexpr int LPR = S::ROW / 16;  // lanes per token row
  constexpr bool ROWK = BF16 && LPR <= 64 && 64 % LPR == 0;
  constexpr int KPITCH = S::ROW + 16;  // LDS bytes per staged row (padded against bank conflicts)
  const int koff = ROWK ? (lane / LPR) * tok + 16 * (lane % LPR) : r16 * tok + 16 * q4;
  const int kstep = ROWK ? (64 / LPR) * tok : 64;
  auto relayout = [&](Tile<BF16, S>& r) __attribute__((always_inline)) {
    if constexpr (ROWK) {
      using V = typename Words<BF16>::vec;
#pragma unroll
      for (int t = 0; t < S::NKL; ++t)
        *reinterpret_cast<V*>(kst + ((64 / LPR) * t + lane / LPR) * KPITCH + 16 * (lane % LPR)) =
            r.k[t];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < S::NKL; ++t)
        r.k[t] = *reinterpret_cast<const V*>(kst + r16 * KPITCH + 64 * t + 16 * q4);
      // the next tile's writes must not overtake these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };
  const int voff = 4 * q4 * tok + r16 * (S::E * S::ESZ);

  auto issue = [&](int t, Tile<BF16, S>& r) __attribute__((always_inline)) {
    const int pb = __builtin_amdgcn_readfirstlane(slice_w[(16 * t) / BS]);
    const int inblk = (16 * t) % BS;
    const long long off = (long long)pb * blk + (long long)inblk * tok;
    load_tile<BF16, S, CPOL>(r, kbase + off, vbase + off, (BS - inblk) * tok, koff, kstep, voff,
                             tok);
  };
  // a partition ends after tile t: write its partial (the run's last
  // partition is written after the loop)
  auto boundary = [&](int t) __attribute__((always_inline)) {
    if ((t + 1) % tpp == 0 && t != last) flush(p0 + t / tpp);
  };
  auto compute_full = [&](int t, Tile<BF16, S>& r) __attribute__((always_inline)) {
    relayout(r);
    tile_update<BF16, S, false>(r, tile_scores<BF16, S>(r, qr), 16, lane, a.scale_log2, m_run,
                                l_run, acc);
    boundary(t);
  };
  auto compute = [&](int t, Tile<BF16, S>& r) __attribute__((always_inline)) {
    if (t == last) relayout(r);
    if (t == last)
      tile_update<BF16, S, true>(r, tile_scores<BF16, S>(r, qr), nvalid_last, lane, a.scale_log2,
                                 m_run, l_run, acc);
    else
      compute_full(t, r);
  };

  {
    // three-tile register ring: while one tile is computed, the next two are
    // in flight.  The steady-state trip is branch free except for the rare
    // partition end, so the wait counts stay tight; the last 1..4 tiles are
    // finished after it.
    Tile<BF16, S> b0, b1, b2;
    if (ntiles > 0) {
      // straight-line prologue (a single-tile run loads its tile twice): a
      // conditional issue on the way into the loop would make every wait in
      // it conservative
      issue(0, b0);
      issue(min(1, last), b1);
      int t = 0;
      // sched_barrier keeps the compiler from hoisting work on a tile whose
      // loads were just issued above the compute of the tile before it
      // (that would turn the ring back into a wait for every load in flight)
      for (; t + 5 <= ntiles; t += 3) {
        issue(t + 2, b2);
        __builtin_amdgcn_sched_barrier(0);
        compute_full(t, b0);
        __builtin_amdgcn_sched_barrier(0);
        issue(t + 3, b0);
        __builtin_amdgcn_sched_barrier(0);
        compute_full(t + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        issue(t + 4, b1);
        __builtin_amdgcn_sched_barrier(0);
        compute_full(t + 2, b2);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int rem = ntiles - t;  // 1..4 tiles left; t, t+1 already issued
      if (rem >= 3) issue(t + 2, b2);
      compute(t, b0);
      if (rem >= 4) issue(t + 3, b0);
      started();  // every load of the unit is out
      if (rem >= 2) compute(t + 1, b1);
      if (rem >= 3) compute(t + 2, b2);
      if (rem >= 4) compute(t + 3, b0);
      // a new token that starts a partition of its own: close the last
      // partition of cached tokens first
      if (owns_new && L % P == 0) flush(L / P - 1);
    } else {
      started();
    }
    if (owns_new) {
      new_token_tile<BF16, S>(b1, lane, knew, vnew);
      tile_update<BF16, S, true>(b1, tile_scores<BF16, S>(b1, qr), 1, lane, a.scale_log2, m_run,
                                 l_run, acc);
    }
  }
  flush(p0 + nparts - 1);
}

// Persistent per-partition kernel: each wave takes units by ticket from the
// work list the plan kernel built, prefetching its next ticket while it
// works (the atomic goes out after the unit's last tile loads: ahead of its
// first ones, the in-order vector-memory counter made the first tile wait
// for it, and ahead of later ones, the later tiles -- step time 148 -> 141
// us on 64 GQA-4 sequences, 1604 -> 1565 us on the long-context batch),
// until the list is exhausted.  No workgroup is launched for an empty
// partition and the tail drains on the shortest units.
template <bool BF16, int D, int BS>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(BF16 ? 2 : 1)))
void decode_partial_kernel(DecodeArgs a) {
  __shared__ int slice[kWaves][kMaxSlice];
  __shared__ float run_state[kWaves][(D / 4 + 2) * 64];  // per lane: D/4 sums, m, l
  __shared__ __attribute__((aligned(16))) char kstage[kWaves][BF16 ? 16 * (D * 2 + 16) : 16];
  const int lane = threadIdx.x & 63;
  // the wave index is uniform; saying so keeps everything derived from it
  // (unit, kv head, block bases, buffer descriptors) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int per_item = a.num_kv_heads * a.head_chunks;
  const unsigned total = (unsigned)a.ctrl[1] * (unsigned)per_item;
  // Tickets are taken per workgroup: ticket T is units kWaves T .. kWaves T +
  // kWaves-1, one per wave -- neighbouring kv heads of the same run, whose
  // rows sit side by side in every block, so the workgroup's loads of a
  // tile land on one contiguous kWaves x head-row span of the block.  Wave 0
  // takes the tickets and passes them on through LDS (double buffered by
  // iteration parity, one barrier per unit).
  __shared__ unsigned s_ticket[2];
  int ticket = (wave == 0 && lane == 0) ? atomicAdd(&a.ctrl[0], 1) : 0;
  for (int it = 0;; ++it) {
    if (wave == 0) s_ticket[it & 1] = (unsigned)__builtin_amdgcn_readfirstlane(ticket);
    __syncthreads();
    const unsigned T = (unsigned)__builtin_amdgcn_readfirstlane(s_ticket[it & 1]);
    if ((unsigned long long)T * kWaves >= total) break;
    const unsigned u = T * kWaves + wave;  // wave 0's unit always exists
    if (u >= total) continue;
    const int4 item = a.items[u / (unsigned)per_item];
    const int r = (int)(u % (unsigned)per_item);
    const int packed = __builtin_amdgcn_readfirstlane(item.y);
    decode_unit<BF16, D, BS, kCpolStream>(a, slice[wave], run_state[wave], kstage[wave], lane,
                             __builtin_amdgcn_readfirstlane(item.x),
                             packed >> 8, packed & 255, __builtin_amdgcn_readfirstlane(item.z),
                             r / a.head_chunks, r % a.head_chunks, [&]() {
                               if (wave == 0 && lane == 0) ticket = atomicAdd(&a.ctrl[0], 1);
                             });
  }
}

// Direct grid for small batches: one wave per (sequence, partition, kv head,
// head chunk) slot of the full grid, no work list; slots past a sequence's
// end exit at once.  For few units the persistent kernel's per-unit work-list
// lookups would not be hidden.
template <bool BF16, int D, int BS>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(BF16 ? 2 : 1)))
void decode_direct_kernel(DecodeArgs a) {
  __shared__ int slice[kWaves][kMaxSlice];
  __shared__ float run_state[kWaves][(D / 4 + 2) * 64];
  __shared__ __attribute__((aligned(16))) char kstage[kWaves][BF16 ? 16 * (D * 2 + 16) : 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned unit = blockIdx.x * kWaves + wave;
  if (unit >= (unsigned)a.total_units) return;
  const int hc = (int)(unit % (unsigned)a.head_chunks);
  unit /= (unsigned)a.head_chunks;
  const int kvh = (int)(unit % (unsigned)a.num_kv_heads);
  unit /= (unsigned)a.num_kv_heads;
  const int part = (int)(unit % (unsigned)a.n_parts);
  const int seq = (int)(unit / (unsigned)a.n_parts);
  const int L = __builtin_amdgcn_readfirstlane(a.cache_seqlens[seq]);
  const int Lp = L + a.has_new;
  const bool bad = L < 0 || (long long)Lp > (long long)a.max_blocks_per_seq * BS;
  if (part > 0 && (bad || part * a.part_tokens >= Lp)) return;
  decode_unit<BF16, D, BS, kCpolStream>(a, slice[wave], run_state[wave], kstage[wave], lane, seq,
                                        part, 1, L, kvh, hc, []() {});
}

// Work list for the persistent kernel, one workgroup.  Every sequence's
// partitions are cut into runs of R consecutive partitions (R chosen so that
// there are at least about two units per resident wave, and at most
// a.max_run: every unit start costs a wave several dependent memory round
// trips with no tile in flight, so fewer, longer units pay while the tail
// still balances).  The runs that do not hold a sequence's end are all R full
// partitions long and come first, in sequence order; then each sequence's
// last run, longest first (bucketed by token count), so that the list ends
// on the shortest units and the waves run dry together.  A sequence with
// nothing to attend or a bad length gets one one-partition run so that its
// output is written.  Items carry (sequence, first partition << 8 |
// partitions, cached length).  Also resets the ticket counter and records
// the run length for the merge.
//
// The sums and scans run inside each wave (lane shuffles) with one exchange
// of the 16 wave totals through LDS, two barriers per scan; the lengths are
// read from memory once (kept in registers for the first kPlanChunks chunks
// of 1024 sequences).  With a barrier per step of an LDS tree instead (~55
// barriers) the kernel took 7.7-7.8 us at 64 and 256 sequences, now 5.9-6.5
// us: what remains is the cold read of the lengths, the stores of the list
// and the dispatch itself.
constexpr int kPlanBuckets = 512;
constexpr int kPlanChunks = 4;

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive prefix of v over the 1024 threads of the workgroup (thread
// order), and the total.  s_w: 16 ints of LDS.  Every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v, lane);
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int x = s_w[k];
    base += k < w ? x : 0;
    tot += x;
  }
  __syncthreads();  // s_w free for the next scan
  total = tot;
  return base + inc - v;
}

__global__ __launch_bounds__(1024) void decode_plan_kernel(DecodeArgs a, int block_size) {
  __shared__ int s_w[16];
  __shared__ int s_hist[kPlanBuckets], s_cur[kPlanBuckets];
  const int tid = threadIdx.x;
  const long long span = (long long)a.max_blocks_per_seq * block_size;
  auto nparts_of = [&](int L) {
    const int Lp = L + a.has_new;
    if (L < 0 || (long long)Lp > span || Lp == 0) return 1;
    return (Lp + a.part_tokens - 1) / a.part_tokens;
  };
  int lens[kPlanChunks];
  // chunk k's length for this thread (selected, not indexed, so that the
  // array stays in registers)
  auto len_of = [&](int k, int i) {
    int v = 0;
    bool hit = false;
#pragma unroll
    for (int c = 0; c < kPlanChunks; ++c)
      if (k == c) {
        v = lens[c];
        hit = true;
      }
    return hit ? v : a.cache_seqlens[i];
  };
  // pass 1: partitions over the batch -> run length
  int my = 0;
#pragma unroll
  for (int k = 0; k < kPlanChunks; ++k) {
    const int i = tid + 1024 * k;
    lens[k] = i < a.batch ? a.cache_seqlens[i] : 0;
    my += i < a.batch ? nparts_of(lens[k]) : 0;
  }
  for (int i = tid + 1024 * kPlanChunks; i < a.batch; i += 1024) my += nparts_of(a.cache_seqlens[i]);
  for (int b = tid; b < kPlanBuckets; b += 1024) s_hist[b] = s_cur[b] = 0;
  int total_parts;
  block_exclusive_scan(my, s_w, total_parts);
  const long long units = (long long)total_parts * a.num_kv_heads * a.head_chunks;
  long long rr = units / (2LL * a.resident_waves);
  const int R = (int)(rr < 1 ? 1 : (rr > a.max_run ? a.max_run : rr));
  if (tid == 0) a.ctrl[0] = 0;
  const long long rp = (long long)R * a.part_tokens;  // tokens of a full run
  // a sequence's last run: its first partition, and the bucket of its token
  // count (0 = a full run's length, kPlanBuckets-1 = nothing)
  auto last_run = [&](int np, int L, int& first) {
    first = ((np - 1) / R) * R;
    const int Lp = L + a.has_new;
    const long long t = (L < 0 || (long long)Lp > span) ? 0 : max(Lp - first * a.part_tokens, 0);
    return (int)((rp - t) * kPlanBuckets / (rp + 1));
  };
  // pass 2: runs before each sequence's last, written in sequence order
  // chunk by chunk; the last runs are counted per bucket
  int carry = 0;
  for (int base = 0, k = 0; base < a.batch; base += 1024, ++k) {
    const int i = base + tid;
    int L = 0, np = 0, first = 0;
    if (i < a.batch) {
      L = len_of(k, i);
      np = nparts_of(L);
      atomicAdd(&s_hist[last_run(np, L, first)], 1);
    }
    const int nc = np > 0 ? (np - 1) / R : 0;
    int chunk_total;
    const int e = carry + block_exclusive_scan(nc, s_w, chunk_total);
    for (int c = 0; c < nc; ++c) a.items[e + c] = make_int4(i, ((c * R) << 8) | R, L, 0);
    carry += chunk_total;
  }
  const int n_lead = carry;
  // bucket starts: exclusive scan of the histogram (kPlanBuckets <= 1024;
  // the scan's barriers also order the histogram's atomics before the reads)
  __syncthreads();
  const int h = tid < kPlanBuckets ? s_hist[tid] : 0;
  int nb;
  const int start = block_exclusive_scan(h, s_w, nb);
  if (tid < kPlanBuckets) s_hist[tid] = start;
  __syncthreads();
  // pass 3: the last runs, longest first (order within a bucket is free)
  for (int base = 0, k = 0; base < a.batch; base += 1024, ++k) {
    const int i = base + tid;
    if (i >= a.batch) break;
    int first;
    const int L = len_of(k, i);
    const int np = nparts_of(L);
    const int b = last_run(np, L, first);
    const int pos = s_hist[b] + atomicAdd(&s_cur[b], 1);
    a.items[n_lead + pos] = make_int4(i, (first << 8) | (np - first), L, 0);
  }
  if (tid == 0) {
    a.ctrl[1] = n_lead + a.batch;
    a.ctrl[2] = R;
  }
}

// Merge of the run partials: one thread per 16-byte piece of a partial (4
// dims of one q head), so a wave reads whole contiguous stretches of the
// [j][q4][head][4] partial layout and every lane is busy whatever the group
// size.  Thread t of a (sequence, kv head, chunk of <= 16 heads) holds head
// t % gc, dims 4E (t / gc % 4) + 4 (t / 4gc) .. +3.  For each head:
// m = max m_k, l = sum l_k 2^(m_k - m), sums likewise, out = sum / l (0 for
// l = 0), taken online over batches of 8 runs (a batch's loads all in
// flight together; the running sums are rescaled when a batch raises m); a
// NaN partial (a data error) makes the output NaN; empty runs (m = -inf)
// contribute nothing.
constexpr int kMergeBatch = 8;
template <bool BF16, int D, int BS>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  using S = Shape<BF16, D>;
  const int per = min(a.group, 16) * (D / 4);  // threads per (sequence, kv head, chunk)
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long grp = gid / per;
  const int t = (int)(gid - grp * per);
  const long long ngroups = (long long)a.batch * a.num_kv_heads * a.head_chunks;
  if (grp >= ngroups) return;
  const int hc = (int)(grp % a.head_chunks);
  const long long sk = grp / a.head_chunks;  // seq * num_kv_heads + kvh
  const int kvh = (int)(sk % a.num_kv_heads);
  const int seq = (int)(sk / a.num_kv_heads);
  const int gc = min(16, a.group - 16 * hc);
  if (t >= gc * (D / 4)) return;
  const int r = t % gc, q4 = (t / gc) & 3, j = t / (4 * gc);
  const int hq = kvh * a.group + 16 * hc + r;
  char* dst = (char*)a.out + (((long long)seq * a.num_heads + hq) * D + 4 * S::E * q4 + 4 * j) *
                                 S::ESZ;
  auto store4 = [&](f32x4 o) {
    if constexpr (BF16)
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    else
      *reinterpret_cast<f32x4*>(dst) = o;
  };

  // the run length and the sequence's length are both requested before
  // either is used, so that the two round trips overlap (the control words
  // always exist; the direct grid leaves them unset and does not use them)
  const int R_plan = a.ctrl[2];
  const int L = a.cache_seqlens[seq];
  asm volatile("" ::"s"(R_plan), "v"(L));
  const int Lp = L + a.has_new;
  if (L < 0 || (long long)Lp > (long long)a.max_blocks_per_seq * BS) {
    const float nan = __builtin_nanf("");
    store4(f32x4{nan, nan, nan, nan});
    return;
  }
  const int np = Lp > 0 ? (Lp + a.part_tokens - 1) / a.part_tokens : 1;
  // each run of R partitions left one partial, at its first slot
  const int R = a.direct ? 1 : R_plan;
  const int nruns = (np + R - 1) / R;
  const long long blk0 = sk * a.n_parts;
  const float* accp = a.ws_acc + blk0 * a.group * D + 16 * hc * D + 4 * t;
  const float2* mlp = a.ws_ml + blk0 * a.group + 16 * hc + r;
  const long long acc_step = (long long)R * a.group * D;  // floats between runs
  const long long ml_step = (long long)R * a.group;

  float M = -INFINITY, Ls = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  bool nan = false;
  for (int k0 = 0; k0 < nruns; k0 += kMergeBatch) {
    float2 ml[kMergeBatch];
    f32x4 v[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const bool in = k0 + i < nruns;
      ml[i] = in ? mlp[(k0 + i) * ml_step] : make_float2(-INFINITY, 0.f);
      v[i] = in ? *reinterpret_cast<const f32x4*>(accp + (k0 + i) * acc_step)
                : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      nan |= ml[i].x != ml[i].x;
      mb = fmaxf(mb, ml[i].x);
    }
    const float mn = fmaxf(M, mb);
    if (mn == -INFINITY) continue;  // nothing but empty runs so far
    if (mn > M) {
      const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mn);
      Ls *= sc;
      o *= sc;
      M = mn;
    }
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (ml[i].x == -INFINITY) continue;
      const float w = fast_exp2(ml[i].x - M);
      Ls += ml[i].y * w;
      o += v[i] * w;
    }
  }
  const float inv = nan ? __builtin_nanf("") : (Ls > 0.f ? 1.f / Ls : 0.f);
  store4(o * inv);
}

// Workgroups of decode_partial_kernel<BF16, D, BS> that fit on the device at
// once (launch geometry only, no other state).  Queried once per device and
// instantiation: the instantiations differ in register use (two waves per
// SIMD for bf16 at head_dim 128, three at 64, one for fp32 at 128), and every
// one of them has the same function type, so the cache is keyed by the
// template arguments, not by the kernel's type.
template <bool BF16, int D, int BS>
int resident_workgroups() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_partial_kernel<BF16, D, BS>,
                                                   kWaves * 64, 0) != hipSuccess)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 256;
  const int v = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 256);
  if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <bool BF16, int D, int BS>
hipError_t launch_one(const DecodeArgs& args, int phases, hipStream_t stream) {
  DecodeArgs a = args;
  const auto kernel = decode_partial_kernel<BF16, D, BS>;
  long long wgs = resident_workgroups<BF16, D, BS>();
  a.resident_waves = (int)(wgs * kWaves);
  // few units (up to two grid slots per resident wave): the direct grid;
  // more: the persistent kernel with runs
  a.direct = a.total_units <= 2LL * a.resident_waves;
  if ((phases & 1) && a.direct) {
    const long long grid = (a.total_units + kWaves - 1) / kWaves;
    if (grid > 0) {
      hipLaunchKernelGGL((decode_direct_kernel<BF16, D, BS>), dim3((unsigned)grid),
                         dim3(kWaves * 64), 0, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else if (phases & 1) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, a, BS);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long need = (a.total_units + kWaves - 1) / kWaves;
    if (wgs > need) wgs = need;
    if (wgs > 0) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(kWaves * 64), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if ((phases & 2) && a.n_parts > 1) {
    const long long threads = (long long)a.batch * a.num_kv_heads * a.head_chunks *
                              (a.group < 16 ? a.group : 16) * (D / 4);
    hipLaunchKernelGGL((decode_merge_kernel<BF16, D, BS>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Workspace of pkv_decode_noalloc: one array per GPU, part of this code
// object, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host that name is only a stand-in); it looks up
// the device address once per device and passes that.
__device__ __align__(256) char scratch[kDecodeScratchBytes];

}  // namespace

hipError_t decode_scratch(void** ptr) {
  static std::atomic<void*> addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

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
