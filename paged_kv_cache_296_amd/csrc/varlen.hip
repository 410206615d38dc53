// Variable-length (packed) attention for gfx950, no mask.
//
// What is computed (HF Transformers "paged attention" page, section "Jalur
// Varlen"): sequences are packed along one token axis; the cumulative
// lengths cu_seq_lens_q / cu_seq_lens_k say which query rows and which
// key/value rows belong to request b.  Every query row attends every key row
// of its own request; a request with no key row outputs zeros.
//
// How:
//  * A workgroup (4 waves) owns 128 query rows of one q head; each wave owns
//    32 rows.  Key tiles of 64 rows stream through LDS, double buffered: K as
//    rows [key][dim], V transposed to [dim][key] so that both MFMA operands
//    are 16-byte LDS reads.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the query rows sit on the
//    lane axis, so a row's max and sum are in-lane reductions plus one
//    exchange between the two 32-lane halves.  P^T from the S^T accumulator
//    is directly the B operand of O^T = V^T P^T (same MFMA), provided the key
//    order in the V^T LDS rows swaps bits 2 and 3 of the key index, which the
//    transposing store does.  O^T keeps one query row per lane, so the
//    online-softmax rescale is lane-local.
//  * Online softmax in the exp2 domain; the final division by the row sum
//    happens once in the epilogue; bf16 output is rounded to nearest even.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_kernels.h"

namespace pkv {
namespace {

using u32 = uint32_t;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 128;       // query rows per workgroup
constexpr int kWaveRows = 32;    // query rows per wave
constexpr int kKeys = 64;        // keys per LDS tile
constexpr unsigned kErrCu = 4u, kErrMaxLen = 8u;

__device__ __forceinline__ float swap32(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32 pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (u32)__builtin_bit_cast(unsigned short, a) |
         ((u32)__builtin_bit_cast(unsigned short, b) << 16);
}

// position of key k (0..63) inside a V^T LDS row: bits 2 and 3 swapped
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D>
struct Lds {
  static constexpr int KROW = D * 2 + 16;        // bytes per K row (padded)
  static constexpr int VROW = kKeys * 2 + 16;    // bytes per V^T row (padded)
  static constexpr int KBYTES = kKeys * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
};

template <int D>
struct Stage {
  // K: 64 keys x D dims in 16-byte row pieces; V: groups of 4 keys x 8 dims
  static constexpr int KPIECES = kKeys * D * 2 / 16 / 256;  // per thread
  static constexpr int VG_TOTAL = (kKeys / 4) * (D / 8);
  static constexpr int VGROUPS = (VG_TOTAL + 255) / 256;
  u32x4 k[KPIECES];
  u32x4 v[VGROUPS][4];
};

// Byte offset of (dim row r, key position p) in the V^T tile.  The 16-byte
// chunk index (p / 8) is XOR-ed with (r / 8) mod 8 so that the transposing
// stores, which hit rows 8 apart, spread over the LDS banks.
template <int D>
__device__ __forceinline__ int vt_off(int r, int p) {
  return r * Lds<D>::VROW + 16 * ((p >> 3) ^ ((r >> 3) & 7)) + 2 * (p & 7);
}

template <int D>
__device__ __forceinline__ void stage_load(Stage<D>& st, const char* kg, const char* vg, int k0,
                                           int k_end, int tok, int tid) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  // K pieces: piece p = tid + 256 * r -> key p / (D/8), 16-byte chunk p % (D/8)
#pragma unroll
  for (int r = 0; r < Stage<D>::KPIECES; ++r) {
    const int p = tid + 256 * r;
    const int key = p / (D / 8), ch = p % (D / 8);
    const int kk = k0 + key;
    st.k[r] = kk < k_end ? *reinterpret_cast<const u32x4*>(kg + (long long)kk * tok + 16 * ch) : z;
  }
  // V groups: g = tid + 256 * r -> dim group g % (D/8), key quad g / (D/8)
#pragma unroll
  for (int r = 0; r < Stage<D>::VGROUPS; ++r) {
    const int g = tid + 256 * r;
    const int dg = g % (D / 8), kq = g / (D / 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = k0 + 4 * kq + i;
      st.v[r][i] = (g < Stage<D>::VG_TOTAL && kk < k_end)
                       ? *reinterpret_cast<const u32x4*>(vg + (long long)kk * tok + 16 * dg)
                       : z;
    }
  }
}

template <int D>
__device__ __forceinline__ void stage_store(const Stage<D>& st, char* buf, int tid) {
#pragma unroll
  for (int r = 0; r < Stage<D>::KPIECES; ++r) {
    const int p = tid + 256 * r;
    const int key = p / (D / 8), ch = p % (D / 8);
    *reinterpret_cast<u32x4*>(buf + key * Lds<D>::KROW + 16 * ch) = st.k[r];
  }
  char* vt = buf + Lds<D>::KBYTES;
#pragma unroll
  for (int r = 0; r < Stage<D>::VGROUPS; ++r) {
    const int g = tid + 256 * r;
    if (g >= Stage<D>::VG_TOTAL) break;
    const int dg = g % (D / 8), kq = g / (D / 8);
    const int pos = vt_pos(4 * kq);  // the 4 keys stay adjacent
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      u32 t01, t23;
      if (e & 1) {
        t01 = (st.v[r][0][w] >> 16) | (st.v[r][1][w] & 0xffff0000u);
        t23 = (st.v[r][2][w] >> 16) | (st.v[r][3][w] & 0xffff0000u);
      } else {
        t01 = (st.v[r][0][w] & 0xffffu) | (st.v[r][1][w] << 16);
        t23 = (st.v[r][2][w] & 0xffffu) | (st.v[r][3][w] << 16);
      }
      *reinterpret_cast<u32x2*>(vt + vt_off<D>(8 * dg + e, pos)) = u32x2{t01, t23};
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void varlen_kernel(VarlenArgs a) {
  constexpr int KS = D / 16;     // QK k-steps of 16 dims
  constexpr int DT = D / 32;     // O^T dim tiles
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps row math scalar
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int n = lane & 31, hh = lane >> 5;

  const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1];
  const int k0s = a.cu_k[b], k1s = a.cu_k[b + 1];
  const int len_q = q1 - q0, len_k = k1s - k0s;
  const bool cu_ok = q0 >= 0 && q1 >= q0 && q1 <= a.total_q && k0s >= 0 && k1s >= k0s &&
                     k1s <= a.total_k && (b != 0 || (q0 == 0 && k0s == 0)) &&
                     (b != a.batch - 1 || (q1 == a.total_q && k1s == a.total_k));
  const bool len_ok = len_q <= a.max_len_q && len_k <= a.max_len_k;
  if (!cu_ok || !len_ok) {
    if (a.err_flag && tid == 0 && qt == 0 && h == 0) atomicOr(a.err_flag, (int)(cu_ok ? kErrMaxLen : kErrCu));
    if (!(q0 >= 0 && q1 >= q0 && q1 <= a.total_q)) return;  // nowhere safe to write
    for (int r = qt * kRows + tid; r < min(len_q, (qt + 1) * kRows); r += 256) {
      __bf16* o = (__bf16*)a.out + ((long long)(q0 + r) * a.num_heads + h) * D;
      for (int d = 0; d < D; ++d) o[d] = (__bf16)__builtin_nanf("");
    }
    return;
  }
  if (qt * kRows >= len_q) return;

  const int kvh = h / a.group;
  const int tok_q = a.num_heads * D * 2;     // bytes between query rows
  const int tok_k = a.num_kv_heads * D * 2;  // bytes between key rows
  const char* kg = (const char*)a.k + (long long)k0s * tok_k + (long long)kvh * D * 2;
  const char* vg = (const char*)a.v + (long long)k0s * tok_k + (long long)kvh * D * 2;

  // this lane's query row as the B operand: dims 16s + 8hh + j
  const int row = qt * kRows + wave * kWaveRows + n;
  const bool row_ok = row < len_q;
  const bool wave_active = qt * kRows + wave * kWaveRows < len_q;
  u32x4 qr[KS];
  {
    const char* qp = (const char*)a.q + (long long)(q0 + (row_ok ? row : 0)) * tok_q + (long long)h * D * 2 + 16 * hh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qr[s] = row_ok ? *reinterpret_cast<const u32x4*>(qp + 32 * s) : z;
    }
  }

  f32x16 acc[DT];
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int nk = (len_k + kKeys - 1) / kKeys;
  Stage<D> st;
  if (nk > 0) {
    stage_load<D>(st, kg, vg, 0, len_k, tok_k, tid);
    stage_store<D>(st, smem, tid);
  }
  __syncthreads();
  for (int j = 0; j < nk; ++j) {
    char* cur = smem + (j & 1) * Lds<D>::BUF;
    if (j + 1 < nk) stage_load<D>(st, kg, vg, (j + 1) * kKeys, len_k, tok_k, tid);
    if (wave_active) {
      // S^T for two 32-key tiles
      f32x16 s[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
        const char* kp = cur + (32 * mt + n) * Lds<D>::KROW + 16 * hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(kp + 32 * ks);
          s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf),
                                                          __builtin_bit_cast(bf16x8, qr[ks]), s[mt], 0, 0, 0);
        }
      }
      // scale, mask the key tail, row max
      const int kbase = j * kKeys;
      float mt_max = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + 32 * mt + 8 * (r >> 2) + 4 * hh + (r & 3);
          float x = s[mt][r] * a.scale_log2;
          if (key >= len_k) x = -INFINITY;
          s[mt][r] = x;
          mt_max = fmaxf(mt_max, x);
        }
      mt_max = fmaxf(mt_max, swap32(mt_max));
      const float m_new = fmaxf(m_run, mt_max);
      const float alpha = fast_exp2(m_run - m_new);
      float psum = 0.f;
      u32 pw[2][8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(s[mt][r] - m_new), p1 = fast_exp2(s[mt][r + 1] - m_new);
          psum += p0 + p1;
          pw[mt][r >> 1] = pack_bf16x2(p0, p1);
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < DT; ++d) acc[d] *= alpha;
      // O^T += V^T P^T, 16 keys per step
      const char* vt = cur + Lds<D>::KBYTES;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int mt = kk >> 1, ap = kk & 1;
        const u32x4 pf = {pw[mt][4 * ap], pw[mt][4 * ap + 1], pw[mt][4 * ap + 2], pw[mt][4 * ap + 3]};
#pragma unroll
        for (int d = 0; d < DT; ++d) {
          const u32x4 vf = *reinterpret_cast<const u32x4*>(
              vt + vt_off<D>(32 * d + n, 32 * mt + 16 * ap + 8 * hh));
          acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, vf),
                                                           __builtin_bit_cast(bf16x8, pf), acc[d], 0, 0, 0);
        }
      }
    }
    if (j + 1 < nk) stage_store<D>(st, smem + ((j + 1) & 1) * Lds<D>::BUF, tid);
    __syncthreads();
  }

  if (!row_ok) return;
  float l_tot = l_run + swap32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  char* op = (char*)a.out + (long long)(q0 + row) * tok_q + (long long)h * D * 2;
#pragma unroll
  for (int d = 0; d < DT; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = 32 * d + 8 * g + 4 * hh;
      const u32x2 w = {pack_bf16x2(acc[d][4 * g] * inv, acc[d][4 * g + 1] * inv),
                       pack_bf16x2(acc[d][4 * g + 2] * inv, acc[d][4 * g + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + 2 * dim) = w;
    }
}

template <int D>
hipError_t launch_v(const VarlenArgs& a, hipStream_t stream) {
  const size_t lds = 2 * Lds<D>::BUF;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)varlen_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(varlen_kernel<D>, dim3(a.q_tiles, a.num_heads, a.batch), dim3(256), lds,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

int varlen_rows_per_workgroup() { return kRows; }

hipError_t launch_varlen(int dtype, int head_dim, const VarlenArgs& a, hipStream_t stream) {
  if (dtype != 1) return hipErrorInvalidValue;
  if (a.q_tiles == 0 || a.batch == 0) return hipSuccess;
  if (head_dim == 128) return launch_v<128>(a, stream);
  if (head_dim == 64) return launch_v<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
