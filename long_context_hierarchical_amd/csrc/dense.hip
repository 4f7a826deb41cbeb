// Dense softmax attention with standard RoPE at the original positions: the comparator the
// RecSA abstract ("Recursive Sparse Attention: Million-Token Length Extrapolation at
// Logarithmic Cost") times its method against, in prefill and in decoding.
//
// Two steps:
//   rotate_keys  keys rotated at their own positions once (a dense cache normally stores them
//                so): cos/sin of p * omega_i from the exact float64 product, rounded to float32,
//                separate multiply and add, rounded to the storage type.
//   attention    bf16: flash attention on MFMA (v_mfma_f32_32x32x16_bf16). A wave owns 32
//                (query, head) rows -- 32/G queries x the G heads of one KV head -- and the 4
//                waves of a workgroup share every K/V tile staged in LDS. Scores are computed
//                transposed, S^T = K Q~^T, so that each lane's probabilities are already in the
//                operand layout of O^T += V^T P^T; V is staged in LDS as stored (key-major) and
//                the V^T operand is read with gfx950's transposing LDS load. The online
//                softmax needs two lane exchanges per tile. Long key ranges are split across
//                workgroups and merged afterwards. float32 storage: a plain VALU kernel.
#include <math.h>

#include "common.hpp"
#include "rope.hpp"
#include "internal.hpp"

namespace recsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16: within each 16-lane block, lane l receives element l % 4 of the 8-byte
// chunks addressed by lanes l / 4, 4 + l / 4, 8 + l / 4, 12 + l / 4 of that block. When those
// lanes point at 4 consecutive rows of a row-major bf16 tile (lane 4j + c at row j, columns
// 4c .. 4c + 3), lane l gets column l of the 4 rows: the k-contiguous MFMA operand layout.
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
}

// ---------------------------------------------------------------- key rotation

template <int D, bool BF16>
__global__ __launch_bounds__(256) void rotate_keys_kernel(const void* K, int64_t cap, void* Kr, int64_t kr_rows,
                                                          int64_t p_lo, int64_t n, int64_t BH, InvFreq iv, int use_rope) {
  constexpr int HALF = D / 2, CPR = HALF / 8;
  const int64_t rows = n - p_lo;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= BH * rows * CPR) return;
  const int c = static_cast<int>(idx % CPR);
  const int64_t row = idx / CPR;
  const int64_t bh = row / rows, p = p_lo + row % rows;
  const int64_t src = (bh * cap + p) * D, dst = (bh * kr_rows + p) * D;
  float lo[8], hi[8], olo[8], ohi[8];
  load8<BF16>(K, src + 8 * c, lo);
  load8<BF16>(K, src + HALF + 8 * c, hi);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (use_rope) {
      float cs, sn;
      rope_cs(p, iv.w[8 * c + e], cs, sn);
      const float p1 = lo[e] * cs, p2 = hi[e] * sn, p3 = hi[e] * cs, p4 = lo[e] * sn;
      olo[e] = round_store<BF16>(p1 - p2);
      ohi[e] = round_store<BF16>(p3 + p4);
    } else {
      olo[e] = lo[e];
      ohi[e] = hi[e];
    }
  }
  store8<BF16>(Kr, dst + 8 * c, olo);
  store8<BF16>(Kr, dst + HALF + 8 * c, ohi);
}

hipError_t launch_rotate_keys(const void* K, int64_t cap, void* Kr, int64_t kr_rows, int64_t n, int64_t BH, int d,
                              bool bf16, const InvFreq& iv, int use_rope, hipStream_t s, int64_t p_lo) {
  if (n <= p_lo) return hipSuccess;
  const int64_t total = BH * (n - p_lo) * (d / 16);
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (d == 128) {
    if (bf16) hipLaunchKernelGGL((rotate_keys_kernel<128, true>), grid, dim3(256), 0, s, K, cap, Kr, kr_rows, p_lo, n, BH, iv, use_rope);
    else hipLaunchKernelGGL((rotate_keys_kernel<128, false>), grid, dim3(256), 0, s, K, cap, Kr, kr_rows, p_lo, n, BH, iv, use_rope);
  } else {
    if (bf16) hipLaunchKernelGGL((rotate_keys_kernel<64, true>), grid, dim3(256), 0, s, K, cap, Kr, kr_rows, p_lo, n, BH, iv, use_rope);
    else hipLaunchKernelGGL((rotate_keys_kernel<64, false>), grid, dim3(256), 0, s, K, cap, Kr, kr_rows, p_lo, n, BH, iv, use_rope);
  }
  return hipGetLastError();
}

// Queries rotated at their positions (causal: q_start + j; otherwise n_tokens), rounded to bf16:
// the same cos/sin, products, sums and rounding as the keys' rotation.
template <int D>
__global__ __launch_bounds__(256) void rotate_queries_kernel(const void* q, void* qr, int64_t rows, int32_t Hq,
                                                             int64_t n_q, int64_t q_start, int64_t n_tokens,
                                                             int32_t causal, InvFreq iv) {
  constexpr int HALF = D / 2, CPR = HALF / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= rows * CPR) return;
  const int c = static_cast<int>(idx % CPR);
  const int64_t row = idx / CPR;                  // (b * n_q + j) * Hq + head
  const int64_t j = (row / Hq) % n_q;
  const int64_t p = causal ? q_start + j : n_tokens;
  float lo[8], hi[8], olo[8], ohi[8];
  load8<true>(q, row * D + 8 * c, lo);
  load8<true>(q, row * D + HALF + 8 * c, hi);
#pragma unroll 1
  for (int e = 0; e < 8; ++e) {
    float cs, sn;
    rope_cs(p, iv.w[8 * c + e], cs, sn);
    const float p1 = lo[e] * cs, p2 = hi[e] * sn, p3 = hi[e] * cs, p4 = lo[e] * sn;
    olo[e] = round_store<true>(p1 - p2);
    ohi[e] = round_store<true>(p3 + p4);
  }
  store8<true>(qr, row * D + 8 * c, olo);
  store8<true>(qr, row * D + HALF + 8 * c, ohi);
}

hipError_t launch_rotate_queries(const DenseArgs& a, void* qr, int64_t B, int d, hipStream_t s) {
  const int64_t rows = B * a.n_q * a.Hq;
  if (rows <= 0) return hipSuccess;
  const int64_t total = rows * (d / 16);
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (d == 128)
    hipLaunchKernelGGL((rotate_queries_kernel<128>), grid, dim3(256), 0, s, a.q, qr, rows, a.Hq, a.n_q, a.q_start,
                       a.n_tokens, a.causal, a.iv);
  else
    hipLaunchKernelGGL((rotate_queries_kernel<64>), grid, dim3(256), 0, s, a.q, qr, rows, a.Hq, a.n_q, a.q_start,
                       a.n_tokens, a.causal, a.iv);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bf16 flash attention (MFMA)

template <int G>
struct DenseGeom {
  static constexpr int QPW = 32 / G;   // queries per wave
  static constexpr int QPB = 4 * QPW;  // queries per workgroup
};



__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// A wave owns 32 (query, head) rows: 32/G queries x the G heads of one KV head. Per 64-key tile:
// S^T = K Q~^T as two 32-key halves of D/16 v_mfma_f32_32x32x16_bf16 (A: 32 key rows x 16 dims
// from LDS; B: the rows' rotated queries, held in registers); lane l then holds 16 logits of row
// l % 32 per half, keys 8 (v / 4) + 4 (l / 32) + v % 4, and P^T's operand for O^T += V^T P^T is
// those values in order (k-slot 8 (l / 32) + e = key 16 ks + 8 (e / 4) + 4 (l / 32) + e % 4).
template <int D, int G>
__global__ __launch_bounds__(256) void dense_mfma_kernel(DenseArgs a) {
  constexpr int QPW = DenseGeom<G>::QPW, QPB = DenseGeom<G>::QPB;
  constexpr int KT = 64;               // keys per tile
  constexpr int KS = D / 16;           // MFMA k-steps over head_dim
  constexpr int DT = D / 32;           // 32-dim output tiles
  constexpr int KPAD = D + 8;          // K tile row stride (bf16): D/2 + 4 dwords
  // V tile row stride (bf16): D/2 + 16 dwords, an odd multiple of 16, so the 4 rows that the
  // 32 lanes of one transposing read touch fall in distinct banks
  constexpr int VPAD = D + 32;
  __shared__ __align__(16) uint16_t Ks[KT * KPAD];
  __shared__ __align__(16) uint16_t Vs[KT * VPAD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, r32 = lane & 31;
  const int64_t qb = blockIdx.x, bh = blockIdx.y, split = blockIdx.z;
  const int64_t b = bh / a.Hkv;
  const int h = static_cast<int>(bh % a.Hkv);

  const int64_t qi = qb * QPB + wave * QPW + r32 / G;
  const bool wave_active = qb * QPB + wave * QPW < a.n_q;   // uniform across the wave
  const int hh = r32 % G;
  const bool row_ok = qi < a.n_q;
  const int64_t pos = a.causal ? a.q_start + qi : a.n_tokens;
  const int64_t row_kmax = a.causal ? pos + 1 : a.n_tokens;
  const int64_t q_last = (qb * QPB + QPB < a.n_q ? qb * QPB + QPB : a.n_q) - 1;
  const int64_t kmax_blk = a.causal ? a.q_start + q_last + 1 : a.n_tokens;
  const int64_t k_lo = split * a.keys_per_split;
  const int64_t k_hi = k_lo + a.keys_per_split < kmax_blk ? k_lo + a.keys_per_split : kmax_blk;

  // rotated, bf16-rounded query fragments (B operand; the queries were rotated beforehand):
  // k-step m holds dims 16m + 8*hl + 0..7 of the lane's row
  bf16x8_t qf[KS];
  {
    const int64_t qoff = ((b * a.n_q + (row_ok ? qi : 0)) * a.Hq + static_cast<int64_t>(h) * G + hh) * D;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qoff + 16 * m + 8 * hl);
      qf[m] = row_ok ? as_bf16x8(u) : as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
    }
  }

  f32x16_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[t][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  // transposing-read addresses: 16-lane block bl reads keys 4*(bl >> 1) + (s >> 2) (+ 8 for the
  // upper 4 k-slots) and dims 16*(bl & 1) + 4*(s & 3) of each 32-dim tile, s = lane & 15
  const int bl = lane >> 4, sl = lane & 15;
  const int vrow = 4 * (bl >> 1) + (sl >> 2), vcol = 16 * (bl & 1) + 4 * (sl & 3);

  for (int64_t k0 = k_lo; k0 < k_hi; k0 += KT) {
    __syncthreads();
    for (int c = tid; c < KT * (D / 8); c += 256) {
      const int r = c / (D / 8), ch = c % (D / 8);
      const int64_t key = k0 + r;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < k_hi) {
        kv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.Kr) + (bh * a.kr_rows + key) * D + ch * 8);
        vv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.V) + (bh * a.v_rows + key) * D + ch * 8);
      }
      *reinterpret_cast<uint4*>(&Ks[r * KPAD + ch * 8]) = kv;
      *reinterpret_cast<uint4*>(&Vs[r * VPAD + ch * 8]) = vv;
    }
    __syncthreads();

    // the tile's two 32-key halves one after the other, each a step of the online softmax; a
    // wave that owns no query (few queries, as in decoding) only helps stage the tiles
#pragma unroll 1
    for (int kh = 0; kh < (wave_active ? 2 : 0); ++kh) {
      f32x16_t st;
#pragma unroll
      for (int v = 0; v < 16; ++v) st[v] = 0.0f;
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&Ks[(32 * kh + r32) * KPAD + 16 * m + 8 * hl]);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), qf[m], st, 0, 0, 0);
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t key = k0 + 32 * kh + 8 * (v >> 2) + 4 * hl + (v & 3);
        float x = st[v] * a.scale;
        if (!row_ok || key >= k_hi || key >= row_kmax) x = -INFINITY;
        st[v] = x;
        tmax = fmaxf(tmax, x);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = m_new == -INFINITY ? 1.0f : __expf(m_run - m_new);
      float lsum = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pr = st[v] == -INFINITY ? 0.0f : __expf(st[v] - m_new);
        st[v] = pr;
        lsum += pr;
      }
      lsum += __shfl_xor(lsum, 32);
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < DT; ++t) o[t] *= alpha;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(st[8 * ks + e]);
        const uint16_t* vr = &Vs[(32 * kh + 16 * ks + vrow) * VPAD + vcol];
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const i16x4_t lo = lds_read_tr16(vr + 32 * t);
          const i16x4_t hi = lds_read_tr16(vr + 8 * VPAD + 32 * t);
          const i16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va), pb, o[t], 0, 0, 0);
        }
      }
    }
  }

  // o[t][v] = O^T[dim 32t + 8(v/4) + 4*hl + v%4][row r32]
  if (!row_ok) return;
  if (a.n_splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* dst = a.out + ((b * a.n_q + qi) * a.Hq + static_cast<int64_t>(h) * G + hh) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(dst + 32 * t + 8 * g4 + 4 * hl) =
            make_float4(o[t][4 * g4] * inv, o[t][4 * g4 + 1] * inv, o[t][4 * g4 + 2] * inv, o[t][4 * g4 + 3] * inv);
    if (a.lse && hl == 0)
      a.lse[(b * a.n_q + qi) * a.Hq + static_cast<int64_t>(h) * G + hh] = l_run > 0.0f ? m_run + logf(l_run) : -INFINITY;
  } else {
    const int64_t rows = a.n_q * G;
    const int64_t prow = (split * gridDim.y + bh) * rows + qi * G + hh;
    float* dst = a.part_o + prow * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(dst + 32 * t + 8 * g4 + 4 * hl) =
            make_float4(o[t][4 * g4], o[t][4 * g4 + 1], o[t][4 * g4 + 2], o[t][4 * g4 + 3]);
    if (hl == 0) {
      a.part_ml[2 * prow] = m_run;
      a.part_ml[2 * prow + 1] = l_run;
    }
  }
}

// Few queries (decoding: every row of a KV head fits one 16-row wave): 16 (query, head) rows per
// wave on v_mfma_f32_16x16x32_bf16, which wastes less of each tile than the 32-row kernel when
// most rows are empty. Same data layout and results; the queries arrive rotated (use_rope = 0)
// or are rotated here.
template <int D, int G>
__global__ __launch_bounds__(256) void dense_mfma16_kernel(DenseArgs a) {
  constexpr int QPW = 16 / G, QPB = 4 * QPW;
  constexpr int KT = 64;               // keys per tile
  constexpr int KSTEPS = D / 32;       // MFMA k-steps over head_dim
  constexpr int DT = D / 16;           // 16-dim output tiles
  constexpr int HALF = D / 2;
  constexpr int KPAD = D + 8;          // K tile row stride (bf16)
  // V tile row stride (bf16): D/2 + 8 dwords, an odd multiple of 8, so the 8 rows that 32
  // lanes of a transposing read touch fall in distinct bank groups
  constexpr int VPAD = D + 16;
  __shared__ __align__(16) uint16_t Ks[KT * KPAD];
  __shared__ __align__(16) uint16_t Vs[KT * VPAD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, r16 = lane & 15;
  const int64_t qb = blockIdx.x, bh = blockIdx.y, split = blockIdx.z;
  const int64_t b = bh / a.Hkv;
  const int h = static_cast<int>(bh % a.Hkv);

  const int64_t qi = qb * QPB + wave * QPW + r16 / G;
  const int hh = r16 % G;
  const bool row_ok = qi < a.n_q;
  const int64_t pos = a.causal ? a.q_start + qi : a.n_tokens;
  const int64_t row_kmax = a.causal ? pos + 1 : a.n_tokens;
  const int64_t q_last = (qb * QPB + QPB < a.n_q ? qb * QPB + QPB : a.n_q) - 1;
  const int64_t kmax_blk = a.causal ? a.q_start + q_last + 1 : a.n_tokens;
  const int64_t k_lo = split * a.keys_per_split;
  const int64_t k_hi = k_lo + a.keys_per_split < kmax_blk ? k_lo + a.keys_per_split : kmax_blk;

  // rotated, bf16-rounded query fragments (B operand): dims 32m + 8*g4 + j
  bf16x8_t qf[KSTEPS];
  {
    float x[KSTEPS][8];
    const int64_t qoff = ((b * a.n_q + (row_ok ? qi : 0)) * a.Hq + static_cast<int64_t>(h) * G + hh) * D;
#pragma unroll
    for (int m = 0; m < KSTEPS; ++m) load8<true>(a.q, qoff + 32 * m + 8 * g4, x[m]);
    if (a.use_rope) {
#pragma unroll
      for (int m = 0; m < KSTEPS / 2; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float c, s;
          rope_cs(pos, a.iv.w[32 * m + 8 * g4 + j], c, s);
          const float x1 = x[m][j], x2 = x[m + KSTEPS / 2][j];
          const float p1 = x1 * c, p2 = x2 * s, p3 = x2 * c, p4 = x1 * s;
          x[m][j] = p1 - p2;
          x[m + KSTEPS / 2][j] = p3 + p4;
        }
    }
#pragma unroll
    for (int m = 0; m < KSTEPS; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[m][j] = static_cast<__bf16>(row_ok ? x[m][j] : 0.0f);
  }

  f32x4_t o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) o[t] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  // K/V tiles are double-buffered in registers: the next tile's rows are requested before this
  // tile is multiplied. Every key row is read by one workgroup only (one query per sequence), so
  // the loads carry the non-temporal hint.
  constexpr int LPT = KT * (D / 8) / 256;   // 16-byte pieces per thread per tile, for K and for V
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  u32x4v kn[LPT], vn[LPT];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int c = tid + 256 * u;
      const int r = c / (D / 8), ch = c % (D / 8);
      const int64_t key = k0 + r < k_hi ? k0 + r : k_hi - 1;   // rows past the range: zeroed when stored
      kn[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(
          static_cast<const uint16_t*>(a.Kr) + (bh * a.kr_rows + key) * D + ch * 8));
      vn[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(
          static_cast<const uint16_t*>(a.V) + (bh * a.v_rows + key) * D + ch * 8));
    }
  };
  if (k_lo < k_hi) fetch(k_lo);
  for (int64_t k0 = k_lo; k0 < k_hi; k0 += KT) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int c = tid + 256 * u;
      const int r = c / (D / 8), ch = c % (D / 8);
      const bool ok = k0 + r < k_hi;
      const u32x4v z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4v*>(&Ks[r * KPAD + ch * 8]) = ok ? kn[u] : z;
      *reinterpret_cast<u32x4v*>(&Vs[r * VPAD + ch * 8]) = ok ? vn[u] : z;
    }
    __syncthreads();
    if (k0 + KT < k_hi) fetch(k0 + KT);

    // S^T: 4 sub-tiles of 16 keys x 16 rows; lane holds keys 16*s4 + 4*g4 + i of row r16
    f32x4_t st[4];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      st[s4] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < KSTEPS; ++m) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&Ks[(16 * s4 + r16) * KPAD + 32 * m + 8 * g4]);
        st[s4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka), qf[m], st[s4], 0, 0, 0);
      }
    }
    float sv[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t key = k0 + 16 * s4 + 4 * g4 + i;
        float v = st[s4][i] * a.scale;
        if (!row_ok || key >= k_hi || key >= row_kmax) v = -INFINITY;
        sv[s4][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_new == -INFINITY ? 1.0f : __expf(m_run - m_new);
    float lsum = 0.0f;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = sv[s4][i] == -INFINITY ? 0.0f : __expf(sv[s4][i] - m_new);
        sv[s4][i] = p;
        lsum += p;
      }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] *= alpha;

    // O^T += V^T P^T over two 32-key blocks; the k-slot order (4*g4 + j, then 16 + 4*g4 + j)
    // is the order the S^T lanes already hold
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = static_cast<__bf16>(sv[2 * kb][i]);
        pb[4 + i] = static_cast<__bf16>(sv[2 * kb + 1][i]);
      }
      // this lane addresses key 32kb + 4*g4 + r16/4 (and 16 keys on), dims 16t + 4*(r16%4) + 0..3;
      // it receives dim 16t + r16 of keys 32kb + 4*g4 + 0..3 and 32kb + 16 + 4*g4 + 0..3
      const uint16_t* vr = &Vs[(32 * kb + 4 * g4 + (r16 >> 2)) * VPAD + 4 * (r16 & 3)];
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const i16x4_t lo = lds_read_tr16(vr + 16 * t);
        const i16x4_t hi = lds_read_tr16(vr + 16 * VPAD + 16 * t);
        const i16x8_t va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va), pb, o[t], 0, 0, 0);
      }
    }
  }

  // o[t][i] = O^T[dim 16t + 4*g4 + i][row r16]
  if (!row_ok) return;
  if (a.n_splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    float* dst = a.out + ((b * a.n_q + qi) * a.Hq + static_cast<int64_t>(h) * G + hh) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      *reinterpret_cast<float4*>(dst + 16 * t + 4 * g4) =
          make_float4(o[t][0] * inv, o[t][1] * inv, o[t][2] * inv, o[t][3] * inv);
    if (a.lse && g4 == 0)
      a.lse[(b * a.n_q + qi) * a.Hq + static_cast<int64_t>(h) * G + hh] = l_run > 0.0f ? m_run + logf(l_run) : -INFINITY;
  } else {
    const int64_t rows = a.n_q * G;
    const int64_t prow = (split * gridDim.y + bh) * rows + qi * G + hh;
    float* dst = a.part_o + prow * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      *reinterpret_cast<float4*>(dst + 16 * t + 4 * g4) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
    if (g4 == 0) {
      a.part_ml[2 * prow] = m_run;
      a.part_ml[2 * prow + 1] = l_run;
    }
  }
}

// merge split partials: one workgroup of D threads per (sequence x KV head, row)
template <int D, int G>
__global__ __launch_bounds__(D) void dense_merge_kernel(DenseArgs a) {
  const int64_t row = blockIdx.x;           // qi * G + hh
  const int64_t bh = blockIdx.y;
  const int64_t rows = a.n_q * G;
  const int64_t BHn = gridDim.y;
  const int dd = threadIdx.x;
  float m = -INFINITY;
  for (int sp = 0; sp < a.n_splits; ++sp) m = fmaxf(m, a.part_ml[2 * ((sp * BHn + bh) * rows + row)]);
  float l = 0.0f, acc = 0.0f;
  for (int sp = 0; sp < a.n_splits; ++sp) {
    const int64_t pr = (sp * BHn + bh) * rows + row;
    const float ms = a.part_ml[2 * pr];
    if (ms == -INFINITY) continue;
    const float w = __expf(ms - m);
    l += a.part_ml[2 * pr + 1] * w;
    acc += a.part_o[pr * D + dd] * w;
  }
  const int64_t b = bh / a.Hkv;
  const int h = static_cast<int>(bh % a.Hkv);
  const int64_t qi = row / G;
  const int hh = static_cast<int>(row % G);
  const int64_t orow = (b * a.n_q + qi) * a.Hq + static_cast<int64_t>(h) * G + hh;
  a.out[orow * D + dd] = l > 0.0f ? acc / l : 0.0f;
  if (a.lse && dd == 0) a.lse[orow] = l > 0.0f ? m + logf(l) : -INFINITY;
}

// ---------------------------------------------------------------- float32 storage: VALU

// One wave per (sequence, query, KV head); 64 keys per round, one key per lane.
template <int D, int G>
__global__ __launch_bounds__(64) void dense_valu_kernel(DenseArgs a) {
  constexpr int HALF = D / 2, DPL = D / 64;
  __shared__ float qs[G][D];
  __shared__ float ps[G][64];
  const int lane = threadIdx.x;
  const int64_t unit = blockIdx.x, b = blockIdx.y;
  const int64_t qi = unit / a.Hkv;
  const int h = static_cast<int>(unit % a.Hkv);
  const int64_t bh = b * a.Hkv + h;
  const int64_t pos = a.causal ? a.q_start + qi : a.n_tokens;
  const int64_t kmax = a.causal ? pos + 1 : a.n_tokens;
  const int64_t qoff = ((b * a.n_q + qi) * a.Hq + static_cast<int64_t>(h) * G) * D;
  for (int idx = lane; idx < G * HALF; idx += 64) {
    const int g = idx / HALF, i = idx % HALF;
    const float x1 = load1<false>(a.q, qoff + g * D + i), x2 = load1<false>(a.q, qoff + g * D + i + HALF);
    if (a.use_rope) {
      float c, s;
      rope_cs(pos, a.iv.w[i], c, s);
      const float p1 = x1 * c, p2 = x2 * s, p3 = x2 * c, p4 = x1 * s;
      qs[g][i] = p1 - p2;
      qs[g][i + HALF] = p3 + p4;
    } else {
      qs[g][i] = x1;
      qs[g][i + HALF] = x2;
    }
  }
  __syncthreads();
  float m_run[G], l_run[G], acc[G][DPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[g][e] = 0.0f;
  }
  const float* Kr = static_cast<const float*>(a.Kr);
  const float* V = static_cast<const float*>(a.V);
  for (int64_t k0 = 0; k0 < kmax; k0 += 64) {
    const int64_t key = k0 + lane;
    const bool ok = key < kmax;
    float z[G];
#pragma unroll
    for (int g = 0; g < G; ++g) z[g] = 0.0f;
    if (ok) {
      const float* kr = Kr + (bh * a.kr_rows + key) * D;
      for (int dd = 0; dd < D; ++dd) {
        const float kv = kr[dd];
#pragma unroll
        for (int g = 0; g < G; ++g) z[g] = fmaf(qs[g][dd], kv, z[g]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float zz = ok ? z[g] * a.scale : -INFINITY;
      const float mx = fmaxf(m_run[g], wave_max(zz));
      const float p = ok ? expf(zz - mx) : 0.0f;
      const float alpha = expf(m_run[g] - mx);
      l_run[g] = l_run[g] * alpha + wave_sum(p);
      m_run[g] = mx;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[g][e] *= alpha;
      ps[g][lane] = p;
    }
    __syncthreads();
    const int64_t kn = kmax - k0 < 64 ? kmax - k0 : 64;
    for (int j = 0; j < kn; ++j) {
      const float* vr = V + (bh * a.v_rows + k0 + j) * D + lane * DPL;
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float v = vr[e];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g][e] = fmaf(ps[g][j], v, acc[g][e]);
      }
    }
    __syncthreads();
  }
  const int64_t orow = (b * a.n_q + qi) * a.Hq + static_cast<int64_t>(h) * G;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) a.out[(orow + g) * D + lane * DPL + e] = l_run[g] > 0.0f ? acc[g][e] / l_run[g] : 0.0f;
    if (a.lse && lane == 0) a.lse[orow + g] = l_run[g] > 0.0f ? m_run[g] + logf(l_run[g]) : -INFINITY;
  }
}

// ---------------------------------------------------------------- launch

template <int D, int G>
static hipError_t launch_dense_bf16(const DenseArgs& a, int64_t B, hipStream_t s) {
  if (a.n_q * G <= 16) {
    const dim3 grid(1u, static_cast<unsigned>(B * a.Hkv), static_cast<unsigned>(a.n_splits));
    hipLaunchKernelGGL((dense_mfma16_kernel<D, G>), grid, dim3(256), 0, s, a);
  } else {
    constexpr int QPB = DenseGeom<G>::QPB;
    const dim3 grid(static_cast<unsigned>((a.n_q + QPB - 1) / QPB), static_cast<unsigned>(B * a.Hkv),
                    static_cast<unsigned>(a.n_splits));
    hipLaunchKernelGGL((dense_mfma_kernel<D, G>), grid, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  const dim3 mg(static_cast<unsigned>(a.n_q * G), static_cast<unsigned>(B * a.Hkv));
  hipLaunchKernelGGL((dense_merge_kernel<D, G>), mg, dim3(D), 0, s, a);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_dense_f32(const DenseArgs& a, int64_t B, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.n_q * a.Hkv), static_cast<unsigned>(B));
  hipLaunchKernelGGL((dense_valu_kernel<D, G>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dense_d(const DenseArgs& a, bool bf16, int G, int64_t B, hipStream_t s) {
  switch (G) {
    case 1: return bf16 ? launch_dense_bf16<D, 1>(a, B, s) : launch_dense_f32<D, 1>(a, B, s);
    case 2: return bf16 ? launch_dense_bf16<D, 2>(a, B, s) : launch_dense_f32<D, 2>(a, B, s);
    case 4: return bf16 ? launch_dense_bf16<D, 4>(a, B, s) : launch_dense_f32<D, 4>(a, B, s);
    case 8: return bf16 ? launch_dense_bf16<D, 8>(a, B, s) : launch_dense_f32<D, 8>(a, B, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dense(const DenseArgs& a, int d, bool bf16, int G, int64_t B, hipStream_t s) {
  if (a.n_q <= 0) return hipSuccess;
  if (d == 128) return launch_dense_d<128>(a, bf16, G, B, s);
  if (d == 64) return launch_dense_d<64>(a, bf16, G, B, s);
  return hipErrorInvalidValue;
}

}  // namespace recsa
