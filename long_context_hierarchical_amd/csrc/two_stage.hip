// Two-stage block-then-token selection over the RecSA cache: a coarse pass over blocks, then
// token selection inside the kept blocks, then attention over the kept tokens only -- the
// indexer summarised in "HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
// Attention", over the pooled block keys of "Recursive Sparse Attention: Million-Token Length
// Extrapolation at Logarithmic Cost" (abstract: one pooled key per node, RoPE positions as
// indices among a level's candidates).
//
// Stage 1 (ts_score_*): every complete block g < n1 is a candidate at index g and the query sits
// at n1, so the block keys rotated at their index do not depend on the query: they are rotated
// once, and stage 1 is a plain product of the rotated queries with them. bf16 runs it on MFMA
// (v_mfma_f32_32x32x16_bf16): a wave owns 32 (query, head) rows -- 32 / G queries -- as the A
// operand in registers and streams 32 block rows per step as the B operand straight from memory;
// each lane then holds 16 logits of one block, and the G heads of a query are G consecutive
// rows, i.e. consecutive accumulator values of the same lane, so the group score needs no lane
// exchange (two halves of the wave for G = 8). The scores of one slab of blocks stay in LDS and
// each query keeps the slab's best s1 blocks, written in ascending block order. float32 storage
// computes the same scores on the vector units.
//
// Stage 2, one workgroup per (query, KV head): ts_merge_kernel merges the slabs' lists into the s1
// kept blocks (every block of the global best s1 is in its slab's best s1); ts_token_kernel
// scores the kept blocks' tokens and the trailing tokens -- 16 lanes per row, rotated at the
// candidate index from the RoPE table, the query at C0 -- keeps the best s0, computes their
// logits again (holding only scores in LDS keeps more workgroups per CU) and runs one softmax
// over them.
//
// Selections (both stages): one wave finds the s-th largest of n ordered-bit scores with an
// 8-bit radix select over an LDS histogram, then emits the kept positions in ascending order
// (every score above the threshold, and the first ones equal to it), which is the order
// "score descending, index ascending" restricted to the kept set.
#include <math.h>

#include <atomic>

#include "common.hpp"
#include "rope.hpp"
#include "internal.hpp"
#include "lanes.hpp"

namespace recsa {

typedef __bf16 ts_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float ts_f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ ts_bf16x8_t ts_bf16x8(uint4 u) { return __builtin_bit_cast(ts_bf16x8_t, u); }

// ---------------------------------------------------------------- wave selection

// Given a 256-bin histogram of the keys that match the prefix so far, the bin holding the
// rem-th largest of them (counting from the top) and its rank inside that bin. Every lane of the
// wave returns the same pair.
__device__ __forceinline__ void radix_bin(const uint32_t* hist, int lane, int rem, int& digit, int& nrem) {
  const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
  const uint32_t tot = c0 + c1 + c2 + c3;
  uint32_t suf = tot;  // keys in bins >= 4 lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(suf, off);
    if (lane + off < 64) suf += o;
  }
  const uint32_t above = suf - tot;  // keys in bins > 4 lane + 3
  const uint32_t r = static_cast<uint32_t>(rem);
  const bool mine = above < r && r <= suf;
  int dg = 0, nr = 0;
  if (mine) {
    uint32_t cum = above;
    bool found = false;
    const uint32_t c[4] = {c0, c1, c2, c3};
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (!found && cum + c[b] >= r) {
        found = true;
        dg = 4 * lane + b;
        nr = static_cast<int>(r - cum);
      }
      cum += c[b];
    }
  }
  const uint64_t bal = __ballot(mine);
  const int src = static_cast<int>(__builtin_ctzll(bal));
  digit = __shfl(dg, src);
  nrem = __shfl(nr, src);
}

// The s-th largest of keys[0..n) (1 <= s < n) and how many keys equal to it are kept (tau,
// need_eq), by one wave: four passes of an 8-bit radix select. hist: 256 words of LDS used by
// this wave alone.
__device__ void wave_threshold(const uint32_t* keys, int n, int s, uint32_t* hist, int lane, uint32_t& tau,
                               int& need_eq) {
  uint32_t prefix = 0u, mask = 0u;
  int rem = s;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = lane; i < 256; i += 64) hist[i] = 0u;
    wave_sync();
#pragma unroll 4
    for (int i = lane; i < n; i += 64) {
      const uint32_t u = keys[i];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    wave_sync();
    int digit, nrem;
    radix_bin(hist, lane, rem, digit, nrem);
    prefix |= static_cast<uint32_t>(digit) << shift;
    mask |= 255u << shift;
    rem = nrem;
    wave_sync();
  }
  tau = prefix;
  need_eq = rem;
}

// The same with the whole 256-thread workgroup building each histogram; every wave then takes the
// same decision from it. Called by every thread of the workgroup.
__device__ void block_threshold(const uint32_t* keys, int n, int s, uint32_t* hist, int tid, uint32_t& tau,
                                int& need_eq) {
  uint32_t prefix = 0u, mask = 0u;
  int rem = s;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
#pragma unroll 4
    for (int i = tid; i < n; i += 256) {
      const uint32_t u = keys[i];
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    int digit, nrem;
    radix_bin(hist, tid & 63, rem, digit, nrem);
    prefix |= static_cast<uint32_t>(digit) << shift;
    mask |= 255u << shift;
    rem = nrem;
    __syncthreads();
  }
  tau = prefix;
  need_eq = rem;
}

// Emits (rank, position), in ascending position, for every key above tau and the first
// need_eq keys equal to it; returns how many were emitted.
template <typename F>
__device__ int wave_compact(const uint32_t* keys, int n, uint32_t tau, int need_eq, int lane, F emit) {
  int base = 0, eq_base = 0;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll 4
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const bool valid = i < n;
    const uint32_t u = valid ? keys[i] : 0u;
    const bool gt = valid && u > tau, eq = valid && u == tau;
    const uint64_t beq = __ballot(eq);
    const int er = eq_base + __popcll(beq & below);
    const bool take = gt || (eq && er < need_eq);
    const uint64_t bt = __ballot(take);
    if (take) emit(base + __popcll(bt & below), i);
    base += __popcll(bt);
    eq_base += __popcll(beq);
  }
  return base;
}

// ---------------------------------------------------------------- query rotation

template <int D, bool BF16>
__global__ __launch_bounds__(256) void ts_rotate_queries_kernel(const void* q, void* q1, void* q0, int64_t rows,
                                                                int64_t p1, int64_t p0, InvFreq iv, int use_rope) {
  constexpr int HALF = D / 2, CPR = HALF / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= 2 * rows * CPR) return;
  const bool second = idx >= rows * CPR;
  const int64_t k = second ? idx - rows * CPR : idx;
  const int c = static_cast<int>(k % CPR);
  const int64_t row = k / CPR;
  const int64_t p = second ? p0 : p1;
  void* dst = second ? q0 : q1;
  float lo[8], hi[8], olo[8], ohi[8];
  load8<BF16>(q, row * D + 8 * c, lo);
  load8<BF16>(q, row * D + HALF + 8 * c, hi);
#pragma unroll 1
  for (int e = 0; e < 8; ++e) {
    if (use_rope) {
      float cs, sn;
      rope_cs(p, iv.w[8 * c + e], cs, sn);
      const float a1 = lo[e] * cs, a2 = hi[e] * sn, a3 = hi[e] * cs, a4 = lo[e] * sn;
      olo[e] = round_store<BF16>(a1 - a2);
      ohi[e] = round_store<BF16>(a3 + a4);
    } else {
      olo[e] = lo[e];
      ohi[e] = hi[e];
    }
  }
  store8<BF16>(dst, row * D + 8 * c, olo);
  store8<BF16>(dst, row * D + HALF + 8 * c, ohi);
}

hipError_t launch_ts_rotate_queries(const void* q, void* q1, void* q0, int64_t rows, int64_t p1, int64_t p0, int d,
                                    bool bf16, const InvFreq& iv, int use_rope, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t total = 2 * rows * (d / 16);
  const dim3 grid(static_cast<unsigned>((total + 255) / 256));
  if (d == 128) {
    if (bf16) hipLaunchKernelGGL((ts_rotate_queries_kernel<128, true>), grid, dim3(256), 0, s, q, q1, q0, rows, p1, p0, iv, use_rope);
    else hipLaunchKernelGGL((ts_rotate_queries_kernel<128, false>), grid, dim3(256), 0, s, q, q1, q0, rows, p1, p0, iv, use_rope);
  } else {
    if (bf16) hipLaunchKernelGGL((ts_rotate_queries_kernel<64, true>), grid, dim3(256), 0, s, q, q1, q0, rows, p1, p0, iv, use_rope);
    else hipLaunchKernelGGL((ts_rotate_queries_kernel<64, false>), grid, dim3(256), 0, s, q, q1, q0, rows, p1, p0, iv, use_rope);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- stage 1: block scores

// Workgroup -> (slice, slab, query group). Consecutive workgroups are dispatched to different
// XCDs in turn; each XCD is given a contiguous range of the logical order (query group fastest),
// so the query groups that read one slab of block keys run on the same XCD, close in time, and
// share its L2.
struct TsTile {
  int64_t bh, slab, qg;
  bool live;
};
__device__ __forceinline__ TsTile ts_tile(const TsArgs& a, int RQ) {
  const int64_t nqg = (a.n_q + RQ - 1) / RQ;
  const int64_t total = a.BH * a.n_slabs * nqg;
  const int64_t per = (total + 7) / 8;
  const int64_t lin = blockIdx.x;
  const int64_t logical = (lin % 8) * per + lin / 8;
  TsTile t;
  t.live = logical < total;
  t.qg = logical % nqg;
  t.slab = (logical / nqg) % a.n_slabs;
  t.bh = logical / (nqg * a.n_slabs);
  return t;
}

// Each query row of the tile keeps its slab's best min(s1, nv) blocks: wave w handles rows
// w, w + 4, ... (ordered-bit scores Sl[row][0..nv)).
__device__ void ts_slab_select(const TsArgs& a, const TsTile& t, const uint32_t* Sl, int SB, int RQ, int nv,
                               uint32_t* hist, int wave, int lane) {
  const int64_t g_lo = t.slab * SB;
  const int s = a.s1 < nv ? a.s1 : nv;
  for (int rq = wave; rq < RQ; rq += 4) {
    const int64_t j = t.qg * RQ + rq;
    if (j >= a.n_q) break;
    const uint32_t* keys = Sl + rq * SB;
    uint2* dst = a.cand + ((t.bh * a.n_q + j) * a.n_slabs + t.slab) * static_cast<int64_t>(a.s1);
    if (s >= nv) {
      for (int i = lane; i < nv; i += 64) dst[i] = make_uint2(keys[i], static_cast<uint32_t>(g_lo + i));
    } else {
      uint32_t tau;
      int need_eq;
      wave_threshold(keys, nv, s, hist, lane, tau, need_eq);
      wave_compact(keys, nv, tau, need_eq, lane,
                   [&](int r, int i) {
                     if (r < s) dst[r] = make_uint2(keys[i], static_cast<uint32_t>(g_lo + i));
                   });
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(256) void ts_score_mfma_kernel(TsArgs a) {
  // TQ tiles of 32 (query, head) rows per wave: every block row loaded serves 32 TQ rows (one tile
  // keeps four workgroups on a CU, which hides the loads' latency better than a second tile saves)
  constexpr int TQ = 1, QT = 32 / G, RQ = TQ * QT, SB = ts_slab_blocks(G), KS = D / 16;
  __shared__ uint32_t Sl[RQ * SB];
  __shared__ uint32_t hist[4 * 256];
  const TsTile t = ts_tile(a, RQ);
  if (!t.live) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hl = lane >> 5, r32 = lane & 31;
  const int64_t b = t.bh / a.Hkv;
  const int h = static_cast<int>(t.bh % a.Hkv);

  // A operands: tile tq, row r32 = (query tq QT + r32 / G, head r32 % G); k-step m holds dims
  // 16 m + 8 hl + 0..7
  ts_bf16x8_t qf[TQ][KS];
#pragma unroll
  for (int tq = 0; tq < TQ; ++tq) {
    const int64_t j = t.qg * RQ + tq * QT + r32 / G;
    const bool row_ok = j < a.n_q;
    const int64_t qoff = ((b * a.n_q + (row_ok ? j : 0)) * a.Hq + static_cast<int64_t>(h) * G + r32 % G) * D;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q1) + qoff + 16 * m + 8 * hl);
      qf[tq][m] = ts_bf16x8(row_ok ? u : make_uint4(0u, 0u, 0u, 0u));
    }
  }
  const int64_t g_lo = t.slab * SB;
  const int nv = static_cast<int>(a.n1 - g_lo < SB ? a.n1 - g_lo : SB);
  const uint16_t* kbase = static_cast<const uint16_t*>(a.kb) + t.bh * a.kb_rows * D;
  // chunk c of 32 blocks goes to wave c % 4; the next chunk's key rows are loaded while this one
  // is multiplied (rows past the slab's end read its last row and are not stored)
  auto load_chunk = [&](int c, uint4 (&kr)[KS]) {
    const int gl = c * 32 + r32;
    const int64_t g = g_lo + (gl < nv ? gl : nv - 1);
#pragma unroll
    for (int m = 0; m < KS; ++m) kr[m] = *reinterpret_cast<const uint4*>(kbase + g * D + 16 * m + 8 * hl);
  };
  uint4 kr[KS], kn[KS];
  if (wave * 32 < nv) load_chunk(wave, kr);
  for (int c = wave; c * 32 < nv; c += 4) {
    const int gl = c * 32 + r32;                              // block within the slab
    if ((c + 4) * 32 < nv) load_chunk(c + 4, kn);
    ts_f32x16_t acc[TQ];
#pragma unroll
    for (int tq = 0; tq < TQ; ++tq)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[tq][v] = 0.0f;
#pragma unroll
    for (int m = 0; m < KS; ++m)
#pragma unroll
      for (int tq = 0; tq < TQ; ++tq)
        acc[tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[tq][m], ts_bf16x8(kr[m]), acc[tq], 0, 0, 0);
    // value v: row 8 (v / 4) + 4 hl + v % 4 of the tile, block gl; logit = fp32(scale * dot)
#pragma unroll
    for (int tq = 0; tq < TQ; ++tq) {
      if constexpr (G <= 4) {
#pragma unroll
        for (int v = 0; v < 16; v += G) {
          float sc = acc[tq][v] * a.scale;
#pragma unroll
          for (int u = 1; u < G; ++u) sc = sc + acc[tq][v + u] * a.scale;
          const int r = 8 * (v >> 2) + 4 * hl + (v & 3);
          if (gl < nv) Sl[(tq * QT + r / G) * SB + gl] = ordered_bits(sc);
        }
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float sc = acc[tq][4 * q4] * a.scale;
#pragma unroll
          for (int u = 1; u < 4; ++u) sc = sc + acc[tq][4 * q4 + u] * a.scale;
          sc = sc + __shfl_xor(sc, 32);                       // heads 4..7 live in the other half
          if (hl == 0 && gl < nv) Sl[(tq * QT + q4) * SB + gl] = ordered_bits(sc);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < KS; ++m) kr[m] = kn[m];
  }
  __syncthreads();
  ts_slab_select(a, t, Sl, SB, RQ, nv, hist + 256 * wave, wave, lane);
}

template <int D, int G>
__global__ __launch_bounds__(256) void ts_score_valu_kernel(TsArgs a) {
  constexpr int RQ = 32 / G, SB = ts_slab_blocks(G);
  __shared__ float qs[32 * D];
  __shared__ uint32_t Sl[RQ * SB];
  __shared__ uint32_t hist[4 * 256];
  const TsTile t = ts_tile(a, RQ);
  if (!t.live) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = t.bh / a.Hkv;
  const int h = static_cast<int>(t.bh % a.Hkv);
  for (int i = tid; i < 32 * D; i += 256) {
    const int r = i / D, e = i % D;
    const int64_t j = t.qg * RQ + r / G;
    qs[i] = j < a.n_q ? static_cast<const float*>(a.q1)[((b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G + r % G) * D + e]
                      : 0.0f;
  }
  __syncthreads();
  const int64_t g_lo = t.slab * SB;
  const int nv = static_cast<int>(a.n1 - g_lo < SB ? a.n1 - g_lo : SB);
  for (int c = wave; c * 64 < nv; c += 4) {
    const int gl = c * 64 + lane;
    const int64_t g = g_lo + (gl < nv ? gl : nv - 1);
    float acc[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) acc[r] = 0.0f;
    for (int e0 = 0; e0 < D; e0 += 8) {
      float x[8];
      load8<false>(a.kb, (t.bh * a.kb_rows + g) * D + e0, x);
#pragma unroll
      for (int r = 0; r < 32; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r] = fmaf(qs[r * D + e0 + e], x[e], acc[r]);
    }
#pragma unroll
    for (int rq = 0; rq < RQ; ++rq) {
      float sc = acc[rq * G] * a.scale;
#pragma unroll
      for (int u = 1; u < G; ++u) sc = sc + acc[rq * G + u] * a.scale;
      if (gl < nv) Sl[rq * SB + gl] = ordered_bits(sc);
    }
  }
  __syncthreads();
  ts_slab_select(a, t, Sl, SB, RQ, nv, hist + 256 * wave, wave, lane);
}

template <int D, int G>
static void ts_score_t(const TsArgs& a, bool bf16, hipStream_t s) {
  const int RQ = 32 / G;                   // queries per workgroup
  const int64_t total = a.BH * a.n_slabs * ((a.n_q + RQ - 1) / RQ);
  const dim3 grid(static_cast<unsigned>((total + 7) / 8 * 8));
  if (bf16) hipLaunchKernelGGL((ts_score_mfma_kernel<D, G>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ts_score_valu_kernel<D, G>), grid, dim3(256), 0, s, a);
}

hipError_t launch_ts_score(const TsArgs& a, int d, bool bf16, int G, hipStream_t s) {
  if (a.n_q <= 0 || a.n_slabs <= 0 || a.s1 <= 0) return hipSuccess;
#define TS_SCORE(DD, GG) \
  if (d == DD && G == GG) { ts_score_t<DD, GG>(a, bf16, s); return hipGetLastError(); }
  TS_SCORE(128, 1) TS_SCORE(128, 2) TS_SCORE(128, 4) TS_SCORE(128, 8)
  TS_SCORE(64, 1) TS_SCORE(64, 2) TS_SCORE(64, 4) TS_SCORE(64, 8)
#undef TS_SCORE
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- stage 2: tokens and softmax

// PPL consecutive storage elements -> float (PPL = 2 or 4).
template <bool BF16, int PPL>
__device__ __forceinline__ void ts_load(const void* base, int64_t off, float (&x)[PPL]) {
  if constexpr (PPL == 4) {
    if constexpr (BF16) {
      const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
      x[0] = __uint_as_float(u.x << 16);
      x[1] = __uint_as_float(u.x & 0xFFFF0000u);
      x[2] = __uint_as_float(u.y << 16);
      x[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
      x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
    }
  } else {
    loadN<BF16, 2>(base, off, x);
  }
}

// Merged list -> the s1 kept blocks, ascending: one workgroup per (query, KV head). Slab t holds
// its first min(s1, SB) entries at t s1 (the last slab possibly fewer), so merged entry x is entry
// x % c of slab x / c with c = min(s1, SB); every block of the global best s1 is in its slab's
// best s1, and the list is in ascending block order, so ties keep the lower block.
__global__ __launch_bounds__(256) void ts_merge_kernel(TsArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  uint32_t* mk = reinterpret_cast<uint32_t*>(lds);
  int32_t* mg = reinterpret_cast<int32_t*>(lds + ts_al16(static_cast<int64_t>(a.merge) * 4));
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds + 2 * ts_al16(static_cast<int64_t>(a.merge) * 4));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t j = blockIdx.x, bh = blockIdx.y;
  const uint2* src = a.cand + (bh * a.n_q + j) * a.n_slabs * static_cast<int64_t>(a.s1);
  int32_t* kept = a.kept + (bh * a.n_q + j) * static_cast<int64_t>(a.s1);
  const int c = a.s1 < a.SB ? a.s1 : a.SB;
  constexpr int MU = 8;   // all of a thread's loads issued before any is used
  for (int x0 = tid; x0 < a.merge; x0 += 256 * MU) {
    uint2 e[MU];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int x = x0 + 256 * u;
      const int xc = x < a.merge ? x : x0;
      e[u] = src[static_cast<int64_t>(xc / c) * a.s1 + xc % c];
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int x = x0 + 256 * u;
      if (x < a.merge) {
        mk[x] = e[u].x;
        mg[x] = static_cast<int32_t>(e[u].y);
      }
    }
  }
  __syncthreads();
  if (a.merge == a.s1) {
    for (int i = tid; i < a.s1; i += 256) kept[i] = mg[i];
  } else {
    uint32_t tau;
    int need_eq;
    block_threshold(mk, a.merge, a.s1, hist, tid, tau, need_eq);
    if (wave == 0)
      wave_compact(mk, a.merge, tau, need_eq, lane, [&](int r, int i) {
        if (r < a.s1) kept[r] = mg[i];
      });
  }
}

// One candidate row's logits: the row (token `row`, 16 lanes, PPL rotation pairs per lane) is
// rotated at its candidate index ic from the RoPE table and rounded to the storage type, then
// dotted with the lane's slice of the rotated query; z_h = fp32(scale * dot). bf16 rounds and
// packs element pairs with one conversion each and takes the dot products with v_dot2 (the
// rotated query is exact in bf16). Scoring and the kept rows' second pass both call this, so
// they produce the same bits.
template <int D, bool BF16, int G>
__device__ __forceinline__ void ts_row_logits(float (&lo)[D / 32], float (&hi)[D / 32], const float2* tab, int ic,
                                              int use_rope, int sub, const float (&qlo)[G][D / 32],
                                              const float (&qhi)[G][D / 32], float scale, float (&z)[G]) {
  constexpr int PPL = D / 32;
  float olo[PPL], ohi[PPL];
  if (use_rope) {
    // (cos, sin) pairs PPL sub .. PPL sub + PPL - 1 of position ic, two pairs per load
    const float4* t4 = reinterpret_cast<const float4*>(tab + static_cast<int64_t>(ic) * (D / 2) + PPL * sub);
#pragma unroll
    for (int p2 = 0; p2 < PPL / 2; ++p2) {
      const float4 cs = t4[p2];
      const float c2[2] = {cs.x, cs.z}, s2[2] = {cs.y, cs.w};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int p = 2 * p2 + e;
        const float a1 = lo[p] * c2[e], a2 = hi[p] * s2[e], a3 = hi[p] * c2[e], a4 = lo[p] * s2[e];
        olo[p] = a1 - a2;
        ohi[p] = a3 + a4;
      }
    }
  } else {
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      olo[p] = lo[p];
      ohi[p] = hi[p];
    }
  }
  if constexpr (BF16) {
    bf16x2_t kp[PPL];
#pragma unroll
    for (int u = 0; u < PPL / 2; ++u) {
      kp[u] = pack_bf16_rne(olo[2 * u], olo[2 * u + 1]);
      kp[PPL / 2 + u] = pack_bf16_rne(ohi[2 * u], ohi[2 * u + 1]);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float dot = 0.0f;
#pragma unroll
      for (int u = 0; u < PPL / 2; ++u) {
        dot = __builtin_amdgcn_fdot2_f32_bf16(kp[u], pack_bf16_rne(qlo[hh][2 * u], qlo[hh][2 * u + 1]), dot, false);
        dot = __builtin_amdgcn_fdot2_f32_bf16(kp[PPL / 2 + u], pack_bf16_rne(qhi[hh][2 * u], qhi[hh][2 * u + 1]), dot,
                                              false);
      }
      z[hh] = lane_group_sum<16>(dot) * scale;
    }
  } else {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float dot = 0.0f;
#pragma unroll
      for (int p = 0; p < PPL; ++p) {
        dot = fmaf(qlo[hh][p], olo[p], dot);
        dot = fmaf(qhi[hh][p], ohi[p], dot);
      }
      z[hh] = lane_group_sum<16>(dot) * scale;
    }
  }
}

template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void ts_token_kernel(TsArgs a) {
  extern __shared__ __align__(16) unsigned char lds[];
  const TsTokenLayout L = ts_token_layout(D, G, a.C0, a.s1, a.s0);
  uint32_t* keys = reinterpret_cast<uint32_t*>(lds + L.keys);
  float* red = reinterpret_cast<float*>(lds + L.red);
  int32_t* kb = reinterpret_cast<int32_t*>(lds + L.kb);
  int32_t* kp = reinterpret_cast<int32_t*>(lds + L.kp);
  float* zk = reinterpret_cast<float*>(lds + L.zk);
  float* qs = reinterpret_cast<float*>(lds + L.qs);
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds + L.hist);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t j = blockIdx.x, bh = blockIdx.y;
  const int64_t b = bh / a.Hkv;
  const int h = static_cast<int>(bh % a.Hkv);
  const int64_t unit = (b * a.n_q + j) * a.Hkv + h;        // row of the selection outputs
  const int64_t qrow = (b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G;

  // 1. the kept blocks (ascending) and the query rotated at C0
  if (a.s1 > 0) {
    const int32_t* kept = a.kept + (bh * a.n_q + j) * static_cast<int64_t>(a.s1);
    for (int i = tid; i < a.s1; i += 256) kb[i] = kept[i];
  }
  for (int i = tid; i < G * D; i += 256) qs[i] = load1<BF16>(a.q0, qrow * D + i);
  __syncthreads();
  if (a.sel_blocks)
    for (int i = tid; i < a.sel_bw; i += 256) a.sel_blocks[unit * a.sel_bw + i] = i < a.s1 ? kb[i] : -1;

  // 2. every token candidate's group score: the kept blocks' tokens, then the trailing ones, at
  // their index; RPI rows per 16-lane group in flight
  const int64_t tail0 = static_cast<int64_t>(a.f) * a.n1;
  const int sf = a.s1 * a.f;
  const int64_t kv = bh * a.cap * D;
  auto token_of = [&](int i) -> int64_t {
    return i < sf ? static_cast<int64_t>(kb[i / a.f]) * a.f + i % a.f : tail0 + (i - sf);
  };
  constexpr int PPL = D / 32;
  constexpr int RPI = 4;
  const int sub = lane & 15, grp = tid >> 4;
  float qlo[G][PPL], qhi[G][PPL];  // the lane's slice of the rotated query, for every row
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int p = 0; p < PPL; ++p) {
      qlo[hh][p] = qs[hh * D + PPL * sub + p];
      qhi[hh][p] = qs[hh * D + D / 2 + PPL * sub + p];
    }
  for (int i0 = 0; i0 < a.C0; i0 += 16 * RPI) {
    float lo[RPI][PPL], hi[RPI][PPL];
#pragma unroll
    for (int u = 0; u < RPI; ++u) {
      const int i = i0 + u * 16 + grp;
      const int64_t row = kv + token_of(i < a.C0 ? i : a.C0 - 1) * D;
      ts_load<BF16, PPL>(a.K, row + PPL * sub, lo[u]);
      ts_load<BF16, PPL>(a.K, row + D / 2 + PPL * sub, hi[u]);
    }
#pragma unroll
    for (int u = 0; u < RPI; ++u) {
      const int i = i0 + u * 16 + grp;
      float z[G];
      ts_row_logits<D, BF16, G>(lo[u], hi[u], a.tab, i < a.C0 ? i : a.C0 - 1, a.use_rope, sub, qlo, qhi, a.scale, z);
      float S = z[0];
#pragma unroll
      for (int hh = 1; hh < G; ++hh) S = S + z[hh];
      if (i < a.C0 && sub == 0) keys[i] = ordered_bits(S);
    }
  }
  __syncthreads();

  // 3. kept tokens, ascending
  if (a.s0 == a.C0) {
    for (int i = tid; i < a.C0; i += 256) kp[i] = i;
  } else if (a.s0 > 0) {
    uint32_t tau;
    int need_eq;
    block_threshold(keys, a.C0, a.s0, hist, tid, tau, need_eq);
    if (wave == 0)
      wave_compact(keys, a.C0, tau, need_eq, lane, [&](int r, int i) {
        if (r < a.s0) kp[r] = i;
      });
  }
  __syncthreads();

  // 4. the kept tokens' logits again (same arithmetic, same bits), then one softmax per head
  for (int r0 = 0; r0 < a.s0; r0 += 16 * RPI) {
    float lo[RPI][PPL], hi[RPI][PPL];
#pragma unroll
    for (int u = 0; u < RPI; ++u) {
      const int r = r0 + u * 16 + grp;
      const int64_t row = kv + token_of(kp[r < a.s0 ? r : a.s0 - 1]) * D;
      ts_load<BF16, PPL>(a.K, row + PPL * sub, lo[u]);
      ts_load<BF16, PPL>(a.K, row + D / 2 + PPL * sub, hi[u]);
    }
#pragma unroll
    for (int u = 0; u < RPI; ++u) {
      const int r = r0 + u * 16 + grp;
      float z[G];
      ts_row_logits<D, BF16, G>(lo[u], hi[u], a.tab, kp[r < a.s0 ? r : a.s0 - 1], a.use_rope, sub, qlo, qhi, a.scale, z);
      if (r < a.s0 && sub == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) zk[r * G + hh] = z[hh];
      }
    }
  }
  __syncthreads();
  constexpr int EPL = D / 64;
  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float mx = -INFINITY;
    for (int r = lane; r < a.s0; r += 64) mx = fmaxf(mx, zk[r * G + hh]);
    m[hh] = wave_max(mx);
    l[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.0f;
  }
  __syncthreads();   // every wave has its maxima before the logits become weights
  for (int x = tid; x < a.s0 * G; x += 256) {
    const int hh = x % G;
    float mh = m[0];
#pragma unroll
    for (int t = 1; t < G; ++t) mh = hh == t ? m[t] : mh;
    zk[x] = expf(zk[x] - mh);
  }
  __syncthreads();
  // wave w sums kept rows w, w + 4, ...: U rows per wave in flight
  constexpr int U = 8;
  for (int r0 = wave; r0 < a.s0; r0 += 4 * U) {
    float v[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + 4 * u;
      loadN<BF16, EPL>(a.V, kv + token_of(kp[r < a.s0 ? r : r0]) * D + EPL * lane, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + 4 * u;
      if (r < a.s0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = zk[r * G + hh];
          l[hh] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[hh][e] = fmaf(p, v[u][e], acc[hh][e]);
        }
      }
    }
  }
  // the partial outputs take the place of the (no longer needed) scores
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) red[(wave * G + hh) * D + EPL * lane + e] = acc[hh][e];
  float* lsum = reinterpret_cast<float*>(hist);   // the selection is done with the histogram
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) lsum[wave * G + hh] = l[hh];
  }
  __syncthreads();
  for (int o = tid; o < G * D; o += 256) {
    const int hh = o / D, e = o % D;
    const float den = (lsum[hh] + lsum[G + hh]) + (lsum[2 * G + hh] + lsum[3 * G + hh]);
    const float num = (red[hh * D + e] + red[(G + hh) * D + e]) + (red[(2 * G + hh) * D + e] + red[(3 * G + hh) * D + e]);
    a.out[qrow * D + o] = a.s0 > 0 ? num / den : 0.0f;
  }
  if (a.lse && tid < G) {
    const int hh = tid;
    const float den = (lsum[hh] + lsum[G + hh]) + (lsum[2 * G + hh] + lsum[3 * G + hh]);
    a.lse[qrow + hh] = a.s0 > 0 ? m[hh] + logf(den) : -INFINITY;
  }
  if (a.sel_tokens)
    for (int i = tid; i < a.sel_tw; i += 256)
      a.sel_tokens[unit * a.sel_tw + i] = i < a.s0 ? static_cast<int32_t>(token_of(kp[i])) : -1;
}

template <int D, int G>
static void ts_tokens_t(const TsArgs& a, bool bf16, size_t lds, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.n_q), static_cast<unsigned>(a.BH));
  if (bf16) hipLaunchKernelGGL((ts_token_kernel<D, true, G>), grid, dim3(256), lds, s, a);
  else hipLaunchKernelGGL((ts_token_kernel<D, false, G>), grid, dim3(256), lds, s, a);
}



hipError_t launch_ts_merge(const TsArgs& a, hipStream_t s) {
  if (a.n_q <= 0 || a.s1 <= 0) return hipSuccess;
  const size_t lds = ts_merge_lds_bytes(a.merge);
  // long lists (many slabs) use up to gfx950's 160 KB of LDS per workgroup; the kernel's limit is
  // raised on each device (the attribute belongs to the current device) to the largest size asked
  // for so far there
  constexpr int kDevices = 64;
  static std::atomic<size_t> allowed[kDevices];   // 0: never raised (64 KB)
  if (lds > 65536) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::atomic<size_t>* lim = dev >= 0 && dev < kDevices ? &allowed[dev] : nullptr;
    if (lim == nullptr || lds > lim->load()) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ts_merge_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
      if (lim != nullptr) {
        size_t cur = lim->load();
        while (lds > cur && !lim->compare_exchange_weak(cur, lds)) {
        }
      }
    }
  }
  const dim3 grid(static_cast<unsigned>(a.n_q), static_cast<unsigned>(a.BH));
  hipLaunchKernelGGL(ts_merge_kernel, grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_ts_tokens(const TsArgs& a, int d, bool bf16, int G, size_t lds, int64_t B, hipStream_t s) {
  (void)B;
  if (a.n_q <= 0) return hipSuccess;
#define TS_TOK(DD, GG) \
  if (d == DD && G == GG) { ts_tokens_t<DD, GG>(a, bf16, lds, s); return hipGetLastError(); }
  TS_TOK(128, 1) TS_TOK(128, 2) TS_TOK(128, 4) TS_TOK(128, 8)
  TS_TOK(64, 1) TS_TOK(64, 2) TS_TOK(64, 4) TS_TOK(64, 8)
#undef TS_TOK
  return hipErrorInvalidValue;
}

}  // namespace recsa
