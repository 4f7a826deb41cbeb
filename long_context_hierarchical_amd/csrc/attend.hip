// RecSA descent + one softmax: one wave (64 lanes) per (sequence, query, KV head).
//
// Method: "Recursive Sparse Attention: Million-Token Length Extrapolation at
// Logarithmic Cost", abstract. Per tree level only k candidates survive, which
// bounds the rows a query touches by a multiple of the tree height; the RoPE
// position of a row is its rank in its level's candidate list, not its token
// position; rows a query drops are not discarded but enter the same softmax,
// as their node's mean value, next to the token rows it reaches. The explainer
// page ("Recursive Sparse Attention RecSA: Million-Token Context Extrapolation
// at Logarithmic Cost", section "Core Idea") describes the same descent: coarse
// filtering near the root, refinement level by level down to the tokens.
//
// Per level (top to bottom):
//   candidates  children of the nodes kept one level up (ascending), then the
//               nodes without a complete parent; at the top every node.
//   score       each candidate key rotated at its index i and rounded to the
//               storage type; the query heads rotated at C and rounded; the
//               logit z = scale * <q~, k~> per head (float32, any order), the
//               group score S = sum over the G heads of the KV group.
//   select      the s = min(k, C) largest (S, -i) keys: the s-th largest score by
//               bisection on its order-preserving bits (ballot counts), then the
//               scores above it and, lowest index first, those equal to it
//               (exact, deterministic).
//   softmax     unkept candidates join the online softmax with their node's
//               mean value; kept ones become the next level's parents.
// Token level: the tokens under the kept level-1 nodes plus the trailing
// partial block, all entries; the query sits at C_0, or C_0 - 1 when its own
// token is one of them (causal prefill).
//
// A unit is a dependent chain of T + 1 rounds, so the kernel runs one wave per
// unit with no workgroup barrier and lets many independent units share a CU;
// calls with few units give each unit four waves instead (same arithmetic).
// Lane layout: in the score phase D/16 lanes per candidate row, a lane holding
// elements [8s, 8s+8) and their rotate-half partners [D/2 + 8s, ...), so the
// rotation needs no lane exchange and the per-row reduction is 3 (d=128) DPP
// steps; bf16 operands are rounded and packed by v_cvt_pk_bf16_f32 and dotted
// by v_dot2 (the G query heads share each loaded row; their rotated operands
// sit in LDS). Each chunk of candidates first gets a candidate -> row table in
// LDS, read by the row loads, the selection and the value phase. Row loads are
// double-buffered and never behind a branch, so the next pass's rows stay in
// flight while the current one is computed. In the value phase D/4 lanes per
// row, a lane holding elements [4s, 4s+4), 8 rows per pass. The kernel is held
// to 128 VGPRs (4 waves per SIMD) for groups of up to 4 query heads.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "lanes.hpp"

namespace recsa {

// 4 consecutive storage elements -> float.
template <bool BF16>
__device__ __forceinline__ void load4(const void* base, int64_t off, float (&x)[4]) {
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
}

typedef __bf16 mf_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float mf_f32x16_t __attribute__((ext_vector_type(16)));
typedef short mv_i16x4_t __attribute__((ext_vector_type(4)));
typedef short mv_i16x8_t __attribute__((ext_vector_type(8)));
typedef float mv_f32x4_t __attribute__((ext_vector_type(4)));

// The value pass on the matrix cores (bf16 storage, G >= 2). O[h][c] += sum over 4 candidate rows
// of P[h][r] V[r][c] is two v_mfma_f32_4x4x4_16b_bf16 per 64 value columns and 4 query heads: their
// 16 blocks (block b = lane / 4) each take 4 columns and all of them the same 4 x 4 block of
// weights. Lane l supplies the weights of head l % 4 for the 4 rows (A) and one column of the 64
// for the same rows (B), and receives O[4 heads][that column] in its 4 accumulators. With one wave
// a lane loads its columns of each row itself (2 lane and 2 lane + 1 at D = 128, lane at D = 64);
// with several waves the rows sit in LDS and a transposing read gives lane l column l. A weight p
// enters as two bf16 terms, hi = bf16(p) and lo = bf16(p - hi) (p - hi is exact in float32), one
// product each: the weight is held to 2^-17 of itself instead of bf16's 2^-9, and the sums stay
// float32. The matrix core forms each output element from its row of A and its column of B alone,
// and every launch shape runs the same sequence of products for an element -- the candidates'
// 4-row quads in ascending order up to the next multiple of 16 rows (hi, then lo), the rows past
// the last candidate and the kept ones with weight 0 -- so results do not depend on the launch.
__device__ __forceinline__ mv_i16x4_t mv_read_tr(const uint16_t* p) {
  // within each 16 lanes, lane 4j + c addresses row j of 4 at its columns 4c .. 4c + 3 and lane l
  // receives column l of the 4 rows (gfx950's ds_read_b64_tr_b16)
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) mv_i16x4_t*)(p));
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return static_cast<uint16_t>(__builtin_bit_cast(uint32_t, pack_bf16_rne(x, 0.0f)) & 0xFFFFu);
}

// orders the surrounding LDS accesses for the compiler (a wave's LDS accesses execute in order)
__device__ __forceinline__ void lds_order() { __asm__ volatile("" ::: "memory"); }

// Candidate index -> node (or token) id: children of the kept parents, then orphans.
// Ids and indices fit in 32 bits (the capacity is at most INT32_MAX); a power-of-two
// fanout splits an index with a shift and a mask.
struct CandMap {
  const int32_t* parents;
  int32_t n_kids;   // f * (number of kept parents)
  int32_t orph;     // first orphan id
  int32_t f;
  int32_t fshift;   // log2(f) when f is a power of two, else -1
  __device__ __forceinline__ int32_t operator()(int32_t i) const {
    if (i >= n_kids) return orph + (i - n_kids);
    int32_t p, c;
    if (fshift >= 0) {
      p = i >> fshift;
      c = i & (f - 1);
    } else {
      p = i / f;
      c = i - p * f;
    }
    return f * parents[p] + c;
  }
};

// One row fragment of 8 storage elements, as loaded (converted later).
template <bool BF16>
struct Raw8 {
  uint4 u[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> raw8_load(const void* base, int64_t off) {
  Raw8<BF16> r;
  if constexpr (BF16) {
    r.u[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + off);
    r.u[0] = p[0];
    r.u[1] = p[1];
  }
  return r;
}

// The same from a wave-uniform byte base and a 32-bit byte offset (the host keeps every slice of
// the caches, the tree and the RoPE table under 4 GiB), so that the load takes its base from
// scalar registers and one 32-bit add per address.
template <bool BF16>
__device__ __forceinline__ Raw8<BF16> raw8_load32(const char* base, uint32_t boff) {
  Raw8<BF16> r;
  const uint4* p = reinterpret_cast<const uint4*>(base + boff);
  r.u[0] = p[0];
  if constexpr (!BF16) r.u[1] = p[1];
  return r;
}

template <bool BF16>
__device__ __forceinline__ Raw8<BF16> raw8_zero() {
  Raw8<BF16> r;
#pragma unroll
  for (int i = 0; i < (BF16 ? 1 : 2); ++i) r.u[i] = make_uint4(0u, 0u, 0u, 0u);
  return r;
}

template <bool BF16>
__device__ __forceinline__ void raw8_cvt(const Raw8<BF16>& r, float (&x)[8]) {
  if constexpr (BF16) {
    const uint32_t w[4] = {r.u[0].x, r.u[0].y, r.u[0].z, r.u[0].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      x[4 * k] = __uint_as_float(r.u[k].x);
      x[4 * k + 1] = __uint_as_float(r.u[k].y);
      x[4 * k + 2] = __uint_as_float(r.u[k].z);
      x[4 * k + 3] = __uint_as_float(r.u[k].w);
    }
  }
}

// One row fragment of 4 storage elements, as loaded (converted later).
template <bool BF16>
struct Raw4 {
  typename std::conditional<BF16, uint2, uint4>::type u;
};

template <bool BF16>
__device__ __forceinline__ Raw4<BF16> raw4_load(const void* base, int64_t off) {
  Raw4<BF16> r;
  if constexpr (BF16) {
    r.u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
  } else {
    r.u = *reinterpret_cast<const uint4*>(static_cast<const float*>(base) + off);
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ Raw4<BF16> raw4_zero() {
  Raw4<BF16> r;
  if constexpr (BF16) {
    r.u = make_uint2(0u, 0u);
  } else {
    r.u = make_uint4(0u, 0u, 0u, 0u);
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ void raw4_cvt(const Raw4<BF16>& r, float (&x)[4]) {
  if constexpr (BF16) {
    x[0] = __uint_as_float(r.u.x << 16);
    x[1] = __uint_as_float(r.u.x & 0xFFFF0000u);
    x[2] = __uint_as_float(r.u.y << 16);
    x[3] = __uint_as_float(r.u.y & 0xFFFF0000u);
  } else {
    x[0] = __uint_as_float(r.u.x);
    x[1] = __uint_as_float(r.u.y);
    x[2] = __uint_as_float(r.u.z);
    x[3] = __uint_as_float(r.u.w);
  }
}

// One value-row fragment of N (1, 2 or 4) storage elements, as loaded.
template <bool BF16, int N>
struct RawV {
  using T = typename std::conditional<
      BF16, typename std::conditional<N == 4, uint2, typename std::conditional<N == 2, uint32_t, uint16_t>::type>::type,
      typename std::conditional<N == 4, uint4, typename std::conditional<N == 2, uint2, uint32_t>::type>::type>::type;
  T u;
  __device__ __forceinline__ void load(const void* base, int64_t off) {
    if constexpr (BF16) u = *reinterpret_cast<const T*>(static_cast<const uint16_t*>(base) + off);
    else u = *reinterpret_cast<const T*>(static_cast<const float*>(base) + off);
  }
  __device__ __forceinline__ void zero() { u = T{}; }
  __device__ __forceinline__ void cvt(float (&x)[N]) const {
    if constexpr (BF16) {
      if constexpr (N == 4) {
        x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xFFFF0000u);
        x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xFFFF0000u);
      } else if constexpr (N == 2) {
        x[0] = __uint_as_float(u << 16); x[1] = __uint_as_float(u & 0xFFFF0000u);
      } else {
        x[0] = __uint_as_float(static_cast<uint32_t>(u) << 16);
      }
    } else {
      if constexpr (N == 4) {
        x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y); x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
      } else if constexpr (N == 2) {
        x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
      } else {
        x[0] = __uint_as_float(u);
      }
    }
  }
};


// The first scored level on the matrix cores (bf16 storage). A unit's first scored level holds all
// n_l nodes of that level at their own index (every level above keeps all its nodes), so the units
// of a workgroup whose first scored level is the same share its rotated keys: one tile
// S = Q~ K~^T per 32 candidates on v_mfma_f32_32x32x16_bf16, the 32 rows being the units' query
// heads rotated at their n_l (G rows per unit, zero rows past them) and the 32 columns 32
// consecutive nodes rotated at their index. scale * S lands in each unit's logit array ([C][G]).
// Every call path that scores this level (one wave per unit, several waves per unit, the decoding
// step) takes its logits from this code, and the matrix core forms each output element from its
// row and its column alone, so a unit's logits do not depend on which units share its workgroup.
//
// k-order: lane l supplies row (A) or column (B) l % 32 and the 8 elements of half kh = l / 32 of
// each 16-wide k-step. Step m < D/32 takes the rotate-half "lo" elements QH kh + 8m + e (QH = D/4,
// e < 8), step D/32 + m their partners HALF + QH kh + 8m + e: a lane rotates its own pairs in
// registers (no lane exchange), and the D/16 steps take every element once.
template <int D, int G>
__device__ void mf_shared_levels(const AttnArgs& a, unsigned char* lds_all, const Lds& L, int slots, int slot, int ls,
                                 int32_t cs, const float* qs, uint16_t* mstage, int64_t bh, int tid, int NT) {
  constexpr int HALF = D / 2, QH = D / 4, MS = D / 32;
  const int lane = static_cast<int>(threadIdx.x) % kWave, r32 = lane & 31, kh = lane >> 5;
  const int nwaves = static_cast<int>(blockDim.x) / kWave, gw = static_cast<int>(threadIdx.x) / kWave;
  auto info_of = [&](int s) { return reinterpret_cast<const int32_t*>(lds_all + s * L.total + L.info); };
  int lv_hi = RECSA_MAX_LEVELS + 1;
  for (;;) {
    // the next (lower) first-scored level among the workgroup's units, and its largest node count
    int L0 = 0;
    int32_t cmax = 0;
    for (int s = 0; s < slots; ++s) {
      const int l = info_of(s)[0];
      if (l < lv_hi && l > L0) L0 = l;
    }
    if (L0 == 0) break;
    for (int s = 0; s < slots; ++s)
      if (info_of(s)[0] == L0 && info_of(s)[1] > cmax) cmax = info_of(s)[1];
    // this unit's G rows: its query heads rotated at its node count and rounded to bf16 (the
    // rotation of the per-unit scoring, element for element); zeros when its level is another one
    const bool mine = ls == L0;
    for (int i = tid; i < G * HALF; i += NT) {
      const int hh = i / HALF, p = i % HALF;
      const float ql = qs[hh * D + p], qh = qs[hh * D + HALF + p];
      float lo = 0.0f, hi = 0.0f;
      if (mine) {
        if (a.use_rope) {
          const float2 t = a.tab[static_cast<int64_t>(cs) * HALF + p];
          const float p1 = ql * t.x, p2 = qh * t.y;
          const float p3 = qh * t.x, p4 = ql * t.y;
          lo = p1 - p2;
          hi = p3 + p4;
        } else {
          lo = ql;
          hi = qh;
        }
      }
      const uint32_t wd = __builtin_bit_cast(uint32_t, pack_bf16_rne(lo, hi));
      uint16_t* row = mstage + (slot * G + hh) * D;
      row[p] = static_cast<uint16_t>(wd & 0xFFFFu);
      row[HALF + p] = static_cast<uint16_t>(wd >> 16);
    }
    for (int i = static_cast<int>(threadIdx.x); i < (32 - slots * G) * D / 8; i += static_cast<int>(blockDim.x))
      reinterpret_cast<uint4*>(mstage + slots * G * D)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const uint16_t* arow = mstage + r32 * D + QH * kh;   // this lane's A fragments, read per k-step
    const int64_t rowbase = bh * a.tree.rows[L0];
    const uint16_t* src = static_cast<const uint16_t*>(a.tree.NK[L0]);
    for (int cb = gw; cb * 32 < cmax; cb += nwaves) {
      const int32_t c = cb * 32 + r32;
      const int64_t cr = c < cmax ? c : cmax - 1;   // a column past the last node loads the last one
      mf_f32x16_t acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        const uint16_t* rp = src + (rowbase + cr) * D + QH * kh + 8 * m;
        const uint4 ulo = *reinterpret_cast<const uint4*>(rp);
        const uint4 uhi = *reinterpret_cast<const uint4*>(rp + HALF);
        const uint32_t wl[4] = {ulo.x, ulo.y, ulo.z, ulo.w}, wh[4] = {uhi.x, uhi.y, uhi.z, uhi.w};
        float klo[8], khi[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          klo[2 * q] = __uint_as_float(wl[q] << 16);
          klo[2 * q + 1] = __uint_as_float(wl[q] & 0xFFFF0000u);
          khi[2 * q] = __uint_as_float(wh[q] << 16);
          khi[2 * q + 1] = __uint_as_float(wh[q] & 0xFFFF0000u);
        }
        float olo[8], ohi[8];
        if (a.use_rope) {
          const float4* t = reinterpret_cast<const float4*>(a.tab + cr * HALF + QH * kh + 8 * m);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 tv = t[q];
            const float cc[2] = {tv.x, tv.z}, ss[2] = {tv.y, tv.w};
#pragma unroll
            for (int v = 0; v < 2; ++v) {
              const int e = 2 * q + v;
              const float p1 = klo[e] * cc[v], p2 = khi[e] * ss[v];
              const float p3 = khi[e] * cc[v], p4 = klo[e] * ss[v];
              olo[e] = p1 - p2;
              ohi[e] = p3 + p4;
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            olo[e] = klo[e];
            ohi[e] = khi[e];
          }
        }
        uint4 bl, bhv;
        bl.x = __builtin_bit_cast(uint32_t, pack_bf16_rne(olo[0], olo[1]));
        bl.y = __builtin_bit_cast(uint32_t, pack_bf16_rne(olo[2], olo[3]));
        bl.z = __builtin_bit_cast(uint32_t, pack_bf16_rne(olo[4], olo[5]));
        bl.w = __builtin_bit_cast(uint32_t, pack_bf16_rne(olo[6], olo[7]));
        bhv.x = __builtin_bit_cast(uint32_t, pack_bf16_rne(ohi[0], ohi[1]));
        bhv.y = __builtin_bit_cast(uint32_t, pack_bf16_rne(ohi[2], ohi[3]));
        bhv.z = __builtin_bit_cast(uint32_t, pack_bf16_rne(ohi[4], ohi[5]));
        bhv.w = __builtin_bit_cast(uint32_t, pack_bf16_rne(ohi[6], ohi[7]));
        const mf_bf16x8_t alo = __builtin_bit_cast(mf_bf16x8_t, *reinterpret_cast<const uint4*>(arow + 8 * m));
        const mf_bf16x8_t ahi = __builtin_bit_cast(mf_bf16x8_t, *reinterpret_cast<const uint4*>(arow + HALF + 8 * m));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, __builtin_bit_cast(mf_bf16x8_t, bl), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, __builtin_bit_cast(mf_bf16x8_t, bhv), acc, 0, 0, 0);
      }
      // lane l holds column c and rows 8 (v / 4) + 4 kh + v % 4 of the tile
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + 4 * kh + (v & 3);
        const int s = r / G, hh = r % G;
        if (s < slots) {
          const int32_t* in = info_of(s);
          if (in[0] == L0 && c < in[1]) {
            float* zs = reinterpret_cast<float*>(lds_all + s * L.total + L.zs);
            zs[c * G + hh] = acc[v] * a.scale;
          }
        }
      }
    }
    __syncthreads();
    lv_hi = L0;
  }
}

// NW waves per unit. NW = 1: one wave does everything. NW > 1 (few units, latency-bound):
// the waves share the score passes, wave 0 alone selects, wave h mod NW computes query head
// h's softmax weights, and each wave owns D / NW of the value dimensions with the same row-group accumulation
// chains as one wave, so every output element is accumulated in exactly the same order and
// the results are bitwise those of NW = 1. When the launcher grants the LDS (pv_stage), the
// value rows of a softmax chunk are staged through LDS by all threads with 16-byte loads
// (the first round is in flight during wave 0's weight pass, each next one during the
// current round's accumulation), and a lane reads its chain's rows 8 at a time without a
// branch (a kept row has weight 0, and adding 0 * v leaves the sum unchanged). Occupancy
// does not matter with so few units, so these kernels may take up to 256 registers.
template <int D, bool BF16, int G, int NW>
__global__ __launch_bounds__(NW == 1 && BF16 ? 512 : 64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 1 && G <= 4 ? 4 : 2))) void attend_kernel(AttnArgs args) {
  // read the arguments in place: the per-level tables are indexed by a run-time level, and a
  // by-value copy of the struct would be placed in scratch memory
  (void)args;
  const AttnArgs& a = *(const AttnArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  constexpr int VE = 4;                // elements per row group lane (one wave), value phase
  constexpr int VEW = VE / NW > 0 ? VE / NW : 1;   // elements per lane of each wave (fmaf value path)
  constexpr int RL = D / VE;           // lanes per row, value phase
  constexpr int RPP = kWave / RL;      // rows per pass, value phase
  constexpr int SL = D / 16;           // lanes per row, score phase (8 rotate-half pairs per lane)
  constexpr int SPP = kWave / SL;      // rows per pass, score phase
  constexpr int HALF = D / 2;
  constexpr int PV_UNROLL = NW == 1 ? 4 : 8;
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int SCPR = D * ESZ / 16;   // 16-byte pieces per row, staged value rows
  constexpr int SR = NW * kWave * 4 / SCPR;   // rows per staging round
  static_assert(NW == 1 || SR % (8 * (kWave / (D / VE))) == 0, "a staging round holds whole 8-row residue steps");

  // bf16 storage: the first level a unit scores holds every node of that level, in order, for
  // every unit of the workgroup; its logits come from one matrix-core tile (see mf_level below)
  constexpr bool MF = BF16;
  // bf16 storage with G >= 2: the value pass on the matrix cores (mv_read_tr above)
  constexpr bool MV = BF16 && G >= 2;
  // the fmaf value path splits a lane's value elements between the waves (NW <= 4); the
  // matrix-core one takes whole (head group, column block) pairs, so it runs with 8 waves too
  static_assert(NW == 1 || NW == 4 || (MV && NW == 8), "waves per unit");
  static_assert(MV || VE % NW == 0, "waves split the value elements of a lane");
  constexpr int HG = G > 4 ? G / 4 : 1;   // groups of 4 query heads
  constexpr int CB = D / 64;              // 64-column blocks of the value rows
  extern __shared__ __align__(16) unsigned char lds_all[];
  // NW = 1: a workgroup holds `slots` units, one wave each; NW > 1: one unit on NW waves
  const int slots = NW == 1 && MF ? static_cast<int>(blockDim.x) / kWave : 1;
  // wave-uniform: held in a scalar register, so the unit's LDS addresses stay scalar too
  const int slot = NW == 1 && MF ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave) : 0;
  const int zcap = a.zcap;
  const Lds L = lds_layout(D, G, a.smax, zcap);
  unsigned char* lds = lds_all + slot * L.total;   // this unit's region
  float* qs = reinterpret_cast<float*>(lds + L.q);
  // rotated query operands, [G][D/16 lane slots][16 words]: bf16 packs 8 pairs
  // (lo0,lo1), (lo2,lo3), .., (hi6,hi7) into words 0..7; float32 keeps lo0..lo7, hi0..hi7
  uint32_t* qr = reinterpret_cast<uint32_t*>(lds + L.qr);
  float* zs = reinterpret_cast<float*>(lds + L.zs);
  float* sc = reinterpret_cast<float*>(lds + L.sc);
  int32_t* cid = reinterpret_cast<int32_t*>(lds + L.cid);
  uint8_t* flags = reinterpret_cast<uint8_t*>(lds + L.flags);
  int32_t* selA = reinterpret_cast<int32_t*>(lds + L.selA);
  int32_t* selB = reinterpret_cast<int32_t*>(lds + L.selB);
  int64_t* nls = reinterpret_cast<int64_t*>(lds + L.nls);
  float* bc = reinterpret_cast<float*>(lds + L.bc);   // wave 0 -> all: alpha[G], l[G]
  int32_t* info = reinterpret_cast<int32_t*>(lds + L.info);
  uint4* vst = reinterpret_cast<uint4*>(lds_all + slots * L.total);   // staged value rows (several waves)
  uint16_t* mstage = reinterpret_cast<uint16_t*>(lds_all + slots * L.total + (NW > 1 ? a.stage_bytes : 0));
  const bool staged = NW > 1 && a.pv_stage == 1;          // rounds of SR rows
  const bool prefetched = NW > 1 && a.pv_stage == 2;      // a chunk's rows, loaded while it is scored
  // matrix-core value pass: the softmax weights as bf16 pairs, [row / 4][head][hi, lo][row % 4]
  // (16 bytes per quad and head, 4 G bytes per row: the size of a row's logits). One wave: in the
  // unit's logit array (an iteration of the weight pass writes the bytes of the logit rows it has
  // just read). Several waves: a region of their own after the tile's rows.
  uint16_t* pw = NW == 1 ? reinterpret_cast<uint16_t*>(zs)
                         : reinterpret_cast<uint16_t*>(lds_all + slots * L.total + a.stage_bytes + mf_stage_bytes(D));
  // the G logits (then weights) of candidate r: one vector LDS access
  auto zrow_load = [&](int32_t r, float (&z)[G]) {
    if constexpr (G % 4 == 0) {
#pragma unroll
      for (int i = 0; i < G / 4; ++i) {
        const float4 t = reinterpret_cast<const float4*>(zs + r * G)[i];
        z[4 * i] = t.x; z[4 * i + 1] = t.y; z[4 * i + 2] = t.z; z[4 * i + 3] = t.w;
      }
    } else if constexpr (G == 2) {
      const float2 t = reinterpret_cast<const float2*>(zs + r * G)[0];
      z[0] = t.x; z[1] = t.y;
    } else {
      z[0] = zs[r];
    }
  };
  auto zrow_store = [&](int32_t r, const float (&z)[G]) {
    if constexpr (G % 4 == 0) {
#pragma unroll
      for (int i = 0; i < G / 4; ++i)
        reinterpret_cast<float4*>(zs + r * G)[i] = make_float4(z[4 * i], z[4 * i + 1], z[4 * i + 2], z[4 * i + 3]);
    } else if constexpr (G == 2) {
      reinterpret_cast<float2*>(zs + r * G)[0] = make_float2(z[0], z[1]);
    } else {
      zs[r] = z[0];
    }
  };

  const int lane = threadIdx.x % kWave;
  // wave within the unit (wave-uniform: a scalar register)
  const int wid = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int tid = NW == 1 ? lane : static_cast<int>(threadIdx.x);         // thread within the unit
  constexpr int NT = NW * kWave;
  auto bsync = [&]() {
    if constexpr (NW == 1) wave_sync();
    else __syncthreads();
  };
  const int sub = lane % RL, rg = lane / RL;       // value phase
  const int ssub = lane % SL, srg = lane / SL;     // score phase
  // units: per (sequence, KV head) its (query, selection group) pairs in order, `slots`
  // consecutive ones per workgroup; consecutive workgroups take consecutive KV heads, so with 8
  // KV heads every XCD keeps to one KV head (workgroup i runs on XCD i mod 8)
  const int64_t b = blockIdx.y;
  const int hkv = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.Hkv_kv));
  const int64_t u = static_cast<int64_t>(blockIdx.x / static_cast<unsigned>(a.Hkv_kv)) * slots + slot;
  const bool active = u < a.n_q * a.kv_div;
  const int64_t j = active ? u / a.kv_div : 0;
  const int h = hkv * a.kv_div + static_cast<int>(u % a.kv_div);   // selection group
  const int64_t n = !active ? 0 : a.prefill ? a.q_start + j + 1 : a.n_fixed;
  const int f = a.f;
  const int64_t bh = b * a.Hkv_kv + hkv;

  // raw query heads of the selection group -> LDS (float)
  if (active) {
    const int64_t qbase = ((b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G) * D;
    for (int i = tid * 4; i < G * D; i += NT * 4) {
      float x[4];
      load4<BF16>(a.q, qbase + i, x);
      *reinterpret_cast<float4*>(qs + i) = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
  if (tid == 0) {
    int T = 0;
    int64_t m = n / f;
    while (m >= 1 && T < RECSA_MAX_LEVELS) {
      nls[++T] = m;
      m /= f;
    }
    nls[T + 1] = 0;
    nls[0] = T;
  }
  bsync();
  const int T = static_cast<int>(nls[0]);
  // the first level this unit scores: every level above it keeps all its nodes (k_l >= n_l), so
  // its candidates are all of its n_l nodes, in order, at their own index; the query sits at n_l
  int ls = 0;
  int32_t cs = 0;
  for (int lv = T; lv >= 1; --lv) {
    const int32_t nl = static_cast<int32_t>(nls[lv]);
    if (a.k.k[lv] < nl) {
      ls = lv;
      cs = nl;
      break;
    }
  }
  // several waves, prefetch mode: the value rows of candidates [0, cn) -- rounded up to whole
  // 8-row residue steps with copies of the last row -- go straight from memory to LDS
  // (row-major, D * ESZ bytes a row) while the chunk is scored and selected
  auto prefetch_values = [&](const void* vsrc, int64_t rowbase, int32_t cn) {
    const int32_t pieces = ((cn + 8 * RPP - 1) / (8 * RPP)) * (8 * RPP) * SCPR;
    for (int32_t jw = wid; jw * kWave < pieces; jw += NW) {
      const int32_t idx = jw * kWave + lane;
      const int32_t r = idx / SCPR;
      const int64_t row = rowbase + cid[r < cn ? r : cn - 1];
      const char* g = static_cast<const char*>(vsrc) + row * (D * ESZ) + (idx % SCPR) * 16;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(g),
                                       (__attribute__((address_space(3))) void*)(vst + jw * kWave), 16, 0, 0);
    }
  };
  if constexpr (MF) {
    if (tid == 0) {
      info[0] = ls;
      info[1] = cs;
    }
    // several waves: the first scored level's candidates are its nodes in order, so their value
    // rows can be requested now, before the tile is computed (as score_rows does for a level it
    // scores)
    if (prefetched && active && ls > 0) {
      for (int32_t r = tid; r < cs; r += NT) cid[r] = r;
      bsync();
      prefetch_values(a.tree.NV[ls], bh * a.tree.rows[ls], cs);
    }
    __syncthreads();
    mf_shared_levels<D, G>(a, lds_all, L, slots, slot, ls, cs, qs, mstage, bh, tid, NT);
  }
  if (!active) return;
  const int64_t sel_row0 = ((b * a.n_q + j) * a.Hkv + h) * a.n_levels;
  if (a.sel) {
    for (int lv = T + 1; lv <= a.n_levels; ++lv)
      for (int c = tid; c < a.sel_width; c += NT) a.sel[(sel_row0 + lv - 1) * a.sel_width + c] = -1;
  }

  float m_run[G], l_run[G], acc[G][VEW];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < VEW; ++e) acc[hh][e] = 0.0f;
  }
  // matrix-core value pass: oacc[hg][cb][i] = O[head 4 hg + i][column]: with one wave, column
  // 2 lane + cb (D = 128) or lane (D = 64); with several waves, column 64 cb + lane
  mv_f32x4_t oacc[HG][CB];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) oacc[hg][cb] = mv_f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // several waves: this lane's 8-byte chunk of a quad's transposed read (row mv_j of the quad,
  // 16-column block mv_bl, chunk mv_c of it)
  const int mv_j = (lane & 15) >> 2, mv_c = lane & 3, mv_bl = lane >> 4;
  // this lane's weight pair (hi, lo) of head group hg for quad qd; heads past G get 0
  auto mv_weights = [&](int32_t qd, int hg) __attribute__((always_inline)) {
    const int hd = 4 * hg + (lane & 3);
    const mv_i16x8_t w = *reinterpret_cast<const mv_i16x8_t*>(pw + (qd * G + (hd < G ? hd : G - 1)) * 8);
    const mv_i16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
    return hd < G ? w : z;
  };
  auto mv_mfma = [&](int hg, int cb, const mv_i16x8_t& w, const mv_i16x4_t& bv) __attribute__((always_inline)) {
    oacc[hg][cb] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_shufflevector(w, w, 0, 1, 2, 3), bv, oacc[hg][cb], 0, 0, 0);
    oacc[hg][cb] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_shufflevector(w, w, 4, 5, 6, 7), bv, oacc[hg][cb], 0, 0, 0);
  };
  // the products of quad qd (rows 4 qd .. 4 qd + 3 of the chunk); bop(cb) is this lane's B
  // operand of column block cb
  auto mv_quad = [&](int32_t qd, auto bop) __attribute__((always_inline)) {
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      const mv_i16x8_t w = mv_weights(qd, hg);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) mv_mfma(hg, cb, w, bop(cb));
    }
  };
  auto mv_weight = [&](int32_t r, int hh, float p) {
    const uint16_t hi = bf16_bits(p);
    uint16_t* w = pw + ((r >> 2) * G + hh) * 8 + (r & 3);
    w[0] = hi;
    w[4] = bf16_bits(p - __uint_as_float(static_cast<uint32_t>(hi) << 16));
  };

  // rotated query operands for the current level -> qr: lane slot ssub holds the 8
  // rotate-half pairs (elements 8*ssub + e and HALF + 8*ssub + e, e < 8) of every head
  auto rotate_query = [&](int64_t pos) __attribute__((always_inline)) {
    float c[8], s[8];
    if (a.use_rope) {
      const float4* t = reinterpret_cast<const float4*>(a.tab + pos * HALF + 8 * ssub);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 tv = t[u];
        c[2 * u] = tv.x; s[2 * u] = tv.y; c[2 * u + 1] = tv.z; s[2 * u + 1] = tv.w;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float ql[8], qh[8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4 xl = *reinterpret_cast<const float4*>(qs + hh * D + 8 * ssub + 4 * u);
        const float4 xh = *reinterpret_cast<const float4*>(qs + hh * D + HALF + 8 * ssub + 4 * u);
        ql[4 * u] = xl.x; ql[4 * u + 1] = xl.y; ql[4 * u + 2] = xl.z; ql[4 * u + 3] = xl.w;
        qh[4 * u] = xh.x; qh[4 * u + 1] = xh.y; qh[4 * u + 2] = xh.z; qh[4 * u + 3] = xh.w;
      }
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (a.use_rope) {
          const float p1 = ql[e] * c[e], p2 = qh[e] * s[e];
          const float p3 = qh[e] * c[e], p4 = ql[e] * s[e];
          lo[e] = p1 - p2;
          hi[e] = p3 + p4;
        } else {
          lo[e] = ql[e];
          hi[e] = qh[e];
        }
      }
      uint32_t* dst = qr + (hh * SL + ssub) * 16;
      if (srg == 0 && wid == 0) {
        if constexpr (BF16) {
          uint32_t w[8];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            w[u] = __builtin_bit_cast(uint32_t, pack_bf16_rne(lo[2 * u], lo[2 * u + 1]));
            w[4 + u] = __builtin_bit_cast(uint32_t, pack_bf16_rne(hi[2 * u], hi[2 * u + 1]));
          }
          reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
          reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
        } else {
          reinterpret_cast<float4*>(dst)[0] = make_float4(lo[0], lo[1], lo[2], lo[3]);
          reinterpret_cast<float4*>(dst)[1] = make_float4(lo[4], lo[5], lo[6], lo[7]);
          reinterpret_cast<float4*>(dst)[2] = make_float4(hi[0], hi[1], hi[2], hi[3]);
          reinterpret_cast<float4*>(dst)[3] = make_float4(hi[4], hi[5], hi[6], hi[7]);
        }
      }
    }
    bsync();
  };

  // logits of candidates [c0, c0 + cn) (index = RoPE position) -> zs[r * G + hh], sc[r].
  // Two row buffers alternate: the rows of the next pass are requested after this pass's
  // RoPE-table entries, so waiting for the table does not wait for them. The loop body has
  // no branch around a load (the rotation is chosen outside the loop; a pass past the end
  // and lanes past the last candidate load the last candidate's row and write nothing), so
  // the loads' completion is tracked exactly.
  auto score_rows_t = [&](const void* src, const void* vsrc, int64_t rowbase, const CandMap& cm, int32_t c0,
                          int32_t cn, int64_t qpos, auto rope) {
    constexpr bool ROPE = decltype(rope)::value;
    // several waves (latency-bound): a pass's RoPE-table entries are fetched with its rows,
    // one pass ahead; one wave fetches them at the start of the pass (fewer registers)
    constexpr bool PT = ROPE && NW > 1;
    float4 ta[PT ? 4 : 1], tb[PT ? 4 : 1];
    // the slice's rows from a wave-uniform base: a row's byte offset fits 32 bits
    const char* sbase = static_cast<const char*>(src) + rowbase * (D * ESZ);
    const char* tbase = reinterpret_cast<const char*>(a.tab);
    auto fetch = [&](int32_t r0, Raw8<BF16>& lo, Raw8<BF16>& hi, float4 (&tn)[PT ? 4 : 1]) {
      const int32_t r = r0 + srg < cn ? r0 + srg : cn - 1;
      const uint32_t boff = static_cast<uint32_t>(cid[r]) * (D * ESZ) + static_cast<uint32_t>(8 * ssub * ESZ);
      lo = raw8_load32<BF16>(sbase, boff);
      hi = raw8_load32<BF16>(sbase, boff + HALF * ESZ);
      if constexpr (PT) {
        const uint32_t toff = (static_cast<uint32_t>(c0 + r) * HALF + 8 * ssub) * static_cast<uint32_t>(sizeof(float2));
        const float4* t = reinterpret_cast<const float4*>(tbase + toff);
#pragma unroll
        for (int u = 0; u < 4; ++u) tn[u] = t[u];
      }
    };
    auto pass = [&](int32_t r0, const Raw8<BF16>& clo, const Raw8<BF16>& chi, const float4 (&tc)[PT ? 4 : 1],
                    Raw8<BF16>& nlo, Raw8<BF16>& nhi, float4 (&tn)[PT ? 4 : 1]) {
      const int32_t r = r0 + srg;
      const bool valid = r < cn;
      float4 tv[4];
      if constexpr (ROPE && !PT) {
        const uint32_t toff = (static_cast<uint32_t>(c0 + (valid ? r : 0)) * HALF + 8 * ssub) * static_cast<uint32_t>(sizeof(float2));
        const float4* t = reinterpret_cast<const float4*>(tbase + toff);
#pragma unroll
        for (int u = 0; u < 4; ++u) tv[u] = t[u];
      }
      fetch(r0 + NW * SPP, nlo, nhi, tn);
      if constexpr (PT) {
#pragma unroll
        for (int u = 0; u < 4; ++u) tv[u] = tc[u];
      }
      float klo[8], khi[8];
      raw8_cvt<BF16>(clo, klo);
      raw8_cvt<BF16>(chi, khi);
      float olo[8], ohi[8];
      if constexpr (ROPE) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float cc[2] = {tv[u].x, tv[u].z}, ss[2] = {tv[u].y, tv[u].w};
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const int e = 2 * u + v;
            const float p1 = klo[e] * cc[v], p2 = khi[e] * ss[v];
            const float p3 = khi[e] * cc[v], p4 = klo[e] * ss[v];
            olo[e] = p1 - p2;
            ohi[e] = p3 + p4;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { olo[e] = klo[e]; ohi[e] = khi[e]; }
      }
      float part[G];
      if constexpr (BF16) {
        bf16x2_t kp[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kp[u] = pack_bf16_rne(olo[2 * u], olo[2 * u + 1]);
          kp[4 + u] = pack_bf16_rne(ohi[2 * u], ohi[2 * u + 1]);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const uint4* src4 = reinterpret_cast<const uint4*>(qr + (hh * SL + ssub) * 16);
          const uint4 qa = src4[0], qb = src4[1];
          const uint32_t qw[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
          float p = 0.0f;
#pragma unroll
          for (int u = 0; u < 8; ++u)
            p = __builtin_amdgcn_fdot2_f32_bf16(kp[u], __builtin_bit_cast(bf16x2_t, qw[u]), p, false);
          part[hh] = p;
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float* qf = reinterpret_cast<const float*>(qr + (hh * SL + ssub) * 16);
          float p = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) p = fmaf(qf[e], olo[e], p);
#pragma unroll
          for (int e = 0; e < 8; ++e) p = fmaf(qf[8 + e], ohi[e], p);
          part[hh] = p;
        }
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) part[hh] = lane_group_sum<SL>(part[hh]);
      if (valid && ssub == 0) {
        if constexpr (NW == 1) {
          zrow_store(r, part);   // scaled, and summed into the group score, after the passes
        } else {
          float S = 0.0f, z[G];
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            z[hh] = part[hh] * a.scale;
            S = S + z[hh];
          }
          zrow_store(r, z);
          sc[r] = S;
        }
      }
    };
    // the chunk's candidate -> row map, read by the row loads, the selection and the values;
    // entries up to the next multiple of 16 repeat the last candidate's row
    for (int32_t r = tid; r < ((cn + 15) & ~15); r += NT) cid[r] = cm(c0 + (r < cn ? r : cn - 1));
    bsync();
    if (prefetched) prefetch_values(vsrc, rowbase, cn);
    Raw8<BF16> alo, ahi, blo, bhi;
    int32_t r0 = wid * SPP;
    fetch(r0, alo, ahi, ta);
    if (qpos >= 0) rotate_query(qpos);   // its table reads overlap the first rows' loads
    for (; r0 < cn; r0 += 2 * NW * SPP) {
      pass(r0, alo, ahi, ta, blo, bhi, tb);
      if (r0 + NW * SPP >= cn) break;
      pass(r0 + NW * SPP, blo, bhi, tb, alo, ahi, ta);
    }
    if constexpr (NW == 1) {
      // one wave: the logits z = scale * dot and the group score S = sum of the G logits in
      // head order, one candidate per lane (the same arithmetic as the several-wave passes)
      wave_sync();
      for (int32_t r = lane; r < cn; r += kWave) {
        float z[G], S = 0.0f;
        zrow_load(r, z);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          z[hh] = z[hh] * a.scale;
          S = S + z[hh];
        }
        zrow_store(r, z);
        sc[r] = S;
      }
    }
    bsync();
  };
  // the first scored level: its logits are already in zs (mf_shared_levels); the candidate -> node
  // map, the group scores (the heads' logits summed in head order, as score_rows does) and, with
  // several waves, the value prefetch
  auto shared_rows = [&](const void* vsrc, int64_t rowbase, const CandMap& cm, int32_t cn) {
    for (int32_t r = tid; r < cn; r += NT) {
      cid[r] = cm(r);
      float z[G];
      zrow_load(r, z);
      float S = 0.0f;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) S = S + z[hh];
      sc[r] = S;
    }
    for (int32_t r = cn + tid; r < ((cn + 15) & ~15); r += NT) cid[r] = cm(cn - 1);   // padding, as score_rows
    bsync();
    (void)vsrc;
    (void)rowbase;   // several waves: its value rows were requested before the tile
  };
  // qpos >= 0: rotate the query heads at qpos first (a level's first chunk)
  auto score_rows = [&](const void* src, const void* vsrc, int64_t rowbase, const CandMap& cm, int32_t c0, int32_t cn,
                        int64_t qpos) {
    if (a.use_rope) score_rows_t(src, vsrc, rowbase, cm, c0, cn, qpos, std::true_type{});
    else score_rows_t(src, vsrc, rowbase, cm, c0, cn, qpos, std::false_type{});
  };
  // NU: candidate slots per lane held in registers (C <= NU * 64 unless GEN); GEN: the slots
  // past NU are read from LDS. Slots past the last candidate hold key 0, which no threshold
  // t > 0 counts, so the result does not depend on NU.
  auto select_top_n = [&](int32_t C, int32_t s, int32_t* sel_out, auto nu_t, auto gen_t) {
    constexpr int NU = decltype(nu_t)::value;
    constexpr bool GEN = decltype(gen_t)::value;
    const int32_t nu = (C + kWave - 1) / kWave;
    uint32_t o[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int32_t r = lane + kWave * u;
      o[u] = r < C ? ordered_bits(sc[r]) : 0u;
    }
    auto key = [&](int u) -> uint32_t {
      const int32_t r = lane + kWave * u;
      return r < C ? ordered_bits(sc[r]) : 0u;
    };
    // candidates with key >= t (t > 0; an empty slot holds 0)
    auto count_ge = [&](uint32_t t) -> int32_t {
      int32_t c = 0;
#pragma unroll
      for (int u = 0; u < NU; ++u) c += __popcll(__ballot(o[u] >= t));
      if constexpr (GEN)
        for (int u = NU; u < nu; ++u) c += __popcll(__ballot(key(u) >= t));
      return c;
    };
    // tau: the largest t with at least s keys >= t; once exactly s keys are >= some t they
    // are the selection (nothing left to tie-break), so the search stops there
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = tau | (1u << bit);
      const int32_t c = count_ge(t);
      if (c >= s) {
        tau = t;
        if (c == s) break;
      }
    }
    int32_t above = 0;
#pragma unroll
    for (int u = 0; u < NU; ++u) above += __popcll(__ballot(o[u] > tau));
    if constexpr (GEN)
      for (int u = NU; u < nu; ++u) above += __popcll(__ballot(key(u) > tau));
    const int32_t need = s - above;   // keys equal to tau to keep, lowest index first
    const uint64_t lt = (1ull << lane) - 1ull;
    int32_t taken = 0, cnt = 0;
    auto emit = [&](int u, uint32_t kv) {
      const int32_t r = lane + kWave * u;
      const bool valid = r < C;
      const uint64_t eq = __ballot(valid && kv == tau);
      const bool keep = valid && (kv > tau || (kv == tau && taken + __popcll(eq & lt) < need));
      const uint64_t km = __ballot(keep);
      if (valid) flags[r] = keep ? 1 : 0;
      if (keep) sel_out[cnt + __popcll(km & lt)] = cid[r];
      taken += __popcll(eq);
      cnt += __popcll(km);
    };
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (u < nu) emit(u, o[u]);
    if constexpr (GEN)
      for (int u = NU; u < nu; ++u) emit(u, key(u));
    wave_sync();
  };
  // Keeps the s largest (S, -r) keys among r < C: flags[r] = 1 and sel_out[0..s) = their
  // node ids in candidate order. A threshold is found by bisection on the scores'
  // order-preserving 32-bit patterns (a ballot count per step, no lane exchange); the
  // candidates above it are kept, then those equal to it in index order. Each step counts
  // only the lane slots that can hold a candidate (two at f = 16, k = 8).
  auto select_top = [&](int32_t C, int32_t s, int32_t* sel_out) {
    if (C <= 2 * kWave) select_top_n(C, s, sel_out, std::integral_constant<int, 2>{}, std::false_type{});
    else if (C <= 3 * kWave) select_top_n(C, s, sel_out, std::integral_constant<int, 3>{}, std::false_type{});
    else if (C <= 4 * kWave) select_top_n(C, s, sel_out, std::integral_constant<int, 4>{}, std::false_type{});
    else select_top_n(C, s, sel_out, std::integral_constant<int, 4>{}, std::true_type{});
  };

  // fold entries r < cn (skipping kept ones when use_flags) into the online softmax: wave 0
  // computes the weights (into zs) and the running max and sum; every wave then accumulates
  // its value elements
  const int dim0 = wid * (D / NW) + sub * VEW;
  auto softmax_pv = [&](const void* vsrc, int64_t rowbase, const CandMap& cm, int32_t c0, int32_t cn,
                        bool use_flags) {
    // several waves: value rows staged through LDS, 4 16-byte pieces per thread and round
    uint4 st0, st1, st2, st3;
    auto piece = [&](int32_t s0, int i) -> uint4 {
      const int idx = tid + i * NT;
      const int32_t r = s0 + idx / SCPR;
      const int64_t row = rowbase + cid[r < cn ? r : cn - 1];
      return *reinterpret_cast<const uint4*>(static_cast<const char*>(vsrc) + row * (D * ESZ) + (idx % SCPR) * 16);
    };
    auto stage_issue = [&](int32_t s0) {
      st0 = piece(s0, 0);
      st1 = piece(s0, 1);
      st2 = piece(s0, 2);
      st3 = piece(s0, 3);
    };
    if constexpr (NW > 1) {
      if (staged) stage_issue(0);   // in flight during the weight pass
      // this wave's prefetched rows have landed in LDS before the barrier below
      if (prefetched) __builtin_amdgcn_s_waitcnt(0);
    }
    if constexpr (NW > 1) {
      // several waves: head hh's weights are computed by wave hh % NW, in the order one wave
      // uses for it (each head's max, exponentials and sum are independent of the other heads),
      // and its running max lives in that wave; every wave takes alpha and the running sum
      // from LDS
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        if (hh % NW != wid) continue;
        float mn = -INFINITY;
        for (int32_t r = lane; r < cn; r += kWave) {
          if (use_flags && flags[r]) continue;
          mn = fmaxf(mn, zs[r * G + hh]);
        }
        mn = fmaxf(m_run[hh], wave_max_dpp(mn));
        float ls = 0.0f;
        for (int32_t r = lane; r < cn; r += kWave) {
          const bool skip = use_flags && flags[r];
          const float p = skip ? 0.0f : expf(zs[r * G + hh] - mn);
          if constexpr (MV) mv_weight(r, hh, p);
          else zs[r * G + hh] = p;
          ls += p;
        }
        if constexpr (MV) {
          for (int32_t r = cn + lane; r < ((cn + 15) & ~15); r += kWave) mv_weight(r, hh, 0.0f);
        }
        const float lsum = wave_sum_dpp(ls);
        const float alpha = expf(m_run[hh] - mn);
        const float lnew = l_run[hh] * alpha + lsum;
        m_run[hh] = mn;
        if (lane == 0) {
          bc[hh] = alpha;
          bc[G + hh] = lnew;
        }
      }
    } else {
      float mnew[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) mnew[hh] = -INFINITY;
      for (int32_t r = lane; r < cn; r += kWave) {
        if (use_flags && flags[r]) continue;
        float z[G];
        zrow_load(r, z);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) mnew[hh] = fmaxf(mnew[hh], z[hh]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) mnew[hh] = fmaxf(m_run[hh], wave_max_dpp(mnew[hh]));
      float ls[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) ls[hh] = 0.0f;
      // matrix-core value pass: the bf16 weight pairs overwrite the logit array (pw); iteration t
      // writes the bytes of logit rows [64 t, 64 t + 64), the ones it has read, and lds_order
      // keeps each iteration's reads before its writes
      if constexpr (MV) lds_order();
      for (int32_t r = lane; r < cn; r += kWave) {
        const bool skip = use_flags && flags[r];
        float z[G];
        zrow_load(r, z);
        if constexpr (MV) lds_order();
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = skip ? 0.0f : expf(z[hh] - mnew[hh]);
          z[hh] = p;
          ls[hh] += p;
        }
        if constexpr (MV) {
#pragma unroll
          for (int hh = 0; hh < G; ++hh) mv_weight(r, hh, z[hh]);
        } else {
          zrow_store(r, z);
        }
      }
      if constexpr (MV) {
        for (int32_t r = cn + lane; r < ((cn + 15) & ~15); r += kWave)
#pragma unroll
          for (int hh = 0; hh < G; ++hh) mv_weight(r, hh, 0.0f);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float lsum = wave_sum_dpp(ls[hh]);
        const float alpha = expf(m_run[hh] - mnew[hh]);
        l_run[hh] = l_run[hh] * alpha + lsum;
        m_run[hh] = mnew[hh];
        if constexpr (MV) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) oacc[hh / 4][cb][hh % 4] *= alpha;
        } else {
#pragma unroll
          for (int e = 0; e < VEW; ++e) acc[hh][e] *= alpha;
        }
      }
    }
    bsync();
    if constexpr (NW > 1) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float alpha = bc[hh];
        l_run[hh] = bc[G + hh];
        if constexpr (MV) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) oacc[hh / 4][cb][hh % 4] *= alpha;
        } else {
#pragma unroll
          for (int e = 0; e < VEW; ++e) acc[hh][e] *= alpha;
        }
      }
      // matrix-core value pass: the quads of LDS rows [0, sn) (copies of a finite row up to the
      // next multiple of 16, weight 0), wave w taking (head group, column block) pair w; four
      // quads' operands are read before their products
      auto chains_mv = [&](int32_t s0, int32_t sn) {
        const uint16_t* vs = reinterpret_cast<const uint16_t*>(vst);
        const int32_t nq = (sn + 15) / 16 * 4;
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            if (hg * CB + cb != wid) continue;
            const uint16_t* bp = vs + mv_j * D + 64 * cb + 16 * mv_bl + 4 * mv_c;
            for (int32_t qd = 0; qd < nq; qd += 4) {
              mv_i16x8_t w[4];
              mv_i16x4_t bv[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                w[t] = mv_weights((s0 >> 2) + qd + t, hg);
                bv[t] = mv_read_tr(bp + (qd + t) * 4 * D);
              }
#pragma unroll
              for (int t = 0; t < 4; ++t) mv_mfma(hg, cb, w[t], bv[t]);
            }
          }
      };
      // 8 rows of the residue per step from LDS rows [0, sn) of vst (rows up to the next
      // multiple of 8 * RPP hold finite copies), their reads issued together and no branch: a
      // kept row has weight 0 and a row past the end gets weight 0, and fmaf(0, v, acc)
      // leaves acc unchanged, exactly as skipping the row does
      auto chains = [&](int32_t s0, int32_t sn) {
        for (int32_t rb = 0; rb < sn; rb += 8 * RPP) {
          float v[8][VEW], pz[8][G];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int32_t rr = rb + u * RPP + rg;
            const bool ok = rr < sn;
            if constexpr (BF16) {
              const uint16_t* vp = reinterpret_cast<const uint16_t*>(vst) + rr * D + dim0;
#pragma unroll
              for (int e = 0; e < VEW; ++e) v[u][e] = __uint_as_float(static_cast<uint32_t>(vp[e]) << 16);
            } else {
              const float* vp = reinterpret_cast<const float*>(vst) + rr * D + dim0;
#pragma unroll
              for (int e = 0; e < VEW; ++e) v[u][e] = vp[e];
            }
            zrow_load(s0 + (ok ? rr : 0), pz[u]);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) pz[u][hh] = ok ? pz[u][hh] : 0.0f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int hh = 0; hh < G; ++hh)
#pragma unroll
              for (int e = 0; e < VEW; ++e) acc[hh][e] = fmaf(pz[u][hh], v[u][e], acc[hh][e]);
        }
      };
      if (prefetched) {
        if constexpr (MV) chains_mv(0, cn);
        else chains(0, cn);
        bsync();
        return;
      }
      if (staged) {
        // rounds of SR rows through LDS; the next round's loads are in flight while this
        // round is accumulated. Each lane keeps its chain: rows of its residue rg mod RPP in
        // ascending order, element dim0 + e, as with one wave.
        for (int32_t s0 = 0; s0 < cn; s0 += SR) {
          vst[tid] = st0;
          vst[tid + NT] = st1;
          vst[tid + 2 * NT] = st2;
          vst[tid + 3 * NT] = st3;
          if (s0 + SR < cn) stage_issue(s0 + SR);
          bsync();
          if constexpr (MV) chains_mv(s0, cn - s0 < SR ? cn - s0 : SR);
          else chains(s0, cn - s0 < SR ? cn - s0 : SR);
          bsync();
        }
        return;
      }
    }
    // value rows: two buffers alternate, the next iteration's rows are requested before this
    // iteration's are accumulated; every row slot loads (a kept or absent row loads a valid
    // row and adds nothing), so no load sits behind a branch
    if constexpr (MV && NW == 1) {
      // matrix-core value pass with one wave: every lane loads its columns of every row -- 4
      // bytes, columns 2 lane and 2 lane + 1 (D = 128; column block cb = the column's parity), or
      // 2 bytes, column lane (D = 64) -- so that a quad's 4 rows at one column pack straight into
      // the B operand. 8 rows (2 quads) per group; the next group's rows are in flight while this
      // group's products run. Rows past the last candidate load the last candidate's row; their
      // weights are 0 (padded to a multiple of 16 rows), like the kept rows'.
      using RT = typename std::conditional<D == 128, uint32_t, uint16_t>::type;
      static_assert(D * 2 == 64 * static_cast<int>(sizeof(RT)), "a row is 64 units of RT");
      const char* vb = static_cast<const char*>(vsrc) + rowbase * (D * 2);   // wave-uniform
      const uint32_t lane_off = static_cast<uint32_t>(lane) * static_cast<uint32_t>(sizeof(RT));
      // the row ids of a group of VG rows in 16-byte LDS reads (the map is padded to a multiple of
      // 16 rows with the last candidate's row; a group past the padding re-reads the last VG)
      constexpr int VG = G <= 4 ? 16 : 8;   // 8 at G = 8 (registers)
      const int32_t cn16 = (cn + 15) & ~15;
      auto gfetch = [&](int32_t r0, RT (&raw)[VG]) {
        const int32_t rc = r0 < cn16 - VG ? r0 : cn16 - VG;
#pragma unroll
        for (int i = 0; i < VG / 4; ++i) {
          const int4 c4 = *reinterpret_cast<const int4*>(cid + rc + 4 * i);
          const int32_t ids[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            raw[4 * i + e] = *reinterpret_cast<const RT*>(vb + static_cast<uint32_t>(ids[e]) * (D * 2) + lane_off);
        }
      };
      auto gcompute = [&](int32_t r0, const RT (&raw)[VG]) {
#pragma unroll
        for (int qq = 0; qq < VG / 4; ++qq) {
          uint32_t w[CB][2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const uint32_t x = raw[4 * qq + 2 * t], y = raw[4 * qq + 2 * t + 1];
            if constexpr (D == 128) {
              // one byte permute each: (x.lo, y.lo) and (x.hi, y.hi)
              w[0][t] = __builtin_amdgcn_perm(y, x, 0x05040100u);
              w[CB - 1][t] = __builtin_amdgcn_perm(y, x, 0x07060302u);
            } else {
              w[0][t] = x | (y << 16);
            }
          }
          mv_quad((r0 >> 2) + qq, [&](int cb) { return __builtin_bit_cast(mv_i16x4_t, make_uint2(w[cb][0], w[cb][1])); });
        }
      };
      // groups of VG rows (the quads up to the padded count, as the several-wave path takes them),
      // the next group's rows in flight during this group's products
      RT ra[VG], rb[VG];
      gfetch(0, ra);
      for (int32_t r0 = 0; r0 < cn; r0 += 2 * VG) {
        gfetch(r0 + VG, rb);
        gcompute(r0, ra);
        if (r0 + VG >= cn16) break;
        gfetch(r0 + 2 * VG, ra);
        gcompute(r0 + VG, rb);
      }
      bsync();
      return;
    }
    auto vfetch = [&](int32_t r0, RawV<BF16, VEW> (&raw)[PV_UNROLL]) {
#pragma unroll
      for (int u = 0; u < PV_UNROLL; ++u) {
        const int32_t r = r0 + u * RPP + rg;
        raw[u].load(vsrc, (rowbase + cid[r < cn ? r : cn - 1]) * D + dim0);
      }
    };
    auto vpass = [&](int32_t r0, const RawV<BF16, VEW> (&cur)[PV_UNROLL], RawV<BF16, VEW> (&nxt)[PV_UNROLL]) {
      vfetch(r0 + RPP * PV_UNROLL, nxt);
#pragma unroll
      for (int u = 0; u < PV_UNROLL; ++u) {
        const int32_t r = r0 + u * RPP + rg;
        if (r >= cn || (use_flags && flags[r])) continue;
        float v[VEW];
        cur[u].cvt(v);
        float pr[G];
        zrow_load(r, pr);
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
#pragma unroll
          for (int e = 0; e < VEW; ++e) acc[hh][e] = fmaf(pr[hh], v[e], acc[hh][e]);
        }
      }
    };
    RawV<BF16, VEW> va[PV_UNROLL], vb[PV_UNROLL];
    vfetch(0, va);
    for (int32_t r0 = 0; r0 < cn; r0 += 2 * RPP * PV_UNROLL) {
      vpass(r0, va, vb);
      if (r0 + RPP * PV_UNROLL >= cn) break;
      vpass(r0 + RPP * PV_UNROLL, vb, va);
    }
    bsync();
  };

  // --- levels T .. 1 -------------------------------------------------------------
  int32_t* sel_prev = selA;
  int32_t* sel_new = selB;
  int32_t s_prev = 0;
  const int32_t fshift = (f & (f - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(f)) : -1;
  for (int lv = T; lv >= 1; --lv) {
    const int32_t n_l = static_cast<int32_t>(nls[lv]), n_up = static_cast<int32_t>(nls[lv + 1]);
    const CandMap cm{sel_prev, f * s_prev, f * n_up, f, fshift};
    const int32_t C = cm.n_kids + (n_l - cm.orph);
    const int32_t kl = a.k.k[lv];
    const int32_t s = kl < C ? kl : C;
    if (s == C) {
      for (int32_t i = tid; i < C; i += NT) sel_new[i] = cm(i);
      bsync();
    } else {
      const int64_t rowbase = bh * a.tree.rows[lv];
      if (MF && lv == ls) shared_rows(a.tree.NV[lv], rowbase, cm, C);
      else score_rows(a.tree.NK[lv], a.tree.NV[lv], rowbase, cm, 0, C, C);
      if (s > 0) {
        if (wid == 0) select_top(C, s, sel_new);
      } else {
        for (int32_t r = tid; r < C; r += NT) flags[r] = 0;
      }
      bsync();
      softmax_pv(a.tree.NV[lv], rowbase, cm, 0, C, true);
    }
    if (a.sel) {
      for (int c = tid; c < a.sel_width; c += NT)
        a.sel[(sel_row0 + lv - 1) * a.sel_width + c] = c < s ? sel_new[c] : -1;
    }
    int32_t* t = sel_prev;
    sel_prev = sel_new;
    sel_new = t;
    s_prev = s;
  }

  // --- token level -------------------------------------------------------------------
  {
    const int32_t n1 = T >= 1 ? static_cast<int32_t>(nls[1]) : 0;
    const CandMap cm{sel_prev, f * s_prev, f * n1, f, fshift};
    const int32_t C0 = cm.n_kids + (static_cast<int32_t>(n) - cm.orph);
    const bool own = a.prefill && C0 > 0 && cm(C0 - 1) == n - 1;
    const int32_t pq = own ? C0 - 1 : C0;
    const int64_t rowbase = bh * a.cap;
    for (int64_t c0 = 0; c0 < C0; c0 += zcap) {
      const int32_t cn = static_cast<int32_t>(C0 - c0 < zcap ? C0 - c0 : zcap);
      score_rows(a.K, a.V, rowbase, cm, static_cast<int32_t>(c0), cn, c0 == 0 ? pq : -1);
      softmax_pv(a.V, rowbase, cm, static_cast<int32_t>(c0), cn, false);
    }
  }

  // --- merge the row groups' partial sums, normalise, write ---------------------------
  const int64_t obase = ((b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G) * D;
  if constexpr (MV) {
    // head 4 hg + i of oacc[hg][cb] (with several waves, of this wave's pair hg * CB + cb)
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hd = 4 * hg + i;
        if (hd >= G) continue;
        const float l = l_run[hd];
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        float* o = a.out + obase + hd * D;
        if constexpr (NW == 1 && D == 128) {
          *reinterpret_cast<float2*>(o + 2 * lane) = make_float2(oacc[hg][0][i] * inv, oacc[hg][1][i] * inv);
        } else if constexpr (NW == 1) {
          o[lane] = oacc[hg][0][i] * inv;
        } else {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            if (hg * CB + cb == wid) o[64 * cb + lane] = oacc[hg][cb][i] * inv;
        }
      }
  }
#pragma unroll
  for (int off = RL; off < kWave; off <<= 1)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < VEW; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], off);
  if (!MV && rg == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float l = l_run[hh];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      float* o = a.out + obase + hh * D + dim0;
      if constexpr (VEW == 4) {
        *reinterpret_cast<float4*>(o) = make_float4(acc[hh][0] * inv, acc[hh][1] * inv, acc[hh][2] * inv, acc[hh][3] * inv);
      } else {
#pragma unroll
        for (int e = 0; e < VEW; ++e) o[e] = acc[hh][e] * inv;
      }
    }
  }
  if (a.lse) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      // the wave that holds head hh's running max (wave 0 alone with one wave)
      if (hh % NW == wid && lane == 0) {
        a.lse[(b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G + hh] =
            l_run[hh] > 0.0f ? m_run[hh] + logf(l_run[hh]) : -INFINITY;
      }
    }
  }
}

// Units (sequence, query, KV head) below which a unit gets several waves: with fewer, the
// GPU is not filled by one wave per unit and the descent's latency dominates.
constexpr int64_t kMultiWaveUnits = 2048;

// gfx950 has 160 KB of LDS per workgroup; a kernel's dynamic LDS limit is 64 KB until raised, and
// the attribute belongs to the current device: raised once per device and instantiation
constexpr size_t kLdsMax = 163840;

template <int D, bool BF16, int G, int NW>
static hipError_t allow_full_lds() {
  constexpr int kDevices = 64;
  static std::atomic<bool> done[kDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kDevices && done[dev].load()) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_kernel<D, BF16, G, NW>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsMax));
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < kDevices) done[dev].store(true);
  return hipSuccess;
}

template <int D, bool BF16, int G>
static hipError_t launch_attend_t(const AttnArgs& a, size_t lds, int64_t B, hipStream_t s) {
  // units per (sequence, KV head): its queries times its selection groups
  const int64_t units_kv = a.n_q * a.kv_div;
  const size_t mf = BF16 ? mf_stage_bytes(D) : 0;   // the matrix-core tile's rows
  if (units_kv * a.Hkv_kv * B < kMultiWaveUnits) {
    const dim3 grid(static_cast<unsigned>(units_kv * a.Hkv_kv), static_cast<unsigned>(B));
    // value rows through LDS when it has room: a whole chunk's rows (zcap of them, rounded up
    // to whole 8-row residue steps -- 8 * 64 / (D / 4) rows -- then to whole 64-lane loads of
    // 16 bytes), prefetched while the chunk is scored; else rounds of 4 waves x 64 lanes x 4
    // pieces of 16 bytes
    // bf16 with G >= 2 (the value pass on the matrix cores): 8 waves per unit, whose score passes
    // cover 64 candidate rows each (a level's 128 in two passes, both in flight at once); else 4
    constexpr bool kMV = BF16 && G >= 2;
    constexpr int kNW = kMV ? 8 : 4;
    constexpr size_t kPiecesPerRow = D * (BF16 ? 2 : 4) / 16;
    constexpr size_t kStep = 8 * kWave / (D / 4);
    const size_t rows = (static_cast<size_t>(a.zcap) + kStep - 1) / kStep * kStep;
    const size_t kFull = (rows * kPiecesPerRow + kWave - 1) / kWave * kWave * 16;
    constexpr size_t kStage = static_cast<size_t>(kNW) * kWave * 4 * 16;
    hipError_t e = allow_full_lds<D, BF16, G, kNW>();
    if (e != hipSuccess) return e;
    // the staged value rows, then the tile's rows (the first scored level's value rows are
    // requested before its tile is computed), then (matrix-core value pass) the bf16 weights;
    // that pass reads the value rows from LDS, and a staging mode is always granted (a unit's
    // LDS is at most 64 KB)
    const size_t pwb = kMV ? static_cast<size_t>(4 * G) * static_cast<size_t>(a.zcap) : 0;
    AttnArgs b = a;
    if (lds + kFull + mf + pwb <= kLdsMax) {
      b.pv_stage = 2;
      b.stage_bytes = static_cast<int32_t>(kFull);
    } else if (lds + kStage + mf + pwb <= kLdsMax) {
      b.pv_stage = 1;
      b.stage_bytes = static_cast<int32_t>(kStage);
    } else {
      if (kMV) return hipErrorInvalidValue;
      b.pv_stage = 0;
      b.stage_bytes = 0;
    }
    hipLaunchKernelGGL((attend_kernel<D, BF16, G, kNW>), grid, dim3(kNW * kWave), lds + b.stage_bytes + mf + pwb, s, b);
  } else {
    // bf16: up to 8 units of one KV head per workgroup, one wave each, whose rows fill the 32
    // rows of the first scored level's tile, as many as LDS holds; float32: one unit
    int slots = BF16 ? std::min(8, 32 / G) : 1;
    while (slots > 1 && slots * lds + mf > kLdsMax) slots /= 2;
    const size_t bytes = slots * lds + mf;
    if (bytes > 65536) {
      hipError_t e = allow_full_lds<D, BF16, G, 1>();
      if (e != hipSuccess) return e;
    }
    const dim3 grid(static_cast<unsigned>((units_kv + slots - 1) / slots * a.Hkv_kv), static_cast<unsigned>(B));
    hipLaunchKernelGGL((attend_kernel<D, BF16, G, 1>), grid, dim3(slots * kWave), bytes, s, a);
  }
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_attend_g(const AttnArgs& a, int G, size_t lds, int64_t B, hipStream_t s) {
  switch (G) {
    case 1: return launch_attend_t<D, BF16, 1>(a, lds, B, s);
    case 2: return launch_attend_t<D, BF16, 2>(a, lds, B, s);
    case 4: return launch_attend_t<D, BF16, 4>(a, lds, B, s);
    case 8: return launch_attend_t<D, BF16, 8>(a, lds, B, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attend(const AttnArgs& a, int d, bool bf16, int G, size_t lds, int64_t B, hipStream_t s) {
  if (a.n_q <= 0 || B <= 0) return hipSuccess;
  if (d == 128) return bf16 ? launch_attend_g<128, true>(a, G, lds, B, s) : launch_attend_g<128, false>(a, G, lds, B, s);
  if (d == 64) return bf16 ? launch_attend_g<64, true>(a, G, lds, B, s) : launch_attend_g<64, false>(a, G, lds, B, s);
  return hipErrorInvalidValue;
}

}  // namespace recsa
