// RecSA descent + one softmax: one wave (64 lanes) per (sequence, query, KV head).
//
// RecSA abstract ("Recursive Sparse Attention: Million-Token Length
// Extrapolation at Logarithmic Cost"): a query keeps at most k candidates per
// level above the tokens, so it reads O(log L) entries; every entry's RoPE
// position is its index among its level's candidates; the summaries of the
// candidates it does not keep share one softmax with the exact tokens.
// Explainer page ("Recursive Sparse Attention RecSA: Million-Token Context
// Extrapolation at Logarithmic Cost", section "Core Idea"): coarse filtering
// at the upper levels, then level by level down to the tokens.
//
// Per level (top to bottom):
//   candidates  children of the nodes kept one level up (ascending), then the
//               nodes without a complete parent; at the top every node.
//   score       each candidate key rotated at its index i and rounded to the
//               storage type; the query heads rotated at C and rounded; the
//               logit z = scale * <q~, k~> per head (float32, any order), the
//               group score S = sum over the G heads of the KV group.
//   select      the s = min(k, C) largest (S, -i) keys: s rounds of a wave-wide
//               64-bit max (exact, deterministic, lowest index wins ties).
//   softmax     unkept candidates join the online softmax with their node's
//               mean value; kept ones become the next level's parents.
// Token level: the tokens under the kept level-1 nodes plus the trailing
// partial block, all entries; the query sits at C_0, or C_0 - 1 when its own
// token is one of them (causal prefill).
//
// A unit is a dependent chain of T + 1 rounds, so the kernel runs one wave per
// unit with no workgroup barrier and lets many independent units share a CU.
// Lane layout: in the score phase D/16 lanes per candidate row, a lane holding
// elements [8s, 8s+8) and their rotate-half partners [D/2 + 8s, ...), so the
// rotation needs no lane exchange and the per-row reduction is 3 (d=128)
// shuffle steps; bf16 operands are rounded and packed by v_cvt_pk_bf16_f32 and
// dotted by v_dot2 (the G query heads share each loaded row). In the value
// phase D/8 lanes per row, a lane holding elements [8s, 8s+8).
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace recsa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest, ties to even) and pack them.
__device__ __forceinline__ bf16x2_t pack_bf16_rne(float lo, float hi) {
  return __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(static_cast<uint32_t>(v)), m));
  const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(static_cast<uint32_t>(v >> 32)), m));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

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

struct Lds {
  uint32_t q, zs, sc, flags, selA, selB, nls, total;
};

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline Lds lds_layout(int d, int G, int smax, int zcap) {
  Lds L;
  uint32_t o = 0;
  L.q = o;     o = align16(o + 4u * G * d);         // raw query heads of the KV group
  L.zs = o;    o = align16(o + 4u * G * zcap);      // logits, then softmax weights, [G][zcap]
  L.sc = o;    o = align16(o + 4u * zcap);          // group scores
  L.flags = o; o = align16(o + zcap);               // kept flags
  L.selA = o;  o = align16(o + 4u * smax);          // kept node ids, two buffers
  L.selB = o;  o = align16(o + 4u * smax);
  L.nls = o;   o = align16(o + 8u * (RECSA_MAX_LEVELS + 2));
  L.total = o;
  return L;
}

size_t attend_lds_bytes(int d, int G, int smax, int zcap) {
  return lds_layout(d, G, smax, zcap).total;
}

// Candidate index -> node (or token) id: children of the kept parents, then orphans.
struct CandMap {
  const int32_t* parents;
  int64_t n_kids;   // f * (number of kept parents)
  int64_t orph;     // first orphan id
  int f;
  __device__ __forceinline__ int64_t operator()(int64_t i) const {
    return i < n_kids ? static_cast<int64_t>(f) * parents[i / f] + i % f : orph + (i - n_kids);
  }
};

template <int D, bool BF16, int G>
__global__ __launch_bounds__(64) void attend_kernel(AttnArgs a) {
  constexpr int RL = D / 8;            // lanes per row, value phase (8 elements per lane)
  constexpr int RPP = kWave / RL;      // rows per pass, value phase
  constexpr int SL = D / 16;           // lanes per row, score phase (8 rotate-half pairs per lane)
  constexpr int SPP = kWave / SL;      // rows per pass, score phase
  constexpr int HALF = D / 2;
  constexpr int PV_UNROLL = 2;

  extern __shared__ __align__(16) unsigned char lds[];
  const int zcap = a.zcap;
  const Lds L = lds_layout(D, G, a.smax, zcap);
  float* qs = reinterpret_cast<float*>(lds + L.q);
  float* zs = reinterpret_cast<float*>(lds + L.zs);
  float* sc = reinterpret_cast<float*>(lds + L.sc);
  uint8_t* flags = reinterpret_cast<uint8_t*>(lds + L.flags);
  int32_t* selA = reinterpret_cast<int32_t*>(lds + L.selA);
  int32_t* selB = reinterpret_cast<int32_t*>(lds + L.selB);
  int64_t* nls = reinterpret_cast<int64_t*>(lds + L.nls);

  const int lane = threadIdx.x;
  const int sub = lane % RL, rg = lane / RL;       // value phase
  const int ssub = lane % SL, srg = lane / SL;     // score phase
  const int64_t unit = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t j = unit / a.Hkv;
  const int h = static_cast<int>(unit % a.Hkv);
  const int64_t n = a.prefill ? a.q_start + j + 1 : a.n_fixed;
  const int f = a.f;
  const int64_t bh = b * a.Hkv + h;

  // raw query heads of the KV group -> LDS (float)
  {
    const int64_t qbase = ((b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G) * D;
    for (int i = lane * 4; i < G * D; i += kWave * 4) {
      float x[4];
      load4<BF16>(a.q, qbase + i, x);
      *reinterpret_cast<float4*>(qs + i) = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
  if (lane == 0) {
    int T = 0;
    int64_t m = n / f;
    while (m >= 1 && T < RECSA_MAX_LEVELS) {
      nls[++T] = m;
      m /= f;
    }
    nls[T + 1] = 0;
    nls[0] = T;
  }
  wave_sync();
  const int T = static_cast<int>(nls[0]);
  const int64_t sel_row0 = ((b * a.n_q + j) * a.Hkv + h) * a.n_levels;
  if (a.sel) {
    for (int lv = T + 1; lv <= a.n_levels; ++lv)
      for (int c = lane; c < a.sel_width; c += kWave) a.sel[(sel_row0 + lv - 1) * a.sel_width + c] = -1;
  }

  float m_run[G], l_run[G], acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;
  }

  // rotated query operands for the current level: this lane's 8 rotate-half pairs
  // (elements 8*ssub + e and HALF + 8*ssub + e, e < 8) of every head
  bf16x2_t qp[G][8];   // bf16: packed (lo0,lo1), (lo2,lo3), .., (hi6,hi7)
  float qf[G][16];     // f32: lo0..lo7, hi0..hi7
  auto rotate_query = [&](int64_t pos) {
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
      if constexpr (BF16) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          qp[hh][u] = pack_bf16_rne(lo[2 * u], lo[2 * u + 1]);
          qp[hh][4 + u] = pack_bf16_rne(hi[2 * u], hi[2 * u + 1]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qf[hh][e] = lo[e];
          qf[hh][8 + e] = hi[e];
        }
      }
    }
  };

  // logits of candidates [c0, c0 + cn) (index = RoPE position) -> zs[hh * zcap + r], sc[r]
  auto score_rows = [&](const void* src, int64_t rowbase, const CandMap& cm, int64_t c0, int64_t cn) {
    for (int64_t r0 = 0; r0 < cn; r0 += SPP) {
      const int64_t r = r0 + srg;
      const bool valid = r < cn;
      const int64_t i = c0 + r;
      float klo[8], khi[8];
      if (valid) {
        const int64_t off = (rowbase + cm(i)) * D + 8 * ssub;
        load8<BF16>(src, off, klo);
        load8<BF16>(src, off + HALF, khi);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { klo[e] = 0.0f; khi[e] = 0.0f; }
      }
      float olo[8], ohi[8];
      if (a.use_rope) {
        const float4* t = reinterpret_cast<const float4*>(a.tab + (valid ? i : 0) * HALF + 8 * ssub);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 tv = t[u];
          const float cc[2] = {tv.x, tv.z}, ss[2] = {tv.y, tv.w};
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
          float p = 0.0f;
#pragma unroll
          for (int u = 0; u < 8; ++u) p = __builtin_amdgcn_fdot2_f32_bf16(kp[u], qp[hh][u], p, false);
          part[hh] = p;
        }
      } else {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float p = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) p = fmaf(qf[hh][e], olo[e], p);
#pragma unroll
          for (int e = 0; e < 8; ++e) p = fmaf(qf[hh][8 + e], ohi[e], p);
          part[hh] = p;
        }
      }
#pragma unroll
      for (int off = SL / 2; off >= 1; off >>= 1)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) part[hh] += __shfl_xor(part[hh], off);
      if (valid && ssub == 0) {
        float S = 0.0f;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float z = part[hh] * a.scale;
          zs[hh * zcap + r] = z;
          S = S + z;
        }
        sc[r] = S;
      }
    }
    wave_sync();
  };

  // flags[r] = 1 for the s largest (S, -r) keys among r < C
  auto select_top = [&](int64_t C, int64_t s) {
    for (int64_t r = lane; r < C; r += kWave) flags[r] = 0;
    wave_sync();
    uint64_t best = 0;
    int64_t slot = -1;
    for (int64_t r = lane; r < C; r += kWave) {
      const uint64_t k = select_key(sc[r], static_cast<uint32_t>(r));
      if (k > best) { best = k; slot = r; }
    }
    for (int64_t it = 0; it < s; ++it) {
      uint64_t w = best;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t o = shfl_xor_u64(w, off);
        w = o > w ? o : w;
      }
      if (best == w) {            // keys are unique: exactly one lane holds the maximum
        flags[slot] = 1;
        best = 0;
        slot = -1;
        for (int64_t r = lane; r < C; r += kWave) {
          if (flags[r]) continue;
          const uint64_t k = select_key(sc[r], static_cast<uint32_t>(r));
          if (k > best) { best = k; slot = r; }
        }
      }
    }
    wave_sync();
  };

  // fold entries r < cn (skipping kept ones when use_flags) into the online softmax
  auto softmax_pv = [&](const void* vsrc, int64_t rowbase, const CandMap& cm, int64_t c0, int64_t cn,
                        bool use_flags) {
    float mnew[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) mnew[hh] = -INFINITY;
    for (int64_t r = lane; r < cn; r += kWave) {
      if (use_flags && flags[r]) continue;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) mnew[hh] = fmaxf(mnew[hh], zs[hh * zcap + r]);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) mnew[hh] = fmaxf(m_run[hh], wave_max(mnew[hh]));
    float ls[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) ls[hh] = 0.0f;
    for (int64_t r = lane; r < cn; r += kWave) {
      const bool skip = use_flags && flags[r];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = skip ? 0.0f : expf(zs[hh * zcap + r] - mnew[hh]);
        zs[hh * zcap + r] = p;
        ls[hh] += p;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float lsum = wave_sum(ls[hh]);
      const float alpha = expf(m_run[hh] - mnew[hh]);
      l_run[hh] = l_run[hh] * alpha + lsum;
      m_run[hh] = mnew[hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
    }
    wave_sync();
    for (int64_t r0 = 0; r0 < cn; r0 += RPP * PV_UNROLL) {
      float v[PV_UNROLL][8];
      bool live[PV_UNROLL];
#pragma unroll
      for (int u = 0; u < PV_UNROLL; ++u) {
        const int64_t r = r0 + u * RPP + rg;
        live[u] = r < cn && !(use_flags && flags[r]);
        if (live[u]) load8<BF16>(vsrc, (rowbase + cm(c0 + r)) * D + 8 * sub, v[u]);
      }
#pragma unroll
      for (int u = 0; u < PV_UNROLL; ++u) {
        if (!live[u]) continue;
        const int64_t r = r0 + u * RPP + rg;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = zs[hh * zcap + r];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(p, v[u][e], acc[hh][e]);
        }
      }
    }
    wave_sync();
  };

  // --- levels T .. 1 -------------------------------------------------------------
  int32_t* sel_prev = selA;
  int32_t* sel_new = selB;
  int64_t s_prev = 0;
  for (int lv = T; lv >= 1; --lv) {
    const int64_t n_l = nls[lv], n_up = nls[lv + 1];
    const CandMap cm{sel_prev, static_cast<int64_t>(f) * s_prev, static_cast<int64_t>(f) * n_up, f};
    const int64_t C = cm.n_kids + (n_l - cm.orph);
    const int64_t kl = a.k.k[lv];
    const int64_t s = kl < C ? kl : C;
    if (s == C) {
      for (int64_t i = lane; i < C; i += kWave) sel_new[i] = static_cast<int32_t>(cm(i));
      wave_sync();
    } else {
      const int64_t rowbase = bh * a.tree.rows[lv];
      rotate_query(C);
      score_rows(a.tree.NK[lv], rowbase, cm, 0, C);
      if (s > 0) {
        select_top(C, s);
      } else {
        for (int64_t r = lane; r < C; r += kWave) flags[r] = 0;
        wave_sync();
      }
      int64_t cnt = 0;
      for (int64_t base = 0; base < C; base += kWave) {
        const int64_t i = base + lane;
        const bool fl = i < C && flags[i];
        const uint64_t bal = __ballot(fl);
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        if (fl) sel_new[cnt + pre] = static_cast<int32_t>(cm(i));
        cnt += __popcll(bal);
      }
      wave_sync();
      softmax_pv(a.tree.NV[lv], rowbase, cm, 0, C, true);
    }
    if (a.sel) {
      for (int c = lane; c < a.sel_width; c += kWave)
        a.sel[(sel_row0 + lv - 1) * a.sel_width + c] = c < s ? sel_new[c] : -1;
    }
    int32_t* t = sel_prev;
    sel_prev = sel_new;
    sel_new = t;
    s_prev = s;
  }

  // --- token level -------------------------------------------------------------------
  {
    const int64_t n1 = T >= 1 ? nls[1] : 0;
    const CandMap cm{sel_prev, static_cast<int64_t>(f) * s_prev, static_cast<int64_t>(f) * n1, f};
    const int64_t C0 = cm.n_kids + (n - cm.orph);
    const bool own = a.prefill && C0 > 0 && cm(C0 - 1) == n - 1;
    const int64_t pq = own ? C0 - 1 : C0;
    const int64_t rowbase = bh * a.cap;
    if (C0 > 0) rotate_query(pq);
    for (int64_t c0 = 0; c0 < C0; c0 += zcap) {
      const int64_t cn = C0 - c0 < zcap ? C0 - c0 : zcap;
      score_rows(a.K, rowbase, cm, c0, cn);
      softmax_pv(a.V, rowbase, cm, c0, cn, false);
    }
  }

  // --- merge the row groups' partial sums, normalise, write ---------------------------
#pragma unroll
  for (int off = RL; off < kWave; off <<= 1)
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], off);
  const int64_t obase = ((b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G) * D;
  if (rg == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float l = l_run[hh];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      float4* o = reinterpret_cast<float4*>(a.out + obase + hh * D + 8 * sub);
      o[0] = make_float4(acc[hh][0] * inv, acc[hh][1] * inv, acc[hh][2] * inv, acc[hh][3] * inv);
      o[1] = make_float4(acc[hh][4] * inv, acc[hh][5] * inv, acc[hh][6] * inv, acc[hh][7] * inv);
    }
  }
  if (a.lse) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (lane == hh) {
        a.lse[(b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G + hh] =
            l_run[hh] > 0.0f ? m_run[hh] + logf(l_run[hh]) : -INFINITY;
      }
    }
  }
}

template <int D, bool BF16, int G>
static hipError_t launch_attend_t(const AttnArgs& a, size_t lds, int64_t B, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.n_q * a.Hkv), static_cast<unsigned>(B));
  hipLaunchKernelGGL((attend_kernel<D, BF16, G>), grid, dim3(kWave), lds, s, a);
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
