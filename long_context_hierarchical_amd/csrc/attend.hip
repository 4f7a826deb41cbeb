// RecSA descent + one softmax, one workgroup per (sequence, query, KV head).
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
//   select      the s = min(k, C) largest (S, -i) keys, by an 8-bit radix
//               select over 64-bit keys in LDS (exact, deterministic).
//   softmax     unkept candidates join the online softmax with their node's
//               mean value; kept ones become the next level's parents.
// Token level: the tokens under the kept level-1 nodes plus the trailing
// partial block, all entries; the query sits at C_0, or C_0 - 1 when its own
// token is one of them (causal prefill).
//
// Work layout (256 threads = 4 waves of 64):
//   score phase  D/8 lanes per candidate row, 8 elements (16 B for bf16) per
//                lane: one coalesced row load, the rotate-half partner via a
//                lane shuffle, G partial dot products reduced by shuffles;
//                the G query heads of the KV group share every loaded row.
//   value phase  a wave per entry, D/64 dims per lane; every wave keeps a
//                partial (acc) for all G heads; waves merge at the end.
#include <math.h>

#include "common.hpp"
#include "internal.hpp"

namespace recsa {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

struct Lds {
  uint32_t qraw, qrot, selA, selB, zs, keys, flags, red, hist, nls, misc, fin, total;
};

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline Lds lds_layout(int d, int G, int smax, int csel, int ch0) {
  const uint32_t zcap = static_cast<uint32_t>(csel > ch0 ? csel : ch0);
  Lds L;
  uint32_t o = 0;
  L.qraw = o;  o = align16(o + 4u * G * d);
  L.qrot = o;  o = align16(o + 4u * G * d);
  L.selA = o;  o = align16(o + 4u * smax);
  L.selB = o;  o = align16(o + 4u * smax);
  L.zs = o;    o = align16(o + 4u * G * zcap);
  L.keys = o;  o = align16(o + 8u * csel);
  L.flags = o; o = align16(o + zcap);
  L.red = o;   o = align16(o + 4u * 2 * kWaves * G);
  L.hist = o;  o = align16(o + 4u * 256);
  L.nls = o;   o = align16(o + 8u * (RECSA_MAX_LEVELS + 2));
  L.misc = o;  o = align16(o + 8u * 4);
  L.fin = o;   o = align16(o + 4u * kWaves * G * d);
  L.total = o;
  return L;
}

size_t attend_lds_bytes(int d, int G, int smax, int csel, int ch0) {
  return lds_layout(d, G, smax, csel, ch0).total;
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

// Exact top-s of C unique 64-bit keys: flags[i] = 1 for the s largest.
__device__ void radix_select(const uint64_t* keys, int64_t C, int64_t s, uint8_t* flags,
                             uint32_t* hist, uint64_t* misc) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix = 0, mask = 0;
  int64_t need = s;
  for (int shift = 56; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < C; i += kThreads) {
      const uint64_t k = keys[i];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) c[q] = hist[255 - 4 * lane - q];  // descending digits
      const uint32_t tot = c[0] + c[1] + c[2] + c[3];
      uint32_t inc = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(inc, off);
        if (lane >= off) inc += t;
      }
      const uint32_t exc = inc - tot;
      if (static_cast<int64_t>(exc) < need && need <= static_cast<int64_t>(inc)) {
        uint32_t cum = exc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (static_cast<int64_t>(cum + c[q]) >= need) {
            misc[0] = static_cast<uint64_t>(255 - 4 * lane - q);
            misc[1] = cum;
            misc[2] = c[q];
            break;
          }
          cum += c[q];
        }
      }
    }
    __syncthreads();
    const uint64_t digit = misc[0];
    const int64_t above = static_cast<int64_t>(misc[1]);
    const int64_t cnt = static_cast<int64_t>(misc[2]);
    __syncthreads();
    need -= above;
    prefix |= digit << shift;
    mask |= 0xFFull << shift;
    if (cnt == need) break;  // every key left in this digit is kept
  }
  for (int64_t i = tid; i < C; i += kThreads) flags[i] = (keys[i] & mask) >= prefix ? 1 : 0;
}

template <int D, bool BF16, int G>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttnArgs a) {
  constexpr int RL = D / 8;            // lanes per candidate row (score phase)
  constexpr int RPW = kWave / RL;      // rows per wave
  constexpr int RPI = RPW * kWaves;    // rows per iteration
  constexpr int DPL = D / kWave;       // dims per lane (value phase)
  constexpr int HALF = D / 2;
  constexpr int PV_UNROLL = 4;

  extern __shared__ __align__(16) unsigned char lds[];
  const Lds L = lds_layout(D, G, a.smax, a.csel, a.ch0);
  float* qraw = reinterpret_cast<float*>(lds + L.qraw);
  float* qrot = reinterpret_cast<float*>(lds + L.qrot);
  int32_t* selA = reinterpret_cast<int32_t*>(lds + L.selA);
  int32_t* selB = reinterpret_cast<int32_t*>(lds + L.selB);
  float* zs = reinterpret_cast<float*>(lds + L.zs);
  uint64_t* keys = reinterpret_cast<uint64_t*>(lds + L.keys);
  uint8_t* flags = reinterpret_cast<uint8_t*>(lds + L.flags);
  float* red = reinterpret_cast<float*>(lds + L.red);
  uint32_t* hist = reinterpret_cast<uint32_t*>(lds + L.hist);
  int64_t* nls = reinterpret_cast<int64_t*>(lds + L.nls);
  uint64_t* misc = reinterpret_cast<uint64_t*>(lds + L.misc);
  float* fin = reinterpret_cast<float*>(lds + L.fin);
  const int zcap = a.csel > a.ch0 ? a.csel : a.ch0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t unit = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t j = unit / a.Hkv;
  const int h = static_cast<int>(unit % a.Hkv);
  const int64_t n = a.prefill ? a.q_start + j + 1 : a.n_fixed;
  const int f = a.f;
  const int64_t bh = b * a.Hkv + h;

  const int64_t qbase = ((b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G) * D;
  for (int i = tid; i < G * D; i += kThreads) qraw[i] = load1<BF16>(a.q, qbase + i);
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
  __syncthreads();
  const int T = static_cast<int>(nls[0]);
  const int64_t sel_row0 = ((b * a.n_q + j) * a.Hkv + h) * a.n_levels;
  if (a.sel) {
    for (int lv = T + 1; lv <= a.n_levels; ++lv)
      for (int c = tid; c < a.sel_width; c += kThreads) a.sel[(sel_row0 + lv - 1) * a.sel_width + c] = -1;
  }

  float m_run[G], l_run[G], acc[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.0f;
  }

  // --- helpers over the current candidate map ---------------------------------
  auto rotate_query = [&](int64_t pos) {
    for (int idx = tid; idx < G * HALF; idx += kThreads) {
      const int hh = idx / HALF, i = idx % HALF;
      const float x1 = qraw[hh * D + i], x2 = qraw[hh * D + i + HALF];
      if (a.use_rope) {
        const float2 cs = a.tab[pos * HALF + i];
        const float p1 = x1 * cs.x, p2 = x2 * cs.y, p3 = x2 * cs.x, p4 = x1 * cs.y;
        qrot[hh * D + i] = round_store<BF16>(p1 - p2);
        qrot[hh * D + i + HALF] = round_store<BF16>(p3 + p4);
      } else {
        qrot[hh * D + i] = x1;
        qrot[hh * D + i + HALF] = x2;
      }
    }
  };

  // logits of candidates [c0, c0 + cn) (index = RoPE position) into zs[hh * zcap + r]
  auto score_rows = [&](const void* src, int64_t rowbase, const CandMap& cm, int64_t c0, int64_t cn,
                        bool want_keys) {
    const int sub = lane % RL, rg = lane / RL;
    float qv[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[hh][e] = qrot[hh * D + sub * 8 + e];
    const int pi0 = (sub % (RL / 2)) * 8;
    const bool first_half = sub < RL / 2;
    for (int64_t r0 = 0; r0 < cn; r0 += RPI) {
      const int64_t r = r0 + wave * RPW + rg;
      const bool valid = r < cn;
      const int64_t i = c0 + r;
      float x[8];
      if (valid) {
        load8<BF16>(src, (rowbase + cm(i)) * D + sub * 8, x);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.0f;
      }
      float kx[8];
      if (a.use_rope) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = __shfl_xor(x[e], RL / 2);
        const float4* t4 = reinterpret_cast<const float4*>(a.tab + (valid ? i : 0) * HALF + pi0);
        float cs[16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 t = t4[u];
          cs[4 * u] = t.x; cs[4 * u + 1] = t.y; cs[4 * u + 2] = t.z; cs[4 * u + 3] = t.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = cs[2 * e], s = cs[2 * e + 1];
          const float p1 = x[e] * c, p2 = y[e] * s;
          kx[e] = round_store<BF16>(first_half ? p1 - p2 : p1 + p2);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) kx[e] = x[e];
      }
      float part[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float p = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) p = fmaf(qv[hh][e], kx[e], p);
        part[hh] = p;
      }
#pragma unroll
      for (int off = RL / 2; off >= 1; off >>= 1)
#pragma unroll
        for (int hh = 0; hh < G; ++hh) part[hh] += __shfl_xor(part[hh], off);
      if (valid && sub == 0) {
        float S = 0.0f;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float z = part[hh] * a.scale;
          zs[hh * zcap + r] = z;
          S = S + z;
        }
        if (want_keys) keys[r] = select_key(S, static_cast<uint32_t>(i));
      }
    }
  };

  // fold entries r in [0, cn) (skipping kept ones when use_flags) into the online softmax
  auto softmax_pv = [&](const void* vsrc, int64_t rowbase, const CandMap& cm, int64_t c0, int64_t cn,
                        bool use_flags) {
    float lm[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) lm[hh] = -INFINITY;
    for (int64_t r = tid; r < cn; r += kThreads) {
      if (use_flags && flags[r]) continue;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) lm[hh] = fmaxf(lm[hh], zs[hh * zcap + r]);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      lm[hh] = wave_max(lm[hh]);
      if (lane == 0) red[wave * G + hh] = lm[hh];
    }
    __syncthreads();
    float mnew[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float mx = m_run[hh];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, red[w * G + hh]);
      mnew[hh] = mx;
    }
    float ls[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) ls[hh] = 0.0f;
    for (int64_t r = tid; r < cn; r += kThreads) {
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
      ls[hh] = wave_sum(ls[hh]);
      if (lane == 0) red[(kWaves + wave) * G + hh] = ls[hh];
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float lsum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) lsum += red[(kWaves + w) * G + hh];
      const float alpha = expf(m_run[hh] - mnew[hh]);
      l_run[hh] = l_run[hh] * alpha + lsum;
      m_run[hh] = mnew[hh];
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] *= alpha;
    }
    // value rows: a wave per entry, PV_UNROLL rows in flight
    for (int64_t r0 = wave; r0 < cn; r0 += kWaves * PV_UNROLL) {
      float v[PV_UNROLL][DPL];
      bool live[PV_UNROLL];
#pragma unroll
      for (int u = 0; u < PV_UNROLL; ++u) {
        const int64_t r = r0 + u * kWaves;
        live[u] = r < cn && !(use_flags && flags[r]);
        if (live[u]) {
          loadN<BF16, DPL>(vsrc, (rowbase + cm(c0 + r)) * D + lane * DPL, v[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < PV_UNROLL; ++u) {
        if (!live[u]) continue;
        const int64_t r = r0 + u * kWaves;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float p = zs[hh * zcap + r];
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[hh][e] = fmaf(p, v[u][e], acc[hh][e]);
        }
      }
    }
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
      for (int64_t i = tid; i < C; i += kThreads) sel_new[i] = static_cast<int32_t>(cm(i));
    } else {
      const int64_t rowbase = bh * a.tree.rows[lv];
      rotate_query(C);
      __syncthreads();
      score_rows(a.tree.NK[lv], rowbase, cm, 0, C, s > 0);
      __syncthreads();
      if (s > 0) {
        radix_select(keys, C, s, flags, hist, misc);
      } else {
        for (int64_t i = tid; i < C; i += kThreads) flags[i] = 0;
      }
      __syncthreads();
      if (wave == 0) {
        int64_t cnt = 0;
        for (int64_t base = 0; base < C; base += kWave) {
          const int64_t i = base + lane;
          const bool fl = i < C && flags[i];
          const uint64_t bal = __ballot(fl);
          const int pre = __popcll(bal & ((1ull << lane) - 1ull));
          if (fl) sel_new[cnt + pre] = static_cast<int32_t>(cm(i));
          cnt += __popcll(bal);
        }
      }
      softmax_pv(a.tree.NV[lv], rowbase, cm, 0, C, true);
    }
    __syncthreads();
    if (a.sel) {
      for (int c = tid; c < a.sel_width; c += kThreads)
        a.sel[(sel_row0 + lv - 1) * a.sel_width + c] = c < s ? sel_new[c] : -1;
    }
    int32_t* t = sel_prev;
    sel_prev = sel_new;
    sel_new = t;
    s_prev = s;
    __syncthreads();
  }

  // --- token level -------------------------------------------------------------------
  {
    const int64_t n1 = T >= 1 ? nls[1] : 0;
    const CandMap cm{sel_prev, static_cast<int64_t>(f) * s_prev, static_cast<int64_t>(f) * n1, f};
    const int64_t C0 = cm.n_kids + (n - cm.orph);
    const bool own = a.prefill && C0 > 0 && cm(C0 - 1) == n - 1;
    const int64_t pq = own ? C0 - 1 : C0;
    const int64_t rowbase = bh * a.cap;
    if (C0 > 0) {
      rotate_query(pq);
      __syncthreads();
    }
    for (int64_t c0 = 0; c0 < C0; c0 += a.ch0) {
      const int64_t cn = C0 - c0 < a.ch0 ? C0 - c0 : a.ch0;
      score_rows(a.K, rowbase, cm, c0, cn, false);
      __syncthreads();
      softmax_pv(a.V, rowbase, cm, c0, cn, false);
      __syncthreads();
    }
  }

  // --- merge the waves' partial sums, normalise, write -----------------------------
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) fin[(wave * G + hh) * D + lane * DPL + e] = acc[hh][e];
  __syncthreads();
  const int64_t obase = ((b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G) * D;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int hh = idx / D;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += fin[(w * G) * D + idx];
    float l = 0.0f;
#pragma unroll
    for (int g2 = 0; g2 < G; ++g2) l = (g2 == hh) ? l_run[g2] : l;
    a.out[obase + idx] = l > 0.0f ? sum / l : 0.0f;
  }
  if (a.lse) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (tid == hh) {
        a.lse[(b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G + hh] =
            l_run[hh] > 0.0f ? m_run[hh] + logf(l_run[hh]) : -INFINITY;
      }
    }
  }
}

template <int D, bool BF16, int G>
static hipError_t launch_attend_t(const AttnArgs& a, size_t lds, int64_t B, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.n_q * a.Hkv), static_cast<unsigned>(B));
  hipLaunchKernelGGL((attend_kernel<D, BF16, G>), grid, dim3(kThreads), lds, s, a);
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
