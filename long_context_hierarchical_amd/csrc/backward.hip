// Gradients of RecSA tree attention with the forward pass's selections held fixed.
//
// RecSA abstract ("Recursive Sparse Attention: Million-Token Length Extrapolation at
// Logarithmic Cost"): the mechanism is trained (its pooler is distilled, the model fine-tuned),
// which needs gradients through the tree attention. The kept candidates of each level are a
// discrete choice; they are taken from the forward pass (its `sel` output) and held fixed, and
// the forward's roundings to the storage type are passed straight through. Per unit (sequence,
// query, KV head) with entries e (logit z = scale * <q~, k~_e>, value v_e) and P = exp(z - lse):
//   dz_h   = P_h (dout_h . v_e - dout_h . out_h) + dlse_h P_h
//   dv_e   = sum_h P_h dout_h                              (added to the entry's value row)
//   dk~_e  = scale sum_h dz_h q~_h  -> rot^T at the entry's candidate index (its key row)
//   dq~_h += scale dz_h k~_e        -> rot^T at the level's query position (dq)
// A node's key is W @ m (m the mean of its children's stored keys) and its value the mean of
// its children's values, so the node gradients are pushed down level by level afterwards
// (tree_push_kernel): dW += outer(dkey, m), each child's key gradient += W^T dkey / f, each
// child's value gradient += dvalue / f.
//
// backward_unit_kernel: one wave per unit; d / 8 lanes per candidate row, each holding 4
// rotate-half pairs, so rotations and their transposes need no lane exchange. The candidate list of a level is rebuilt from the kept parents recorded
// one level up; the logit is recomputed from the same rotated, rounded operands. Row gradients
// go out with float32 atomic adds (many queries share the upper levels' nodes); a pass's rows
// are first transposed through LDS so that each atomic instruction covers 64 consecutive floats
// of one row (whole cache lines: 3.6x faster than one instruction per 4-float stride).
#include <math.h>

#include "common.hpp"
#include "internal.hpp"
#include "lanes.hpp"

namespace recsa {

// 4 consecutive storage elements at element `off` -> float
template <bool BF16>
__device__ __forceinline__ void load4s(const void* base, int64_t off, float* x) {
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    x[0] = __uint_as_float(u.x << 16);
    x[1] = __uint_as_float(u.x & 0xFFFF0000u);
    x[2] = __uint_as_float(u.y << 16);
    x[3] = __uint_as_float(u.y & 0xFFFF0000u);
  } else {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
  }
}

size_t backward_unit_lds_bytes(int zcap, int smax) {
  return static_cast<size_t>((zcap + 15) / 16 * 16) + 4u * static_cast<size_t>(smax);
}

template <int D, bool BF16, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void backward_unit_kernel(BwdArgs args) {
  (void)args;
  const BwdArgs& a = *(const BwdArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  constexpr int SL = D / 8;           // lanes per candidate row
  constexpr int SPP = kWave / SL;     // rows per pass
  constexpr int HALF = D / 2;
  __shared__ float qs[G * D];         // raw query heads
  __shared__ float qt[G * D];         // the current level's rotated, rounded query heads
  __shared__ float dos[G * D];        // dout
  __shared__ float dqs[G * D];        // dq, summed over levels
  __shared__ float hs[3 * G];         // lse, dlse, dout . out per head
  __shared__ int64_t nls[RECSA_MAX_LEVELS + 2];
  __shared__ float rst[SPP][2][D];     // a pass's key and value row gradients
  __shared__ int64_t roff[SPP];        // their row offsets (-1: not an entry)
  extern __shared__ __align__(16) unsigned char dyn[];
  uint8_t* flags = dyn;                                                     // kept flags [zcap]
  int32_t* par = reinterpret_cast<int32_t*>(dyn + (a.zcap + 15) / 16 * 16);  // kept parents [smax]

  const int lane = threadIdx.x;
  const int ssub = lane % SL, srg = lane / SL;
  const int64_t unit = blockIdx.x, b = blockIdx.y;
  const int64_t j = unit / a.Hkv;
  const int h = static_cast<int>(unit % a.Hkv);
  const int64_t n = a.causal ? a.q_start + j + 1 : a.n_fixed;
  const int f = a.f;
  const int64_t bh = b * a.Hkv + h;
  const int64_t hbase = (b * a.n_q + j) * a.Hq + static_cast<int64_t>(h) * G;   // first head row
  const float scale = a.scale;

  for (int i = lane; i < G * D; i += kWave) {
    qs[i] = load1<BF16>(a.q, hbase * D + i);
    dos[i] = a.dout[hbase * D + i];
    dqs[i] = 0.0f;
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    float p = 0.0f;
    for (int i = lane; i < D; i += kWave) p = fmaf(a.dout[(hbase + hh) * D + i], a.out[(hbase + hh) * D + i], p);
    const float dd = wave_sum_dpp(p);
    if (lane == 0) {
      hs[hh] = a.lse[hbase + hh];
      hs[G + hh] = a.dlse ? a.dlse[hbase + hh] : 0.0f;
      hs[2 * G + hh] = dd;
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
  const int32_t* selu = a.sel + ((b * a.n_q + j) * a.Hkv + h) * static_cast<int64_t>(a.n_levels) * a.sel_width;

  // the query heads rotated at position p and rounded to the storage type, as the forward
  auto rotate_query = [&](int64_t p) {
    for (int i = lane; i < G * HALF; i += kWave) {
      const int hh = i / HALF, e = i % HALF;
      const float x1 = qs[hh * D + e], x2 = qs[hh * D + HALF + e];
      float lo = x1, hi = x2;
      if (a.use_rope) {
        const float2 cs = a.tab[p * HALF + e];
        const float p1 = x1 * cs.x, p2 = x2 * cs.y, p3 = x2 * cs.x, p4 = x1 * cs.y;
        lo = p1 - p2;
        hi = p3 + p4;
      }
      qt[hh * D + e] = round_store<BF16>(lo);
      qt[hh * D + HALF + e] = round_store<BF16>(hi);
    }
    wave_sync();
  };

  // entries among candidates [0, C) (kept ones skipped when use_flags); candidate i is row
  // cm(i) of krows / vrows and sits at position i; query position qpos. A row is held by SL
  // lanes, each with 4 rotate-half pairs (elements 4 * ssub + e and HALF + 4 * ssub + e); the
  // heads are taken one at a time (each head's logit and gradients depend only on that head).
  auto entries = [&](const void* krows, const void* vrows, float* gk, float* gv, int64_t rowbase, int32_t C,
                     int32_t n_kids, int32_t orph, bool use_flags, int64_t qpos) {
    float dqt[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) dqt[hh][e] = 0.0f;
    for (int32_t r0 = 0; r0 < C; r0 += SPP) {
      const int32_t i = r0 + srg;
      const bool valid = i < C && !(use_flags && flags[i]);
      const int32_t ic = i < C ? i : C - 1;
      int32_t g;
      if (ic < n_kids) g = f * par[ic / f] + ic % f;
      else g = orph + (ic - n_kids);
      const int64_t off = (rowbase + g) * D + 4 * ssub;
      float k4[8], v4[8];
      load4s<BF16>(krows, off, k4);
      load4s<BF16>(krows, off + HALF, k4 + 4);
      load4s<BF16>(vrows, off, v4);
      load4s<BF16>(vrows, off + HALF, v4 + 4);
      float c[4], s[4], o[8];
      if (a.use_rope) {
        const float4* t = reinterpret_cast<const float4*>(a.tab + static_cast<int64_t>(ic) * HALF + 4 * ssub);
        const float4 t0 = t[0], t1 = t[1];
        c[0] = t0.x; s[0] = t0.y; c[1] = t0.z; s[1] = t0.w;
        c[2] = t1.x; s[2] = t1.y; c[3] = t1.z; s[3] = t1.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p1 = k4[e] * c[e], p2 = k4[4 + e] * s[e], p3 = k4[4 + e] * c[e], p4 = k4[e] * s[e];
          o[e] = round_store<BF16>(p1 - p2);
          o[4 + e] = round_store<BF16>(p3 + p4);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[e] = 1.0f;
          s[e] = 0.0f;
          o[e] = k4[e];
          o[4 + e] = k4[4 + e];
        }
      }
      float dk[8], du[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dk[e] = 0.0f;
        du[e] = 0.0f;
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float qv[8], dv8[8];
        const float4* qp = reinterpret_cast<const float4*>(qt + hh * D + 4 * ssub);
        const float4* qp2 = reinterpret_cast<const float4*>(qt + hh * D + HALF + 4 * ssub);
        const float4* dp = reinterpret_cast<const float4*>(dos + hh * D + 4 * ssub);
        const float4* dp2 = reinterpret_cast<const float4*>(dos + hh * D + HALF + 4 * ssub);
        const float4 qa = qp[0], qb = qp2[0], da = dp[0], db = dp2[0];
        qv[0] = qa.x; qv[1] = qa.y; qv[2] = qa.z; qv[3] = qa.w; qv[4] = qb.x; qv[5] = qb.y; qv[6] = qb.z; qv[7] = qb.w;
        dv8[0] = da.x; dv8[1] = da.y; dv8[2] = da.z; dv8[3] = da.w; dv8[4] = db.x; dv8[5] = db.y; dv8[6] = db.z; dv8[7] = db.w;
        float zq = 0.0f, dv = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          zq = fmaf(qv[e], o[e], zq);
          dv = fmaf(dv8[e], v4[e], dv);
        }
        zq = lane_group_sum<SL>(zq);
        dv = lane_group_sum<SL>(dv);
        const float p = valid ? expf(zq * scale - hs[hh]) : 0.0f;
        const float dz = p * (dv - hs[2 * G + hh]) + hs[G + hh] * p;
        const float w = scale * dz;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dk[e] = fmaf(dz, qv[e], dk[e]);
          du[e] = fmaf(p, dv8[e], du[e]);
          dqt[hh][e] = fmaf(w, o[e], dqt[hh][e]);
        }
      }
      // this pass's row gradients through LDS, then added row by row with each wave
      // instruction covering 64 consecutive floats of one row
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float dl = dk[e] * scale, dh = dk[4 + e] * scale;
        rst[srg][0][4 * ssub + e] = dl * c[e] + dh * s[e];
        rst[srg][0][HALF + 4 * ssub + e] = dh * c[e] - dl * s[e];
        rst[srg][1][4 * ssub + e] = du[e];
        rst[srg][1][HALF + 4 * ssub + e] = du[4 + e];
      }
      if (ssub == 0) {
        roff[srg] = valid && gk != nullptr ? (rowbase + g) * D : -1;   // no row gradients wanted: skip
      }
      wave_sync();
#pragma unroll
      for (int r = 0; r < SPP; ++r) {
        const int64_t ro = roff[r];
        if (ro < 0) continue;
#pragma unroll
        for (int e = lane; e < D; e += kWave) {
          unsafeAtomicAdd(gk + ro + e, rst[r][0][e]);
          unsafeAtomicAdd(gv + ro + e, rst[r][1][e]);
        }
      }
      wave_sync();
    }
    // sum over the row groups (lanes with the same slot), back through the query rotation
#pragma unroll
    for (int off = SL; off < kWave; off <<= 1)
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) dqt[hh][e] += __shfl_xor(dqt[hh][e], off);
    if (srg == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float c = 1.0f, s = 0.0f;
        if (a.use_rope) {
          const float2 cs = a.tab[qpos * HALF + 4 * ssub + e];
          c = cs.x;
          s = cs.y;
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float g1 = dqt[hh][e], g2 = dqt[hh][4 + e];
          dqs[hh * D + 4 * ssub + e] += g1 * c + g2 * s;
          dqs[hh * D + HALF + 4 * ssub + e] += g2 * c - g1 * s;
        }
      }
    }
    wave_sync();
  };

  const bool any = hs[0] > -INFINITY;   // no entry at all (n = 0): every gradient is 0
  int32_t s_up = 0;
  for (int lv = T; lv >= 1 && any; --lv) {
    const int32_t n_l = static_cast<int32_t>(nls[lv]), n_up = static_cast<int32_t>(nls[lv + 1]);
    const int32_t n_kids = f * s_up, orph = f * n_up;
    const int32_t C = n_kids + (n_l - orph);
    const int32_t* row = selu + static_cast<int64_t>(lv - 1) * a.sel_width;
    int32_t s = 0;
    for (int c0 = 0; c0 < a.sel_width; c0 += kWave) {
      const int c = c0 + lane;
      s += __popcll(__ballot(c < a.sel_width && row[c < a.sel_width ? c : 0] >= 0));
    }
    if (s < C) {
      for (int32_t i = lane; i < C; i += kWave) flags[i] = 0;
      wave_sync();
      for (int32_t c = lane; c < s; c += kWave) {
        const int32_t id = row[c];
        int32_t idx;
        if (id < orph) {
          const int32_t p = id / f;
          int32_t lo = 0, hi = s_up;   // rank of p among the kept parents (ascending)
          while (lo < hi) {
            const int32_t mid = (lo + hi) >> 1;
            if (par[mid] < p) lo = mid + 1;
            else hi = mid;
          }
          idx = f * lo + (id - f * p);
        } else {
          idx = n_kids + (id - orph);
        }
        flags[idx] = 1;
      }
      wave_sync();
      rotate_query(C);
      entries(a.tree.NK[lv], a.tree.NV[lv], a.gNK[lv], a.gNV[lv], bh * a.tree.rows[lv], C, n_kids, orph, true, C);
    }
    for (int32_t c = lane; c < s; c += kWave) par[c] = row[c];
    wave_sync();
    s_up = s;
  }
  if (any) {
    const int32_t n1 = T >= 1 ? static_cast<int32_t>(nls[1]) : 0;
    const int32_t n_kids = f * s_up, orph = f * n1;
    const int32_t C0 = n_kids + (static_cast<int32_t>(n) - orph);
    int32_t last = -1;
    if (C0 > 0) last = C0 - 1 < n_kids ? f * par[(C0 - 1) / f] + (C0 - 1) % f : orph + (C0 - 1 - n_kids);
    const bool own = a.causal && C0 > 0 && last == n - 1;
    const int64_t pq = own ? C0 - 1 : C0;
    if (C0 > 0) {
      rotate_query(pq);
      entries(a.K, a.V, a.dK, a.dV, bh * a.cap, C0, n_kids, orph, false, pq);
    }
  }
  for (int i = lane; i < G * D; i += kWave) a.dq[hbase * D + i] = dqs[i];
}

template <int D, bool BF16, int G>
static hipError_t launch_bwd_t(const BwdArgs& a, int64_t B, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.n_q * a.Hkv), static_cast<unsigned>(B));
  hipLaunchKernelGGL((backward_unit_kernel<D, BF16, G>), grid, dim3(kWave), backward_unit_lds_bytes(a.zcap, a.smax),
                     s, a);
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_bwd_g(const BwdArgs& a, int G, int64_t B, hipStream_t s) {
  switch (G) {
    case 1: return launch_bwd_t<D, BF16, 1>(a, B, s);
    case 2: return launch_bwd_t<D, BF16, 2>(a, B, s);
    case 4: return launch_bwd_t<D, BF16, 4>(a, B, s);
    case 8: return launch_bwd_t<D, BF16, 8>(a, B, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_backward_units(const BwdArgs& a, int d, bool bf16, int G, int64_t B, hipStream_t s) {
  if (a.n_q <= 0 || B <= 0) return hipSuccess;
  if (d == 128) return bf16 ? launch_bwd_g<128, true>(a, G, B, s) : launch_bwd_g<128, false>(a, G, B, s);
  if (d == 64) return bf16 ? launch_bwd_g<64, true>(a, G, B, s) : launch_bwd_g<64, false>(a, G, B, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- top-down push

// One level. Persistent workgroups take tiles of NB nodes of one slice in turn (the grid strides
// over (slice, tile) pairs). Per tile: the nodes' key gradients a go to LDS (a node whose key
// and value gradients are both 0 is skipped); each thread sums one 16-byte piece of one node's
// children in child order and divides by f (the forward's m); thread t adds
// sum_nodes a[t / TPR] * m[...] into its CPT entries of row t / TPR of dW; W^T a comes from W
// in LDS (bf16 storage; float32 W is read through the cache); then each thread adds its
// 4-float pieces of W^T a / f and of the value gradient / f to every child, as float4
// read-modify-writes (a child has one parent, so nothing else writes it in this launch).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void tree_push_kernel(TreePushArgs a) {
  constexpr int NT = 256, NB = 16;
  constexpr int TPR = NT / D, CPT = D / TPR;     // dW: threads per row, columns per thread
  constexpr int NPG = NB / TPR;                  // W^T a: nodes per thread
  constexpr int EPC = 8;                         // elements per child piece (16 bytes of bf16)
  constexpr int PPR = D / EPC;                   // pieces per row
  constexpr int Q4 = D / 4;                      // float4 pieces per row
  __shared__ uint16_t Ws[BF16 ? D * D : 1];
  __shared__ float ag[NB][D], mg[NB][D], dmg[NB][D];
  __shared__ int touched[NB];
  const int tid = threadIdx.x;
  const int f = a.f;
  const float ff = static_cast<float>(f);
  const bool pow2 = (f & (f - 1)) == 0;
  const float inv_f = 1.0f / ff;
  if constexpr (BF16) {
    for (int i = tid; i < D * D / 8; i += NT)
      reinterpret_cast<uint4*>(Ws)[i] = reinterpret_cast<const uint4*>(a.W)[i];
  }
  const int wr = tid / TPR, wc0 = (tid % TPR) * CPT;
  float dw[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) dw[c] = 0.0f;
  const int64_t tiles = (a.n_nodes + NB - 1) / NB;
  for (int64_t job = blockIdx.x; job < tiles * a.BH; job += gridDim.x) {
    const int64_t slice = job / tiles, tile = job % tiles;
    const int64_t g0 = tile * NB;
    if (tid < NB) touched[tid] = 0;
    __syncthreads();
    for (int idx = tid; idx < NB * Q4; idx += NT) {
      const int nd = idx / Q4, q = idx % Q4;
      float4 va = make_float4(0.0f, 0.0f, 0.0f, 0.0f), vb = va;
      if (g0 + nd < a.n_nodes) {
        va = reinterpret_cast<const float4*>(a.gk + (slice * a.rows + g0 + nd) * D)[q];
        vb = reinterpret_cast<const float4*>(a.gv + (slice * a.rows + g0 + nd) * D)[q];
      }
      reinterpret_cast<float4*>(ag[nd])[q] = va;
      if (va.x != 0.0f || va.y != 0.0f || va.z != 0.0f || va.w != 0.0f || vb.x != 0.0f || vb.y != 0.0f ||
          vb.z != 0.0f || vb.w != 0.0f)
        touched[nd] = 1;
    }
    __syncthreads();
    // m: the forward's mean of the children's stored keys (child order, float32, / f)
    for (int idx = tid; idx < NB * PPR; idx += NT) {
      const int nd = idx / PPR, pc = idx % PPR;
      float m[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) m[e] = 0.0f;
      if (touched[nd]) {
        const int64_t cbase = (slice * a.child_rows + (g0 + nd) * f) * D + pc * EPC;
        for (int c = 0; c < f; ++c) {
          float x[EPC];
          load8<BF16>(a.childK, cbase + static_cast<int64_t>(c) * D, x);
#pragma unroll
          for (int e = 0; e < EPC; ++e) m[e] = m[e] + x[e];
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e) m[e] = pow2 ? m[e] * inv_f : m[e] / ff;
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) mg[nd][pc * EPC + e] = m[e];
    }
    __syncthreads();
#pragma unroll 1
    for (int nd = 0; nd < NB; ++nd) {
      if (!touched[nd]) continue;
      const float ai = ag[nd][wr];
#pragma unroll
      for (int c = 0; c < CPT; ++c) dw[c] = fmaf(ai, mg[nd][wc0 + c], dw[c]);
    }
    {
      const int i = tid % D, nd0 = (tid / D) * NPG;
      float dm[NPG];
#pragma unroll
      for (int u = 0; u < NPG; ++u) dm[u] = 0.0f;
#pragma unroll 4
      for (int k = 0; k < D; ++k) {
        float w;
        if constexpr (BF16) w = __uint_as_float(static_cast<uint32_t>(Ws[k * D + i]) << 16);
        else w = static_cast<const float*>(a.W)[static_cast<int64_t>(k) * D + i];
#pragma unroll
        for (int u = 0; u < NPG; ++u) dm[u] = fmaf(w, ag[nd0 + u][k], dm[u]);
      }
#pragma unroll
      for (int u = 0; u < NPG; ++u) dmg[nd0 + u][i] = dm[u] / ff;
    }
    __syncthreads();
    for (int idx = tid; idx < NB * Q4 && a.ck != nullptr; idx += NT) {
      const int nd = idx / Q4, q = idx % Q4;
      if (!touched[nd]) continue;
      const float4 dk = reinterpret_cast<const float4*>(dmg[nd])[q];
      float4 dv = reinterpret_cast<const float4*>(a.gv + (slice * a.rows + g0 + nd) * D)[q];
      dv = make_float4(dv.x / ff, dv.y / ff, dv.z / ff, dv.w / ff);
      const int64_t cbase = (slice * a.child_rows + (g0 + nd) * f) * D;
      for (int c = 0; c < f; ++c) {
        float4* pk = reinterpret_cast<float4*>(a.ck + cbase + static_cast<int64_t>(c) * D) + q;
        float4* pv = reinterpret_cast<float4*>(a.cv + cbase + static_cast<int64_t>(c) * D) + q;
        const float4 ok = *pk, ov = *pv;
        *pk = make_float4(ok.x + dk.x, ok.y + dk.y, ok.z + dk.z, ok.w + dk.w);
        *pv = make_float4(ov.x + dv.x, ov.y + dv.y, ov.z + dv.z, ov.w + dv.w);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c)
    if (dw[c] != 0.0f) unsafeAtomicAdd(a.dW + static_cast<int64_t>(wr) * D + wc0 + c, dw[c]);
}

static int push_grid() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return 2 * cus;
}

template <int D, bool BF16>
static hipError_t launch_push_t(const TreePushArgs& a, hipStream_t s) {
  if (a.n_nodes <= 0 || a.BH <= 0) return hipSuccess;
  const int64_t jobs = (a.n_nodes + 15) / 16 * a.BH;
  const int64_t g = jobs < push_grid() ? jobs : push_grid();
  hipLaunchKernelGGL((tree_push_kernel<D, BF16>), dim3(static_cast<unsigned>(g)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tree_push(const TreePushArgs& a, int d, bool bf16, hipStream_t s) {
  if (d == 128) return bf16 ? launch_push_t<128, true>(a, s) : launch_push_t<128, false>(a, s);
  if (d == 64) return bf16 ? launch_push_t<64, true>(a, s) : launch_push_t<64, false>(a, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- zero fill

__global__ __launch_bounds__(256) void fill_zero_kernel(float4* p, int64_t n4) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t n4 = n / 4;   // n is a multiple of 4 (whole rows of d floats)
  const int64_t blocks = (n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<float4*>(p), n4);
  return hipGetLastError();
}

}  // namespace recsa
