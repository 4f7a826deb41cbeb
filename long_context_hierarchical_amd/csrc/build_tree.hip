// Tree build: pooled node keys and mean node values, one level per launch.
//
// RecSA abstract ("Recursive Sparse Attention: Million-Token Length
// Extrapolation at Logarithmic Cost"): every node summarises its subtree with
// one key from the layer's pooler, shared by all levels, and one mean-pooled
// value. Here the pooler is key = W @ m, m the mean of the node's f children's
// stored keys; the value is the mean of the children's stored values.
//
// HBM-bound: a tile reads f * (nodes per tile) child rows of K and V once and
// writes 1/f as many node rows. Each workgroup keeps W (transposed, float32)
// in LDS and loops over tiles, so W is fetched once per workgroup.
//
// Rounding (decides selections, so it is fixed): child sums in child order in
// float32, one correctly rounded division by f (an exact multiply by 1/f when f
// is a power of two: same value), then for each output
// acc = fmaf(W[i][j], m[j], acc) over j = 0..d-1 (one rounding per term; the
// file is compiled with -ffp-contract=off so nothing else is fused), rounded to
// the storage type.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace recsa {

// Workgroup barrier that orders LDS only: the waves' outstanding global loads (the next
// tile's prefetch) and stores stay in flight across it, where __syncthreads() would wait for
// all of them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Streaming accesses: the child rows are read once and the node rows written once per build, so
// both go through the caches with the non-temporal hint (no allocation for reuse); measured, the
// full build at 512K took 1.67 ms with the hint on loads and stores against 1.79 ms without.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));

// 8 storage elements (exact in the storage type) stored non-temporally at element `off`.
template <bool BF16>
__device__ __forceinline__ void store8_nt(void* base, int64_t off, const float (&x)[8]) {
  if constexpr (BF16) {
    nt_u32x4 u;
    u.x = (__float_as_uint(x[0]) >> 16) | (__float_as_uint(x[1]) & 0xFFFF0000u);
    u.y = (__float_as_uint(x[2]) >> 16) | (__float_as_uint(x[3]) & 0xFFFF0000u);
    u.z = (__float_as_uint(x[4]) >> 16) | (__float_as_uint(x[5]) & 0xFFFF0000u);
    u.w = (__float_as_uint(x[6]) >> 16) | (__float_as_uint(x[7]) & 0xFFFF0000u);
    __builtin_nontemporal_store(u, reinterpret_cast<nt_u32x4*>(static_cast<uint16_t*>(base) + off));
  } else {
    nt_f32x4* p = reinterpret_cast<nt_f32x4*>(static_cast<float*>(base) + off);
    __builtin_nontemporal_store(nt_f32x4{x[0], x[1], x[2], x[3]}, p);
    __builtin_nontemporal_store(nt_f32x4{x[4], x[5], x[6], x[7]}, p + 1);
  }
}

template <bool BF16>
__device__ __forceinline__ void store1_nt(void* base, int64_t off, float x) {
  if constexpr (BF16) {
    __builtin_nontemporal_store(static_cast<uint16_t>(__float_as_uint(x) >> 16), static_cast<uint16_t*>(base) + off);
  } else {
    __builtin_nontemporal_store(x, static_cast<float*>(base) + off);
  }
}

template <bool BF16>
struct Chunk;  // raw storage of 8 consecutive elements
template <>
struct Chunk<true> {
  uint4 u;
  __device__ __forceinline__ void load(const void* base, int64_t off) {   // streamed child rows
    const nt_u32x4 t =
        __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(static_cast<const uint16_t*>(base) + off));
    u = make_uint4(t.x, t.y, t.z, t.w);
  }
  __device__ __forceinline__ void load_cached(const void* base, int64_t off) {
    u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  }
  __device__ __forceinline__ void add_to(float (&s)[8]) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      s[2 * k] = s[2 * k] + __uint_as_float(w[k] << 16);
      s[2 * k + 1] = s[2 * k + 1] + __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
};
template <>
struct Chunk<false> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* base, int64_t off) {   // streamed child rows
    const nt_f32x4* p = reinterpret_cast<const nt_f32x4*>(static_cast<const float*>(base) + off);
    const nt_f32x4 x = __builtin_nontemporal_load(p), y = __builtin_nontemporal_load(p + 1);
    a = make_float4(x.x, x.y, x.z, x.w);
    b = make_float4(y.x, y.y, y.z, y.w);
  }
  __device__ __forceinline__ void load_cached(const void* base, int64_t off) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    a = p[0];
    b = p[1];
  }
  __device__ __forceinline__ void add_to(float (&s)[8]) const {
    s[0] = s[0] + a.x; s[1] = s[1] + a.y; s[2] = s[2] + a.z; s[3] = s[3] + a.w;
    s[4] = s[4] + b.x; s[5] = s[5] + b.y; s[6] = s[6] + b.z; s[7] = s[7] + b.w;
  }
};

template <int D>
struct PoolGeom {
  static constexpr int T = 512;           // threads per workgroup
  static constexpr int CH = D / 8;        // 8-element chunks per row (phase 1)
  static constexpr int NPW = T / CH;      // nodes per tile: 32 (d=128) / 64 (d=64)
  static constexpr int OG = D / 4;        // groups of 4 outputs (phase 2)
  static constexpr int NGR = T / OG;      // node groups
  static constexpr int NPT = NPW / NGR;   // nodes per thread
};

// One pass over level-l nodes [g_lo, g_hi) of every (sequence, KV head); tiles of NPW
// nodes aligned to multiples of NPW. Phase 1: a thread sums one 8-element chunk of one
// node's children in child order; the first PF children of its next tile are loaded into
// registers before the matrix-vector phase of the current tile, the rest in batches of PF.
// Phase 2: W @ m for the tile's nodes from LDS. With FUSE (f divides NPW) the tile holds
// NPW / f whole parents at level l+1, which are built in the same pass from the tile's node
// rows as stored (re-read through the cache in 16-byte chunks; rows below g_lo come from
// earlier calls).
// Two workgroups of 512 threads per CU (W and the tile's key means fill the LDS), at most
// 128 VGPRs each.
template <int D, bool BF16, bool FUSE>
__global__ __launch_bounds__(512, 4) void pool_kernel(PoolArgs a) {
  using Gm = PoolGeom<D>;
  constexpr int T = Gm::T, CH = Gm::CH, NPW = Gm::NPW, NPT = Gm::NPT;
  constexpr int PF = BF16 ? 2 : 1;        // children per register batch
  static_assert(NPT == 2, "phase 2 tiles 4 outputs x 2 nodes per thread");
  // bf16 storage keeps W as stored (bf16, exact) and stages the tile's node rows for the
  // fused parents; float32 storage keeps W as float32 and re-reads the node rows
  constexpr bool STAGE = BF16 && FUSE;
  using WT = typename std::conditional<BF16, uint16_t, float>::type;
  __shared__ WT wt[D][D];                 // wt[j][i] = W[i][j]
  __shared__ float mt[D][NPW];            // mt[j][node] = mean of the node's child keys
  __shared__ uint16_t k1s[STAGE ? NPW : 1][D];   // the tile's node keys / values (bf16 bits)
  __shared__ uint16_t v1s[STAGE ? NPW : 1][D];
  float* const m2s = &mt[0][0];           // parents' key means [P][D] reuse mt after phase 2
  auto wload = [&](int j, int i) -> float {
    if constexpr (BF16) return bf16_to_f32(wt[j][i]);
    else return wt[j][i];
  };

  const int tid = threadIdx.x;
  const int f = a.f;
  const int64_t base0 = (a.g_lo / NPW) * NPW;
  const int64_t tiles_per_bh = (a.g_hi - base0 + NPW - 1) / NPW;
  const int64_t total = tiles_per_bh * a.BH;

  for (int idx = tid; idx < D * CH; idx += T) {
    const int i = idx / CH, j0 = (idx % CH) * 8;
    float x[8];
    load8<BF16>(a.W, static_cast<int64_t>(i) * D + j0, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (BF16) wt[j0 + e][i] = static_cast<uint16_t>(__float_as_uint(x[e]) >> 16);
      else wt[j0 + e][i] = x[e];
    }
  }

  const float ff = static_cast<float>(f);
  const bool pow2 = (f & (f - 1)) == 0;
  const float inv_f = 1.0f / ff;                // exact for a power of two
  auto div_f = [&](float x) { return pow2 ? x * inv_f : x / ff; };
  const int nl = tid / CH, ch = tid % CH;       // phase 1: node slot, 8-element chunk
  const int og = tid % Gm::OG, ng = tid / Gm::OG;
  const int o0 = og * 4, n0 = ng * NPT;         // phase 2: outputs o0.., node slots n0..

  Chunk<BF16> rk[PF], rv[PF];
  auto prefetch = [&](int64_t tile) {
    if (tile >= total) return;
    const int64_t bh = tile / tiles_per_bh;
    const int64_t g = base0 + (tile % tiles_per_bh) * NPW + nl;
    if (g < a.g_lo || g >= a.g_hi) return;
    const int64_t cb = (bh * a.src_rows + g * f) * D + ch * 8;
#pragma unroll
    for (int c = 0; c < PF; ++c) {
      if (c < f) {
        rk[c].load(a.srcK, cb + static_cast<int64_t>(c) * D);
        rv[c].load(a.srcV, cb + static_cast<int64_t>(c) * D);
      }
    }
  };
  prefetch(blockIdx.x);
  lds_barrier();

  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int64_t bh = tile / tiles_per_bh;
    const int64_t tb = base0 + (tile % tiles_per_bh) * NPW;
    const int64_t g = tb + nl;

    // phase 1: child sums in child order -> node value (stored) and key mean (LDS)
    if (g >= a.g_lo && g < a.g_hi) {
      float sk[8], sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { sk[e] = 0.0f; sv[e] = 0.0f; }
#pragma unroll
      for (int c = 0; c < PF; ++c) {
        if (c < f) {
          rk[c].add_to(sk);
          rv[c].add_to(sv);
        }
      }
      const int64_t cb = (bh * a.src_rows + g * f) * D + ch * 8;
      for (int c0 = PF; c0 < f; c0 += PF) {
        Chunk<BF16> xk[PF], xv[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          if (c0 + u < f) {
            xk[u].load(a.srcK, cb + static_cast<int64_t>(c0 + u) * D);
            xv[u].load(a.srcV, cb + static_cast<int64_t>(c0 + u) * D);
          }
        }
#pragma unroll
        for (int u = 0; u < PF; ++u) {
          if (c0 + u < f) {
            xk[u].add_to(sk);
            xv[u].add_to(sv);
          }
        }
      }
      float nv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mt[ch * 8 + e][nl] = div_f(sk[e]);
        nv[e] = round_store<BF16>(div_f(sv[e]));
      }
      store8_nt<BF16>(a.dstV, (bh * a.dst_rows + g) * D + ch * 8, nv);
      if constexpr (STAGE) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v1s[nl][ch * 8 + e] = static_cast<uint16_t>(__float_as_uint(nv[e]) >> 16);
      }
    } else if (STAGE && g < a.g_lo) {
      // a node built by an earlier call: its stored key and value feed the parent
      const int64_t off = (bh * a.dst_rows + g) * D + ch * 8;
      const uint4 xk = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.dstK) + off);
      const uint4 xv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.dstV) + off);
      *reinterpret_cast<uint4*>(&k1s[nl][ch * 8]) = xk;
      *reinterpret_cast<uint4*>(&v1s[nl][ch * 8]) = xv;
    }
    lds_barrier();
    prefetch(tile + gridDim.x);

    // phase 2: key_i = sum_j W[i][j] m_j, accumulated in input order j = 0..D-1, one
    // fused multiply-add per term; 4 outputs x 2 node slots per thread
    float acc[NPT][4];
#pragma unroll
    for (int u = 0; u < NPT; ++u)
#pragma unroll
      for (int o = 0; o < 4; ++o) acc[u][o] = 0.0f;
#pragma unroll 8
    for (int j = 0; j < D; ++j) {
      float wv[4];
      if constexpr (BF16) {
        const uint2 w4 = *reinterpret_cast<const uint2*>(&wt[j][o0]);
        wv[0] = __uint_as_float(w4.x << 16); wv[1] = __uint_as_float(w4.x & 0xFFFF0000u);
        wv[2] = __uint_as_float(w4.y << 16); wv[3] = __uint_as_float(w4.y & 0xFFFF0000u);
      } else {
        const float4 w4 = *reinterpret_cast<const float4*>(&wt[j][o0]);
        wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
      }
      const float2 m2 = *reinterpret_cast<const float2*>(&mt[j][n0]);
      const float mv[2] = {m2.x, m2.y};
#pragma unroll
      for (int u = 0; u < NPT; ++u)
#pragma unroll
        for (int o = 0; o < 4; ++o) acc[u][o] = fmaf(wv[o], mv[u], acc[u][o]);
    }
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int64_t gg = tb + n0 + u;
      if (gg >= a.g_lo && gg < a.g_hi) {
        const int64_t off = (bh * a.dst_rows + gg) * D + o0;
        if constexpr (BF16) {
          const uint32_t b0 = f32_to_bf16_bits(acc[u][0]), b1 = f32_to_bf16_bits(acc[u][1]);
          const uint32_t b2 = f32_to_bf16_bits(acc[u][2]), b3 = f32_to_bf16_bits(acc[u][3]);
          __builtin_nontemporal_store(nt_u32x2{b0 | (b1 << 16), b2 | (b3 << 16)},
                                      reinterpret_cast<nt_u32x2*>(static_cast<uint16_t*>(a.dstK) + off));
          if constexpr (STAGE)
            *reinterpret_cast<uint2*>(&k1s[n0 + u][o0]) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
          __builtin_nontemporal_store(nt_f32x4{acc[u][0], acc[u][1], acc[u][2], acc[u][3]},
                                      reinterpret_cast<nt_f32x4*>(static_cast<float*>(a.dstK) + off));
        }
      }
    }

    if constexpr (FUSE) {
      // the tile's parents one level up, [pb, pb + P), those in [g_lo / f, g_hi / f)
      const int P = NPW / f;
      const int64_t p_lo = a.g_lo / f, p_hi = a.g_hi / f, pb = tb / f;
      if (pb + P > p_lo && pb < p_hi) {
        if constexpr (STAGE) lds_barrier();   // the tile's node rows are in LDS
        else __syncthreads();                 // the tile's node rows are stored and visible
        if constexpr (STAGE) {
          for (int it = tid; it < P * 2 * D; it += T) {
            const int p = it / (2 * D), rem = it % (2 * D), which = rem / D, dd = rem % D;
            const int64_t g2 = pb + p;
            if (g2 < p_lo || g2 >= p_hi) continue;
            const uint16_t(*src)[D] = which ? v1s : k1s;
            float s1 = 0.0f;
            for (int c = 0; c < f; ++c) s1 = s1 + bf16_to_f32(src[p * f + c][dd]);
            if (which == 0) m2s[p * D + dd] = div_f(s1);
            else store1_nt<BF16>(a.dst2V, (bh * a.dst2_rows + g2) * D + dd, round_store<BF16>(div_f(s1)));
          }
        } else {
          for (int it = tid; it < P * 2 * CH; it += T) {
            const int p = it / (2 * CH), rem = it % (2 * CH), which = rem / CH, cc = rem % CH;
            const int64_t g2 = pb + p;
            if (g2 < p_lo || g2 >= p_hi) continue;
            const void* src = which ? a.dstV : a.dstK;
            const int64_t rb = (bh * a.dst_rows + g2 * f) * D + cc * 8;
            float s8[8];
  #pragma unroll
            for (int e = 0; e < 8; ++e) s8[e] = 0.0f;
            for (int c0 = 0; c0 < f; c0 += 4) {
              Chunk<BF16> x[4];
  #pragma unroll
              for (int u = 0; u < 4; ++u)
                if (c0 + u < f) x[u].load_cached(src, rb + static_cast<int64_t>(c0 + u) * D);
  #pragma unroll
              for (int u = 0; u < 4; ++u)
                if (c0 + u < f) x[u].add_to(s8);
            }
            if (which == 0) {
  #pragma unroll
              for (int e = 0; e < 8; ++e) m2s[p * D + cc * 8 + e] = div_f(s8[e]);
            } else {
              float o8[8];
  #pragma unroll
              for (int e = 0; e < 8; ++e) o8[e] = round_store<BF16>(div_f(s8[e]));
              store8_nt<BF16>(a.dst2V, (bh * a.dst2_rows + g2) * D + cc * 8, o8);
            }
          }
        }
        lds_barrier();
        for (int it = tid; it < P * D; it += T) {
          const int p = it / D, i = it % D;
          const int64_t g2 = pb + p;
          if (g2 < p_lo || g2 >= p_hi) continue;
          float acc2 = 0.0f;
#pragma unroll 8
          for (int j = 0; j < D; ++j) acc2 = fmaf(wload(j, i), m2s[p * D + j], acc2);
          store1_nt<BF16>(a.dst2K, (bh * a.dst2_rows + g2) * D + i, round_store<BF16>(acc2));
        }
      }
    }
    lds_barrier();
  }
}

int pool_nodes_per_tile(int d) { return d == 128 ? PoolGeom<128>::NPW : PoolGeom<64>::NPW; }

static int persistent_grid() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return 2 * cus;  // two 512-thread workgroups fit a CU's LDS
}

template <int D, bool BF16>
static hipError_t launch_pool_t(const PoolArgs& a, hipStream_t s) {
  constexpr int NPW = PoolGeom<D>::NPW;
  const int64_t base0 = (a.g_lo / NPW) * NPW;
  const int64_t tiles = (a.g_hi - base0 + NPW - 1) / NPW * a.BH;
  if (a.g_hi <= a.g_lo || tiles <= 0) return hipSuccess;
  const int64_t cap = a.grid > 0 ? a.grid : persistent_grid();
  const int64_t grid = tiles < cap ? tiles : cap;
  if (a.fuse_next) {
    hipLaunchKernelGGL((pool_kernel<D, BF16, true>), dim3(static_cast<unsigned>(grid)), dim3(PoolGeom<D>::T), 0, s, a);
  } else {
    hipLaunchKernelGGL((pool_kernel<D, BF16, false>), dim3(static_cast<unsigned>(grid)), dim3(PoolGeom<D>::T), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_pool_level(const PoolArgs& a, int d, bool bf16, hipStream_t s) {
  if (d == 128) return bf16 ? launch_pool_t<128, true>(a, s) : launch_pool_t<128, false>(a, s);
  if (d == 64) return bf16 ? launch_pool_t<64, true>(a, s) : launch_pool_t<64, false>(a, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- RoPE table

__global__ __launch_bounds__(256) void rope_table_kernel(float2* tab, int64_t P, int half, InvFreq iv) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= (P + 1) * half) return;
  const int64_t p = idx / half;
  const int i = static_cast<int>(idx % half);
  const double ang = static_cast<double>(p) * static_cast<double>(iv.w[i]);  // exact product
  tab[idx] = make_float2(static_cast<float>(cos(ang)), static_cast<float>(sin(ang)));
}

hipError_t launch_rope_table(float2* tab, int64_t P, int half, const InvFreq& iv, hipStream_t s) {
  const int64_t n = (P + 1) * half;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, tab, P, half, iv);
  return hipGetLastError();
}

}  // namespace recsa
