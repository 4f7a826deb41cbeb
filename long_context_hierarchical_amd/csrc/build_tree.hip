// Tree build: pooled node keys and mean node values, one level per launch.
//
// RecSA abstract ("Recursive Sparse Attention: Million-Token Length
// Extrapolation at Logarithmic Cost"): every node summarises its subtree with
// one key from the layer's pooler, shared by all levels, and one mean-pooled
// value. Here the pooler is key = W @ m, m the mean of the node's f children's
// stored keys; the value is the mean of the children's stored values.
//
// HBM-bound: a tile reads f * (rows per tile) child rows of K and V once and
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

template <bool BF16>
struct Chunk;  // raw storage of 8 consecutive elements
template <>
struct Chunk<true> {
  uint4 u;
  __device__ __forceinline__ void load(const void* base, int64_t off) {
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
  __device__ __forceinline__ void load(const void* base, int64_t off) {
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
  static constexpr int CH = D / 8;        // 8-element chunks per row (phase 1)
  static constexpr int NPW = 256 / CH;    // nodes per tile: 16 (d=128) / 32 (d=64)
  static constexpr int OG = D / 4;        // groups of 4 outputs (phase 2)
  static constexpr int NGR = 256 / OG;    // node groups
  static constexpr int NPT = NPW / NGR;   // nodes per thread
};

// One pass over level-l nodes [g_lo, g_hi) of every (sequence, KV head); tiles of NPW
// nodes aligned to multiples of NPW. Each thread prefetches its next tile's children into
// registers before the matrix-vector phase of the current one, so loads stay in flight.
// With FUSE (f == NPW) the tile's parent at level l+1 is built from the tile's nodes too
// (reading already-stored nodes below g_lo back from the tree).
template <int D, bool BF16, bool FUSE>
__global__ __launch_bounds__(256, 2) void pool_kernel(PoolArgs a) {
  using Gm = PoolGeom<D>;
  constexpr int CH = Gm::CH, NPW = Gm::NPW, NPT = Gm::NPT;
  constexpr int PF = BF16 ? 16 : 8;       // children held in registers per thread
  using ST = typename std::conditional<BF16, uint16_t, float>::type;
  static_assert(NPT == 2, "phase 2 tiles 4 outputs x 2 nodes per thread");
  __shared__ float wt[D][D];              // wt[j][i] = W[i][j], float32
  __shared__ float mt[D][NPW];            // mt[j][node] = mean of the node's child keys
  __shared__ ST k1s[FUSE ? NPW : 1][D];   // this tile's node keys / values (storage values)
  __shared__ ST v1s[FUSE ? NPW : 1][D];
  float* const m2s = &mt[0][0];           // the parent's key mean reuses mt after phase 2

  const int tid = threadIdx.x;
  const int f = a.f;
  const int64_t base0 = (a.g_lo / NPW) * NPW;
  const int64_t tiles_per_bh = (a.g_hi - base0 + NPW - 1) / NPW;
  const int64_t total = tiles_per_bh * a.BH;

  for (int idx = tid; idx < D * CH; idx += 256) {
    const int i = idx / CH, j0 = (idx % CH) * 8;
    float x[8];
    load8<BF16>(a.W, static_cast<int64_t>(i) * D + j0, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) wt[j0 + e][i] = x[e];
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
  __syncthreads();

  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int64_t bh = tile / tiles_per_bh;
    const int64_t tb = base0 + (tile % tiles_per_bh) * NPW;
    const int64_t g = tb + nl;
    const bool fresh = g >= a.g_lo && g < a.g_hi;

    // phase 1: child sums in child order -> node value (stored) and key mean (LDS)
    if (fresh) {
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
      for (int c = PF; c < f; ++c) {
        Chunk<BF16> xk, xv;
        xk.load(a.srcK, cb + static_cast<int64_t>(c) * D);
        xv.load(a.srcV, cb + static_cast<int64_t>(c) * D);
        xk.add_to(sk);
        xv.add_to(sv);
      }
      float nv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mt[ch * 8 + e][nl] = div_f(sk[e]);
        nv[e] = round_store<BF16>(div_f(sv[e]));
      }
      store8<BF16>(a.dstV, (bh * a.dst_rows + g) * D + ch * 8, nv);
      if constexpr (FUSE) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (BF16) v1s[nl][ch * 8 + e] = static_cast<uint16_t>(__float_as_uint(nv[e]) >> 16);
          else v1s[nl][ch * 8 + e] = nv[e];
        }
      }
    } else if (FUSE && g < a.g_lo) {
      // node built by an earlier call: its stored key and value feed the parent
      const int64_t off = (bh * a.dst_rows + g) * D + ch * 8;
      float xk[8], xv[8];
      load8<BF16>(a.dstK, off, xk);
      load8<BF16>(a.dstV, off, xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (BF16) {
          k1s[nl][ch * 8 + e] = static_cast<uint16_t>(__float_as_uint(xk[e]) >> 16);
          v1s[nl][ch * 8 + e] = static_cast<uint16_t>(__float_as_uint(xv[e]) >> 16);
        } else {
          k1s[nl][ch * 8 + e] = xk[e];
          v1s[nl][ch * 8 + e] = xv[e];
        }
      }
    }
    __syncthreads();
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
      const float4 w4 = *reinterpret_cast<const float4*>(&wt[j][o0]);
      const float2 m2 = *reinterpret_cast<const float2*>(&mt[j][n0]);
      const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
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
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dstK) + off) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
          if constexpr (FUSE) {
            k1s[n0 + u][o0] = b0; k1s[n0 + u][o0 + 1] = b1; k1s[n0 + u][o0 + 2] = b2; k1s[n0 + u][o0 + 3] = b3;
          }
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.dstK) + off) =
              make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
          if constexpr (FUSE) {
#pragma unroll
            for (int o = 0; o < 4; ++o) k1s[n0 + u][o0 + o] = acc[u][o];
          }
        }
      }
    }

    if constexpr (FUSE) {
      // the tile's parent one level up: children = the NPW (= f) node slots of this tile
      const int64_t g2 = tb / NPW;
      if (g2 >= a.g_lo / NPW && g2 < a.g_hi / NPW) {
        __syncthreads();
        if (tid < 2 * D) {
          const int dd = tid % D;
          float s = 0.0f;
          if (tid < D) {
#pragma unroll 4
            for (int c = 0; c < NPW; ++c) {
              if constexpr (BF16) s = s + bf16_to_f32(k1s[c][dd]);
              else s = s + k1s[c][dd];
            }
            m2s[dd] = div_f(s);
          } else {
#pragma unroll 4
            for (int c = 0; c < NPW; ++c) {
              if constexpr (BF16) s = s + bf16_to_f32(v1s[c][dd]);
              else s = s + v1s[c][dd];
            }
            store1<BF16>(a.dst2V, (bh * a.dst2_rows + g2) * D + dd, round_store<BF16>(div_f(s)));
          }
        }
        __syncthreads();
        if (tid < D) {
          float acc2 = 0.0f;
#pragma unroll 8
          for (int j = 0; j < D; ++j) acc2 = fmaf(wt[j][tid], m2s[j], acc2);
          store1<BF16>(a.dst2K, (bh * a.dst2_rows + g2) * D + tid, round_store<BF16>(acc2));
        }
      }
    }
    __syncthreads();
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
  return 2 * cus;  // two 256-thread workgroups fit a CU's LDS
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
    hipLaunchKernelGGL((pool_kernel<D, BF16, true>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((pool_kernel<D, BF16, false>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
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
