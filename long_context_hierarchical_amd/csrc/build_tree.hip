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
// float32, one correctly rounded division by f, then for each output the
// products W[i][j] * m[j] added in input order with separate multiply and add
// (the file is compiled with -ffp-contract=off), rounded to the storage type.
#include "common.hpp"
#include "internal.hpp"

namespace recsa {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void pool_level_kernel(PoolArgs a) {
  constexpr int CH = D / 8;            // 8-element chunks per row (phase 1)
  constexpr int NPW = 256 / CH;        // nodes per tile: 16 (d=128) / 32 (d=64)
  constexpr int OG = D / 4;            // groups of 4 outputs (phase 2)
  constexpr int NGR = 256 / OG;        // node groups
  constexpr int NPT = NPW / NGR;       // nodes per thread
  static_assert(NPT == 2, "phase 2 tiles 4 outputs x 2 nodes per thread");
  __shared__ float wt[D][D];           // wt[j][i] = W[i][j], float32
  __shared__ float mt[D][NPW];         // mt[j][node] = mean of the node's child keys

  const int tid = threadIdx.x;
  const int f = a.f;
  const int64_t n_nodes = a.g_hi - a.g_lo;
  const int64_t tiles_per_bh = (n_nodes + NPW - 1) / NPW;
  const int64_t total = tiles_per_bh * a.BH;

  for (int idx = tid; idx < D * CH; idx += 256) {
    const int i = idx / CH, j0 = (idx % CH) * 8;
    float x[8];
    load8<BF16>(a.W, static_cast<int64_t>(i) * D + j0, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) wt[j0 + e][i] = x[e];
  }

  const float ff = static_cast<float>(f);
  const int nl = tid / CH, ch = tid % CH;       // phase 1: node, 8-element chunk
  const int og = tid % OG, ng = tid / OG;       // phase 2: outputs og*4.., nodes ng*NPT..
  const int o0 = og * 4, n0 = ng * NPT;

  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int64_t bh = tile / tiles_per_bh;
    const int64_t g0 = a.g_lo + (tile % tiles_per_bh) * NPW;
    const int64_t g = g0 + nl;

    // phase 1: child sums in child order -> node value (stored) and key mean (LDS)
    if (g < a.g_hi) {
      float sk[8], sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { sk[e] = 0.0f; sv[e] = 0.0f; }
      const int64_t base = (bh * a.src_rows + g * f) * D + ch * 8;
#pragma unroll 4
      for (int c = 0; c < f; ++c) {
        float xk[8], xv[8];
        load8<BF16>(a.srcK, base + static_cast<int64_t>(c) * D, xk);
        load8<BF16>(a.srcV, base + static_cast<int64_t>(c) * D, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) { sk[e] = sk[e] + xk[e]; sv[e] = sv[e] + xv[e]; }
      }
      float nv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mt[ch * 8 + e][nl] = sk[e] / ff;
        nv[e] = round_store<BF16>(sv[e] / ff);
      }
      store8<BF16>(a.dstV, (bh * a.dst_rows + g) * D + ch * 8, nv);
    }
    __syncthreads();

    // phase 2: key_i = sum_j W[i][j] m_j, accumulated in input order j = 0..D-1 with
    // separate multiply and add; 4 outputs x 2 nodes per thread
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
        for (int o = 0; o < 4; ++o) {
          const float t = wv[o] * mv[u];
          acc[u][o] = acc[u][o] + t;
        }
    }
#pragma unroll
    for (int u = 0; u < NPT; ++u) {
      const int64_t gg = g0 + n0 + u;
      if (gg < a.g_hi) {
        const int64_t off = (bh * a.dst_rows + gg) * D + o0;
        if constexpr (BF16) {
          uint2 pk;
          pk.x = f32_to_bf16_bits(acc[u][0]) | (f32_to_bf16_bits(acc[u][1]) << 16);
          pk.y = f32_to_bf16_bits(acc[u][2]) | (f32_to_bf16_bits(acc[u][3]) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dstK) + off) = pk;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.dstK) + off) =
              make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
        }
      }
    }
    __syncthreads();
  }
}

template <int D, bool BF16>
static hipError_t launch_pool_t(const PoolArgs& a, hipStream_t s) {
  constexpr int NPW = 256 / (D / 8);
  const int64_t n_nodes = a.g_hi - a.g_lo;
  const int64_t tiles = (n_nodes + NPW - 1) / NPW * a.BH;
  if (tiles <= 0) return hipSuccess;
  const int64_t grid = tiles < 2048 ? tiles : 2048;
  hipLaunchKernelGGL((pool_level_kernel<D, BF16>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, a);
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
