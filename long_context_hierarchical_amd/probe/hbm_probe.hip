// HBM bandwidth probe: the achievable read and copy rates of this GPU, measured with plain
// streaming kernels (16-byte loads, grid-stride, 8 (read) or 4 (copy) loads in flight per
// thread), as the practical ceiling beside the nameplate peak. Also a read stream that writes
// one 16-byte row per 16 rows read (the traffic mix of a tree build at fanout 16: every child
// row read once, one node row written per 16), in 512-thread workgroups that read their tile
// two rows per thread at a time and then write. Prints one JSON line:
//   {"read_GBps": R, "copy_GBps": C, "read16_write1_GBps": M, "bytes": N, "grid": G}
// with the best rate over grid sizes; copy and the mix count bytes read plus bytes written.
// Usage: hbm_probe [GiB to read, default 8]
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#define CK(x)                                                                    \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "hbm_probe: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, size_t n, uint32_t* sink) {
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; practically never taken
}

template <int U>
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ p, uint4* __restrict__ q, size_t n) {
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) q[i + u * stride] = v[u];
  }
  for (; i < n; i += stride) q[i] = p[i];
}

// The read/write mix: 512-thread workgroups stream tiles of 512 x 16 rows of 16 bytes; each
// thread reads its 16 rows two at a time, then writes one 16-byte row per 16 read.
__global__ __launch_bounds__(512) void mix_kernel(const uint4* __restrict__ p, uint4* __restrict__ q, size_t tiles) {
  const int tid = threadIdx.x;
  for (size_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const uint4* src = p + t * 8192 + tid;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    for (int c = 0; c < 16; c += 2) {
      const uint4 v0 = src[c * 512], v1 = src[(c + 1) * 512];
      x.x ^= v0.x ^ v1.x; x.y ^= v0.y ^ v1.y; x.z ^= v0.z ^ v1.z; x.w ^= v0.w ^ v1.w;
    }
    q[t * 512 + tid] = x;
  }
}

int main(int argc, char** argv) {
  const double gib = argc > 1 ? atof(argv[1]) : 8.0;
  if (!(gib > 0.0 && gib <= 64.0)) {
    fprintf(stderr, "hbm_probe: size must be in (0, 64] GiB\n");
    return 2;
  }
  const size_t bytes = static_cast<size_t>(gib * 1073741824.0) / 4096 * 4096;
  const size_t n = bytes / 16;
  uint4 *a = nullptr, *b = nullptr;
  uint32_t* sink = nullptr;
  CK(hipMalloc(&a, bytes));
  CK(hipMalloc(&b, bytes / 2));
  CK(hipMalloc(&sink, 4));
  CK(hipMemset(a, 1, bytes));
  CK(hipMemset(b, 0, bytes / 2));
  hipEvent_t e0, e1;
  CK(hipEventCreate(&e0));
  CK(hipEventCreate(&e1));
  const int grids[] = {1024, 2048, 4096, 8192};
  double best_read = 0.0, best_copy = 0.0, best_mix = 0.0;
  int best_grid = 0;
  for (int g : grids) {
    hipLaunchKernelGGL((read_kernel<8>), dim3(g), dim3(256), 0, 0, a, n, sink);
    CK(hipEventRecord(e0));
    for (int rep = 0; rep < 5; ++rep) hipLaunchKernelGGL((read_kernel<8>), dim3(g), dim3(256), 0, 0, a, n, sink);
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double gbps = bytes / (ms / 5 * 1e-3) / 1e9;
    if (gbps > best_read) {
      best_read = gbps;
      best_grid = g;
    }
    const size_t nc = n / 2;
    hipLaunchKernelGGL((copy_kernel<4>), dim3(g), dim3(256), 0, 0, a, b, nc);
    CK(hipEventRecord(e0));
    for (int rep = 0; rep < 5; ++rep) hipLaunchKernelGGL((copy_kernel<4>), dim3(g), dim3(256), 0, 0, a, b, nc);
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double cgbps = 2.0 * nc * 16 / (ms / 5 * 1e-3) / 1e9;
    if (cgbps > best_copy) best_copy = cgbps;
    // the mix: whole tiles of 8192 rows read, 512 rows written per tile
    const size_t tiles = n / 8192;
    const int mg = g / 2;   // 512-thread workgroups
    hipLaunchKernelGGL(mix_kernel, dim3(mg), dim3(512), 0, 0, a, b, tiles);
    CK(hipEventRecord(e0));
    for (int rep = 0; rep < 5; ++rep) hipLaunchKernelGGL(mix_kernel, dim3(mg), dim3(512), 0, 0, a, b, tiles);
    CK(hipEventRecord(e1));
    CK(hipEventSynchronize(e1));
    CK(hipEventElapsedTime(&ms, e0, e1));
    const double mbytes = (tiles * 8192.0 + tiles * 512.0) * 16.0;
    const double mgbps = mbytes / (ms / 5 * 1e-3) / 1e9;
    if (mgbps > best_mix) best_mix = mgbps;
  }
  CK(hipGetLastError());
  printf("{\"read_GBps\": %.1f, \"copy_GBps\": %.1f, \"read16_write1_GBps\": %.1f, \"bytes\": %zu, \"grid\": %d}\n",
         best_read, best_copy, best_mix, bytes, best_grid);
  CK(hipFree(a));
  CK(hipFree(b));
  CK(hipFree(sink));
  return 0;
}
