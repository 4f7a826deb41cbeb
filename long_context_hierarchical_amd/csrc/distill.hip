// Pooler distillation, the two pieces around the tree attention's forward and gradient:
//
// "Recursive Sparse Attention: Million-Token Length Extrapolation at Logarithmic Cost",
// abstract, and the explainer's section "Core Idea: Compressing the KV Cache with a Tree
// Structure": the pooler is learned by distilling from full attention. With the loss read as
// the mean squared difference between RecSA's output and full attention's (selections held
// fixed), a step needs dL/dout = 2 (out - target) / N, the loss itself, and a gradient-descent
// update of a float32 master copy of W followed by rounding to the storage type.
#include "common.hpp"
#include "internal.hpp"
#include "lanes.hpp"

namespace recsa {



// dout = 2 (out - target) / N; partial[block] = sum of (out - target)^2 over the block's
// grid-stride elements (fixed order within a thread, then the block's fixed reduction)
__global__ __launch_bounds__(256) void distill_loss_kernel(const float* out, const float* target, float* dout,
                                                          float* partial, int64_t n) {
  __shared__ float ws[4];
  const float two_over_n = 2.0f / static_cast<float>(n);
  float acc = 0.0f;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const float d = out[i] - target[i];
    dout[i] = two_over_n * d;
    acc = fmaf(d, d, acc);
  }
  acc = wave_sum_dpp(acc);
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) partial[blockIdx.x] = (ws[0] + ws[1]) + (ws[2] + ws[3]);
}

// loss = (sum of the partials, in float64, in block order) / N
__global__ __launch_bounds__(64) void distill_loss_final_kernel(const float* partial, int nb, int64_t n, float* loss) {
  if (threadIdx.x != 0) return;
  double s = 0.0;
  for (int b = 0; b < nb; ++b) s += static_cast<double>(partial[b]);
  *loss = static_cast<float>(s / static_cast<double>(n));
}

// W_master -= lr * dW; W = W_master rounded to the storage type
template <bool BF16>
__global__ __launch_bounds__(256) void distill_update_kernel(float* Wm, const float* dW, void* W, float lr, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const float w = Wm[i] - lr * dW[i];
  Wm[i] = w;
  store1<BF16>(W, i, round_store<BF16>(w));
}


hipError_t launch_distill_loss(const float* out, const float* target, float* dout, float* partial, float* loss,
                               int64_t n, hipStream_t s) {
  const int nb = distill_loss_blocks(n);
  hipLaunchKernelGGL(distill_loss_kernel, dim3(nb), dim3(256), 0, s, out, target, dout, partial, n);
  hipLaunchKernelGGL(distill_loss_final_kernel, dim3(1), dim3(64), 0, s, partial, nb, n, loss);
  return hipGetLastError();
}

hipError_t launch_distill_update(float* Wm, const float* dW, void* W, float lr, int64_t n, bool bf16, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (bf16) hipLaunchKernelGGL((distill_update_kernel<true>), grid, dim3(256), 0, s, Wm, dW, W, lr, n);
  else hipLaunchKernelGGL((distill_update_kernel<false>), grid, dim3(256), 0, s, Wm, dW, W, lr, n);
  return hipGetLastError();
}

}  // namespace recsa
