// One step of autoregressive decoding, first part: the new token joins the cache and the nodes
// its arrival completes are built (the attention that follows is attend.hip's kernel).
//
// RecSA abstract ("Recursive Sparse Attention: Million-Token Length Extrapolation at
// Logarithmic Cost"): the tree lives over the KV cache; a node holds a key from the layer's
// pooler (one pooler for every level) and the average of the values it spans, and a decoding
// step touches a number of rows that grows with the tree height only. Here the pooler is key = W @ m, m the mean of the
// node's f children's stored keys, and the value is the mean of the children's stored values.
#include "common.hpp"
#include "internal.hpp"

namespace recsa {

// ---------------------------------------------------------------- decoding step

// A generated token joins the cache; when its arrival completes a node (n + 1 a multiple of f),
// that node is built from its f children -- the new row last -- and may in turn complete its
// parent, so a step builds at most one node per level. The arithmetic is pool_kernel's: child
// sums in child order in float32, one division by f, acc = fmaf(W[i][j], m[j], acc) over
// j = 0..d-1, rounding to the storage type; the level above uses each new node in its rounded,
// stored form. One thread per dimension (= per pooler output); a step pools one node per level,
// so W's rows are read straight from memory. Arguments are read in place from the kernel
// argument segment (the per-level tables are indexed by a run-time level).
template <int D, bool BF16>
__global__ __launch_bounds__(128) void append_step_kernel(StepArgs) {
  const StepArgs& a = *(const StepArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  const int tid = threadIdx.x;
  if (static_cast<int>(blockIdx.x) >= a.BH) {  // RoPE table rows, as rope_table_kernel
    const int64_t idx = static_cast<int64_t>(blockIdx.x - a.BH) * 128 + tid;
    if (idx < (a.P + 1) * a.half) {
      const int64_t p = idx / a.half;
      const int i = static_cast<int>(idx % a.half);
      const double ang = static_cast<double>(p) * static_cast<double>(a.iv.w[i]);
      a.tab[idx] = make_float2(static_cast<float>(cos(ang)), static_cast<float>(sin(ang)));
    }
    return;
  }
  __shared__ float m[D];
  const int64_t bh = blockIdx.x;
  const bool act = tid < D;
  const int f = a.f;
  const float ff = static_cast<float>(f);
  const bool pow2 = (f & (f - 1)) == 0;
  const float inv_f = 1.0f / ff;
  float kc = 0.0f, vc = 0.0f;  // this thread's dimension of the newest child
  if (act) {
    kc = load1<BF16>(a.k_new, bh * D + tid);
    vc = load1<BF16>(a.v_new, bh * D + tid);
    store1<BF16>(a.K, (bh * a.cap + a.n) * D + tid, kc);
    store1<BF16>(a.V, (bh * a.cap + a.n) * D + tid, vc);
  }
  int64_t idx = a.n;  // index of the newest child one level down
  for (int lv = 1; lv <= a.levels && (idx + 1) % f == 0; ++lv) {
    const int64_t g = idx / f;
    const void* sK = lv == 1 ? a.K : a.NK[lv - 1];
    const void* sV = lv == 1 ? a.V : a.NV[lv - 1];
    const int64_t srows = lv == 1 ? a.cap : a.rows[lv - 1];
    float sk = 0.0f, sv = 0.0f;
    if (act) {
      const int64_t base = (bh * srows + g * f) * D + tid;
      for (int c = 0; c < f - 1; ++c) {
        sk = sk + load1<BF16>(sK, base + static_cast<int64_t>(c) * D);
        sv = sv + load1<BF16>(sV, base + static_cast<int64_t>(c) * D);
      }
      sk = sk + kc;
      sv = sv + vc;
      m[tid] = pow2 ? sk * inv_f : sk / ff;
    }
    __syncthreads();
    if (act) {
      float acc = 0.0f;
#pragma unroll 4
      for (int j = 0; j < D; j += 8) {
        float w[8];
        load8<BF16>(a.W, static_cast<int64_t>(tid) * D + j, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(w[e], m[j + e], acc);
      }
      kc = round_store<BF16>(acc);
      vc = round_store<BF16>(pow2 ? sv * inv_f : sv / ff);
      const int64_t o = (bh * a.rows[lv] + g) * D + tid;
      store1<BF16>(a.NK[lv], o, kc);
      store1<BF16>(a.NV[lv], o, vc);
    }
    __syncthreads();
    idx = g;
  }
}

template <int D, bool BF16>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t s) {
  const int64_t tab_blocks = a.tab ? ((a.P + 1) * a.half + 127) / 128 : 0;
  hipLaunchKernelGGL((append_step_kernel<D, BF16>), dim3(static_cast<unsigned>(a.BH + tab_blocks)), dim3(128), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_append_step(const StepArgs& a, int d, bool bf16, hipStream_t s) {
  if (d == 128) return bf16 ? launch_step_t<128, true>(a, s) : launch_step_t<128, false>(a, s);
  if (d == 64) return bf16 ? launch_step_t<64, true>(a, s) : launch_step_t<64, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace recsa
