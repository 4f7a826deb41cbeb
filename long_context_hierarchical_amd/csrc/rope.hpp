// RoPE angle helper shared by the kernels that rotate rows at arbitrary positions on the fly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace recsa {

// RoPE cos/sin at integer position p for inverse frequency w: the exact float64 product, float64
// cos and sin, each rounded once to float32.
__device__ __forceinline__ void rope_cs(int64_t p, float w, float& c, float& s) {
  double sd, cd;
  sincos(static_cast<double>(p) * static_cast<double>(w), &sd, &cd);
  c = static_cast<float>(cd);
  s = static_cast<float>(sd);
}

}  // namespace recsa
