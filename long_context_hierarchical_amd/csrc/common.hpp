// Device helpers shared by the RecSA kernels (gfx950, wave64).
//
// The whole library is compiled with -ffp-contract=off: a multiply followed
// by an add stays two rounded operations unless a kernel asks for a fused
// multiply-add explicitly (fmaf). The tree build and the RoPE rotation rely on
// that, because their float32 roundings decide which nodes a query keeps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace recsa {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <bool BF16>
__device__ __forceinline__ float round_store(float x) {
  if constexpr (BF16) {
    return bf16_to_f32(f32_to_bf16_bits(x));
  } else {
    return x;
  }
}

// 8 consecutive storage elements starting at element `off` -> float.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&x)[8]) {
  if constexpr (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Store 8 floats (already exact in the storage type) at element `off`.
template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t off, const float (&x)[8]) {
  if constexpr (BF16) {
    uint4 u;
    u.x = (__float_as_uint(x[0]) >> 16) | (__float_as_uint(x[1]) & 0xFFFF0000u);
    u.y = (__float_as_uint(x[2]) >> 16) | (__float_as_uint(x[3]) & 0xFFFF0000u);
    u.z = (__float_as_uint(x[4]) >> 16) | (__float_as_uint(x[5]) & 0xFFFF0000u);
    u.w = (__float_as_uint(x[6]) >> 16) | (__float_as_uint(x[7]) & 0xFFFF0000u);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = u;
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(x[0], x[1], x[2], x[3]);
    p[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// N (1 or 2) consecutive storage elements -> float.
template <bool BF16, int N>
__device__ __forceinline__ void loadN(const void* base, int64_t off, float (&x)[N]) {
  static_assert(N == 1 || N == 2, "loadN");
  if constexpr (BF16) {
    if constexpr (N == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + off);
      x[0] = __uint_as_float(w << 16);
      x[1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      x[0] = bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
    }
  } else {
    if constexpr (N == 2) {
      const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(base) + off);
      x[0] = v.x;
      x[1] = v.y;
    } else {
      x[0] = static_cast<const float*>(base)[off];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, int64_t off) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[off]);
  } else {
    return static_cast<const float*>(base)[off];
  }
}

template <bool BF16>
__device__ __forceinline__ void store1(void* base, int64_t off, float x) {
  if constexpr (BF16) {
    static_cast<uint16_t*>(base)[off] = static_cast<uint16_t>(__float_as_uint(x) >> 16);
  } else {
    static_cast<float*>(base)[off] = x;
  }
}

// Monotone map float32 -> uint32 (larger float -> larger key); -0 and +0 map alike.
__device__ __forceinline__ uint32_t ordered_bits(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Selection key: higher score first, then lower candidate index.
__device__ __forceinline__ uint64_t select_key(float s, uint32_t idx) {
  return (static_cast<uint64_t>(ordered_bits(s)) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

}  // namespace recsa
