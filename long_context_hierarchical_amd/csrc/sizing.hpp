// Host-side sizing of the kernels' launches: tiles, LDS layouts and scratch sizes. Shared by the
// kernels' sources and the host code, so that the argument checks and the launches agree (and a
// host-only build of the checks uses the same arithmetic).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "recsa.h"

namespace recsa {

// ---------------------------------------------------------------- tree build
// Nodes per tile of the pool kernel: 512 threads, one 8-element chunk of a row each (32 nodes at
// d = 128, 64 at d = 64); the next level is fused into the pass when the fanout divides it.
__host__ __device__ inline int pool_nodes_per_tile(int d) { return 512 / (d / 8); }

// ---------------------------------------------------------------- descent + softmax
// LDS of one unit of the attention kernel (byte offsets of its regions).
struct Lds {
  uint32_t q, qr, zs, sc, cid, flags, selA, selB, nls, bc, info, total;
};

__host__ __device__ inline uint32_t align16(uint32_t x) { return (x + 15u) & ~15u; }

__host__ __device__ inline Lds lds_layout(int d, int G, int smax, int zcap) {
  Lds L;
  uint32_t o = 0;
  L.q = o;     o = align16(o + 4u * G * d);         // raw query heads of the selection group
  L.qr = o;    o = align16(o + 4u * G * d);         // rotated query operands of the current level
  L.zs = o;    o = align16(o + 4u * G * zcap);      // logits, then softmax weights, [zcap][G]
  L.sc = o;    o = align16(o + 4u * zcap);          // group scores
  L.cid = o;   o = align16(o + 4u * zcap);          // node (or token) id of each scored candidate
  L.flags = o; o = align16(o + zcap);               // kept flags
  L.selA = o;  o = align16(o + 4u * smax);          // kept node ids, two buffers
  L.selB = o;  o = align16(o + 4u * smax);
  L.nls = o;   o = align16(o + 8u * (RECSA_MAX_LEVELS + 2));
  L.bc = o;    o = align16(o + 4u * 2 * G);         // softmax rescale and sum, wave 0 -> all
  L.info = o;  o = align16(o + 4u * 2);             // the first scored level and its node count
  L.total = o;
  return L;
}

__host__ __device__ inline size_t attend_lds_bytes(int d, int G, int smax, int zcap) { return lds_layout(d, G, smax, zcap).total; }

// The rows of the matrix-core tile of the first scored level: 32 (query, head) rows of d bf16.
__host__ __device__ inline uint32_t mf_stage_bytes(int d) { return 32u * d * 2u; }

// ---------------------------------------------------------------- pooler distillation
constexpr int kLossBlocks = 1024;
// Workgroups of the loss reduction (256 elements each, at most kLossBlocks partial sums).
__host__ __device__ inline int distill_loss_blocks(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return static_cast<int>(b < kLossBlocks ? b : kLossBlocks);
}

// ---------------------------------------------------------------- dense reference attention
// Query rows per workgroup of the dense kernel: 4 waves of 32 (query, head) rows.
__host__ __device__ inline int dense_queries_per_block(int G) { return 4 * (32 / G); }

// ---------------------------------------------------------------- allocation-free decode
// Bytes of the library's per-device scratch array: the RoPE table for up to 8191 positions at d = 128.
constexpr size_t kNoallocScratchBytes = size_t(4) << 20;

// ---------------------------------------------------------------- RoPE table cache
// Rows (positions 0 .. kRopeCacheRows - 1) of the per-device RoPE table cache, for head sizes up
// to kRopeCacheHeadDim: 4 MiB of (cos, sin) pairs.
constexpr int64_t kRopeCacheRows = 8192;
constexpr int kRopeCacheHeadDim = 128;

}  // namespace recsa
