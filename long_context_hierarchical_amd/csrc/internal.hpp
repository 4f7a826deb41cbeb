// Host <-> kernel interface of the RecSA library (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "recsa.h"
#include "sizing.hpp"

namespace recsa {

// ---------------------------------------------------------------- tree build
// One launch pools the nodes [g_lo, g_hi) of one level for every (sequence, KV head).
struct PoolArgs {
  const void* srcK;     // children: token rows (level 1) or level-(l-1) node keys
  const void* srcV;
  int64_t src_rows;     // child rows per (sequence, KV head) slice
  void* dstK;           // level-l node keys / values
  void* dstV;
  int64_t dst_rows;     // node rows per slice
  const void* W;        // [d][d] pooler
  int64_t g_lo, g_hi;   // node range to build
  int32_t f;
  int32_t BH;           // batch * n_kv_heads
  // Optional fused next level (f divides the nodes per tile): the level-(l+1) nodes, whose
  // children all fall in one tile, are built in the same pass, nodes [g_lo / f, g_hi / f).
  int32_t fuse_next;
  void* dst2K;
  void* dst2V;
  int64_t dst2_rows;
  int32_t grid;         // persistent grid size (0 = library default)
  int32_t one_tile;     // 1: one 1024-thread workgroup per tile (pool_tile_kernel); 0: persistent
  // Tile queue: with sched set, a workgroup's first tile is its index and each later one comes
  // from an atomic counter that reads sched_base at the launch's start (tiles in the order
  // workgroups ask for them); null: tiles blockIdx.x, + gridDim.x, ...
  unsigned long long* sched;
  unsigned long long sched_base;
};
hipError_t launch_pool_level(const PoolArgs& a, int d, bool bf16, hipStream_t s);
// workgroups of the persistent build grid (two per CU)
int pool_persistent_grid();

// ---------------------------------------------------------------- RoPE table
struct InvFreq {
  float w[64];  // omega_i, i < d/2
};
// tab[p * (d/2) + i] = (cos(p * omega_i), sin(p * omega_i)), evaluated in float64, for p = 0..P.
hipError_t launch_rope_table(float2* tab, int64_t P, int half, const InvFreq& iv, hipStream_t s);

// ---------------------------------------------------------------- decoding step
// Workgroups 0..BH-1 (one per sequence x KV head) write the new token at row n of K and V and
// build the nodes its arrival completes, at most one per level, bottom level first. Workgroups
// BH.. of the same grid fill the RoPE table rows 0..P when `tab` is set.
struct StepArgs {
  const void* k_new;    // [B*H_kv][d]
  const void* v_new;
  void* K;              // [B*H_kv][cap][d]
  void* V;
  int64_t cap;
  int64_t n;            // row of the new token
  const void* W;        // [d][d] pooler
  void* NK[RECSA_MAX_LEVELS + 1];  // index = level (1-based); [B*H_kv][rows[l]][d]
  void* NV[RECSA_MAX_LEVELS + 1];
  int64_t rows[RECSA_MAX_LEVELS + 1];
  int32_t levels;       // levels the tree buffer holds
  int32_t f;
  int32_t BH;
  int32_t half;         // d / 2
  float2* tab;          // RoPE table or null
  int64_t P;
  InvFreq iv;
};
hipError_t launch_append_step(const StepArgs& a, int d, bool bf16, hipStream_t s);

// ---------------------------------------------------------------- descent + softmax
struct TreeLevels {
  const void* NK[RECSA_MAX_LEVELS + 1];  // index = level (1-based); [B*H_kv][rows[l]][d]
  const void* NV[RECSA_MAX_LEVELS + 1];
  int64_t rows[RECSA_MAX_LEVELS + 1];
};

struct LevelK {
  int32_t k[RECSA_MAX_LEVELS + 1];  // index = level (1-based)
};

struct AttnArgs {
  const void* q;        // [B][n_q][H_q][d]
  const void* K;        // [B*H_kv][cap][d]
  const void* V;
  float* out;           // [B][n_q][H_q][d]
  float* lse;           // [B][n_q][H_q] or null
  int32_t* sel;         // [B][n_q][H_kv][n_levels][sel_width] or null
  const float2* tab;    // RoPE table, rows 0..P
  int64_t cap;
  int64_t n_q;
  int64_t n_fixed;      // decode: visible tokens
  int64_t q_start;      // prefill: position of query 0
  int32_t prefill;      // 1: query j sees n = q_start + j + 1 tokens, own token included
  int32_t Hkv, Hq, f;   // Hkv: selection groups per sequence (= KV heads unless heads select alone)
  int32_t Hkv_kv;       // KV heads per sequence
  int32_t kv_div;       // selection groups per KV head (group h reads KV head h / kv_div)
  int32_t n_levels, sel_width;
  float scale;
  int32_t use_rope;
  int32_t smax;         // capacity of a kept-node list
  int32_t zcap;         // capacity of a scored candidate list (selecting levels and token-level chunks)
  int32_t pv_stage;     // set by the launcher, several waves per unit: value rows through LDS in
                        // rounds (1) or prefetched for a whole chunk while it is scored (2)
  int32_t stage_bytes;  // set by the launcher: LDS bytes of that value staging (the matrix-core
                        // tile's rows follow it)
  LevelK k;
  TreeLevels tree;
};


// ---------------------------------------------------------------- gradients (selections held fixed)
struct BwdArgs {
  const void* q;        // [B][n_q][H_q][d] storage type
  const void* K;        // [B*H_kv][cap][d]
  const void* V;
  const float* out;     // forward outputs [B][n_q][H_q][d]
  const float* lse;     // forward log-sum-exp [B][n_q][H_q]
  const int32_t* sel;   // forward selections [B][n_q][H_kv][n_levels][sel_width]
  const float* dout;    // [B][n_q][H_q][d]
  const float* dlse;    // [B][n_q][H_q] or null
  float* dq;            // [B][n_q][H_q][d] (written)
  float* dK;            // [B*H_kv][cap][d] (added to)
  float* dV;
  const float2* tab;    // RoPE table, rows 0..P
  int64_t cap;
  int64_t n_q;
  int64_t n_fixed;      // decode: visible tokens
  int64_t q_start;      // causal: position of query 0
  int32_t causal;
  int32_t Hkv, Hq, f;
  int32_t n_levels, sel_width;
  float scale;
  int32_t use_rope;
  int32_t zcap;         // capacity of the kept-flag list
  int32_t smax;         // capacity of the kept-parent list
  TreeLevels tree;      // forward node rows
  float* gNK[RECSA_MAX_LEVELS + 1];   // node-key gradients, [B*H_kv][rows[l]][d] (added to)
  float* gNV[RECSA_MAX_LEVELS + 1];
};
size_t backward_unit_lds_bytes(int zcap, int smax);
hipError_t launch_backward_units(const BwdArgs& a, int d, bool bf16, int G, int64_t B, hipStream_t s);

// One level of the top-down push: every node of level `level` with a nonzero gradient adds
// outer(dkey, m) to dW, W^T dkey / f to each child's key gradient and dvalue / f to each
// child's value gradient (children: token rows at level 1, level-(l-1) nodes above).
struct TreePushArgs {
  const void* childK;   // stored child keys [BH][child_rows][d] (token rows or level l-1 nodes)
  int64_t child_rows;
  const float* gk;      // this level's node gradients [BH][rows][d]
  const float* gv;
  int64_t rows;
  int64_t n_nodes;      // nodes of this level per slice
  float* ck;            // child gradients [BH][child_rows][d] (added to)
  float* cv;
  const void* W;        // [d][d]
  float* dW;            // [d][d] (added to)
  int32_t f;
  int32_t BH;
};
hipError_t launch_tree_push(const TreePushArgs& a, int d, bool bf16, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

// ---------------------------------------------------------------- pooler distillation
// dout = 2 (out - target) / n and loss = mean of (out - target)^2 (partial: distill_loss_blocks(n) floats)
hipError_t launch_distill_loss(const float* out, const float* target, float* dout, float* partial, float* loss,
                               int64_t n, hipStream_t s);
// W_master -= lr * dW; W = W_master rounded to the storage type (n = d * d)
hipError_t launch_distill_update(float* Wm, const float* dW, void* W, float lr, int64_t n, bool bf16, hipStream_t s);

// ---------------------------------------------------------------- dense reference attention
// Keys rotated at their own positions: Kr[bh][p] = round(rot(K[bh][p], p)), p_lo <= p < n
// (K rows per slice: cap; Kr rows per slice: kr_rows).
hipError_t launch_rotate_keys(const void* K, int64_t cap, void* Kr, int64_t kr_rows, int64_t n, int64_t BH, int d,
                              bool bf16, const InvFreq& iv, int use_rope, hipStream_t s, int64_t p_lo = 0);

struct DenseArgs {
  const void* q;        // [B][n_q][H_q][d]
  const void* Kr;       // rotated keys [B*H_kv][kr_rows][d]
  const void* V;        // [B*H_kv][v_rows][d]
  float* out;           // [B][n_q][H_q][d]
  float* lse;           // [B][n_q][H_q] or null
  float* part_o;        // split partials [splits][B*H_kv][n_q*G][d] (null when one split)
  float* part_ml;       // [splits][B*H_kv][n_q*G][2]
  int64_t kr_rows, v_rows;
  int64_t n_q, q_start, n_tokens;
  int32_t causal;
  int32_t Hkv, Hq;
  int64_t keys_per_split;
  int32_t n_splits;
  float scale;
  int32_t use_rope;
  InvFreq iv;
};
hipError_t launch_dense(const DenseArgs& a, int d, bool bf16, int G, int64_t B, hipStream_t s);
// bf16 queries rotated at their positions into qr ([B][n_q][H_q][d], bf16), for the MFMA kernel.
hipError_t launch_rotate_queries(const DenseArgs& a, void* qr, int64_t B, int d, hipStream_t s);
hipError_t launch_attend(const AttnArgs& a, int d, bool bf16, int G, size_t lds, int64_t B, hipStream_t s);

// ---------------------------------------------------------------- two-stage block-then-token selection
// Stage 1 scores every complete block (level-1 node) of a slice for every query and keeps, per
// slab of SB blocks, the slab's best s1c = min(s1, blocks in the slab) as (ordered score bits,
// block id) in ascending block order. Stage 2, one workgroup per (query, KV head), merges the
// slabs' lists into the s1 kept blocks, then scores their tokens and the trailing tokens, keeps
// the best s0 and takes one softmax over them.
struct TsArgs {
  const void* q1;       // queries rotated at n1 [B][n_q][H_q][d], storage type
  const void* q0;       // queries rotated at C0
  const void* kb;       // block keys rotated at their index [BH][kb_rows][d]
  int64_t kb_rows;
  const void* K;        // token rows [BH][cap][d], pre-RoPE
  const void* V;
  int64_t cap;
  uint2* cand;          // [BH][n_q][n_slabs][s1] (ordered score bits, block id)
  int32_t* kept;        // [BH][n_q][s1] kept block ids, ascending
  const float2* tab;    // RoPE table rows 0..C0, or null without rotation
  float* out;           // [B][n_q][H_q][d]
  float* lse;           // [B][n_q][H_q] or null
  int32_t* sel_blocks;  // [B][n_q][H_kv][sel_bw] or null
  int32_t* sel_tokens;  // [B][n_q][H_kv][sel_tw] or null
  int32_t sel_bw, sel_tw;
  int64_t n;            // visible tokens
  int64_t n1;           // complete blocks, floor(n / f)
  int64_t n_q;
  int64_t BH;
  int32_t Hkv, Hq, f;
  int32_t s1;           // blocks kept, min(k_block, n1)
  int32_t C0;           // token candidates, f s1 + n - f n1
  int32_t s0;           // tokens kept, min(k_token, C0)
  int32_t SB, n_slabs;  // blocks per slab of stage 1, slabs
  int32_t merge;        // entries of the merged list, sum over slabs of s1c
  int32_t use_rope;
  float scale;
};

// Blocks per stage-1 slab: 256 G, i.e. 32 KB of scores for the 32 / G queries of a workgroup.
__host__ __device__ constexpr int ts_slab_blocks(int G) { return 256 * G; }

// Byte offsets of the token workgroup's LDS regions. The candidates' scores and, at the end, the
// waves' partial outputs share the first region.
struct TsTokenLayout {
  int64_t keys, red, kb, kp, zk, qs, hist, total;
};
__host__ __device__ inline int64_t ts_al16(int64_t x) { return (x + 15) / 16 * 16; }
__host__ __device__ inline TsTokenLayout ts_token_layout(int d, int G, int64_t C0, int64_t s1, int64_t s0) {
  TsTokenLayout L{};
  const int64_t sc = ts_al16(C0 * 4), red = ts_al16(4 * static_cast<int64_t>(G) * d * 4);
  int64_t off = sc > red ? sc : red;
  L.keys = 0;
  L.red = 0;
  L.kb = off;
  off += ts_al16(s1 * 4);
  L.kp = off;
  off += ts_al16(s0 * 4);
  L.zk = off;
  off += ts_al16(s0 * G * 4);
  L.qs = off;
  off += ts_al16(static_cast<int64_t>(G) * d * 4);
  L.hist = off;
  off += 256 * 4;
  L.total = off;
  return L;
}
// LDS of the merge workgroup: the merged list (scores, ids) and a histogram.
inline size_t ts_merge_lds_bytes(int64_t merge) { return static_cast<size_t>(2 * ts_al16(merge * 4) + 256 * 4); }

// q1[row] = round(rot(q[row], p1)), q0[row] = round(rot(q[row], p0)) for rows = B n_q H_q (copies
// without rotation).
hipError_t launch_ts_rotate_queries(const void* q, void* q1, void* q0, int64_t rows, int64_t p1, int64_t p0, int d,
                                    bool bf16, const InvFreq& iv, int use_rope, hipStream_t s);
hipError_t launch_ts_score(const TsArgs& a, int d, bool bf16, int G, hipStream_t s);
hipError_t launch_ts_merge(const TsArgs& a, hipStream_t s);
hipError_t launch_ts_tokens(const TsArgs& a, int d, bool bf16, int G, size_t lds, int64_t B, hipStream_t s);

// ---------------------------------------------------------------- allocation-free decode
// Device address of the library's scratch array (kNoallocScratchBytes) on the current device
// (looked up once per device).
hipError_t noalloc_scratch_address(void** out);

// The RoPE table cache (rope_cache.hip): *tab = its device rows when this device's cache holds
// (d, theta) and covers positions 0..P (filling it on `st` if no call has yet), else nullptr (the
// caller fills its own table). Waits on `st` for a fill enqueued by another stream until that fill
// is known to be complete; under graph capture only a completed cache is used.
hipError_t rope_cache_table(int d, float theta, const InvFreq& iv, int64_t P, hipStream_t st, const float2** tab);

}  // namespace recsa
