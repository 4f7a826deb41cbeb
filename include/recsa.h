/*
 * recsa.h -- RecSA tree attention on AMD Instinct MI355X (gfx950): C ABI.
 *
 * Method, cited by page title and section:
 *   [Abstract]  "Recursive Sparse Attention: Million-Token Length Extrapolation
 *               at Logarithmic Cost", abstract.
 *   [Core Idea] "Recursive Sparse Attention RecSA: Million-Token Context
 *               Extrapolation at Logarithmic Cost", section "Core Idea:
 *               Compressing the KV Cache with a Tree Structure".
 *   [Position]  the same page, section "Position Encoding Ingenuity: Making
 *               Extrapolation Possible".
 *
 * A tree is kept over each (sequence, KV head) of the KV cache. A node at
 * level l >= 1 covers f^l consecutive tokens and exists once all f children
 * exist; it holds one pooled key, W @ (mean of its children's stored keys),
 * and one value, the mean of its children's stored values [Abstract, Core
 * Idea]. A query descends from the top level; at each level its candidates
 * are the children of the nodes it kept one level up, followed by the nodes
 * that have no complete parent; it keeps the min(k_l, C_l) candidates with
 * the highest score (the scaled RoPE logit summed over the query heads that
 * share the KV head, ties to the lower candidate index) [Abstract]. The
 * candidate at position i of a level's list is rotated at i, the query at C_l
 * [Abstract, Position]; at the token level the candidates are the tokens
 * under the kept level-1 nodes plus the trailing partial block, and the query
 * sits at C_0, or C_0 - 1 when its own token is a candidate. Per query head a
 * single softmax weighs the dropped candidates (with their nodes' mean values)
 * together with the token-level candidates [Abstract].
 *
 * Conventions for every entry point:
 *   - Pointers marked [dev] are caller-owned HIP device memory; [host] are
 *     host memory read during the call only. The library never frees caller
 *     memory and allocates no device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls validate all
 *     arguments on the host first, then enqueue kernels on `stream` and return
 *     without waiting; outputs are valid once the stream reaches that point.
 *   - Storage type `dtype` (RECSA_F32 or RECSA_BF16) applies to K, V, q, the
 *     pooler W and the tree nodes. Outputs are float32.
 *   - Arrays are dense, row-major, with the innermost dimension head_dim;
 *     device pointers must be 16-byte aligned.
 *   - Every argument error is reported before any launch, as a negative
 *     status; recsa_last_error() then returns a message (thread-local). A
 *     failed HIP launch returns RECSA_ERR_HIP. No exceptions cross the ABI.
 *   - Calls on distinct streams with distinct output buffers may run
 *     concurrently; a workspace must not be shared by calls in flight.
 */
#ifndef RECSA_H
#define RECSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RECSA_ABI_VERSION 3
#define RECSA_MAX_LEVELS 32

typedef enum {
  RECSA_OK = 0,
  RECSA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned pointer, k < 0, ... */
  RECSA_ERR_CAPACITY = -2,     /* token count beyond the cache capacity */
  RECSA_ERR_UNSUPPORTED = -3,  /* shape outside what the kernels are built for */
  RECSA_ERR_HIP = -4,          /* a HIP runtime call or launch failed */
  RECSA_ERR_WORKSPACE = -5     /* workspace smaller than required */
} recsa_status_t;

typedef enum { RECSA_F32 = 0, RECSA_BF16 = 1 } recsa_dtype_t;

typedef struct {
  int32_t batch;          /* B sequences */
  int32_t n_kv_heads;     /* H_kv */
  int32_t n_q_heads;      /* H_q, a multiple of H_kv; G = H_q / H_kv query heads share a KV head (G <= 8) */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t fanout;         /* f: 2..64 */
  int32_t dtype;          /* recsa_dtype_t */
  int64_t capacity;       /* tokens per (sequence, KV head) slice of K and V; sizes the tree */
  float softmax_scale;    /* 0 => 1/sqrt(d), rounded to float32 */
  float rope_theta;       /* RoPE base (1e6 for Qwen3-style models); 0 disables the rotation */
  int32_t select_heads;   /* query heads that select together: 0 (or G) = the G heads of a KV head
                             share one selection (their logits summed); a divisor of G makes smaller
                             groups select independently over the same tree and cache (1 = every
                             head alone). recsa_decode and recsa_prefill support every divisor;
                             the other entry points need 0 or G. */
} recsa_shape_t;

/* ABI version (RECSA_ABI_VERSION). */
int32_t recsa_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* recsa_last_error(void);

/* T = max{l : floor(n / f^l) >= 1}, 0 when n < f (the complete-node forest). */
int32_t recsa_num_levels(int64_t n_tokens, int32_t fanout);

/* Bytes of the tree buffer for `capacity` tokens: for l = 1..T(capacity), the node keys
 * NK_l [B][H_kv][floor(capacity/f^l)][d] followed by the node values NV_l of the same shape,
 * level after level, in the storage type. Returns -1 on an invalid shape. */
int64_t recsa_tree_bytes(const recsa_shape_t* shape);

/* Byte offset of NK_l (which = 0) or NV_l (which = 1) inside the tree buffer; -1 if invalid. */
int64_t recsa_level_offset(const recsa_shape_t* shape, int32_t level, int32_t which);

/* Columns the `sel` output needs: the largest number of nodes kept at any level by any query
 * whose visible prefix has between n_min and n_max tokens. -1 if invalid. */
int32_t recsa_sel_width(const recsa_shape_t* shape, int64_t n_min, int64_t n_max,
                        const int32_t* k_per_level /*[host] n_levels*/, int32_t n_levels);

/* Workspace bytes needed by recsa_decode / recsa_prefill for visible prefixes of up to
 * n_max tokens (the RoPE table for candidate positions). -1 if invalid. */
int64_t recsa_workspace_bytes(const recsa_shape_t* shape, int64_t n_max,
                              const int32_t* k_per_level /*[host]*/, int32_t n_levels);

/* Step 1, tree build [Abstract, Core Idea].
 * Builds every node that is complete at n_new tokens but not at n_old, bottom level first:
 *   m = (sum of the f children's stored keys, in child order, float32) / f
 *   NK = round(W @ m)      (each output accumulated input by input in float32, one fused
 *                           multiply-add -- a single rounding -- per term)
 *   NV = round((sum of the f children's stored values, in child order, float32) / f)
 * Children are token rows at level 1 and stored level-(l-1) nodes above. Nodes complete at
 * n_old are left untouched, so growing the cache in any number of steps gives the same tree.
 *   K, V [dev]: [B][H_kv][capacity][d] pre-RoPE; W [dev]: [d][d] (key_i = sum_j W[i][j] m_j);
 *   tree [dev]: recsa_tree_bytes(shape) bytes.
 * Builds of different trees may run at once on different streams and may be captured in a HIP
 * graph. Large launches hand their tiles out through one of a few device-resident counters, each
 * serving one launch at a time (a launch that finds none free, or runs under graph capture, or
 * with RECSA_BUILD_QUEUE=0 in the environment, takes its tiles in a fixed order); the nodes do
 * not depend on the order. Allocates nothing.
 * Errors: INVALID_ARG (null, misaligned, n_old > n_new, n_old < 0), CAPACITY (n_new > capacity),
 * UNSUPPORTED (d, f or dtype). */
int32_t recsa_build_tree(const recsa_shape_t* shape, const void* K, const void* V, const void* W,
                         int64_t n_old, int64_t n_new, void* tree, void* stream);

/* Steps 2-4 for decoding [Abstract]: n_q queries per sequence, all at position n_tokens and
 * not in the cache, against the first n_tokens cached tokens (the tree must hold every node
 * complete at n_tokens).
 *   q [dev]: [B][n_q][H_q][d]; k_per_level [host]: k_l for l = 1..n_levels (n_levels >= T(n_tokens),
 *   k_l >= 0, INT32_MAX = keep everything).
 *   out [dev]: float32 [B][n_q][H_q][d]; lse [dev] (nullable): float32 [B][n_q][H_q], log of the
 *   softmax denominator (-inf and out = 0 when there is no entry, i.e. n_tokens = 0).
 *   sel [dev] (nullable): int32 [B][n_q][groups][n_levels][sel_width], the kept node ids of level
 *   l in row l-1, ascending, padded with -1; sel_width >= recsa_sel_width(n_tokens, n_tokens);
 *   groups = H_q / select_heads (H_kv by default).
 *   workspace [dev]: ws_bytes >= recsa_workspace_bytes(shape, n_tokens, k, n_levels).
 * Errors: INVALID_ARG, CAPACITY, UNSUPPORTED (candidate lists too long for on-chip memory, or
 * a slice of capacity * head_dim elements -- or its RoPE table -- of 4 GiB or more: the kernels
 * address a slice with 32-bit byte offsets), WORKSPACE. */
int32_t recsa_decode(const recsa_shape_t* shape, const void* q, int64_t n_q,
                     const void* K, const void* V, const void* tree, int64_t n_tokens,
                     const int32_t* k_per_level, int32_t n_levels,
                     float* out, float* lse, int32_t* sel, int32_t sel_width,
                     void* workspace, int64_t ws_bytes, void* stream);

/* recsa_decode for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not allocate, harnesses that forbid it): the same arguments minus the
 * workspace, the same kernels and results. The RoPE table goes to a scratch array the library
 * holds on each GPU (4 MiB, kept until the process ends), so no allocation happens in the call.
 * Calls on one GPU share that array: calls that overlap in time on one GPU (several streams or
 * threads) race and must be serialised by the caller. Calls whose table would exceed the array
 * (about 8K candidate positions at d = 128, e.g. a call that keeps every token of a long prefix)
 * are rejected with RECSA_ERR_UNSUPPORTED before any launch.
 * Errors: as recsa_decode, and UNSUPPORTED as above; HIP when the array's address cannot be
 * looked up. */
int32_t recsa_decode_noalloc(const recsa_shape_t* shape, const void* q, int64_t n_q,
                             const void* K, const void* V, const void* tree, int64_t n_tokens,
                             const int32_t* k_per_level, int32_t n_levels,
                             float* out, float* lse, int32_t* sel, int32_t sel_width, void* stream);

/* Steps 2-4 for causal prefill [Abstract]: query j sits at position t = q_start + j and sees
 * tokens 0..t, its own token included, through the nodes complete at t + 1 (the tree must hold
 * every node complete at q_start + n_q; nodes beyond a query's prefix are ignored). The result
 * does not depend on how a caller splits positions into calls.
 *   q [dev]: [B][n_q][H_q][d]; out float32 [B][n_q][H_q][d]; lse [B][n_q][H_q] (nullable);
 *   sel [B][n_q][H_kv][n_levels][sel_width] (nullable),
 *   sel_width >= recsa_sel_width(q_start + 1, q_start + n_q).
 *   workspace: recsa_workspace_bytes(shape, q_start + n_q, k, n_levels).
 * Errors as recsa_decode. */
int32_t recsa_prefill(const recsa_shape_t* shape, const void* q, int64_t q_start, int64_t n_q,
                      const void* K, const void* V, const void* tree,
                      const int32_t* k_per_level, int32_t n_levels,
                      float* out, float* lse, int32_t* sel, int32_t sel_width,
                      void* workspace, int64_t ws_bytes, void* stream);

/* One step of autoregressive decoding [Abstract: the tree kept over the KV cache, logarithmic
 * cost per decoding step; Core Idea: nodes summarise complete spans of the cache]. Three parts,
 * in order, on `stream`:
 *   1. append: K[b][h][n_tokens] = k_new[b][h] and V[b][h][n_tokens] = v_new[b][h];
 *   2. build: the nodes complete at n_tokens + 1 but not at n_tokens -- at most one per level,
 *      bottom level first, each a parent of the one below -- with recsa_build_tree's arithmetic
 *      (the tree must already hold every node complete at n_tokens);
 *   3. attend: q, the new token's query at position n_tokens, over tokens 0..n_tokens with its
 *      own token included: recsa_prefill with q_start = n_tokens and n_q = 1.
 * Calling it for n_tokens = n, n + 1, ... gives, bit for bit, the caches, tree and outputs that
 * writing the tokens, recsa_build_tree and recsa_prefill give for the same positions.
 *   q [dev]: [B][H_q][d]; k_new, v_new [dev]: [B][H_kv][d] pre-RoPE, storage type, not inside K or V;
 *   K, V [dev]: [B][H_kv][capacity][d], written at row n_tokens; W [dev]: [d][d] pooler;
 *   tree [dev]: updated in place; out float32 [B][H_q][d]; lse float32 [B][H_q] (nullable);
 *   sel [dev] (nullable): int32 [B][H_kv][n_levels][sel_width],
 *   sel_width >= recsa_sel_width(n_tokens + 1, n_tokens + 1);
 *   workspace: recsa_workspace_bytes(shape, n_tokens + 1, k, n_levels).
 * Errors: as recsa_prefill; CAPACITY when n_tokens + 1 > capacity; INVALID_ARG when k_new or
 * v_new overlaps a cache. Nothing is written when an error is returned. */
int32_t recsa_decode_step(const recsa_shape_t* shape, const void* q, const void* k_new, const void* v_new,
                          void* K, void* V, const void* W, void* tree, int64_t n_tokens,
                          const int32_t* k_per_level, int32_t n_levels,
                          float* out, float* lse, int32_t* sel, int32_t sel_width,
                          void* workspace, int64_t ws_bytes, void* stream);

/* Gradients of a recsa_decode (causal = 0) or recsa_prefill (causal = 1) call with respect to
 * q, K, V and the pooler W [Abstract: RecSA is trained -- its pooler distilled, the model
 * fine-tuned]. The pages do not say how gradients pass the selection. Reading: which candidates
 * a level keeps is taken from the forward call's `sel` and held fixed (a discrete choice, not
 * differentiated), and the forward's roundings to the storage type are passed straight through.
 * Per query head and entry e (logit z, weight P, value v_e):
 *   dz = P (dout . v_e - dout . out) + dlse P; v_e gets sum_h P dout_h; the entry's key row gets
 *   the transposed rotation (at its candidate index) of scale sum_h dz q~_h; q gets the
 *   transposed rotations (at each level's query position) of scale sum_e dz k~_e.
 * A node's key is W @ m (m the mean of its children's stored keys), its value the mean of its
 * children's values: a node's key gradient a adds outer(a, m) to dW and W^T a / f to each
 * child's key gradient, its value gradient adds 1/f of itself to each child's, level by level
 * down to the token rows.
 *   causal = 0: n_q queries at position n_tokens (q_start ignored); causal = 1: query j at
 *   q_start + j over tokens 0..q_start + j (n_tokens ignored). q, K, V, W, tree, k_per_level
 *   and n_levels as in the forward call.
 *   out, lse, sel [dev]: the forward call's outputs (sel is required; sel_width as given there).
 *   dout [dev]: float32 [B][n_q][H_q][d]; dlse [dev]: float32 [B][n_q][H_q] (nullable: zero).
 *   dq [dev]: float32 [B][n_q][H_q][d], written.
 *   dK, dV [dev]: float32 [B][H_kv][capacity][d], and dW [dev]: float32 [d][d], added to (zero
 *   them before the first call; calls over successive chunks of queries accumulate). dK and dV
 *   may both be NULL: the token rows' gradients are then not computed (dq and dW are).
 *   workspace: recsa_backward_workspace_bytes(shape, n_max, k, n_levels) with n_max = n_tokens
 *   (decode) or q_start + n_q: the RoPE table and float32 node gradients.
 * Row gradients are summed with float32 atomic adds, in an order the hardware chooses, so they
 * are not bitwise reproducible from run to run.
 * Errors: INVALID_ARG, CAPACITY, UNSUPPORTED, WORKSPACE. */
int64_t recsa_backward_workspace_bytes(const recsa_shape_t* shape, int64_t n_max,
                                       const int32_t* k_per_level, int32_t n_levels);
int32_t recsa_backward(const recsa_shape_t* shape, int32_t causal, const void* q, int64_t q_start,
                       int64_t n_q, int64_t n_tokens, const void* K, const void* V, const void* W,
                       const void* tree, const int32_t* k_per_level, int32_t n_levels,
                       const float* out, const float* lse, const int32_t* sel, int32_t sel_width,
                       const float* dout, const float* dlse,
                       float* dq, float* dK, float* dV, float* dW,
                       void* workspace, int64_t ws_bytes, void* stream);

/* One step of pooler distillation on a fixed batch of decode queries [Abstract; Core Idea: the
 * pooler is learned by distilling from full attention]. The pages give neither loss nor
 * optimiser. Reading: loss = mean over (sequence, query, query head, dimension) of
 * (out - target)^2, out being recsa_decode's output and target full attention's (e.g.
 * recsa_dense_ref_attn on the same queries); the gradient is taken with the selections held
 * fixed (recsa_backward), and W is updated by plain gradient descent on a float32 master copy.
 * In order on `stream`: the tree is rebuilt with the current W (all nodes complete at
 * n_tokens), the queries are decoded (selections recorded), dL/dout = 2 (out - target) / N and
 * the loss are formed, dW is computed, then W_master -= lr * dW and W = round(W_master).
 *   q [dev]: [B][n_q][H_q][d]; K, V [dev]: caches; target [dev]: float32 [B][n_q][H_q][d].
 *   W_master [dev]: float32 [d][d], updated; W [dev]: [d][d] storage type, the pooler this step
 *   uses, overwritten with the rounded update; tree [dev]: rebuilt (recsa_tree_bytes).
 *   loss [dev]: one float32, the loss at the W this step used.
 *   workspace: recsa_distill_workspace_bytes(shape, n_tokens, n_q, k, n_levels).
 * Errors: INVALID_ARG, CAPACITY, UNSUPPORTED, WORKSPACE. */
int64_t recsa_distill_workspace_bytes(const recsa_shape_t* shape, int64_t n_tokens, int64_t n_q,
                                      const int32_t* k_per_level, int32_t n_levels);
int32_t recsa_distill_step(const recsa_shape_t* shape, const void* q, int64_t n_q, const void* K,
                           const void* V, int64_t n_tokens, const int32_t* k_per_level, int32_t n_levels,
                           const float* target, float lr, float* W_master, void* W, void* tree,
                           float* loss, void* workspace, int64_t ws_bytes, void* stream);

/* Two-stage block-then-token selection for decoding, over the same cache and tree: a coarse pass
 * keeps the best blocks, a token pass keeps the best tokens inside them, and attention runs over
 * the kept tokens only ["HISA: Efficient Hierarchical Indexing for Fine-Grained Sparse
 * Attention", summary: block-level filtering, then the token-level indexer inside the kept blocks,
 * with the same top-k token pattern downstream], with RecSA's pooled keys and index positions
 * [Abstract, Position]. The pages give no formulas for it. Reading: the blocks are the level-1
 * nodes (f tokens each, key W @ mean of the token keys, built by recsa_build_tree); with n1 =
 * floor(n_tokens / f):
 *   1. every block g < n1 is a candidate at index g, the query at n1; the s1 = min(k_block, n1)
 *      blocks with the highest group score are kept (ties to the lower index), the rest dropped;
 *   2. the kept blocks' tokens (ascending), then the trailing tokens f n1 .. n_tokens - 1, are
 *      candidates at their index i, the query at C0 = f s1 + n_tokens - f n1; the
 *      s0 = min(k_token, C0) best are kept, the rest dropped;
 *   3. one softmax per query head over the kept tokens with the logits of step 2.
 * Scores and logits are those of recsa_decode (same rotation, rounding and scale). Queries as
 * recsa_decode: n_q per sequence, all at position n_tokens, not in the cache. select_heads must
 * be 0 (or G).
 *   q [dev]: [B][n_q][H_q][d]; K, V [dev]: caches; tree [dev]: built up to n_tokens (level 1 is read).
 *   block_keys [dev] (nullable): [B][H_kv][floor(capacity / f)][d] storage type, the level-1 keys
 *   rotated at their block index (recsa_two_stage_rotate_blocks), valid for every block below n1;
 *   NULL rotates them into the workspace on every call.
 *   out [dev]: float32 [B][n_q][H_q][d]; lse [dev] (nullable): float32 [B][n_q][H_q] (-inf and out = 0
 *   when nothing is kept).
 *   sel_blocks [dev] (nullable): int32 [B][n_q][H_kv][sel_block_width], kept block ids ascending,
 *   -1 padded, sel_block_width >= s1; sel_tokens [dev] (nullable): int32 [B][n_q][H_kv][sel_token_width],
 *   kept token ids ascending, -1 padded, sel_token_width >= s0.
 *   workspace: recsa_two_stage_workspace_bytes(shape, n_tokens, n_q, k_block, k_token,
 *   block_keys != NULL): RoPE table, rotated queries, rotated block keys (when not given), the
 *   per-slab candidate lists and the kept block ids.
 * Errors: INVALID_ARG, CAPACITY, UNSUPPORTED (select_heads, or k_block / k_token so large that a
 * query's candidate lists exceed on-chip memory), WORKSPACE. */
int64_t recsa_two_stage_workspace_bytes(const recsa_shape_t* shape, int64_t n_tokens, int64_t n_q, int32_t k_block,
                                        int32_t k_token, int32_t blocks_rotated);
int32_t recsa_two_stage_decode(const recsa_shape_t* shape, const void* q, int64_t n_q, const void* K, const void* V,
                               const void* tree, const void* block_keys, int64_t n_tokens, int32_t k_block,
                               int32_t k_token, float* out, float* lse, int32_t* sel_blocks, int32_t sel_block_width,
                               int32_t* sel_tokens, int32_t sel_token_width, void* workspace, int64_t ws_bytes,
                               void* stream);

/* Rotates the level-1 keys of the blocks complete at n_new but not at n_old into block_keys
 * (block g at position g, recsa_rotate_keys' arithmetic): a cache of rotated block keys kept next
 * to the tree, for recsa_two_stage_decode.
 *   tree [dev]: built up to n_new; block_keys [dev]: [B][H_kv][floor(capacity / f)][d] storage type.
 * Errors: INVALID_ARG (null, misaligned, overlap, n_old > n_new), CAPACITY. */
int32_t recsa_two_stage_rotate_blocks(const recsa_shape_t* shape, const void* tree, int64_t n_old, int64_t n_new,
                                      void* block_keys, void* stream);

/* Dense softmax attention with standard RoPE at the original positions -- the comparator the
 * method is timed against [Abstract]; also RecSA's limit when every level keeps everything.
 * mode: RECSA_DENSE_CAUSAL (bit 0) and/or RECSA_DENSE_KEYS_ROTATED (bit 1).
 *   not causal: decode, every query at position n_tokens against keys 0..n_tokens-1 (q_start ignored).
 *   causal: query j at position t = q_start + j against keys 0..t (q_start + n_q <= n_tokens).
 *   keys rotated: K already holds each key rotated at its own position (recsa_rotate_keys), as a
 *   dense cache usually stores it; otherwise K is pre-RoPE and is rotated into the workspace first.
 *   q [dev]: [B][n_q][H_q][d] pre-RoPE; out float32 [B][n_q][H_q][d]; lse float32 [B][n_q][H_q] (nullable).
 *   bf16 runs on the matrix cores with the probabilities rounded to bf16 for P V; float32 runs on
 *   the vector units. workspace: recsa_dense_workspace_bytes(shape, n_tokens, n_q, mode).
 * Errors: INVALID_ARG, CAPACITY, UNSUPPORTED, WORKSPACE. */
#define RECSA_DENSE_CAUSAL 1
#define RECSA_DENSE_KEYS_ROTATED 2
int64_t recsa_dense_workspace_bytes(const recsa_shape_t* shape, int64_t n_tokens, int64_t n_q, int32_t mode);
int32_t recsa_dense_ref_attn(const recsa_shape_t* shape, const void* q, int64_t q_start, int64_t n_q,
                             const void* K, const void* V, int64_t n_tokens, int32_t mode,
                             float* out, float* lse, void* workspace, int64_t ws_bytes, void* stream);

/* Rotates the first n_tokens keys of every slice at their own positions (standard RoPE, the
 * same rounding as the tree path): K_rot[b][h][p] = round(rot(K[b][h][p], p)).
 *   K, K_rot [dev]: [B][H_kv][capacity][d]; they must not overlap.
 * Errors: INVALID_ARG, CAPACITY, UNSUPPORTED. */
int32_t recsa_rotate_keys(const recsa_shape_t* shape, const void* K, int64_t n_tokens, void* K_rot, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RECSA_H */
