// RecSA C ABI: argument validation, tree layout, workspace sizing and launch order.
// Every entry point validates everything before the first launch and reports errors
// as negative status codes with a thread-local message.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.hpp"
#include "recsa.h"

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(RECSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxList = 4096;     // kept-node / candidate list capacity in LDS
constexpr int64_t kMaxSliceBytes = int64_t(1) << 32;   // attention: 32-bit offsets within a slice
constexpr size_t kMaxLds = 65536;
constexpr size_t kMaxLdsMerge = 163840;   // gfx950: 160 KB of LDS per workgroup
constexpr int64_t kTableAlign = 256;

struct Info {
  int64_t B, Hkv, Hq, d, f, G, cap;
  int64_t Gs;     // query heads per selection group (G by default)
  bool bf16;
  int64_t esz;
  float scale, theta;
};

int32_t check_shape(const recsa_shape_t* s, Info* o) {
  if (!s) return fail(RECSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->batch <= 0 || s->n_kv_heads <= 0 || s->n_q_heads <= 0)
    return fail(RECSA_ERR_INVALID_ARG, "batch, n_kv_heads and n_q_heads must be positive");
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(RECSA_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", s->n_q_heads,
                s->n_kv_heads);
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(RECSA_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(RECSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", s->head_dim);
  if (s->fanout < 2 || s->fanout > 64) return fail(RECSA_ERR_UNSUPPORTED, "fanout must be in 2..64 (got %d)", s->fanout);
  if (s->dtype != RECSA_F32 && s->dtype != RECSA_BF16) return fail(RECSA_ERR_UNSUPPORTED, "dtype %d", s->dtype);
  if (s->capacity < 0 || s->capacity > INT32_MAX)
    return fail(RECSA_ERR_INVALID_ARG, "capacity must be in 0..2^31-1");
  if (!(s->softmax_scale >= 0.0f) || !std::isfinite(s->softmax_scale))
    return fail(RECSA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (!(s->rope_theta >= 0.0f) || !std::isfinite(s->rope_theta) || (s->rope_theta > 0.0f && s->rope_theta <= 1.0f))
    return fail(RECSA_ERR_INVALID_ARG, "rope_theta must be 0 or > 1");
  o->B = s->batch;
  o->Hkv = s->n_kv_heads;
  o->Hq = s->n_q_heads;
  o->d = s->head_dim;
  o->f = s->fanout;
  o->G = G;
  o->cap = s->capacity;
  o->bf16 = s->dtype == RECSA_BF16;
  o->esz = o->bf16 ? 2 : 4;
  o->scale = s->softmax_scale > 0.0f ? s->softmax_scale : static_cast<float>(1.0 / std::sqrt(static_cast<double>(s->head_dim)));
  o->theta = s->rope_theta;
  if (s->select_heads < 0 || (s->select_heads > 0 && G % s->select_heads != 0))
    return fail(RECSA_ERR_INVALID_ARG, "select_heads (%d) must be 0 or divide the %d query heads of a KV head",
                s->select_heads, G);
  o->Gs = s->select_heads > 0 ? s->select_heads : G;
  return RECSA_OK;
}

// entry points whose kernels select per whole KV head group only
int32_t need_group_selection(const Info& I) {
  if (I.Gs != I.G) return fail(RECSA_ERR_UNSUPPORTED, "this entry point needs select_heads = 0 (or %lld)", (long long)I.G);
  return RECSA_OK;
}

int levels_of(int64_t n, int64_t f) {
  int T = 0;
  for (int64_t m = n / f; m >= 1; m /= f) ++T;
  return T;
}

int64_t nodes_at(int64_t n, int64_t f, int lv) {
  int64_t m = n;
  for (int i = 0; i < lv; ++i) m /= f;
  return m;
}

int64_t level_offset_bytes(const Info& I, int lv, int which) {
  int64_t off = 0;
  for (int l = 1; l < lv; ++l) off += 2 * I.B * I.Hkv * nodes_at(I.cap, I.f, l) * I.d * I.esz;
  if (which) off += I.B * I.Hkv * nodes_at(I.cap, I.f, lv) * I.d * I.esz;
  return off;
}

int32_t check_k(const int32_t* k, int32_t n_levels, int T) {
  if (n_levels < 0 || n_levels > RECSA_MAX_LEVELS)
    return fail(RECSA_ERR_INVALID_ARG, "n_levels must be in 0..%d", RECSA_MAX_LEVELS);
  if (n_levels < T) return fail(RECSA_ERR_INVALID_ARG, "n_levels (%d) is below the tree height (%d)", n_levels, T);
  if (n_levels > 0 && !k) return fail(RECSA_ERR_INVALID_ARG, "k_per_level is NULL");
  for (int i = 0; i < n_levels; ++i)
    if (k[i] < 0) return fail(RECSA_ERR_INVALID_ARG, "k_per_level[%d] = %d is negative", i, k[i]);
  return RECSA_OK;
}

// Data-independent bounds over every visible prefix n <= n_max:
// B_l >= C_l(n), S_l = min(k_l, B_l) >= s_l(n); C_0 <= c0.
struct Bounds {
  int64_t smax = 1, csel = 1, c0 = 0, P = 0;
  int T = 0;
};

Bounds bounds_for(const Info& I, int64_t n_max, const int32_t* k) {
  Bounds bd;
  const int T = levels_of(n_max, I.f);
  bd.T = T;
  int64_t S_up = 0, Pmax = 0;
  for (int lv = T; lv >= 1; --lv) {
    const int64_t Bl = std::min(nodes_at(n_max, I.f, lv), I.f * S_up + I.f - 1);
    const int64_t Sl = std::min<int64_t>(k[lv - 1], Bl);
    bd.smax = std::max(bd.smax, Sl);
    if (k[lv - 1] < Bl) bd.csel = std::max(bd.csel, Bl);
    Pmax = std::max(Pmax, Bl);
    S_up = Sl;
  }
  bd.c0 = T ? std::min(n_max, I.f * S_up + I.f - 1) : n_max;
  bd.P = std::max(Pmax, bd.c0);
  return bd;
}

int32_t max_kept(int64_t n, int64_t f, const int32_t* k) {
  const int T = levels_of(n, f);
  int64_t s_up = 0, best = 0;
  for (int lv = T; lv >= 1; --lv) {
    const int64_t C = f * s_up + (nodes_at(n, f, lv) - f * nodes_at(n, f, lv + 1));
    const int64_t s = std::min<int64_t>(k[lv - 1], C);
    best = std::max(best, s);
    s_up = s;
  }
  return static_cast<int32_t>(best);
}

// The largest max_kept(n) over n_min <= n <= n_max. Level counts above the tokens depend on n
// only through n_1 = floor(n / f), so one n per n_1 is enough, and the walk (from the top of the
// range down) stops once it reaches the data-independent bound min(k_l, B_l) of bounds_for:
// usually at its first step.
int32_t max_kept_range(const Info& I, int64_t n_min, int64_t n_max, const int32_t* k) {
  const Bounds bd = bounds_for(I, n_max, k);
  int64_t ub = 0;
  {
    int64_t S_up = 0;
    for (int lv = bd.T; lv >= 1; --lv) {
      const int64_t Bl = std::min(nodes_at(n_max, I.f, lv), I.f * S_up + I.f - 1);
      const int64_t Sl = std::min<int64_t>(k[lv - 1], Bl);
      ub = std::max(ub, Sl);
      S_up = Sl;
    }
  }
  int32_t best = 0;
  for (int64_t n1 = n_max / I.f; n1 >= n_min / I.f && n1 >= 0; --n1) {
    best = std::max(best, max_kept(std::max(n1 * I.f, n_min), I.f, k));
    if (best >= ub) break;
  }
  return best;
}

int64_t table_bytes(const Info& I, int64_t P) {
  if (I.theta == 0.0f) return 0;
  return ((P + 1) * (I.d / 2) * static_cast<int64_t>(sizeof(float2)) + kTableAlign - 1) / kTableAlign * kTableAlign;
}

recsa::InvFreq inv_freq_of(const Info& I) {
  recsa::InvFreq iv{};
  for (int i = 0; i < I.d / 2; ++i)
    iv.w[i] = static_cast<float>(std::pow(static_cast<double>(I.theta), -2.0 * i / static_cast<double>(I.d)));
  return iv;
}

int32_t fill_table(const Info& I, int64_t P, void* ws, hipStream_t st) {
  if (I.theta == 0.0f) return RECSA_OK;
  hipError_t e = recsa::launch_rope_table(static_cast<float2*>(ws), P, static_cast<int>(I.d / 2), inv_freq_of(I), st);
  if (e != hipSuccess) return hip_fail(e, "RoPE table launch");
  return RECSA_OK;
}

// The table of positions 0..P from the device's RoPE table cache when it covers them (nullptr:
// the call fills its own table in its workspace).
int32_t cached_table(const Info& I, int64_t P, hipStream_t st, const float2** tab) {
  *tab = nullptr;
  if (I.theta == 0.0f) return RECSA_OK;
  hipError_t e = recsa::rope_cache_table(static_cast<int>(I.d), I.theta, inv_freq_of(I), P, st, tab);
  if (e != hipSuccess) return hip_fail(e, "RoPE table cache");
  return RECSA_OK;
}

// A validated attention call: its kernel arguments, LDS bytes and RoPE table rows.
struct AttendPlan {
  Info I;
  recsa::AttnArgs a{};
  size_t lds = 0;
  int64_t P = 0;
  bool empty = false;  // nothing to launch (no queries)
};

// Validates one decode / prefill call and fills its plan; launches nothing.
int32_t prepare_attend(const recsa_shape_t* shape, const void* q, int64_t n_q, const void* K, const void* V,
                       const void* tree, int64_t n_fixed, int64_t q_start, bool prefill, const int32_t* k,
                       int32_t n_levels, float* out, float* lse, int32_t* sel, int32_t sel_width, void* ws,
                       int64_t ws_bytes, AttendPlan* pl) {
  Info& I = pl->I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  if (n_q < 0) return fail(RECSA_ERR_INVALID_ARG, "n_q must be >= 0");
  if (n_q * I.Hq > INT32_MAX || I.B > 65535) return fail(RECSA_ERR_UNSUPPORTED, "grid too large");
  const int64_t n_max = prefill ? q_start + n_q : n_fixed;
  const int64_t n_min = prefill ? q_start + 1 : n_fixed;
  if (prefill && q_start < 0) return fail(RECSA_ERR_INVALID_ARG, "q_start must be >= 0");
  if (!prefill && n_fixed < 0) return fail(RECSA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_max > I.cap) return fail(RECSA_ERR_CAPACITY, "%lld tokens exceed the capacity %lld", (long long)n_max,
                                 (long long)I.cap);
  rc = check_k(k, n_levels, levels_of(n_max, I.f));
  if (rc) return rc;
  if (n_q == 0) {
    pl->empty = true;
    return RECSA_OK;
  }
  if (!q || !out || (n_max > 0 && (!K || !V)) || (levels_of(n_max, I.f) > 0 && !tree))
    return fail(RECSA_ERR_INVALID_ARG, "q, K, V, tree or out is NULL");
  if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(tree) || !aligned16(out) || !aligned16(ws))
    return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (sel) {
    const int32_t need = max_kept_range(I, n_min, n_max, k);
    if (sel_width < need) return fail(RECSA_ERR_INVALID_ARG, "sel_width %d < %d kept nodes", sel_width, need);
  }
  const Bounds bd = bounds_for(I, n_max, k);
  if (bd.smax > kMaxList || bd.csel > kMaxList)
    return fail(RECSA_ERR_UNSUPPORTED, "candidate lists up to %lld entries exceed %lld", (long long)std::max(bd.smax, bd.csel),
                (long long)kMaxList);
  // the attention kernels address a slice's rows (one sequence and KV head of the caches or of a
  // tree level) and the RoPE table with 32-bit byte offsets
  if (I.cap * I.d * I.esz >= kMaxSliceBytes || table_bytes(I, bd.P) >= kMaxSliceBytes)
    return fail(RECSA_ERR_UNSUPPORTED, "a cache slice of %lld tokens (or its RoPE table) reaches 4 GiB", (long long)I.cap);
  // scored-candidate buffers: every selecting level fits whole; the token level is processed in
  // chunks of zcap candidates, so an unbounded token list (no pruning) takes chunks of 256
  const int64_t zneed = std::max<int64_t>(bd.csel, std::min<int64_t>(bd.c0, 256));
  const int zcap = static_cast<int>((zneed + 15) / 16 * 16);
  const size_t lds = recsa::attend_lds_bytes(static_cast<int>(I.d), static_cast<int>(I.Gs), static_cast<int>(bd.smax),
                                             zcap);
  if (lds > kMaxLds) return fail(RECSA_ERR_UNSUPPORTED, "needs %zu bytes of LDS (max %zu)", lds, kMaxLds);
  const int64_t need_ws = table_bytes(I, bd.P);
  if (ws_bytes < need_ws) return fail(RECSA_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes, (long long)need_ws);
  if (need_ws > 0 && !ws) return fail(RECSA_ERR_INVALID_ARG, "workspace is NULL");

  pl->lds = lds;
  pl->P = bd.P;
  recsa::AttnArgs& a = pl->a;
  a.q = q;
  a.K = K;
  a.V = V;
  a.out = out;
  a.lse = lse;
  a.sel = sel;
  a.tab = static_cast<const float2*>(ws);
  a.cap = I.cap;
  a.n_q = n_q;
  a.n_fixed = n_fixed;
  a.q_start = q_start;
  a.prefill = prefill ? 1 : 0;
  a.Hkv = static_cast<int32_t>(I.Hq / I.Gs);
  a.Hkv_kv = static_cast<int32_t>(I.Hkv);
  a.kv_div = static_cast<int32_t>(I.G / I.Gs);
  a.Hq = static_cast<int32_t>(I.Hq);
  a.f = static_cast<int32_t>(I.f);
  a.n_levels = n_levels;
  a.sel_width = sel_width;
  a.scale = I.scale;
  a.use_rope = I.theta != 0.0f;
  a.smax = static_cast<int32_t>(bd.smax);
  a.zcap = zcap;
  for (int lv = 1; lv <= RECSA_MAX_LEVELS; ++lv) a.k.k[lv] = lv <= n_levels ? k[lv - 1] : 0;
  const int Tc = levels_of(I.cap, I.f);
  for (int lv = 1; lv <= Tc && lv <= RECSA_MAX_LEVELS; ++lv) {
    a.tree.NK[lv] = static_cast<const char*>(tree) + level_offset_bytes(I, lv, 0);
    a.tree.NV[lv] = static_cast<const char*>(tree) + level_offset_bytes(I, lv, 1);
    a.tree.rows[lv] = nodes_at(I.cap, I.f, lv);
  }
  return RECSA_OK;
}

int32_t launch_planned_attend(const AttendPlan& pl, hipStream_t st) {
  hipError_t e = recsa::launch_attend(pl.a, static_cast<int>(pl.I.d), pl.I.bf16, static_cast<int>(pl.I.Gs), pl.lds,
                                      pl.I.B, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return RECSA_OK;
}

// use_cache: take the RoPE table from the device's cache when it covers the call (the
// allocation-free entry point always fills its own table in its scratch)
int32_t run_attend(const recsa_shape_t* shape, const void* q, int64_t n_q, const void* K, const void* V,
                   const void* tree, int64_t n_fixed, int64_t q_start, bool prefill, const int32_t* k,
                   int32_t n_levels, float* out, float* lse, int32_t* sel, int32_t sel_width, void* ws,
                   int64_t ws_bytes, void* stream, bool use_cache = true) {
  AttendPlan pl;
  int32_t rc = prepare_attend(shape, q, n_q, K, V, tree, n_fixed, q_start, prefill, k, n_levels, out, lse, sel,
                              sel_width, ws, ws_bytes, &pl);
  if (rc || pl.empty) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float2* tab = nullptr;
  if (use_cache) {
    rc = cached_table(pl.I, pl.P, st, &tab);
    if (rc) return rc;
  }
  if (tab) {
    pl.a.tab = tab;
  } else {
    rc = fill_table(pl.I, pl.P, ws, st);
    if (rc) return rc;
  }
  return launch_planned_attend(pl, st);
}

}  // namespace

extern "C" {

int32_t recsa_abi_version(void) { return RECSA_ABI_VERSION; }

const char* recsa_last_error(void) { return g_err.c_str(); }

int32_t recsa_num_levels(int64_t n_tokens, int32_t fanout) {
  if (n_tokens < 0 || fanout < 2) return -1;
  return levels_of(n_tokens, fanout);
}

int64_t recsa_tree_bytes(const recsa_shape_t* shape) {
  Info I;
  if (check_shape(shape, &I)) return -1;
  return level_offset_bytes(I, levels_of(I.cap, I.f) + 1, 0);
}

int64_t recsa_level_offset(const recsa_shape_t* shape, int32_t level, int32_t which) {
  Info I;
  if (check_shape(shape, &I)) return -1;
  if (level < 1 || level > levels_of(I.cap, I.f) || (which != 0 && which != 1)) {
    fail(RECSA_ERR_INVALID_ARG, "level %d / which %d out of range", level, which);
    return -1;
  }
  return level_offset_bytes(I, level, which);
}

int32_t recsa_sel_width(const recsa_shape_t* shape, int64_t n_min, int64_t n_max, const int32_t* k, int32_t n_levels) {
  Info I;
  if (check_shape(shape, &I)) return -1;
  if (n_min < 0 || n_max < n_min) {
    fail(RECSA_ERR_INVALID_ARG, "need 0 <= n_min <= n_max");
    return -1;
  }
  if (check_k(k, n_levels, levels_of(n_max, I.f))) return -1;
  return max_kept_range(I, n_min, n_max, k);
}

int64_t recsa_workspace_bytes(const recsa_shape_t* shape, int64_t n_max, const int32_t* k, int32_t n_levels) {
  Info I;
  if (check_shape(shape, &I)) return -1;
  if (n_max < 0) {
    fail(RECSA_ERR_INVALID_ARG, "n_max must be >= 0");
    return -1;
  }
  if (check_k(k, n_levels, levels_of(n_max, I.f))) return -1;
  return table_bytes(I, bounds_for(I, n_max, k).P);
}

int32_t recsa_build_tree(const recsa_shape_t* shape, const void* K, const void* V, const void* W, int64_t n_old,
                         int64_t n_new, void* tree, void* stream) {
  Info I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  if (n_old < 0 || n_new < n_old) return fail(RECSA_ERR_INVALID_ARG, "need 0 <= n_old <= n_new");
  if (n_new > I.cap) return fail(RECSA_ERR_CAPACITY, "n_new %lld exceeds the capacity %lld", (long long)n_new, (long long)I.cap);
  const int T = levels_of(n_new, I.f);
  if (nodes_at(n_old, I.f, 1) == nodes_at(n_new, I.f, 1)) return RECSA_OK;  // no node completes
  if (!K || !V || !W || !tree) return fail(RECSA_ERR_INVALID_ARG, "K, V, W or tree is NULL");
  if (!aligned16(K) || !aligned16(V) || !aligned16(W) || !aligned16(tree))
    return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int Tc = levels_of(I.cap, I.f);
  const bool can_fuse = recsa::pool_nodes_per_tile(static_cast<int>(I.d)) % I.f == 0;
  // every launch of this call takes the one-tile form when the first (the largest) has at most
  // one tile per CU: a short build is latency-bound. Otherwise every launch is persistent.
  const int64_t npw = recsa::pool_nodes_per_tile(static_cast<int>(I.d));
  const int64_t first_span = nodes_at(n_new, I.f, 1) - nodes_at(n_old, I.f, 1) / npw * npw;
  const int64_t first_tiles = (first_span + npw - 1) / npw * I.B * I.Hkv;
  const int32_t one_tile = first_tiles * 2 <= recsa::pool_persistent_grid() ? 1 : 0;
  for (int lv = 1; lv <= T;) {
    const int64_t lo = nodes_at(n_old, I.f, lv), hi = nodes_at(n_new, I.f, lv);
    const bool fuse = can_fuse && lv + 1 <= Tc;
    if (hi > lo) {
      recsa::PoolArgs p{};
      if (lv == 1) {
        p.srcK = K;
        p.srcV = V;
        p.src_rows = I.cap;
      } else {
        p.srcK = static_cast<const char*>(tree) + level_offset_bytes(I, lv - 1, 0);
        p.srcV = static_cast<const char*>(tree) + level_offset_bytes(I, lv - 1, 1);
        p.src_rows = nodes_at(I.cap, I.f, lv - 1);
      }
      p.dstK = static_cast<char*>(tree) + level_offset_bytes(I, lv, 0);
      p.dstV = static_cast<char*>(tree) + level_offset_bytes(I, lv, 1);
      p.dst_rows = nodes_at(I.cap, I.f, lv);
      p.W = W;
      p.g_lo = lo;
      p.g_hi = hi;
      p.f = static_cast<int32_t>(I.f);
      p.BH = static_cast<int32_t>(I.B * I.Hkv);
      p.one_tile = one_tile;
      if (fuse) {
        p.fuse_next = 1;
        p.dst2K = static_cast<char*>(tree) + level_offset_bytes(I, lv + 1, 0);
        p.dst2V = static_cast<char*>(tree) + level_offset_bytes(I, lv + 1, 1);
        p.dst2_rows = nodes_at(I.cap, I.f, lv + 1);
      }
      hipError_t e = recsa::launch_pool_level(p, static_cast<int>(I.d), I.bf16, st);
      if (e != hipSuccess) return hip_fail(e, "tree build launch");
    }
    lv += fuse ? 2 : 1;
  }
  return RECSA_OK;
}

int32_t recsa_decode(const recsa_shape_t* shape, const void* q, int64_t n_q, const void* K, const void* V,
                     const void* tree, int64_t n_tokens, const int32_t* k, int32_t n_levels, float* out, float* lse,
                     int32_t* sel, int32_t sel_width, void* workspace, int64_t ws_bytes, void* stream) {
  return run_attend(shape, q, n_q, K, V, tree, n_tokens, 0, false, k, n_levels, out, lse, sel, sel_width, workspace,
                    ws_bytes, stream);
}

int32_t recsa_decode_noalloc(const recsa_shape_t* shape, const void* q, int64_t n_q, const void* K, const void* V,
                             const void* tree, int64_t n_tokens, const int32_t* k, int32_t n_levels, float* out,
                             float* lse, int32_t* sel, int32_t sel_width, void* stream) {
  // size check first: the scratch holds what recsa_decode's workspace would
  Info I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  if (n_tokens < 0) return fail(RECSA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens > I.cap)
    return fail(RECSA_ERR_CAPACITY, "%lld tokens exceed the capacity %lld", (long long)n_tokens, (long long)I.cap);
  rc = check_k(k, n_levels, levels_of(n_tokens, I.f));
  if (rc) return rc;
  const int64_t need = table_bytes(I, bounds_for(I, n_tokens, k).P);
  const int64_t have = static_cast<int64_t>(recsa::kNoallocScratchBytes);
  if (need > have)
    return fail(RECSA_ERR_UNSUPPORTED,
                "this call needs %lld bytes of scratch; the allocation-free entry point has %lld (use recsa_decode "
                "with a workspace)", (long long)need, (long long)have);
  void* scratch = nullptr;
  if (n_q > 0) {
    hipError_t e = recsa::noalloc_scratch_address(&scratch);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
  }
  return run_attend(shape, q, n_q, K, V, tree, n_tokens, 0, false, k, n_levels, out, lse, sel, sel_width, scratch,
                    have, stream, false);
}

int32_t recsa_prefill(const recsa_shape_t* shape, const void* q, int64_t q_start, int64_t n_q, const void* K,
                      const void* V, const void* tree, const int32_t* k, int32_t n_levels, float* out, float* lse,
                      int32_t* sel, int32_t sel_width, void* workspace, int64_t ws_bytes, void* stream) {
  return run_attend(shape, q, n_q, K, V, tree, 0, q_start, true, k, n_levels, out, lse, sel, sel_width, workspace,
                    ws_bytes, stream);
}

int32_t recsa_decode_step(const recsa_shape_t* shape, const void* q, const void* k_new, const void* v_new, void* K,
                          void* V, const void* W, void* tree, int64_t n_tokens, const int32_t* k, int32_t n_levels,
                          float* out, float* lse, int32_t* sel, int32_t sel_width, void* workspace, int64_t ws_bytes,
                          void* stream) {
  Info I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  if (n_tokens < 0) return fail(RECSA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens + 1 > I.cap)
    return fail(RECSA_ERR_CAPACITY, "the new token's row %lld is beyond the capacity %lld", (long long)n_tokens,
                (long long)I.cap);
  if (!k_new || !v_new || !K || !V || !W) return fail(RECSA_ERR_INVALID_ARG, "k_new, v_new, K, V or W is NULL");
  if (levels_of(n_tokens + 1, I.f) > 0 && !tree) return fail(RECSA_ERR_INVALID_ARG, "tree is NULL");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(W))
    return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  AttendPlan pl;
  rc = prepare_attend(shape, q, 1, K, V, tree, 0, n_tokens, true, k, n_levels, out, lse, sel, sel_width, workspace,
                      ws_bytes, &pl);
  if (rc) return rc;
  const char* kn = static_cast<const char*>(k_new);
  const char* vn = static_cast<const char*>(v_new);
  const int64_t row_bytes = I.B * I.Hkv * I.d * I.esz;
  const int64_t cache_bytes = I.B * I.Hkv * I.cap * I.d * I.esz;
  auto overlaps = [](const char* p, int64_t pn, const void* c, int64_t cn) {
    const char* cc = static_cast<const char*>(c);
    return p < cc + cn && cc < p + pn;
  };
  if (overlaps(kn, row_bytes, K, cache_bytes) || overlaps(kn, row_bytes, V, cache_bytes) ||
      overlaps(vn, row_bytes, K, cache_bytes) || overlaps(vn, row_bytes, V, cache_bytes))
    return fail(RECSA_ERR_INVALID_ARG, "k_new and v_new must not overlap the caches");

  recsa::StepArgs sa{};
  sa.k_new = k_new;
  sa.v_new = v_new;
  sa.K = K;
  sa.V = V;
  sa.cap = I.cap;
  sa.n = n_tokens;
  sa.W = W;
  const int Tc = levels_of(I.cap, I.f);
  for (int lv = 1; lv <= Tc && lv <= RECSA_MAX_LEVELS; ++lv) {
    sa.NK[lv] = static_cast<char*>(tree) + level_offset_bytes(I, lv, 0);
    sa.NV[lv] = static_cast<char*>(tree) + level_offset_bytes(I, lv, 1);
    sa.rows[lv] = nodes_at(I.cap, I.f, lv);
  }
  sa.levels = std::min(Tc, RECSA_MAX_LEVELS);
  sa.f = static_cast<int32_t>(I.f);
  sa.BH = static_cast<int32_t>(I.B * I.Hkv);
  sa.half = static_cast<int32_t>(I.d / 2);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the RoPE table: from the device's cache when it covers the call (the append launch then has
  // no table rows to fill), else filled into the workspace by the append launch's extra workgroups
  const float2* cached = nullptr;
  rc = cached_table(I, pl.P, st, &cached);
  if (rc) return rc;
  if (cached) {
    pl.a.tab = cached;
  } else if (I.theta != 0.0f) {
    sa.tab = static_cast<float2*>(workspace);
    sa.P = pl.P;
    sa.iv = inv_freq_of(I);
  }
  hipError_t e = recsa::launch_append_step(sa, static_cast<int>(I.d), I.bf16, st);
  if (e != hipSuccess) return hip_fail(e, "append step launch");
  return launch_planned_attend(pl, st);
}

// Gradient workspace: the RoPE table, then float32 node-key and node-value gradients laid out
// like the tree (levels 1..T(capacity), keys then values per level).
static int64_t grad_level_offset(const Info& I, int lv, int which) {
  Info J = I;
  J.esz = 4;
  return level_offset_bytes(J, lv, which);
}

static int32_t backward_bounds(const Info& I, int64_t n_max, const int32_t* k, int32_t n_levels, Bounds* bd) {
  int32_t rc = check_k(k, n_levels, levels_of(n_max, I.f));
  if (rc) return rc;
  *bd = bounds_for(I, n_max, k);
  if (bd->smax > kMaxList || bd->csel > kMaxList)
    return fail(RECSA_ERR_UNSUPPORTED, "candidate lists up to %lld entries exceed %lld",
                (long long)std::max(bd->smax, bd->csel), (long long)kMaxList);
  return RECSA_OK;
}

int64_t recsa_backward_workspace_bytes(const recsa_shape_t* shape, int64_t n_max, const int32_t* k, int32_t n_levels) {
  Info I;
  if (check_shape(shape, &I)) return -1;
  if (n_max < 0) {
    fail(RECSA_ERR_INVALID_ARG, "n_max must be >= 0");
    return -1;
  }
  Bounds bd;
  if (backward_bounds(I, n_max, k, n_levels, &bd)) return -1;
  return table_bytes(I, bd.P) + grad_level_offset(I, levels_of(I.cap, I.f) + 1, 0);
}

int32_t recsa_backward(const recsa_shape_t* shape, int32_t causal, const void* q, int64_t q_start, int64_t n_q,
                       int64_t n_tokens, const void* K, const void* V, const void* W, const void* tree,
                       const int32_t* k, int32_t n_levels, const float* out, const float* lse, const int32_t* sel,
                       int32_t sel_width, const float* dout, const float* dlse, float* dq, float* dK, float* dV,
                       float* dW, void* workspace, int64_t ws_bytes, void* stream) {
  Info I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  rc = need_group_selection(I);
  if (rc) return rc;
  if (causal != 0 && causal != 1) return fail(RECSA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (n_q < 0) return fail(RECSA_ERR_INVALID_ARG, "n_q must be >= 0");
  if (n_q * I.Hkv > INT32_MAX || I.B > 65535) return fail(RECSA_ERR_UNSUPPORTED, "grid too large");
  if (causal && q_start < 0) return fail(RECSA_ERR_INVALID_ARG, "q_start must be >= 0");
  if (!causal && n_tokens < 0) return fail(RECSA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  const int64_t n_max = causal ? q_start + n_q : n_tokens;
  const int64_t n_min = causal ? q_start + 1 : n_tokens;
  if (n_max > I.cap)
    return fail(RECSA_ERR_CAPACITY, "%lld tokens exceed the capacity %lld", (long long)n_max, (long long)I.cap);
  Bounds bd;
  rc = backward_bounds(I, n_max, k, n_levels, &bd);
  if (rc) return rc;
  if (n_q == 0) return RECSA_OK;
  const int T = levels_of(n_max, I.f);
  if (!q || !out || !lse || !sel || !dout || !dq || !dW || (n_max > 0 && (!K || !V)) || (T > 0 && (!tree || !W)))
    return fail(RECSA_ERR_INVALID_ARG, "q, K, V, W, tree, out, lse, sel, dout, dq or dW is NULL");
  if ((dK == nullptr) != (dV == nullptr)) return fail(RECSA_ERR_INVALID_ARG, "dK and dV must both be given or both be NULL");
  if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(W) || !aligned16(tree) || !aligned16(out) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dK) || !aligned16(dV) || !aligned16(dW) || !aligned16(workspace))
    return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int32_t need = max_kept_range(I, n_min, n_max, k);
  if (sel_width < std::max(need, 1)) return fail(RECSA_ERR_INVALID_ARG, "sel_width %d < %d kept nodes", sel_width, need);
  const int64_t tab = table_bytes(I, bd.P);
  const int64_t need_ws = tab + grad_level_offset(I, levels_of(I.cap, I.f) + 1, 0);
  if (ws_bytes < need_ws) return fail(RECSA_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes, (long long)need_ws);
  if (!workspace) return fail(RECSA_ERR_INVALID_ARG, "workspace is NULL");

  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = fill_table(I, bd.P, workspace, st);
  if (rc) return rc;
  char* gbase = static_cast<char*>(workspace) + tab;
  const int Tc = levels_of(I.cap, I.f);
  for (int lv = 1; lv <= T; ++lv) {
    hipError_t e = recsa::launch_fill_zero(reinterpret_cast<float*>(gbase + grad_level_offset(I, lv, 0)),
                                           2 * I.B * I.Hkv * nodes_at(I.cap, I.f, lv) * I.d, st);
    if (e != hipSuccess) return hip_fail(e, "gradient workspace clear");
  }
  recsa::BwdArgs a{};
  a.q = q;
  a.K = K;
  a.V = V;
  a.out = out;
  a.lse = lse;
  a.sel = sel;
  a.dout = dout;
  a.dlse = dlse;
  a.dq = dq;
  a.dK = dK;
  a.dV = dV;
  a.tab = static_cast<const float2*>(workspace);
  a.cap = I.cap;
  a.n_q = n_q;
  a.n_fixed = n_tokens;
  a.q_start = causal ? q_start : 0;
  a.causal = causal;
  a.Hkv = static_cast<int32_t>(I.Hkv);
  a.Hq = static_cast<int32_t>(I.Hq);
  a.f = static_cast<int32_t>(I.f);
  a.n_levels = n_levels;
  a.sel_width = sel_width;
  a.scale = I.scale;
  a.use_rope = I.theta != 0.0f;
  a.zcap = static_cast<int32_t>((bd.csel + 15) / 16 * 16);
  a.smax = static_cast<int32_t>(bd.smax);
  for (int lv = 1; lv <= Tc && lv <= RECSA_MAX_LEVELS; ++lv) {
    a.tree.NK[lv] = static_cast<const char*>(tree) + level_offset_bytes(I, lv, 0);
    a.tree.NV[lv] = static_cast<const char*>(tree) + level_offset_bytes(I, lv, 1);
    a.tree.rows[lv] = nodes_at(I.cap, I.f, lv);
    a.gNK[lv] = reinterpret_cast<float*>(gbase + grad_level_offset(I, lv, 0));
    a.gNV[lv] = reinterpret_cast<float*>(gbase + grad_level_offset(I, lv, 1));
  }
  hipError_t e = recsa::launch_backward_units(a, static_cast<int>(I.d), I.bf16, static_cast<int>(I.G), I.B, st);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  for (int lv = T; lv >= 1; --lv) {
    recsa::TreePushArgs p{};
    p.childK = lv == 1 ? K : a.tree.NK[lv - 1];
    p.child_rows = lv == 1 ? I.cap : nodes_at(I.cap, I.f, lv - 1);
    p.gk = a.gNK[lv];
    p.gv = a.gNV[lv];
    p.rows = nodes_at(I.cap, I.f, lv);
    p.n_nodes = nodes_at(n_max, I.f, lv);
    p.ck = lv == 1 ? dK : a.gNK[lv - 1];
    p.cv = lv == 1 ? dV : a.gNV[lv - 1];
    p.W = W;
    p.dW = dW;
    p.f = static_cast<int32_t>(I.f);
    p.BH = static_cast<int32_t>(I.B * I.Hkv);
    e = recsa::launch_tree_push(p, static_cast<int>(I.d), I.bf16, st);
    if (e != hipSuccess) return hip_fail(e, "tree gradient launch");
  }
  return RECSA_OK;
}

// Pooler distillation step: workspace sub-buffers, each 256-byte aligned.
struct DistillPlan {
  int64_t dec_ws, out, lse, sel, dout, dq, dW, partial, bwd_ws, total;
  int32_t width;
};

static int64_t al256(int64_t x) { return (x + 255) / 256 * 256; }

static int32_t distill_plan(const recsa_shape_t* shape, int64_t n_tokens, int64_t n_q, const int32_t* k,
                            int32_t n_levels, DistillPlan* p) {
  Info I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  if (n_q < 1) return fail(RECSA_ERR_INVALID_ARG, "n_q must be >= 1");
  if (n_tokens < 0) return fail(RECSA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens > I.cap)
    return fail(RECSA_ERR_CAPACITY, "n_tokens %lld exceeds the capacity %lld", (long long)n_tokens, (long long)I.cap);
  rc = check_k(k, n_levels, levels_of(n_tokens, I.f));
  if (rc) return rc;
  const int64_t dec = recsa_workspace_bytes(shape, n_tokens, k, n_levels);
  const int64_t bwd = recsa_backward_workspace_bytes(shape, n_tokens, k, n_levels);
  if (dec < 0 || bwd < 0) return RECSA_ERR_UNSUPPORTED;
  p->width = std::max<int32_t>(max_kept(n_tokens, I.f, k), 1);
  const int64_t rows = I.B * n_q * I.Hq;
  int64_t o = 0;
  p->dec_ws = o; o += al256(dec);
  p->out = o; o += al256(rows * I.d * 4);
  p->lse = o; o += al256(rows * 4);
  p->sel = o; o += al256(I.B * n_q * I.Hkv * std::max(n_levels, 1) * static_cast<int64_t>(p->width) * 4);
  p->dout = o; o += al256(rows * I.d * 4);
  p->dq = o; o += al256(rows * I.d * 4);
  p->dW = o; o += al256(I.d * I.d * 4);
  p->partial = o; o += al256(static_cast<int64_t>(recsa::distill_loss_blocks(rows * I.d)) * 4);
  p->bwd_ws = o; o += al256(bwd);
  p->total = o;
  return RECSA_OK;
}

int64_t recsa_distill_workspace_bytes(const recsa_shape_t* shape, int64_t n_tokens, int64_t n_q, const int32_t* k,
                                      int32_t n_levels) {
  DistillPlan p;
  if (distill_plan(shape, n_tokens, n_q, k, n_levels, &p)) return -1;
  return p.total;
}

int32_t recsa_distill_step(const recsa_shape_t* shape, const void* q, int64_t n_q, const void* K, const void* V,
                           int64_t n_tokens, const int32_t* k, int32_t n_levels, const float* target, float lr,
                           float* W_master, void* W, void* tree, float* loss, void* workspace, int64_t ws_bytes,
                           void* stream) {
  DistillPlan p;
  int32_t rc = distill_plan(shape, n_tokens, n_q, k, n_levels, &p);
  if (rc) return rc;
  Info I;
  check_shape(shape, &I);
  rc = need_group_selection(I);
  if (rc) return rc;
  if (!std::isfinite(lr)) return fail(RECSA_ERR_INVALID_ARG, "lr must be finite");
  if (!q || !target || !W_master || !W || !loss || !workspace || (n_tokens > 0 && (!K || !V)) ||
      (levels_of(I.cap, I.f) > 0 && !tree))
    return fail(RECSA_ERR_INVALID_ARG, "q, K, V, target, W_master, W, tree, loss or workspace is NULL");
  if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(target) || !aligned16(W_master) || !aligned16(W) ||
      !aligned16(tree) || !aligned16(workspace))
    return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (ws_bytes < p.total)
    return fail(RECSA_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes, (long long)p.total);
  char* ws = static_cast<char*>(workspace);
  float* out = reinterpret_cast<float*>(ws + p.out);
  float* lse = reinterpret_cast<float*>(ws + p.lse);
  int32_t* sel = reinterpret_cast<int32_t*>(ws + p.sel);
  float* dout = reinterpret_cast<float*>(ws + p.dout);
  float* dq = reinterpret_cast<float*>(ws + p.dq);
  float* dW = reinterpret_cast<float*>(ws + p.dW);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = recsa_build_tree(shape, K, V, W, 0, n_tokens, tree, stream);
  if (rc) return rc;
  rc = recsa_decode(shape, q, n_q, K, V, tree, n_tokens, k, n_levels, out, lse, sel, p.width, ws + p.dec_ws,
                    p.out - p.dec_ws, stream);
  if (rc) return rc;
  const int64_t n = I.B * n_q * I.Hq * I.d;
  hipError_t e = recsa::launch_distill_loss(out, target, dout, reinterpret_cast<float*>(ws + p.partial), loss, n, st);
  if (e != hipSuccess) return hip_fail(e, "distillation loss launch");
  e = recsa::launch_fill_zero(dW, I.d * I.d, st);
  if (e != hipSuccess) return hip_fail(e, "gradient clear");
  rc = recsa_backward(shape, 0, q, 0, n_q, n_tokens, K, V, W, tree, k, n_levels, out, lse, sel, p.width, dout, nullptr,
                      dq, nullptr, nullptr, dW, ws + p.bwd_ws, p.total - p.bwd_ws, stream);
  if (rc) return rc;
  e = recsa::launch_distill_update(W_master, dW, W, lr, I.d * I.d, I.bf16, st);
  if (e != hipSuccess) return hip_fail(e, "pooler update launch");
  return RECSA_OK;
}

struct DensePlan {
  int64_t kr_bytes = 0, qr_bytes = 0, part_o_bytes = 0, part_ml_bytes = 0, total = 0, keys_per_split = 0;
  int32_t splits = 1;
};

static DensePlan dense_plan(const Info& I, int64_t n_tokens, int64_t n_q, int32_t mode) {
  DensePlan p;
  const bool causal = mode & RECSA_DENSE_CAUSAL;
  const bool rotated = mode & RECSA_DENSE_KEYS_ROTATED;
  if (!rotated && I.theta != 0.0f) p.kr_bytes = ((I.B * I.Hkv * n_tokens * I.d * I.esz) + 255) / 256 * 256;
  // bf16 runs on the matrix cores with the queries rotated beforehand
  if (I.bf16 && I.theta != 0.0f) p.qr_bytes = ((I.B * n_q * I.Hq * I.d * 2) + 255) / 256 * 256;
  p.keys_per_split = std::max<int64_t>(n_tokens, 1);
  if (I.bf16 && !causal && n_tokens > 0 && n_q > 0) {
    const int64_t qpb = recsa::dense_queries_per_block(static_cast<int>(I.G));
    const int64_t wgs = (n_q + qpb - 1) / qpb * I.B * I.Hkv;
    int64_t splits = std::max<int64_t>(1, (2048 + wgs - 1) / wgs);
    splits = std::min<int64_t>(splits, (n_tokens + 255) / 256);
    int64_t kps = (n_tokens + splits - 1) / splits;
    kps = (kps + 63) / 64 * 64;
    splits = (n_tokens + kps - 1) / kps;
    p.splits = static_cast<int32_t>(splits);
    p.keys_per_split = kps;
  }
  if (p.splits > 1) {
    const int64_t rows = p.splits * I.B * I.Hkv * n_q * I.G;
    p.part_o_bytes = (rows * I.d * 4 + 255) / 256 * 256;
    p.part_ml_bytes = (rows * 2 * 4 + 255) / 256 * 256;
  }
  p.total = p.kr_bytes + p.qr_bytes + p.part_o_bytes + p.part_ml_bytes;
  return p;
}

int64_t recsa_dense_workspace_bytes(const recsa_shape_t* shape, int64_t n_tokens, int64_t n_q, int32_t mode) {
  Info I;
  if (check_shape(shape, &I)) return -1;
  if (n_tokens < 0 || n_q < 0 || (mode & ~3)) {
    fail(RECSA_ERR_INVALID_ARG, "need n_tokens >= 0, n_q >= 0 and mode in 0..3");
    return -1;
  }
  return dense_plan(I, n_tokens, n_q, mode).total;
}

int32_t recsa_rotate_keys(const recsa_shape_t* shape, const void* K, int64_t n_tokens, void* K_rot, void* stream) {
  Info I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  if (n_tokens < 0) return fail(RECSA_ERR_INVALID_ARG, "n_tokens must be >= 0");
  if (n_tokens > I.cap) return fail(RECSA_ERR_CAPACITY, "n_tokens %lld exceeds the capacity %lld", (long long)n_tokens,
                                    (long long)I.cap);
  if (n_tokens == 0) return RECSA_OK;
  if (!K || !K_rot) return fail(RECSA_ERR_INVALID_ARG, "K or K_rot is NULL");
  if (!aligned16(K) || !aligned16(K_rot)) return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int64_t bytes = I.B * I.Hkv * I.cap * I.d * I.esz;
  const char* a = static_cast<const char*>(K);
  const char* b = static_cast<const char*>(K_rot);
  if (a < b + bytes && b < a + bytes) return fail(RECSA_ERR_INVALID_ARG, "K and K_rot overlap");
  hipError_t e = recsa::launch_rotate_keys(K, I.cap, K_rot, I.cap, n_tokens, I.B * I.Hkv, static_cast<int>(I.d), I.bf16,
                                           inv_freq_of(I), I.theta != 0.0f, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "key rotation launch");
  return RECSA_OK;
}

// ---------------------------------------------------------------- two-stage block-then-token selection

struct TsPlan {
  Info I;
  int64_t n1 = 0, s1 = 0, C0 = 0, s0 = 0, SB = 0, n_slabs = 0, merge = 0;
  int64_t tab_bytes = 0, q_bytes = 0, kb_bytes = 0, cand_bytes = 0, kept_bytes = 0, total = 0;
  size_t lds = 0;
};

static int32_t ts_plan(const recsa_shape_t* shape, int64_t n_tokens, int64_t n_q, int32_t k_block, int32_t k_token,
                       bool own_blocks, TsPlan* p) {
  Info& I = p->I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  rc = need_group_selection(I);
  if (rc) return rc;
  if (n_tokens < 0 || n_q < 0) return fail(RECSA_ERR_INVALID_ARG, "n_tokens and n_q must be >= 0");
  if (k_block < 0 || k_token < 0) return fail(RECSA_ERR_INVALID_ARG, "k_block and k_token must be >= 0");
  if (n_tokens > I.cap) return fail(RECSA_ERR_CAPACITY, "n_tokens %lld exceeds the capacity %lld", (long long)n_tokens,
                                    (long long)I.cap);
  if (n_q > INT32_MAX || I.B * I.Hkv > 65535) return fail(RECSA_ERR_UNSUPPORTED, "grid too large");
  p->n1 = n_tokens / I.f;
  p->s1 = std::min<int64_t>(k_block, p->n1);
  p->C0 = I.f * p->s1 + (n_tokens - I.f * p->n1);
  p->s0 = std::min<int64_t>(k_token, p->C0);
  p->SB = recsa::ts_slab_blocks(static_cast<int>(I.G));
  p->n_slabs = (p->n1 + p->SB - 1) / p->SB;
  // stage 1 launches one workgroup per (slice, slab, group of 32 / G queries), in one grid dimension
  if (I.B * I.Hkv * p->n_slabs * ((n_q + 32 / I.G - 1) / (32 / I.G)) + 7 > INT32_MAX)
    return fail(RECSA_ERR_UNSUPPORTED, "too many (query group, block slab) pairs for one launch");
  for (int64_t t = 0; t < p->n_slabs; ++t) p->merge += std::min<int64_t>(p->s1, std::min<int64_t>(p->SB, p->n1 - t * p->SB));
  const recsa::TsTokenLayout L = recsa::ts_token_layout(static_cast<int>(I.d), static_cast<int>(I.G), p->C0, p->s1,
                                                        p->s0);
  p->lds = static_cast<size_t>(L.total);
  if (p->lds > kMaxLds)
    return fail(RECSA_ERR_UNSUPPORTED,
                "k_block = %d and k_token = %d need %zu bytes of LDS per query (max %zu): %lld token candidates",
                k_block, k_token, p->lds, kMaxLds, (long long)p->C0);
  if (recsa::ts_merge_lds_bytes(p->merge) > kMaxLdsMerge)
    return fail(RECSA_ERR_UNSUPPORTED, "%lld merged block candidates per query need %zu bytes of LDS (max %zu)",
                (long long)p->merge, recsa::ts_merge_lds_bytes(p->merge), kMaxLdsMerge);
  p->tab_bytes = p->C0 > 0 ? table_bytes(I, p->C0) : 0;
  p->q_bytes = al256(I.B * n_q * I.Hq * I.d * I.esz);
  p->kb_bytes = own_blocks && p->s1 > 0 ? al256(I.B * I.Hkv * p->n1 * I.d * I.esz) : 0;
  p->cand_bytes = p->s1 > 0 ? al256(I.B * I.Hkv * n_q * p->n_slabs * p->s1 * 8) : 0;
  p->kept_bytes = p->s1 > 0 ? al256(I.B * I.Hkv * n_q * p->s1 * 4) : 0;
  p->total = p->tab_bytes + 2 * p->q_bytes + p->kb_bytes + p->cand_bytes + p->kept_bytes;
  return RECSA_OK;
}

int64_t recsa_two_stage_workspace_bytes(const recsa_shape_t* shape, int64_t n_tokens, int64_t n_q, int32_t k_block,
                                        int32_t k_token, int32_t blocks_rotated) {
  TsPlan p;
  if (ts_plan(shape, n_tokens, n_q, k_block, k_token, blocks_rotated == 0, &p)) return -1;
  return p.total;
}

int32_t recsa_two_stage_rotate_blocks(const recsa_shape_t* shape, const void* tree, int64_t n_old, int64_t n_new,
                                      void* block_keys, void* stream) {
  Info I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  if (n_old < 0 || n_new < n_old) return fail(RECSA_ERR_INVALID_ARG, "need 0 <= n_old <= n_new");
  if (n_new > I.cap) return fail(RECSA_ERR_CAPACITY, "n_new %lld exceeds the capacity %lld", (long long)n_new,
                                 (long long)I.cap);
  const int64_t lo = n_old / I.f, hi = n_new / I.f;
  if (hi <= lo) return RECSA_OK;
  if (!tree || !block_keys) return fail(RECSA_ERR_INVALID_ARG, "tree or block_keys is NULL");
  if (!aligned16(tree) || !aligned16(block_keys)) return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const int64_t rows = nodes_at(I.cap, I.f, 1);
  const char* nk = static_cast<const char*>(tree) + level_offset_bytes(I, 1, 0);
  const int64_t bytes = I.B * I.Hkv * rows * I.d * I.esz;
  const char* bk = static_cast<const char*>(block_keys);
  if (nk < bk + bytes && bk < nk + bytes) return fail(RECSA_ERR_INVALID_ARG, "block_keys overlaps the tree's block keys");
  hipError_t e = recsa::launch_rotate_keys(nk, rows, block_keys, rows, hi, I.B * I.Hkv, static_cast<int>(I.d), I.bf16,
                                           inv_freq_of(I), I.theta != 0.0f, static_cast<hipStream_t>(stream), lo);
  if (e != hipSuccess) return hip_fail(e, "block key rotation launch");
  return RECSA_OK;
}

int32_t recsa_two_stage_decode(const recsa_shape_t* shape, const void* q, int64_t n_q, const void* K, const void* V,
                               const void* tree, const void* block_keys, int64_t n_tokens, int32_t k_block,
                               int32_t k_token, float* out, float* lse, int32_t* sel_blocks, int32_t sel_block_width,
                               int32_t* sel_tokens, int32_t sel_token_width, void* workspace, int64_t ws_bytes,
                               void* stream) {
  TsPlan p;
  int32_t rc = ts_plan(shape, n_tokens, n_q, k_block, k_token, block_keys == nullptr, &p);
  if (rc) return rc;
  const Info& I = p.I;
  if (n_q == 0) return RECSA_OK;
  if (!q || !out || (n_tokens > 0 && (!K || !V)) || (p.n1 > 0 && !tree))
    return fail(RECSA_ERR_INVALID_ARG, "q, K, V, tree or out is NULL");
  if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(tree) || !aligned16(block_keys) ||
      !aligned16(out) || !aligned16(workspace))
    return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  if (sel_blocks && sel_block_width < p.s1)
    return fail(RECSA_ERR_INVALID_ARG, "sel_block_width %d < %lld kept blocks", sel_block_width, (long long)p.s1);
  if (sel_tokens && sel_token_width < p.s0)
    return fail(RECSA_ERR_INVALID_ARG, "sel_token_width %d < %lld kept tokens", sel_token_width, (long long)p.s0);
  if (ws_bytes < p.total) return fail(RECSA_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes,
                                      (long long)p.total);
  if (p.total > 0 && !workspace) return fail(RECSA_ERR_INVALID_ARG, "workspace is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const recsa::InvFreq iv = inv_freq_of(I);
  const int use_rope = I.theta != 0.0f;
  recsa::TsArgs a{};
  a.tab = p.tab_bytes > 0 ? reinterpret_cast<const float2*>(ws) : nullptr;
  char* q1 = ws + p.tab_bytes;
  char* q0 = q1 + p.q_bytes;
  a.q1 = q1;
  a.q0 = q0;
  a.kb = block_keys ? block_keys : static_cast<const void*>(q0 + p.q_bytes);
  a.kb_rows = block_keys ? nodes_at(I.cap, I.f, 1) : p.n1;
  a.cand = reinterpret_cast<uint2*>(q0 + p.q_bytes + p.kb_bytes);
  a.kept = reinterpret_cast<int32_t*>(q0 + p.q_bytes + p.kb_bytes + p.cand_bytes);
  a.K = K;
  a.V = V;
  a.cap = I.cap;
  a.out = out;
  a.lse = lse;
  a.sel_blocks = sel_blocks;
  a.sel_tokens = sel_tokens;
  a.sel_bw = sel_blocks ? sel_block_width : 0;
  a.sel_tw = sel_tokens ? sel_token_width : 0;
  a.n = n_tokens;
  a.n1 = p.n1;
  a.n_q = n_q;
  a.BH = I.B * I.Hkv;
  a.Hkv = static_cast<int32_t>(I.Hkv);
  a.Hq = static_cast<int32_t>(I.Hq);
  a.f = static_cast<int32_t>(I.f);
  a.s1 = static_cast<int32_t>(p.s1);
  a.C0 = static_cast<int32_t>(p.C0);
  a.s0 = static_cast<int32_t>(p.s0);
  a.SB = static_cast<int32_t>(p.SB);
  a.n_slabs = static_cast<int32_t>(p.n_slabs);
  a.merge = static_cast<int32_t>(p.merge);
  a.use_rope = use_rope && p.C0 > 0;
  a.scale = I.scale;
  hipError_t e;
  if (a.tab) {
    e = recsa::launch_rope_table(reinterpret_cast<float2*>(ws), p.C0, static_cast<int>(I.d / 2), iv, st);
    if (e != hipSuccess) return hip_fail(e, "RoPE table launch");
  }
  e = recsa::launch_ts_rotate_queries(q, q1, q0, I.B * n_q * I.Hq, p.n1, p.C0, static_cast<int>(I.d), I.bf16, iv,
                                      use_rope, st);
  if (e != hipSuccess) return hip_fail(e, "query rotation launch");
  if (p.s1 > 0) {
    if (!block_keys) {
      e = recsa::launch_rotate_keys(static_cast<const char*>(tree) + level_offset_bytes(I, 1, 0), nodes_at(I.cap, I.f, 1),
                                    q0 + p.q_bytes, p.n1, p.n1, I.B * I.Hkv, static_cast<int>(I.d), I.bf16, iv, use_rope,
                                    st);
      if (e != hipSuccess) return hip_fail(e, "block key rotation launch");
    }
    e = recsa::launch_ts_score(a, static_cast<int>(I.d), I.bf16, static_cast<int>(I.G), st);
    if (e != hipSuccess) return hip_fail(e, "block scoring launch");
    e = recsa::launch_ts_merge(a, st);
    if (e != hipSuccess) return hip_fail(e, "block merge launch");
  }
  e = recsa::launch_ts_tokens(a, static_cast<int>(I.d), I.bf16, static_cast<int>(I.G), p.lds, I.B, st);
  if (e != hipSuccess) return hip_fail(e, "token stage launch");
  return RECSA_OK;
}

int32_t recsa_dense_ref_attn(const recsa_shape_t* shape, const void* q, int64_t q_start, int64_t n_q, const void* K,
                             const void* V, int64_t n_tokens, int32_t mode, float* out, float* lse, void* workspace,
                             int64_t ws_bytes, void* stream) {
  Info I;
  int32_t rc = check_shape(shape, &I);
  if (rc) return rc;
  if (mode & ~3) return fail(RECSA_ERR_INVALID_ARG, "mode must be in 0..3");
  const bool causal = mode & RECSA_DENSE_CAUSAL;
  const bool rotated = mode & RECSA_DENSE_KEYS_ROTATED;
  if (n_q < 0 || n_tokens < 0) return fail(RECSA_ERR_INVALID_ARG, "n_q and n_tokens must be >= 0");
  if (causal && (q_start < 0 || q_start + n_q > n_tokens))
    return fail(RECSA_ERR_INVALID_ARG, "causal queries need 0 <= q_start and q_start + n_q <= n_tokens");
  if (n_tokens > I.cap) return fail(RECSA_ERR_CAPACITY, "n_tokens %lld exceeds the capacity %lld", (long long)n_tokens,
                                    (long long)I.cap);
  if (n_q * I.Hkv > INT32_MAX || I.B * I.Hkv > 65535) return fail(RECSA_ERR_UNSUPPORTED, "grid too large");
  if (n_q == 0) return RECSA_OK;
  if (!q || !out || (n_tokens > 0 && (!K || !V))) return fail(RECSA_ERR_INVALID_ARG, "q, K, V or out is NULL");
  if (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(out) || !aligned16(workspace))
    return fail(RECSA_ERR_INVALID_ARG, "device pointers must be 16-byte aligned");
  const DensePlan pl = dense_plan(I, n_tokens, n_q, mode);
  if (ws_bytes < pl.total) return fail(RECSA_ERR_WORKSPACE, "workspace %lld < %lld bytes", (long long)ws_bytes,
                                       (long long)pl.total);
  if (pl.total > 0 && !workspace) return fail(RECSA_ERR_INVALID_ARG, "workspace is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const recsa::InvFreq iv = inv_freq_of(I);
  recsa::DenseArgs a{};
  a.q = q;
  a.V = V;
  a.out = out;
  a.lse = lse;
  a.v_rows = I.cap;
  a.n_q = n_q;
  a.q_start = causal ? q_start : 0;
  a.n_tokens = n_tokens;
  a.causal = causal ? 1 : 0;
  a.Hkv = static_cast<int32_t>(I.Hkv);
  a.Hq = static_cast<int32_t>(I.Hq);
  a.scale = I.scale;
  a.use_rope = I.theta != 0.0f;
  a.iv = iv;
  a.n_splits = pl.splits;
  a.keys_per_split = pl.keys_per_split;
  char* ws = static_cast<char*>(workspace);
  if (rotated || I.theta == 0.0f) {
    a.Kr = K;
    a.kr_rows = I.cap;
  } else {
    hipError_t e = recsa::launch_rotate_keys(K, I.cap, ws, n_tokens, n_tokens, I.B * I.Hkv, static_cast<int>(I.d),
                                             I.bf16, iv, 1, st);
    if (e != hipSuccess) return hip_fail(e, "key rotation launch");
    a.Kr = ws;
    a.kr_rows = n_tokens;
  }
  if (pl.splits > 1) {
    a.part_o = reinterpret_cast<float*>(ws + pl.kr_bytes + pl.qr_bytes);
    a.part_ml = reinterpret_cast<float*>(ws + pl.kr_bytes + pl.qr_bytes + pl.part_o_bytes);
  }
  if (pl.qr_bytes > 0) {
    hipError_t e = recsa::launch_rotate_queries(a, ws + pl.kr_bytes, I.B, static_cast<int>(I.d), st);
    if (e != hipSuccess) return hip_fail(e, "query rotation launch");
    a.q = ws + pl.kr_bytes;
    a.use_rope = 0;   // the keys and now the queries are rotated
  }
  hipError_t e = recsa::launch_dense(a, static_cast<int>(I.d), I.bf16, static_cast<int>(I.G), I.B, st);
  if (e != hipSuccess) return hip_fail(e, "dense attention launch");
  return RECSA_OK;
}

}  // extern "C"
