// Host-only stand-ins for the library's kernel launches, for checking the C ABI's host code
// (argument checks, sizing, offsets, launch planning) under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU. Every launch is a no-op that
// succeeds; nothing here reads or writes the (fake) device pointers it is given.
#include "internal.hpp"

namespace recsa {

hipError_t launch_pool_level(const PoolArgs&, int, bool, hipStream_t) { return hipSuccess; }
int pool_persistent_grid() { return 512; }
hipError_t launch_rope_table(float2*, int64_t, int, const InvFreq&, hipStream_t) { return hipSuccess; }
hipError_t launch_append_step(const StepArgs&, int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_attend(const AttnArgs& a, int, bool, int, size_t, int64_t, hipStream_t) {
  // the launch plan's level tables are read up to the deepest level a call can reach
  volatile int64_t sink = 0;
  for (int lv = 1; lv <= RECSA_MAX_LEVELS; ++lv) sink = sink + a.k.k[lv] + a.tree.rows[lv];
  (void)sink;
  return hipSuccess;
}
hipError_t launch_backward_units(const BwdArgs&, int, bool, int, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_tree_push(const TreePushArgs&, int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_fill_zero(float*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_distill_loss(const float*, const float*, float*, float*, float*, int64_t, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_distill_update(float*, const float*, void*, float, int64_t, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_rotate_keys(const void*, int64_t, void*, int64_t, int64_t, int64_t, int, bool, const InvFreq&, int,
                              hipStream_t, int64_t) {
  return hipSuccess;
}
hipError_t launch_dense(const DenseArgs&, int, bool, int, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_rotate_queries(const DenseArgs&, void*, int64_t, int, hipStream_t) { return hipSuccess; }
hipError_t launch_ts_rotate_queries(const void*, void*, void*, int64_t, int64_t, int64_t, int, bool, const InvFreq&, int,
                                    hipStream_t) {
  return hipSuccess;
}
hipError_t launch_ts_score(const TsArgs&, int, bool, int, hipStream_t) { return hipSuccess; }
hipError_t launch_ts_merge(const TsArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_ts_tokens(const TsArgs&, int, bool, int, size_t, int64_t, hipStream_t) { return hipSuccess; }

// no device: the cache never holds a table, so every call takes the workspace path
hipError_t rope_cache_table(int, float, const InvFreq&, int64_t, hipStream_t, const float2** tab) {
  *tab = nullptr;
  return hipSuccess;
}

alignas(256) static unsigned char fake_scratch[256];
hipError_t noalloc_scratch_address(void** out) {
  *out = fake_scratch;
  return hipSuccess;
}

}  // namespace recsa
