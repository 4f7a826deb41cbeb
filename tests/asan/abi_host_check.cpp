// Drives the C ABI's host code through many shapes and calls -- sizing queries, successful calls
// (their launches are the no-op stand-ins of host_stubs.cpp) and rejected ones -- so that
// AddressSanitizer and UndefinedBehaviorSanitizer see every offset, size and table the entry points
// compute. Device pointers are fake, aligned addresses that are never dereferenced. Prints "ok"
// and returns 0 when every status has the expected sign.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "recsa.h"

static int failures = 0;

static void expect(bool ok, const char* what, long long v) {
  if (!ok) {
    ++failures;
    fprintf(stderr, "unexpected: %s -> %lld (%s)\n", what, v, recsa_last_error());
  }
}

// fake device buffers 1 TB apart: no two of them overlap at any size used here
static void* fake(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t(1) << 46) + (i << 40)); }

int main() {
  const int fans[] = {2, 3, 4, 16, 32, 64};
  const int dims[] = {64, 128};
  const int64_t caps[] = {0, 1, 15, 16, 4096, 131072 + 37, 2097152, 2147483647};
  for (int f : fans)
    for (int d : dims)
      for (int64_t cap : caps)
        for (int dt = 0; dt < 2; ++dt) {
          recsa_shape_t sh{2, 8, 32, d, f, dt, cap, 0.0f, 1.0e6f, 0};
          const int64_t tb = recsa_tree_bytes(&sh);
          expect(tb >= 0, "tree_bytes", tb);
          const int T = recsa_num_levels(cap, f);
          for (int lv = 1; lv <= T; ++lv)
            for (int which = 0; which < 2; ++which) {
              const int64_t off = recsa_level_offset(&sh, lv, which);
              expect(off >= 0 && off < tb, "level_offset", off);
            }
          expect(recsa_level_offset(&sh, T + 1, 0) == -1, "level_offset past the top", 0);
          for (int kk : {0, 1, 8, 16, 2147483647}) {
            std::vector<int32_t> k(RECSA_MAX_LEVELS, kk);
            const int nl = T > 0 ? T : 1;
            for (int64_t n : {int64_t(0), int64_t(1), cap / 3, cap - 1, cap}) {
              if (n < 0 || n > cap) continue;
              const int Tn = recsa_num_levels(n, f);
              const int64_t ws = recsa_workspace_bytes(&sh, n, k.data(), nl);
              expect(ws >= 0 || Tn > nl, "workspace_bytes", ws);
              const int32_t w = recsa_sel_width(&sh, n > 300 ? n - 300 : 0, n, k.data(), nl);
              expect(w >= 0, "sel_width", w);
              const int64_t bw = recsa_backward_workspace_bytes(&sh, n, k.data(), nl);
              (void)bw;
              if (kk != 2147483647 && n > 0 && cap <= 2097152) {
                // decode and prefill over the whole prefix, with selections
                const int32_t width = recsa_sel_width(&sh, n, n, k.data(), nl);
                const int32_t rc = recsa_decode(&sh, fake(1), 3, fake(2), fake(3), fake(4), n, k.data(), nl,
                                                static_cast<float*>(fake(5)), static_cast<float*>(fake(6)),
                                                static_cast<int32_t*>(fake(7)), width > 0 ? width : 1, fake(8),
                                                ws > 0 ? ws : 16, nullptr);
                expect(rc == RECSA_OK || rc == RECSA_ERR_UNSUPPORTED, "decode", rc);
                const int64_t qs = n > 5 ? n - 5 : 0;
                const int32_t pw = recsa_sel_width(&sh, qs + 1, n, k.data(), nl);
                const int32_t rp = recsa_prefill(&sh, fake(1), qs, n - qs, fake(2), fake(3), fake(4), k.data(), nl,
                                                 static_cast<float*>(fake(5)), nullptr, static_cast<int32_t*>(fake(7)),
                                                 pw > 0 ? pw : 1, fake(8), ws > 0 ? ws : 16, nullptr);
                expect(rp == RECSA_OK || rp == RECSA_ERR_UNSUPPORTED, "prefill", rp);
                const int32_t rn = recsa_decode_noalloc(&sh, fake(1), 2, fake(2), fake(3), fake(4), n, k.data(), nl,
                                                        static_cast<float*>(fake(5)), nullptr, nullptr, 0, nullptr);
                expect(rn == RECSA_OK || rn == RECSA_ERR_UNSUPPORTED, "decode_noalloc", rn);
                if (n < cap) {
                  const int32_t sw = recsa_sel_width(&sh, n + 1, n + 1, k.data(), nl);
                  const int64_t sws = recsa_workspace_bytes(&sh, n + 1, k.data(), nl);
                  const int32_t rs = recsa_decode_step(&sh, fake(1), fake(20), fake(21), fake(2), fake(3), fake(9),
                                                       fake(4), n, k.data(), nl, static_cast<float*>(fake(5)), nullptr,
                                                       static_cast<int32_t*>(fake(7)), sw > 0 ? sw : 1, fake(8),
                                                       sws > 0 ? sws : 16, nullptr);
                  expect(rs == RECSA_OK || rs == RECSA_ERR_UNSUPPORTED || rs == RECSA_ERR_INVALID_ARG, "decode_step",
                         rs);
                }
                if (bw > 0) {
                  const int32_t rb = recsa_backward(&sh, 0, fake(1), 0, 2, n, fake(2), fake(3), fake(9), fake(4),
                                                    k.data(), nl, static_cast<float*>(fake(5)),
                                                    static_cast<float*>(fake(6)), static_cast<int32_t*>(fake(7)),
                                                    width > 0 ? width : 1, static_cast<float*>(fake(10)), nullptr,
                                                    static_cast<float*>(fake(11)), static_cast<float*>(fake(12)),
                                                    static_cast<float*>(fake(13)), static_cast<float*>(fake(14)),
                                                    fake(8), bw, nullptr);
                  expect(rb == RECSA_OK || rb == RECSA_ERR_UNSUPPORTED, "backward", rb);
                }
              }
            }
          }
          if (cap > 0 && cap <= 2097152) {
            expect(recsa_build_tree(&sh, fake(2), fake(3), fake(9), 0, cap, fake(4), nullptr) == RECSA_OK, "build", 0);
            expect(recsa_build_tree(&sh, fake(2), fake(3), fake(9), cap / 2, cap, fake(4), nullptr) == RECSA_OK,
                   "build (incremental)", 0);
            const int64_t dws = recsa_dense_workspace_bytes(&sh, cap, 4, RECSA_DENSE_CAUSAL);
            expect(dws >= 0, "dense_workspace_bytes", dws);
            expect(recsa_dense_ref_attn(&sh, fake(1), cap > 4 ? cap - 4 : 0, cap > 4 ? 4 : cap, fake(2), fake(3), cap,
                                        RECSA_DENSE_CAUSAL, static_cast<float*>(fake(5)), nullptr, fake(8),
                                        dws > 0 ? dws : 16, nullptr) == RECSA_OK,
                   "dense causal", 0);
            expect(recsa_rotate_keys(&sh, fake(2), cap, fake(3), nullptr) == RECSA_OK, "rotate_keys", 0);
            if (cap >= f) {
              const int64_t tws = recsa_two_stage_workspace_bytes(&sh, cap, 2, 16, 64, 0);
              if (tws > 0) {
                const int32_t rt = recsa_two_stage_decode(&sh, fake(1), 2, fake(2), fake(3), fake(4), nullptr, cap, 16,
                                                          64, static_cast<float*>(fake(5)), nullptr,
                                                          static_cast<int32_t*>(fake(6)), 16,
                                                          static_cast<int32_t*>(fake(7)), 64, fake(8), tws, nullptr);
                expect(rt == RECSA_OK || rt == RECSA_ERR_UNSUPPORTED, "two_stage_decode", rt);
              }
            }
          }
        }
  // rejected calls: every one returns a negative status before any launch
  recsa_shape_t sh{2, 8, 32, 128, 16, RECSA_BF16, 4096, 0.0f, 1.0e6f, 0};
  int32_t k3[3] = {8, 8, 8};
  expect(recsa_decode(&sh, fake(1), 2, fake(2), fake(3), fake(4), 5000, k3, 3, static_cast<float*>(fake(5)), nullptr,
                      nullptr, 0, fake(8), 1 << 20, nullptr) == RECSA_ERR_CAPACITY, "capacity", 0);
  expect(recsa_decode(&sh, fake(1), 2, fake(2), fake(3), fake(4), 4096, k3, 2, static_cast<float*>(fake(5)), nullptr,
                      nullptr, 0, fake(8), 1 << 20, nullptr) == RECSA_ERR_INVALID_ARG, "levels", 0);
  expect(recsa_decode(&sh, fake(1), 2, fake(2), fake(3), fake(4), 4096, k3, 3, static_cast<float*>(fake(5)), nullptr,
                      nullptr, 0, fake(8), 16, nullptr) == RECSA_ERR_WORKSPACE, "workspace", 0);
  // a slice (one sequence and KV head) of 4 GiB or more: the attention kernels' 32-bit offsets
  // would not reach it, so decode, prefill, the decoding step and the allocation-free decode
  // refuse it; one row less is accepted
  for (int dt = 0; dt < 2; ++dt) {
    const int64_t big = (int64_t(1) << 32) / (128 * (dt == RECSA_BF16 ? 2 : 4));
    for (int64_t cap : {big, big - 1}) {
      recsa_shape_t s4{1, 8, 32, 128, 16, dt, cap, 0.0f, 1.0e6f, 0};
      const int32_t want = cap == big ? RECSA_ERR_UNSUPPORTED : RECSA_OK;
      const int64_t ws4 = recsa_workspace_bytes(&s4, 4096, k3, 3);
      expect(recsa_decode(&s4, fake(1), 2, fake(2), fake(3), fake(4), 4096, k3, 3, static_cast<float*>(fake(5)),
                          nullptr, nullptr, 0, fake(8), ws4 > 0 ? ws4 : 16, nullptr) == want, "4 GiB decode", cap);
      expect(recsa_prefill(&s4, fake(1), 4090, 6, fake(2), fake(3), fake(4), k3, 3, static_cast<float*>(fake(5)),
                           nullptr, nullptr, 0, fake(8), ws4 > 0 ? ws4 : 16, nullptr) == want, "4 GiB prefill", cap);
      expect(recsa_decode_noalloc(&s4, fake(1), 2, fake(2), fake(3), fake(4), 4096, k3, 3,
                                  static_cast<float*>(fake(5)), nullptr, nullptr, 0, nullptr) == want,
             "4 GiB decode_noalloc", cap);
      expect(recsa_decode_step(&s4, fake(1), fake(20), fake(21), fake(2), fake(3), fake(9), fake(4), 4095, k3, 3,
                               static_cast<float*>(fake(5)), nullptr, nullptr, 0, fake(8), ws4 > 0 ? ws4 : 16,
                               nullptr) == want,
             "4 GiB decode_step", cap);
    }
  }
  recsa_shape_t bad = sh;
  bad.n_q_heads = 30;
  expect(recsa_tree_bytes(&bad) == -1, "bad heads", 0);
  bad = sh;
  bad.head_dim = 96;
  expect(recsa_tree_bytes(&bad) == -1, "bad head_dim", 0);
  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
