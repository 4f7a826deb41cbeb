/*
 * RecSA oracle: node summaries (TEST INFRASTRUCTURE ONLY; the GPU library never uses this).
 *
 * "Recursive Sparse Attention: Million-Token Length Extrapolation at Logarithmic Cost",
 * abstract: a node holds a key produced by the layer's pooler and the average of the
 * values below it. Reading: key = W m, m = mean of the f children's stored keys; value =
 * mean of the children's stored values; both rounded to the storage type.
 *
 * Arithmetic, written out so that every rounding is visible:
 *   a = 0; for c in 0..f-1: a = a + child_c        (float32 adds, child order)
 *   m = a / f                                      (one correctly rounded division)
 *   acc = 0; for j in 0..d-1: acc = fmaf(W[i][j], m[j], acc)   (one rounding per term)
 *   key_i = round(acc); value = round((sum of child values) / f)
 * Build with -ffp-contract=off so that the compiler adds no fusion of its own.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float round_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  u &= 0xFFFF0000u;
  memcpy(&x, &u, 4);
  return x;
}

/* cK, cV: [g][f][d] children (float32 values exact in the storage type); W: [d][d];
 * NK, NV: [g][d] outputs. bf16 != 0 rounds the outputs to bf16. */
void oracle_pool(int64_t g, int32_t f, int32_t d, const float* cK, const float* cV, const float* W,
                 int32_t bf16, float* NK, float* NV) {
  float a[256], b[256], m[256];
  for (int64_t n = 0; n < g; ++n) {
    const float* kk = cK + n * (int64_t)f * d;
    const float* vv = cV + n * (int64_t)f * d;
    for (int j = 0; j < d; ++j) { a[j] = 0.0f; b[j] = 0.0f; }
    for (int c = 0; c < f; ++c)
      for (int j = 0; j < d; ++j) {
        a[j] = a[j] + kk[c * d + j];
        b[j] = b[j] + vv[c * d + j];
      }
    for (int j = 0; j < d; ++j) {
      m[j] = a[j] / (float)f;
      float v = b[j] / (float)f;
      NV[n * d + j] = bf16 ? round_bf16(v) : v;
    }
    for (int i = 0; i < d; ++i) {
      float acc = 0.0f;
      for (int j = 0; j < d; ++j) acc = fmaf(W[i * d + j], m[j], acc);
      NK[n * d + i] = bf16 ? round_bf16(acc) : acc;
    }
  }
}
