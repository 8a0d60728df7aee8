/*
 * Ideal attention in binary64 -- the reference every head's output is
 * compared against (attention-numerics project page, first section: exact
 * causal attention computed in binary64).  TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Plain definition: for query i, logits z_j = (q_i . k_j) * scale over the
 * visible keys (j <= i when causal, every key otherwise), weights
 * w_j = exp(z_j - max z) / sum exp(z - max z), output sum_j w_j v_j.
 * Grouped-query heads: query head h reads KV head h / (Hq / Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include "oracle.h"
#include "threads.h"

typedef struct {
  const double *q, *k, *v;
  int64_t B, Hq, Hkv, N, d, nrows;
  int causal;
  double scale;
  const int32_t* rows;
  double* out;
} ideal_args;

static void ideal_row(void* p, int64_t item, double* scratch) {
  const ideal_args* a = (const ideal_args*)p;
  int64_t r = item % a->nrows, bh = item / a->nrows;
  int64_t b = bh / a->Hq, h = bh % a->Hq, g = h / (a->Hq / a->Hkv);
  int64_t i = a->rows ? a->rows[r] : r;
  const double* q = a->q + ((b * a->Hq + h) * a->N + i) * a->d;
  const double* K = a->k + (b * a->Hkv + g) * a->N * a->d;
  const double* V = a->v + (b * a->Hkv + g) * a->N * a->d;
  int64_t nvis = a->causal ? i + 1 : a->N;
  double* z = scratch;
  double m = -INFINITY;
  for (int64_t j = 0; j < nvis; ++j) {
    double s = 0.0;
    for (int64_t c = 0; c < a->d; ++c) s += q[c] * K[j * a->d + c];
    z[j] = s * a->scale;
    if (z[j] > m) m = z[j];
  }
  double den = 0.0;
  for (int64_t j = 0; j < nvis; ++j) { z[j] = exp(z[j] - m); den += z[j]; }
  double* o = a->out + (bh * a->nrows + r) * a->d;
  for (int64_t c = 0; c < a->d; ++c) o[c] = 0.0;
  for (int64_t j = 0; j < nvis; ++j) {
    double w = z[j] / den;
    for (int64_t c = 0; c < a->d; ++c) o[c] += w * V[j * a->d + c];
  }
}

int orc_attention_f64(const double* q, const double* k, const double* v,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                      int causal, double softmax_scale,
                      const int32_t* rows, int64_t nrows, double* out, int nthreads) {
  if (!q || !k || !v || !out || B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || Hq % Hkv) return -1;
  if (!rows) nrows = N;
  for (int64_t r = 0; rows && r < nrows; ++r) if (rows[r] < 0 || rows[r] >= N) return -2;
  ideal_args a = {q, k, v, B, Hq, Hkv, N, d, nrows, causal, softmax_scale, rows, out};
  return orc_parallel_for(ideal_row, &a, B * Hq * nrows, N, nthreads);
}
