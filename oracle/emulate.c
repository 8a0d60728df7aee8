/*
 * Step-by-step binary32 emulation of the quantised attention forward.
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Every floating-point step below is
 * one IEEE binary32 operation with round-to-nearest-even (the file is built
 * with -ffp-contract=off; fused multiply-adds are written as fmaf).
 *
 * Prologue (attention-numerics pages: project page, second section; study
 * page, "See the vectors and the arithmetic"):
 *   1. mean key over the full sequence per (batch, KV head) when centring;
 *      K' = K - mean (the exact softmax is unchanged by it);
 *   2. a fixed random-sign Hadamard rotation applied to Q and K', never V;
 *   3. one maximum-based scale per (batch, head) over the full sequence;
 *   4. E4M3FN codes, round-to-nearest-even, saturating at +-448.
 * Main loop (P-Cast summary, Probleemstelling and Methodologie):
 *   online softmax over KV blocks visited forward (0 -> N) or reverse
 *   (N -> 0); P multiplied by the static scale S, cast to E4M3 before the
 *   P.V product, S divided out in the epilogue.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include "oracle.h"
#include "threads.h"

/* ---------------------------------------------------------------- prologue */

void orc_fwht_row(float* x, const int8_t* signs, int64_t d) {
  for (int64_t c = 0; c < d; ++c) x[c] = x[c] * (float)signs[c];
  for (int64_t h = 1; h < d; h <<= 1)
    for (int64_t i = 0; i < d; ++i)
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
}

/* Mean of column c of one [N,d] KV head: binary64 partial sums over chunks of
 * 64 tokens (tokens in increasing order, starting from +0.0), the partials
 * added in a pairwise tree over chunk index (padded with +0.0 to a power of
 * two), one binary64 division by N, then rounding to binary32. */
static float column_mean(const float* K, int64_t N, int64_t d, int64_t c, double* part) {
  int64_t nchunk = (N + 63) / 64, np2 = 1;
  while (np2 < nchunk) np2 <<= 1;
  for (int64_t t = 0; t < np2; ++t) {
    double s = 0.0;
    if (t < nchunk) {
      int64_t n1 = (t + 1) * 64 < N ? (t + 1) * 64 : N;
      for (int64_t n = t * 64; n < n1; ++n) s += (double)K[n * d + c];
    }
    part[t] = s;
  }
  for (int64_t w = np2; w > 1; w >>= 1)
    for (int64_t t = 0; t < w / 2; ++t) part[t] = part[2 * t] + part[2 * t + 1];
  return (float)(part[0] / (double)N);
}

int8_t orc_i8_encode(float x) {
  float r = rintf(x);  /* the default rounding mode: to nearest, ties to even */
  if (r > 127.0f) r = 127.0f;
  if (r < -127.0f) r = -127.0f;
  return (int8_t)r;
}

/* qmax: the largest code magnitude, 448 for E4M3 and 127 for int8. */
static void scales_from_amax(float A, int rotated, int64_t d, float qmax, float* inv, float* desc) {
  if (A == 0.0f) { *inv = 1.0f; *desc = 1.0f; return; }
  *inv = qmax / A;
  *desc = A / qmax;
  if (rotated) *desc = *desc * (float)(1.0 / sqrt((double)d));
}

int orc_prepare(const float* q, const float* k, const float* v,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                uint32_t flags, const int8_t* signs,
                uint8_t* q8, uint8_t* k8, uint8_t* v8,
                float* q_desc, float* k_desc, float* v_desc, float* k_mean) {
  if (!q || !k || !v || !q8 || !k8 || !v8 || !q_desc || !k_desc || !v_desc) return -1;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || Hq % Hkv || (d & (d - 1))) return -1;
  int rotate = (flags & ORC_ROTATE) != 0, center = (flags & ORC_CENTER) != 0;
  int tiled = (flags & ORC_TILE) != 0, prefix = (flags & ORC_PREFIX) != 0, i8 = (flags & ORC_INT8) != 0;
  if (prefix && !tiled) return -1;
  /* tokens the mean key is taken over: all N, or with prefix scales the
   * first 128-token tile only (no key shift may depend on later tokens) */
  int64_t n_mean = prefix ? (N < ORC_TILE_TOKENS ? N : ORC_TILE_TOKENS) : N;
  /* scale groups: the whole sequence, or 128-token tiles */
  int64_t span = tiled ? ORC_TILE_TOKENS : N, ngroup = (N + span - 1) / span;
  if (rotate && !signs) return -1;
  int64_t nchunk = (N + 63) / 64, np2 = 1;
  while (np2 < nchunk) np2 <<= 1;
  double* part = (double*)malloc(sizeof(double) * (size_t)np2);
  float* row = (float*)malloc(sizeof(float) * (size_t)d);
  float* mu = (float*)malloc(sizeof(float) * (size_t)d);
  float* buf = (float*)malloc(sizeof(float) * (size_t)(N * d));
  if (!part || !row || !mu || !buf) { free(part); free(row); free(mu); free(buf); return -3; }

  const float qk_max = i8 ? 127.0f : 448.0f;
  /* Q: rotate, amax per scale group, quantise. */
  for (int64_t bh = 0; bh < B * Hq; ++bh) {
    const float* src = q + bh * N * d;
    for (int64_t n = 0; n < N; ++n) {
      memcpy(buf + n * d, src + n * d, sizeof(float) * (size_t)d);
      if (rotate) orc_fwht_row(buf + n * d, signs, d);
    }
    float Apre = 0.0f;
    for (int64_t t = 0; t < ngroup; ++t) {
      int64_t e0 = t * span * d, e1 = ((t + 1) * span < N ? (t + 1) * span : N) * d;
      float A = 0.0f;
      for (int64_t e = e0; e < e1; ++e) { float a = fabsf(buf[e]); if (a > A) A = a; }
      if (prefix) { if (A > Apre) Apre = A; A = Apre; }
      float inv, desc;
      scales_from_amax(A, rotate, d, qk_max, &inv, &desc);
      q_desc[bh * ngroup + t] = desc;
      for (int64_t e = e0; e < e1; ++e)
        q8[bh * N * d + e] = i8 ? (uint8_t)orc_i8_encode(buf[e] * inv) : orc_e4m3_encode(buf[e] * inv);
    }
  }
  /* K: centre, rotate, amax, quantise.  V: amax, quantise (never rotated). */
  for (int64_t bg = 0; bg < B * Hkv; ++bg) {
    const float* src = k + bg * N * d;
    for (int64_t c = 0; c < d; ++c) mu[c] = center ? column_mean(src, n_mean, d, c, part) : 0.0f;
    if (center && k_mean) memcpy(k_mean + bg * d, mu, sizeof(float) * (size_t)d);
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t c = 0; c < d; ++c) buf[n * d + c] = center ? src[n * d + c] - mu[c] : src[n * d + c];
      if (rotate) orc_fwht_row(buf + n * d, signs, d);
    }
    float inv, desc, A, Apre = 0.0f;
    for (int64_t t = 0; t < ngroup; ++t) {
      int64_t e0 = t * span * d, e1 = ((t + 1) * span < N ? (t + 1) * span : N) * d;
      A = 0.0f;
      for (int64_t e = e0; e < e1; ++e) { float a = fabsf(buf[e]); if (a > A) A = a; }
      if (prefix) { if (A > Apre) Apre = A; A = Apre; }
      scales_from_amax(A, rotate, d, qk_max, &inv, &desc);
      k_desc[bg * ngroup + t] = desc;
      for (int64_t e = e0; e < e1; ++e)
        k8[bg * N * d + e] = i8 ? (uint8_t)orc_i8_encode(buf[e] * inv) : orc_e4m3_encode(buf[e] * inv);
    }

    const float* vs = v + bg * N * d;
    A = 0.0f;
    for (int64_t e = 0; e < N * d; ++e) { float a = fabsf(vs[e]); if (a > A) A = a; }
    scales_from_amax(A, 0, d, 448.0f, &inv, &desc);  /* V is always E4M3 */
    v_desc[bg] = desc;
    for (int64_t e = 0; e < N * d; ++e) v8[bg * N * d + e] = orc_e4m3_encode(vs[e] * inv);
  }
  free(part); free(row); free(mu); free(buf);
  return 0;
}

/* ------------------------------------------------------------- score model */

/* An E4M3 code as sign * s * 2^(E-3): s is the 4-bit significand (8 + mantissa
 * for normal codes, the mantissa for subnormals) and E the scale exponent
 * (exponent field - 7, or -6 for subnormals). */
static inline void split_code(uint8_t c, int* sign, int* s, int* E) {
  int e = (c >> 3) & 15, m = c & 7;
  *sign = (c & 0x80) ? -1 : 1;
  if (e == 0) { *s = m; *E = -6; } else { *s = 8 + m; *E = e - 7; }
}

/* Products of two codes are exact multiples of 2^-18 and bounded by 448^2,
 * so every quantity below is an integer number of units of 2^-25 that fits
 * comfortably in int64 (|sum| < 2^50). */
#define UNIT_SHIFT 25

static inline int64_t rn32_units(int64_t v) {
  float f = (float)ldexp((double)v, -UNIT_SHIFT); /* exact in binary64, one rounding to binary32 */
  return (int64_t)ldexp((double)f, UNIT_SHIFT);
}

/* Sum of the eight products a[k]*b[k], k in [k0, k0+8), in the matrix unit's
 * precision: each product magnitude is truncated (toward zero) to a multiple
 * of 2^(R-13), R being the largest scale exponent E_a + E_b among the
 * non-zero products of the group; the truncated products are then added
 * exactly.  *rmax receives max(*rmax, R). */
static int64_t group8_units(const uint8_t* a, const uint8_t* b, int k0, int* rmax) {
  int sg[8], sp[8], ep[8], R = -1000;
  for (int i = 0; i < 8; ++i) {
    int s1, m1, e1, s2, m2, e2;
    split_code(a[k0 + i], &s1, &m1, &e1);
    split_code(b[k0 + i], &s2, &m2, &e2);
    sg[i] = s1 * s2; sp[i] = m1 * m2; ep[i] = e1 + e2;
    if (sp[i] != 0 && ep[i] > R) R = ep[i];
  }
  if (R > *rmax) *rmax = R;
  int64_t sum = 0;
  if (R == -1000) return 0;
  int lsb = R - 13 + UNIT_SHIFT; /* truncation quantum, in units (>= 0 because R >= -12) */
  for (int i = 0; i < 8; ++i) {
    if (sp[i] == 0) continue;
    int64_t mag = (int64_t)sp[i] << (ep[i] - 6 + UNIT_SHIFT); /* sp * 2^(ep-6), exact */
    mag = (mag >> lsb) << lsb;
    sum += sg[i] * mag;
  }
  return sum;
}

/* Largest multiple of 2^(anchor-24) not above v (two's-complement
 * truncation); v is in units of 2^-25, so quanta finer than one unit leave it
 * unchanged. */
static inline int64_t floor_window(int64_t v, int anchor) {
  int s = anchor - 24 + UNIT_SHIFT;
  if (s <= 0) return v;
  return v & ~(((int64_t)1 << s) - 1);
}

float orc_fp8_dot128(const uint8_t* a, const uint8_t* b, int mode) {
  if (mode == 1) { /* RN32 of the exact dot product */
    int64_t s = 0;
    for (int k = 0; k < 128; ++k) {
      int s1, m1, e1, s2, m2, e2;
      split_code(a[k], &s1, &m1, &e1);
      split_code(b[k], &s2, &m2, &e2);
      s += (int64_t)(s1 * s2) * ((int64_t)(m1 * m2) << (e1 + e2 - 6 + UNIT_SHIFT));
    }
    return (float)ldexp((double)s, -UNIT_SHIFT);
  }
  /* The 128 products are taken as eight passes of sixteen (two groups of
   * eight each): passes 0, 2, 4, 6 cover k = 0-15, 32-47, 64-79, 96-111 and
   * come first, then passes 1, 3, 5, 7 (k = 16-31, 48-63, 80-95, 112-127).
   * In each pass the two group sums are added and the result truncated
   * (floor) to a multiple of 2^(R-24), R the largest product scale exponent
   * of the pass; that is added to the running binary32 value, truncated the
   * same way, and rounded to binary32 (nearest-even).  A pass whose products
   * are all zero leaves the running value unchanged. */
  static const int pass_order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
  int64_t acc = 0;
  for (int t = 0; t < 8; ++t) {
    int p = pass_order[t], R = -1000;
    int64_t ga = group8_units(a, b, 16 * p, &R);
    int64_t gb = group8_units(a, b, 16 * p + 8, &R);
    if (R == -1000) continue;
    int64_t part = floor_window(ga + gb, R);
    acc = rn32_units(floor_window(acc + part, R));
  }
  return (float)ldexp((double)acc, -UNIT_SHIFT);
}

/* -------------------------------------------------------------- main loop */

typedef struct {
  /* fp8 path */
  const uint8_t *q8, *k8, *v8;
  const float *q_desc, *k_desc, *v_desc;
  /* fp32 path */
  const float *qf, *kf, *vf;
  int64_t B, Hq, Hkv, N, d, nrows;
  float softmax_scale, p_scale;
  int kv_order, block_n, causal, score_mode, p_cast, tiles;
  const int32_t* rows;
  float* out;          /* NULL: no output (the P~ codes, counts and checksums only) */
  uint8_t* p_out;
  uint32_t* row_zeros;
  uint64_t* row_hash;
  double* lse;         /* NULL or per row: natural-log sum-exp of the scaled logits */
  int32_t k_sink;
} loop_args;

/* Weight of key j in the P~ row checksum: the (j+1)-th output of the
 * splitmix64 generator seeded with 0 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), made odd. */
static uint64_t key_weight(int64_t j) {
  uint64_t z = (uint64_t)(j + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (z ^ (z >> 31)) | 1ull;
}

/* log2(e) to binary64 precision. */
#define LOG2E 1.4426950408889634

/* One query row.  scratch holds N scores (as doubles), then d accumulators. */
static void attn_row(void* p, int64_t item, double* scratch) {
  const loop_args* a = (const loop_args*)p;
  int64_t d = a->d, N = a->N;
  int64_t r = item % a->nrows, bh = item / a->nrows;
  int64_t b = bh / a->Hq, h = bh % a->Hq, g = h / (a->Hq / a->Hkv), bg = b * a->Hkv + g;
  int64_t i = a->rows ? a->rows[r] : r;
  int fp8 = a->q8 != NULL;
  int64_t nvis = a->causal ? i + 1 : N;

  /* Base-2 logit factor c = (desc_q * desc_k) * RN32(scale * log2 e); with
   * per-tile scales it is formed per block from the row's and block's tiles. */
  float ls2 = (float)((double)a->softmax_scale * LOG2E);
  int64_t ntile = (N + ORC_TILE_TOKENS - 1) / ORC_TILE_TOKENS;
  float c = fp8 ? (a->tiles ? 0.0f : (a->q_desc[bh] * a->k_desc[bg]) * ls2) : ls2;

  double* s = scratch;
  float* acc = (float*)(scratch + N);
  uint8_t qpad[128], kpad[128];
  if (fp8) {
    memset(qpad, 0, sizeof qpad);
    memcpy(qpad, a->q8 + (bh * N + i) * d, (size_t)d);
    memset(kpad, 0, sizeof kpad);
  }
  for (int64_t j = 0; j < nvis; ++j) {
    if (fp8) {
      memcpy(kpad, a->k8 + (bg * N + j) * d, (size_t)d);
      if (a->score_mode == 2) { /* int8 codes: exact integer dot */
        int64_t t = 0;
        for (int64_t cc = 0; cc < d; ++cc) t += (int64_t)(int8_t)qpad[cc] * (int64_t)(int8_t)kpad[cc];
        s[j] = (double)(float)t;
      } else {
        s[j] = orc_fp8_dot128(qpad, kpad, a->score_mode);
      }
    } else { /* ordered binary32 fused multiply-add chain over the channels */
      const float* qr = a->qf + (bh * N + i) * d;
      const float* kr = a->kf + (bg * N + j) * d;
      float t = 0.0f;
      for (int64_t cc = 0; cc < d; ++cc) t = fmaf(qr[cc], kr[cc], t);
      s[j] = t;
    }
  }

  int64_t Bc = a->block_n, J = (nvis - 1) / Bc;
  float ms = -INFINITY, mc_prev = -INFINITY, l = 0.0f;
  for (int64_t cc = 0; cc < d; ++cc) acc[cc] = 0.0f;
  uint8_t* prow = a->p_out ? a->p_out + (bh * a->nrows + r) * N : NULL;
  if (prow) memset(prow, 0, (size_t)N);
  uint32_t zeros = 0;
  uint64_t hash = 0;
  float S = a->p_scale;

  for (int64_t t = 0; t <= J; ++t) {
    int64_t blk = a->kv_order == 0 ? t : J - t;
    int64_t j0 = blk * Bc, j1 = (blk + 1) * Bc < nvis ? (blk + 1) * Bc : nvis;
    if (j0 >= j1) continue; /* no visible key: the block changes nothing */
    float bm = -INFINITY;
    for (int64_t j = j0; j < j1; ++j) if ((float)s[j] > bm) bm = (float)s[j];
    float mnew, mc, alpha;
    if (a->tiles) {
      /* running max in scaled units: m = max(m, RN32(bm * c_block)) */
      c = (a->q_desc[bh * ntile + i / ORC_TILE_TOKENS] * a->k_desc[bg * ntile + j0 / ORC_TILE_TOKENS]) * ls2;
      float bmc = bm * c;
      mnew = -INFINITY; /* the raw max is not tracked here */
      mc = mc_prev > bmc ? mc_prev : bmc;
      alpha = (mc_prev == -INFINITY) ? 0.0f : orc_exp2_rn32(mc_prev - mc);
    } else {
      mnew = ms > bm ? ms : bm;
      mc = mnew * c;
      alpha = (ms == -INFINITY) ? 0.0f : orc_exp2_rn32(mc_prev - mc);
    }
    l = l * alpha;
    if (a->out)
      for (int64_t cc = 0; cc < d; ++cc) acc[cc] = acc[cc] * alpha;
    for (int64_t j = j0; j < j1; ++j) {
      float x = fmaf((float)s[j], c, -mc);
      float pj = orc_exp2_rn32(x);
      float pt; /* the value that enters P.V */
      if (a->p_cast) {
        uint8_t code = orc_e4m3_encode(S * pj);
        if (prow) prow[j] = code;
        if (j >= a->k_sink && code == 0) ++zeros;
        hash += (uint64_t)code * key_weight(j);
        pt = orc_e4m3_decode(code);
      } else {
        pt = S * pj;
      }
      l = l + pj;
      if (!a->out) continue;
      if (fp8) {
        const uint8_t* vr = a->v8 + (bg * N + j) * d;
        for (int64_t cc = 0; cc < d; ++cc) acc[cc] = acc[cc] + pt * orc_e4m3_decode(vr[cc]);
      } else {
        const float* vr = a->vf + (bg * N + j) * d;
        for (int64_t cc = 0; cc < d; ++cc) acc[cc] = acc[cc] + pt * vr[cc];
      }
    }
    if (!a->tiles) ms = mnew;
    mc_prev = mc;
  }
  if (a->out) {
    float vd = fp8 ? a->v_desc[bg] : 1.0f;
    float f = vd / (S * l);
    float* o = a->out + (bh * a->nrows + r) * d;
    for (int64_t cc = 0; cc < d; ++cc) o[cc] = acc[cc] * f;
  }
  if (a->row_zeros) a->row_zeros[bh * a->nrows + r] = zeros;
  if (a->row_hash) a->row_hash[bh * a->nrows + r] = hash;
  /* sum_j exp(z_j) = 2^mc * l with z_j the scaled logits in natural units and
   * mc the running max in base-2 units, so lse = (mc + log2 l) * ln 2 */
  if (a->lse) a->lse[bh * a->nrows + r] = ((double)mc_prev + log2((double)l)) * 0.69314718055994530942;
}

static int check_loop(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, float p_scale,
                      int kv_order, int block_n, const int32_t* rows, int64_t nrows) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || d <= 0 || Hq % Hkv) return -1;
  if (!(p_scale > 0.0f) || kv_order < 0 || kv_order > 1 || block_n <= 0) return -1;
  for (int64_t r = 0; rows && r < nrows; ++r) if (rows[r] < 0 || rows[r] >= N) return -2;
  return 0;
}

int orc_attention_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                      const float* q_desc, const float* k_desc, const float* v_desc,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                      float softmax_scale, float p_scale, int kv_order, int block_n, int causal,
                      const int32_t* rows, int64_t nrows,
                      float* out, uint8_t* p_out, uint32_t* row_zeros, int32_t k_sink,
                      int score_mode, int nthreads, double* lse) {
  if (!q8 || !k8 || !v8 || !q_desc || !k_desc || !v_desc || !out || d > 128) return -1;
  if (!rows) nrows = N;
  int rc = check_loop(B, Hq, Hkv, N, d, p_scale, kv_order, block_n, rows, nrows);
  if (rc) return rc;
  loop_args a;
  memset(&a, 0, sizeof a);
  a.q8 = q8; a.k8 = k8; a.v8 = v8; a.q_desc = q_desc; a.k_desc = k_desc; a.v_desc = v_desc;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d; a.nrows = nrows;
  a.softmax_scale = softmax_scale; a.p_scale = p_scale; a.kv_order = kv_order; a.block_n = block_n;
  a.causal = causal; a.score_mode = score_mode; a.p_cast = 1; a.rows = rows; a.out = out;
  a.p_out = p_out; a.row_zeros = row_zeros; a.k_sink = k_sink; a.lse = lse;
  return orc_parallel_for(attn_row, &a, B * Hq * nrows, N + d, nthreads);
}

int orc_attention_fp8_rowhash(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                              const float* q_desc, const float* k_desc, const float* v_desc,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                              float softmax_scale, float p_scale, int kv_order, int block_n, int causal,
                              const int32_t* rows, int64_t nrows,
                              uint64_t* row_hash, uint32_t* row_zeros, int32_t k_sink,
                              int score_mode, int nthreads) {
  if (!q8 || !k8 || !v8 || !q_desc || !k_desc || !v_desc || !row_hash || d > 128) return -1;
  if (!rows) nrows = N;
  int rc = check_loop(B, Hq, Hkv, N, d, p_scale, kv_order, block_n, rows, nrows);
  if (rc) return rc;
  loop_args a;
  memset(&a, 0, sizeof a);
  a.q8 = q8; a.k8 = k8; a.v8 = v8; a.q_desc = q_desc; a.k_desc = k_desc; a.v_desc = v_desc;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d; a.nrows = nrows;
  a.softmax_scale = softmax_scale; a.p_scale = p_scale; a.kv_order = kv_order; a.block_n = block_n;
  a.causal = causal; a.score_mode = score_mode; a.p_cast = 1; a.rows = rows; a.out = NULL;
  a.row_hash = row_hash; a.row_zeros = row_zeros; a.k_sink = k_sink;
  return orc_parallel_for(attn_row, &a, B * Hq * nrows, N + d, nthreads);
}

int orc_attention_fp8_tiles(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                            const float* q_desc, const float* k_desc, const float* v_desc,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                            float softmax_scale, float p_scale, int kv_order, int block_n, int causal,
                            const int32_t* rows, int64_t nrows,
                            float* out, uint8_t* p_out, uint32_t* row_zeros, int32_t k_sink,
                            int score_mode, int nthreads, double* lse) {
  if (!q8 || !k8 || !v8 || !q_desc || !k_desc || !v_desc || !out || d > 128) return -1;
  if (block_n <= 0 || ORC_TILE_TOKENS % block_n) return -1;
  if (!rows) nrows = N;
  int rc = check_loop(B, Hq, Hkv, N, d, p_scale, kv_order, block_n, rows, nrows);
  if (rc) return rc;
  loop_args a;
  memset(&a, 0, sizeof a);
  a.q8 = q8; a.k8 = k8; a.v8 = v8; a.q_desc = q_desc; a.k_desc = k_desc; a.v_desc = v_desc;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d; a.nrows = nrows;
  a.softmax_scale = softmax_scale; a.p_scale = p_scale; a.kv_order = kv_order; a.block_n = block_n;
  a.causal = causal; a.score_mode = score_mode; a.p_cast = 1; a.tiles = 1; a.rows = rows; a.out = out;
  a.p_out = p_out; a.row_zeros = row_zeros; a.k_sink = k_sink; a.lse = lse;
  return orc_parallel_for(attn_row, &a, B * Hq * nrows, N + d, nthreads);
}

int orc_attention_pcast_f32(const float* q, const float* k, const float* v,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                            float softmax_scale, float p_scale, int kv_order, int block_n, int causal,
                            const int32_t* rows, int64_t nrows,
                            float* out, uint8_t* p_out, uint32_t* row_zeros, int32_t k_sink,
                            int p_cast, int nthreads, double* lse) {
  if (!q || !k || !v || !out) return -1;
  if (!rows) nrows = N;
  int rc = check_loop(B, Hq, Hkv, N, d, p_scale, kv_order, block_n, rows, nrows);
  if (rc) return rc;
  loop_args a;
  memset(&a, 0, sizeof a);
  a.qf = q; a.kf = k; a.vf = v;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.N = N; a.d = d; a.nrows = nrows;
  a.softmax_scale = softmax_scale; a.p_scale = p_scale; a.kv_order = kv_order; a.block_n = block_n;
  a.causal = causal; a.p_cast = p_cast; a.rows = rows; a.out = out;
  a.p_out = p_out; a.row_zeros = row_zeros; a.k_sink = k_sink; a.lse = lse;
  return orc_parallel_for(attn_row, &a, B * Hq * nrows, N + d, nthreads);
}
