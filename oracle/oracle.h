/*
 * CPU oracle for the causal FP8 (E4M3FN) attention forward studied on the
 * "attention-numerics" pages and the "P-Cast Precisie in FP8 Attention"
 * summary.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this library: only the test suite, the package smoke check and the
 * bench's CPU-baseline leg do.  It shares no source with the HIP library.
 *
 * Two engines:
 *   - orc_attention_f64: the plain definition of ideal (causal) attention in
 *     binary64, the error reference the pages measure every head against.
 *   - orc_prepare / orc_attention_fp8 / orc_attention_pcast_f32: a step-by-
 *     step binary32 emulation of the quantised pipeline (per-head max scales,
 *     optional mean-key centring, optional random-sign Hadamard on Q and K,
 *     E4M3 codes, online softmax over KV blocks with the static P scale S).
 *
 * All arrays are dense, row-major, owned by the caller.
 */
#ifndef PAN_ORACLE_H
#define PAN_ORACLE_H
#include <stdint.h>

#define ORC_ROTATE 1u
#define ORC_CENTER 2u
/* One scale per 128-token tile for Q and K instead of per (batch, head): the
 * earlier emulator's granularity, which the attention-numerics project page
 * (second section) contrasts with FA3's full-sequence per-head scales.  V
 * keeps one scale per (batch, KV head). */
#define ORC_TILE 4u
#define ORC_TILE_TOKENS 128
/* With TILE: tile t's Q and K scales come from the largest tile maximum among
 * tiles 0..t (prefix scales: no scale depends on tokens past its tile's end,
 * the caveat the project page raises about full-sequence means and scales).
 * With CENTER as well, the mean key is taken over the first 128-token tile
 * only: one shift common to every key (exact softmax is unchanged by it) that
 * depends on no token past tile 0.  So every quantity used for tile t depends
 * only on tokens in tiles 0..t. */
#define ORC_PREFIX 8u
/* INT8 Q/K (the INT8-QK / FP8-PV kernel family the attention-numerics project
 * page measures, named without its quantisation): Q and K codes are
 * two's-complement int8 = clamp(RNE(x * 127/A), -127, 127) with the same scale
 * groups, descale A/127 (times RN32(1/sqrt d) when rotated); V stays E4M3.
 * The score of two int8 rows is their exact integer dot product (|s| <=
 * 127^2 * 128 < 2^24, exact in binary32): orc_attention_fp8 with score_mode 2. */
#define ORC_INT8 16u

/* int8 code of a binary32 value: round to nearest even, clamp to +-127. */
int8_t orc_i8_encode(float x);

/* E4M3FN codec: round to nearest, ties to even, saturating at +-448. */
uint8_t orc_e4m3_encode(float x);
float orc_e4m3_decode(uint8_t c);
void orc_e4m3_encode_n(const float* x, uint8_t* out, int64_t n);
void orc_e4m3_decode_n(const uint8_t* c, float* out, int64_t n);

/* RN32(2^x): 2^x correctly rounded to binary32. */
float orc_exp2_rn32(float x);
void orc_exp2_rn32_n(const float* x, float* out, int64_t n);

/* Score dot product of two 128-long E4M3 code vectors.
 * mode 0: in the precision of the gfx950 FP8 matrix instruction (see
 *         emulate.c for the arithmetic); mode 1: RN32 of the exact sum. */
float orc_fp8_dot128(const uint8_t* a, const uint8_t* b, int mode);

/* Unnormalised Sylvester Walsh-Hadamard transform of one binary32 row, in the
 * stage order h = 1, 2, 4, ..., d/2 (after the sign flip). */
void orc_fwht_row(float* x, const int8_t* signs, int64_t d);

/* Ideal attention in binary64.  q [B,Hq,N,d], k/v [B,Hkv,N,d];
 * rows: query positions to evaluate (NULL = all N); out [B,Hq,nrows,d]. */
int orc_attention_f64(const double* q, const double* k, const double* v,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                      int causal, double softmax_scale,
                      const int32_t* rows, int64_t nrows, double* out, int nthreads);

/* Prologue emulation.  Inputs binary32 (BF16 inputs are widened exactly by
 * the caller).  Outputs: codes [B,H,N,d], descales [B*H] (with TILE: q_desc
 * [B*Hq*T], k_desc [B*Hkv*T], T = ceil(N/128); v_desc stays [B*Hkv]), k_mean
 * [B*Hkv*d] (written when CENTER is set and k_mean is not NULL). */
int orc_prepare(const float* q, const float* k, const float* v,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                uint32_t flags, const int8_t* signs,
                uint8_t* q8, uint8_t* k8, uint8_t* v8,
                float* q_desc, float* k_desc, float* v_desc, float* k_mean);

/* Main-loop emulation on E4M3 codes.  lse (NULL or per row, binary64):
 * (running max in base-2 scaled units + log2 l) * ln 2, the natural-log
 * sum-exp of the scaled logits from the loop's own max and row sum. */
int orc_attention_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                      const float* q_desc, const float* k_desc, const float* v_desc,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                      float softmax_scale, float p_scale, int kv_order, int block_n, int causal,
                      const int32_t* rows, int64_t nrows,
                      float* out, uint8_t* p_out, uint32_t* row_zeros, int32_t k_sink,
                      int score_mode, int nthreads, double* lse);

/* The main loop of orc_attention_fp8 for its P~ codes only: per row the
 * checksum sum_j code_j * W_j mod 2^64 (W_j = splitmix64 output j+1 from seed
 * 0, made odd) and the count of zero codes among keys j >= k_sink; the output
 * accumulation is skipped. */
int orc_attention_fp8_rowhash(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                              const float* q_desc, const float* k_desc, const float* v_desc,
                              int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                              float softmax_scale, float p_scale, int kv_order, int block_n, int causal,
                              const int32_t* rows, int64_t nrows,
                              uint64_t* row_hash, uint32_t* row_zeros, int32_t k_sink,
                              int score_mode, int nthreads);

/* Main loop with per-tile Q/K descales (from a TILE prologue); block_n must
 * divide 128.  The logit factor c depends on the row's query tile and the
 * block's key tile, so the running max is kept in scaled units: per block
 * m <- max(m, RN32(max_j s * c)), x = fma(s, c, -m), alpha = 2^(m_old - m).
 * With one scale per head this is the per-head loop bit for bit (x -> RN32(x*c)
 * is monotone for c > 0, so RN32(max_s * c) is the max of the blocks' values). */
int orc_attention_fp8_tiles(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                            const float* q_desc, const float* k_desc, const float* v_desc,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                            float softmax_scale, float p_scale, int kv_order, int block_n, int causal,
                            const int32_t* rows, int64_t nrows,
                            float* out, uint8_t* p_out, uint32_t* row_zeros, int32_t k_sink,
                            int score_mode, int nthreads, double* lse);

/* Main-loop emulation with binary32 Q/K/V (only P is cast). p_cast = 0
 * replaces the cast by the identity (structure checks). */
int orc_attention_pcast_f32(const float* q, const float* k, const float* v,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                            float softmax_scale, float p_scale, int kv_order, int block_n, int causal,
                            const int32_t* rows, int64_t nrows,
                            float* out, uint8_t* p_out, uint32_t* row_zeros, int32_t k_sink,
                            int p_cast, int nthreads, double* lse);

#endif
