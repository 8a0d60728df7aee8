/*
 * fp8_attn.h -- C ABI of the MI355X (gfx950) causal FP8 (OCP E4M3FN) attention
 * forward studied on the "attention-numerics" pages (mottopanikeiku.github.io)
 * and in the "P-Cast Precisie in FP8 Attention" summary (gist.science).
 *
 * General conventions
 *   - Every pointer argument named as "device" is device memory owned by the
 *     caller; its lifetime must cover the work enqueued on `stream`.  The
 *     library allocates and frees nothing; scratch memory comes from the
 *     caller through a workspace argument sized by the *_workspace_bytes call,
 *     except for fp8_attn_prepare_noalloc, which uses a fixed device array of
 *     the library (FP8A_NOALLOC_SCRATCH_BYTES on every GPU it runs on).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call validates its arguments on the host first; a failed check
 *     returns a negative status and enqueues nothing.  No call synchronises.
 *   - Layout: operands are [batch, head, token, channel] with the channel axis
 *     contiguous; the other axes use the element strides in fp8a_shape (a
 *     stride triple of zeros means dense).  Grouped-query attention: query
 *     head h reads KV head h / (hq / hkv).
 *   - Quantised operands use a padded token count Np = fp8_attn_padded_seqlen(N)
 *     (a multiple of 128); rows/columns past N hold code 0.
 *   - Thread safety: concurrent calls on different streams with disjoint
 *     outputs are independent, except fp8_attn_prepare_noalloc calls that
 *     overlap on one GPU (they share that GPU's scratch array and race).
 */
#ifndef FP8_ATTN_H
#define FP8_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FP8A_OK = 0,
  FP8A_ERR_NULL = -1,        /* a required pointer is NULL */
  FP8A_ERR_SHAPE = -2,       /* sizes or strides outside what the kernels support */
  FP8A_ERR_UNSUPPORTED = -3, /* a valid request this library does not implement */
  FP8A_ERR_PARAM = -4,       /* a scalar parameter out of range */
  FP8A_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  FP8A_ERR_HIP = -6          /* the HIP runtime reported an error at launch */
} fp8a_status;

typedef enum { FP8A_F32 = 0, FP8A_BF16 = 1, FP8A_F64 = 2, FP8A_E4M3 = 3, FP8A_I8QK = 4 } fp8a_dtype;

/* Prologue flags.  ROTATE: fixed random-sign Hadamard on Q and K, never V
 * (attention-numerics study page, "See the vectors and the arithmetic").
 * CENTER: subtract the full-sequence mean key before rotation (project page,
 * second section; study page, same panel). */
#define FP8A_ROTATE_QK 1u
#define FP8A_CENTER_K 2u
/* TILE_SCALES: one Q scale per (batch, query head, 128-token tile) and one K
 * scale per (batch, KV head, tile) instead of per (batch, head) -- the earlier
 * emulator's granularity, which the project page (second section) contrasts
 * with FA3's full-sequence per-head scales; V keeps per-head scales.  Codes
 * prepared this way go to fp8_attn_fwd_tile_scaled. */
#define FP8A_TILE_SCALES 4u
/* PREFIX_SCALES (with TILE_SCALES): tile t's Q and K scales come from the
 * largest tile maximum among tiles 0..t, so no scale depends on tokens past
 * its own tile (the project page notes that full-sequence means and scales see
 * future tokens).  With CENTER_K the mean key is taken over the first
 * 128-token tile only (min(N, 128) tokens): one shift common to every key, so
 * exact softmax is unchanged, that depends on no token past tile 0.  Every
 * quantity used for tile t then depends only on tokens in tiles 0..t: causal
 * at the 128-token tile granularity.  Error: FP8A_ERR_PARAM without
 * TILE_SCALES. */
#define FP8A_PREFIX_SCALES 8u
/* INT8_QK: Q and K become two's-complement int8 codes, clamp(RNE(x * 127/A),
 * -127, 127), with descale A/127 (times RN32(1/sqrt d) when rotated); V stays
 * E4M3.  This is the INT8-QK / FP8-PV kernel family the project page measures
 * besides FA3 (SageAttention); the pages give none of its quantisation, so the
 * scale groups are FA3's per (batch, head).  Such codes go to fp8_attn_fwd with
 * qkv_dtype FP8A_I8QK.  Not combined with TILE_SCALES (FP8A_ERR_UNSUPPORTED). */
#define FP8A_INT8_QK 16u

typedef struct {
  int32_t batch;     /* B >= 1; B * (hq + 2 hkv) <= 65535 */
  int32_t hq;        /* query heads >= 1 */
  int32_t hkv;       /* KV heads >= 1, hq % hkv == 0 */
  int32_t seqlen;    /* 1 <= N <= 2^30 (token count of every head) */
  int32_t head_dim;  /* d: 64 or 128 */
  int64_t q_stride[3], k_stride[3], v_stride[3]; /* element strides of (batch, head, token) */
} fp8a_shape;

/* Np: the token count padded to a multiple of 128; 0 for a count outside
 * [1, 2^30] (the range every entry point accepts). */
int32_t fp8_attn_padded_seqlen(int32_t seqlen);

/* Workspace needed by fp8_attn_prepare for this shape and flags (bytes). */
size_t fp8_attn_prepare_workspace_bytes(const fp8a_shape* shape, uint32_t flags);

/*
 * fp8_attn_prepare -- quantisation prologue.
 *
 * Computes, per (batch, head) over the full sequence (project page, second
 * section: one max-based scale per (batch, head) for each of Q, K and V, taken
 * over all tokens):
 *   1. if CENTER: mu[b,g,:] = mean over all N tokens of K[b,g,:,:] (over the
 *      first min(N, 128) with PREFIX_SCALES), in binary64 (chunks of 64 tokens
 *      summed in order, chunk sums added in a pairwise tree), rounded to
 *      binary32; K' = K - mu.
 *   2. if ROTATE: for Q and K' (never V) each row is multiplied by
 *      rot_signs and passed through the unnormalised Sylvester Walsh-Hadamard
 *      transform (stages h = 1, 2, ..., d/2) in binary32.
 *   3. A = max |x| per head of the transformed Q, K and of raw V; the scale
 *      448/A quantises, the descale A/448 (times RN32(1/sqrt(d)) for the
 *      rotated Q and K) is written out.  A = 0 gives scale and descale 1.
 *   4. codes = E4M3FN(x * 448/A), round-to-nearest-even, saturating at +-448
 *      (study page, "See the vectors and the arithmetic").
 *
 * Arguments
 *   in_dtype   FP8A_F32 or FP8A_BF16: element type of q, k, v (device).
 *   q, k, v    device, [B,hq,N,d] / [B,hkv,N,d] with the shape's strides.
 *   rot_signs  device int8[d] of +-1; required with ROTATE, else ignored.
 *   q8         device out, [B,hq,Np,d] E4M3FN codes.
 *   k8         device out, [B,hkv,Np,d] codes.
 *   v8t        device out, [B,hkv,d,Np] codes (V transposed: token axis contiguous).
 *   q_desc     device out, float[B*hq];  k_desc, v_desc: float[B*hkv].  With
 *              TILE_SCALES, q_desc float[B*hq*T] and k_desc float[B*hkv*T],
 *              T = Np/128 (tile t covers tokens [128t, 128t+128); step 3's
 *              max is taken per tile for Q and K).
 *   k_mean     device out, float[B*hkv*d]; written when CENTER (may be NULL).
 *   status_word device out, int32 (may be NULL): bit 0 is set when any input
 *              element was NaN or infinite; the codes are then unspecified.
 *   workspace  device scratch of fp8_attn_prepare_workspace_bytes().
 */
int fp8_attn_prepare(const fp8a_shape* shape, fp8a_dtype in_dtype,
                     const void* q, const void* k, const void* v, uint32_t flags,
                     const int8_t* rot_signs,
                     uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                     float* q_desc, float* k_desc, float* v_desc, float* k_mean,
                     int32_t* status_word, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8_attn_prepare_noalloc -- fp8_attn_prepare without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments (minus workspace), results and errors as fp8_attn_prepare; its
 * scratch is a static device array of FP8A_NOALLOC_SCRATCH_BYTES per GPU that
 * the library holds until the process ends.  The call allocates nothing.
 *
 *   - FP8A_ERR_WORKSPACE when fp8_attn_prepare_workspace_bytes(shape, flags)
 *     exceeds FP8A_NOALLOC_SCRATCH_BYTES (8 MiB: with CENTER_K, d = 128 and
 *     8 KV heads, up to 32768 tokens); FP8A_ERR_HIP when the array's device
 *     address cannot be looked up (done once per device, on the first call
 *     made with that device current).
 *   - Every call on a GPU uses the same array; the call clears what must
 *     start at zero.  Calls that overlap on one GPU (several streams or host
 *     threads) race on it and give unspecified results: serialise them.
 */
#define FP8A_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int fp8_attn_prepare_noalloc(const fp8a_shape* shape, fp8a_dtype in_dtype,
                             const void* q, const void* k, const void* v, uint32_t flags,
                             const int8_t* rot_signs,
                             uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                             float* q_desc, float* k_desc, float* v_desc, float* k_mean,
                             int32_t* status_word, void* stream);

/*
 * fp8_attn_fwd -- attention main loop and epilogue.
 *
 * For every query row i, the KV blocks [jB, (j+1)B) holding a visible key
 * (j <= i when causal) are visited in forward (0 -> N) or reverse (N -> 0)
 * order (P-Cast summary, Probleemstelling, item 1).  With E4M3 operands the
 * score is the FP8 matrix-core dot product of the codes; c = (q_desc*k_desc)
 * * RN32(softmax_scale*log2 e); per block the running max m (over raw scores)
 * is updated, x = fma(s, c, -RN32(m*c)), p = 2^x (binary32, correctly
 * rounded wherever it decides a code), l <- l*alpha + sum p, and
 * P~ = E4M3(S*p) enters the FP8 product with V (P-Cast summary, item 2: the
 * static scale S is applied before the E4M3 cast and divided out in the
 * epilogue): out = acc * (v_desc / (S*l)).
 *
 * Arguments
 *   qkv_dtype  FP8A_E4M3: q = q8 [B,hq,Np,d], k = k8 [B,hkv,Np,d], v = v8t
 *              [B,hkv,d,Np] as written by fp8_attn_prepare, descales required.
 *              FP8A_I8QK: the same with int8 q and k codes (an INT8_QK
 *              prologue); the score is their exact integer dot product.
 *              FP8A_F32: dense binary32 q/k/v [B,h,N,d], only P is cast
 *              (the P-Cast summary's simulation that follows the kernel step
 *              by step, Bijdragen item 4); scores are an ordered binary32 fma chain over the
 *              channels; descales must be NULL.
 *   softmax_scale  > 0, usually 1/sqrt(d).
 *   p_scale    S: a power of two in [1, 256] or 448.
 *   kv_order   0 forward, 1 reverse.   block_n: 64 or 128.   causal: 0 or 1.
 *   out        device out, float [B,hq,N,d].
 *   lse        device out, float [B,hq,N] natural-log sum-exp of the scaled
 *              logits (may be NULL).
 *   p_dump     device out, uint8 [B,hq,N,N] P~ codes (may be NULL): every key of
 *              every visited block is written (0 for masked keys); keys of
 *              unvisited blocks are left untouched, so zero it first.
 *   row_hash   device out, uint64 [B,hq,N] (may be NULL): a checksum of the
 *              row's P~ codes for verification, sum over keys j of
 *              code_ij * W_j modulo 2^64 (masked keys have code 0), with
 *              W_j = splitmix64(j) | 1, the (j+1)-th output of a splitmix64
 *              generator seeded with 0 (Steele, Lea and Flood, OOPSLA 2014).
 *              It does not depend on the visit order, and the odd weights make
 *              any single changed code change it.
 *   row_zeros  device out, uint32 [B,hq,N] (may be NULL): number of visible
 *              keys j >= k_sink whose P~ code is 0.
 * Errors: FP8A_ERR_SHAPE also when, with E4M3 operands, one head's codes
 * (Np*d bytes) exceed 2^31 - 1.
 */
int fp8_attn_fwd(const fp8a_shape* shape, fp8a_dtype qkv_dtype,
                 const void* q, const void* k, const void* v,
                 const float* q_desc, const float* k_desc, const float* v_desc,
                 float softmax_scale, float p_scale, int32_t kv_order, int32_t block_n, int32_t causal,
                 float* out, float* lse, uint8_t* p_dump, uint64_t* row_hash, uint32_t* row_zeros,
                 int32_t k_sink, void* stream);

/*
 * fp8_attn_fwd_tile_scaled -- fp8_attn_fwd for codes from a TILE_SCALES
 * prologue (E4M3 operands only).  q_desc is float[B*hq*T] and k_desc
 * float[B*hkv*T] (T = Np/128); v_desc float[B*hkv].  The logit factor of query
 * row i and block j is c = (q_desc[tile(i)] * k_desc[tile of block j]) *
 * RN32(softmax_scale*log2 e), and the running max is kept in those scaled
 * units: per block m <- max(m, RN32(max_j s * c)), x = fma(s, c, -m),
 * alpha = 2^(m_old - m).  With equal scales in every tile this is
 * fp8_attn_fwd bit for bit (x -> RN32(x*c) is monotone for c > 0).  Other
 * arguments, outputs and errors as fp8_attn_fwd.
 */
int fp8_attn_fwd_tile_scaled(const fp8a_shape* shape, const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                             const float* q_desc, const float* k_desc, const float* v_desc,
                             float softmax_scale, float p_scale, int32_t kv_order, int32_t block_n,
                             int32_t causal, float* out, float* lse, uint8_t* p_dump, uint64_t* row_hash,
                             uint32_t* row_zeros, int32_t k_sink, void* stream);

/* Workspace needed by fp8_attn_head_error (bytes). */
size_t fp8_attn_head_error_workspace_bytes(const fp8a_shape* shape, int64_t nrows);

/*
 * fp8_attn_head_error -- relative Frobenius output error per (batch, head):
 * rel_err[b*hq+h] = ||O - R||_F / ||R||_F over the head's rows, sums in
 * binary64 (project page: each head's output against exact causal attention
 * in binary64; study page, "What do these scores mean?").
 *
 *   out        device, float [B,hq,N,d] (as written by fp8_attn_fwd).
 *   ref        device, [B,hq,nrows,d] of ref_dtype FP8A_F32 or FP8A_F64.
 *   rows       device int32[nrows] of query positions in [0, N), or NULL for
 *              all rows (then nrows must equal N).
 *   rel_err    device out, double [B*hq].
 */
int fp8_attn_head_error(const fp8a_shape* shape, const float* out, const void* ref, fp8a_dtype ref_dtype,
                        const int32_t* rows, int64_t nrows, double* rel_err,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* fp8_attn_strerror(int status);

/* Static string identifying the build: "source_sha256=<hex> arch=gfx950",
 * the SHA-256 the build script computed over the library's sources, headers
 * and itself, so a caller can check that a shipped binary matches a source
 * tree.  Not part of the computation; never fails. */
const char* fp8_attn_build_info(void);

#ifdef __cplusplus
}
#endif
#endif /* FP8_ATTN_H */
