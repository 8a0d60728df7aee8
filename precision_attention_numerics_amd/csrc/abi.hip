// extern "C" entry points of libfp8attn: host-side validation, workspace
// layout and kernel launches.  See include/fp8_attn.h for the contract.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/fp8_attn.h"
#include "attn.hpp"
#include "prepare.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const fp8a_shape* s) {
  if (!s) return FP8A_ERR_NULL;
  if (s->batch < 1 || s->hq < 1 || s->hkv < 1 || s->seqlen < 1) return FP8A_ERR_SHAPE;
  if (s->hq % s->hkv != 0) return FP8A_ERR_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return FP8A_ERR_SHAPE;
  if (s->seqlen > (1 << 30)) return FP8A_ERR_SHAPE;
  // the prologue's max pass indexes (tensor, batch, head) by its grid's second
  // dimension (at most 65535 blocks): B*hq query heads and B*hkv key and value
  // heads each; the forward grid is one workgroup per (batch, query head,
  // 128-token query tile), counted in 31 bits
  const int64_t bh = static_cast<int64_t>(s->batch) * s->hq;
  if (static_cast<int64_t>(s->batch) * (s->hq + 2 * static_cast<int64_t>(s->hkv)) > 65535) return FP8A_ERR_SHAPE;
  if (bh * ((static_cast<int64_t>(s->seqlen) + 127) / 128) > INT32_MAX) return FP8A_ERR_SHAPE;
  return FP8A_OK;
}

// Resolves a stride triple (zeros = dense) and checks the 16-byte row
// alignment the vector loads need.
int resolve_strides(const int64_t in[3], int32_t H, const fp8a_shape* s, int64_t out[3]) {
  const int64_t N = s->seqlen, d = s->head_dim;
  if (in[0] == 0 && in[1] == 0 && in[2] == 0) {
    out[0] = H * N * d; out[1] = N * d; out[2] = d;
    return FP8A_OK;
  }
  for (int i = 0; i < 3; ++i) {
    if (in[i] < 0 || in[i] % 8 != 0) return FP8A_ERR_SHAPE;
    out[i] = in[i];
  }
  if (out[2] < d) return FP8A_ERR_SHAPE;
  return FP8A_OK;
}

int32_t np2_chunks(int32_t N) {
  const int32_t nchunk = (N + 63) / 64;
  int32_t np2 = 1;
  while (np2 < nchunk) np2 <<= 1;
  return np2;
}

int32_t err_chunks(int32_t BH, int64_t nrows) {
  int64_t n = (2048 + BH - 1) / BH;
  if (n > nrows) n = nrows;
  if (n < 1) n = 1;
  return static_cast<int32_t>(n);
}

// exp2 patch table: binary32 patterns of x where v_exp_f32 would flip the
// E4M3 code of S * 2^x (see the attention kernel), and for each the adjacent
// binary32 pattern whose v_exp_f32 result is the correctly rounded 2^x of the
// listed x (both measured on gfx950 by running v_exp_f32 on every candidate).
bool p_scale_setup(float S, bool* pow2, float* inv_S, uint32_t* bad0, uint32_t* bad1, uint32_t* rep0,
                   uint32_t* rep1) {
  if (S == 448.0f) {
    *pow2 = false; *inv_S = 0.0f; *bad0 = 0xbf5a689au; *bad1 = 0xbfed344du;
    *rep0 = 0xbf5a6899u; *rep1 = 0xbfed344cu;
    return true;
  }
  for (int k = 0; k <= 8; ++k) {
    if (S == ldexpf(1.0f, k)) {
      *pow2 = true; *inv_S = ldexpf(1.0f, -k); *bad0 = 0xbd3b9cb2u; *bad1 = 0xbef3efb2u;
      *rep0 = 0xbd3b9cb1u; *rep1 = 0xbef3efb3u;
      return true;
    }
  }
  return false;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP8A_OK : FP8A_ERR_HIP; }

// Workspace of fp8_attn_prepare_noalloc: one copy in every GPU's memory, held
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol); it uses the
// device address looked up once per device below.
constexpr size_t kNoAllocScratch = FP8A_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kNoAllocScratch];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of the current device's scratch, looked up on the first
// call made on that device.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8A_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FP8A_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FP8A_OK;
}

size_t prepare_ws_bytes(const fp8a_shape* s, uint32_t flags) {
  if (check_shape(s) != FP8A_OK) return 0;
  const size_t B = s->batch, hq = s->hq, hkv = s->hkv, d = s->head_dim;
  const size_t nt = (flags & FP8A_TILE_SCALES) ? static_cast<size_t>(fp8_attn_padded_seqlen(s->seqlen)) / 128 : 1;
  size_t bytes = align_up(B * (hq * nt + hkv * nt + hkv) * sizeof(uint32_t));
  if (flags & FP8A_CENTER_K) {
    bytes += align_up(B * hkv * static_cast<size_t>(np2_chunks(s->seqlen)) * d * sizeof(double));
    bytes += align_up(B * hkv * d * sizeof(float));
  }
  return bytes;
}

// fp8_attn_prepare with the workspace given; with noalloc the workspace is
// the current device's scratch (looked up once all arguments have passed).
int prepare_common(const fp8a_shape* s, fp8a_dtype in_dtype, const void* q, const void* k, const void* v,
                   uint32_t flags, const int8_t* rot_signs, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                   float* q_desc, float* k_desc, float* v_desc, float* k_mean, int32_t* status_word,
                   void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (in_dtype != FP8A_F32 && in_dtype != FP8A_BF16) return FP8A_ERR_UNSUPPORTED;
  if (flags & ~(FP8A_ROTATE_QK | FP8A_CENTER_K | FP8A_TILE_SCALES | FP8A_PREFIX_SCALES | FP8A_INT8_QK))
    return FP8A_ERR_PARAM;
  if ((flags & FP8A_INT8_QK) && (flags & FP8A_TILE_SCALES)) return FP8A_ERR_UNSUPPORTED;
  if ((flags & FP8A_PREFIX_SCALES) && !(flags & FP8A_TILE_SCALES)) return FP8A_ERR_PARAM;
  if (!q || !k || !v || !q8 || !k8 || !v8t || !q_desc || !k_desc || !v_desc) return FP8A_ERR_NULL;
  if ((flags & FP8A_ROTATE_QK) && !rot_signs) return FP8A_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(k8) || !aligned16(v8t))
    return FP8A_ERR_SHAPE;
  const size_t need = prepare_ws_bytes(s, flags);
  if (noalloc) {
    if (need > kNoAllocScratch) return FP8A_ERR_WORKSPACE;
    if ((rc = device_scratch(&workspace))) return rc;
    workspace_bytes = kNoAllocScratch;
  }
  if (!workspace || workspace_bytes < need) return FP8A_ERR_WORKSPACE;
  fp8a::PrepareArgs a;
  memset(&a, 0, sizeof a);
  if ((rc = resolve_strides(s->q_stride, s->hq, s, a.qs))) return rc;
  if ((rc = resolve_strides(s->k_stride, s->hkv, s, a.ks))) return rc;
  if ((rc = resolve_strides(s->v_stride, s->hkv, s, a.vs))) return rc;
  a.B = s->batch; a.hq = s->hq; a.hkv = s->hkv; a.N = s->seqlen; a.Np = fp8_attn_padded_seqlen(s->seqlen);
  a.D = s->head_dim;
  a.bf16 = in_dtype == FP8A_BF16;
  a.rotate = (flags & FP8A_ROTATE_QK) != 0;
  a.center = (flags & FP8A_CENTER_K) != 0;
  a.ntile = (flags & FP8A_TILE_SCALES) ? a.Np / 128 : 1;
  a.prefix = (flags & FP8A_PREFIX_SCALES) != 0;
  a.int8 = (flags & FP8A_INT8_QK) != 0;
  a.q = q; a.k = k; a.v = v;
  a.signs = rot_signs;
  a.cd = static_cast<float>(1.0 / sqrt(static_cast<double>(s->head_dim)));
  a.q8 = q8; a.k8 = k8; a.v8t = v8t;
  a.q_desc = q_desc; a.k_desc = k_desc; a.v_desc = v_desc;
  a.status = status_word;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.amax = reinterpret_cast<uint32_t*>(ws);
  ws += align_up(static_cast<size_t>(a.B) * (a.hq * a.ntile + a.hkv * a.ntile + a.hkv) * sizeof(uint32_t));
  // tokens the mean key is taken over: all N, or with prefix scales the first
  // 128-token tile only (no key shift may depend on later tokens)
  a.n_mean = a.prefix ? (a.N < 128 ? a.N : 128) : a.N;
  a.np2 = np2_chunks(a.n_mean);
  if (a.center) {
    a.mean_part = reinterpret_cast<double*>(ws);
    ws += align_up(static_cast<size_t>(a.B) * a.hkv * a.np2 * a.D * sizeof(double));
    a.k_mean = k_mean ? k_mean : reinterpret_cast<float*>(ws);
  }
  return hip_status(fp8a::launch_prepare(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int32_t fp8_attn_padded_seqlen(int32_t seqlen) {
  if (seqlen < 1 || seqlen > (1 << 30)) return 0;
  return (seqlen + 127) / 128 * 128;
}

size_t fp8_attn_prepare_workspace_bytes(const fp8a_shape* s, uint32_t flags) { return prepare_ws_bytes(s, flags); }

int fp8_attn_prepare(const fp8a_shape* s, fp8a_dtype in_dtype, const void* q, const void* k, const void* v,
                     uint32_t flags, const int8_t* rot_signs, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                     float* q_desc, float* k_desc, float* v_desc, float* k_mean, int32_t* status_word,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return prepare_common(s, in_dtype, q, k, v, flags, rot_signs, q8, k8, v8t, q_desc, k_desc, v_desc, k_mean,
                        status_word, workspace, workspace_bytes, stream, false);
}

int fp8_attn_prepare_noalloc(const fp8a_shape* s, fp8a_dtype in_dtype, const void* q, const void* k,
                             const void* v, uint32_t flags, const int8_t* rot_signs, uint8_t* q8, uint8_t* k8,
                             uint8_t* v8t, float* q_desc, float* k_desc, float* v_desc, float* k_mean,
                             int32_t* status_word, void* stream) {
  return prepare_common(s, in_dtype, q, k, v, flags, rot_signs, q8, k8, v8t, q_desc, k_desc, v_desc, k_mean,
                        status_word, nullptr, 0, stream, true);
}

}  // extern "C"

namespace {

// Both forward entry points: tiles selects per-tile Q/K descales (E4M3 only).
int fwd_common(const fp8a_shape* s, fp8a_dtype qkv_dtype, const void* q, const void* k, const void* v,
               const float* q_desc, const float* k_desc, const float* v_desc, float softmax_scale,
               float p_scale, int32_t kv_order, int32_t block_n, int32_t causal, float* out, float* lse,
               uint8_t* p_dump, uint64_t* row_hash, uint32_t* row_zeros, int32_t k_sink, void* stream,
               bool tiles) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (qkv_dtype != FP8A_E4M3 && qkv_dtype != FP8A_F32 && qkv_dtype != FP8A_I8QK) return FP8A_ERR_UNSUPPORTED;
  if (tiles && qkv_dtype != FP8A_E4M3) return FP8A_ERR_UNSUPPORTED;
  const bool codes = qkv_dtype == FP8A_E4M3 || qkv_dtype == FP8A_I8QK;
  if (!q || !k || !v || !out) return FP8A_ERR_NULL;
  // the E4M3 kernel addresses one head's K8 / V8t through a buffer resource
  // with a 31-bit byte range
  if (codes && static_cast<int64_t>(fp8_attn_padded_seqlen(s->seqlen)) * s->head_dim > INT32_MAX)
    return FP8A_ERR_SHAPE;
  if (codes && (!q_desc || !k_desc || !v_desc)) return FP8A_ERR_NULL;
  if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return FP8A_ERR_PARAM;
  if (!(p_scale > 0.0f) || !(p_scale <= 448.0f)) return FP8A_ERR_PARAM;
  if (kv_order != 0 && kv_order != 1) return FP8A_ERR_PARAM;
  if (block_n != 64 && block_n != 128) return FP8A_ERR_PARAM;
  if (causal != 0 && causal != 1) return FP8A_ERR_PARAM;
  if (k_sink < 0) return FP8A_ERR_PARAM;
  bool pow2 = false;
  float inv_S = 0.0f;
  uint32_t bad0 = 0, bad1 = 0;
  uint32_t rep0 = 0, rep1 = 0;
  if (!p_scale_setup(p_scale, &pow2, &inv_S, &bad0, &bad1, &rep0, &rep1)) return FP8A_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return FP8A_ERR_SHAPE;
  const float ls2 = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (qkv_dtype == FP8A_F32) {
    fp8a::PcastParams p;
    memset(&p, 0, sizeof p);
    p.q = static_cast<const float*>(q); p.k = static_cast<const float*>(k); p.v = static_cast<const float*>(v);
    p.out = out; p.lse = lse; p.p_dump = p_dump; p.row_hash = row_hash; p.row_zeros = row_zeros;
    p.B = s->batch; p.hq = s->hq; p.hkv = s->hkv; p.N = s->seqlen; p.block_n = block_n;
    p.kv_order = kv_order; p.causal = causal; p.k_sink = k_sink;
    p.ls2 = ls2; p.S = p_scale; p.inv_S = inv_S; p.bad0 = bad0; p.bad1 = bad1;
    return hip_status(fp8a::launch_pcast_f32(p, s->head_dim, pow2, st));
  }
  fp8a::FwdParams p;
  memset(&p, 0, sizeof p);
  p.q8 = static_cast<const uint8_t*>(q); p.k8 = static_cast<const uint8_t*>(k); p.v8t = static_cast<const uint8_t*>(v);
  p.q_desc = q_desc; p.k_desc = k_desc; p.v_desc = v_desc;
  p.out = out; p.lse = lse; p.p_dump = p_dump; p.row_hash = row_hash; p.row_zeros = row_zeros;
  p.B = s->batch; p.hq = s->hq; p.hkv = s->hkv; p.N = s->seqlen; p.Np = fp8_attn_padded_seqlen(s->seqlen);
  p.n_qtiles = p.Np / 128; p.kv_order = kv_order; p.k_sink = k_sink;
  p.tiles = tiles ? 1 : 0;
  p.int8 = qkv_dtype == FP8A_I8QK ? 1 : 0;
  p.ls2 = ls2; p.S = p_scale; p.inv_S = inv_S; p.bad0 = bad0; p.bad1 = bad1;
  {
    float x0, x1;
    memcpy(&x0, &bad0, 4);
    memcpy(&x1, &bad1, 4);
    p.xcheck = x0 < x1 ? x0 : x1;
    p.rep0 = rep0;
    p.rep1 = rep1;
  }
  const bool dump = p_dump != nullptr || row_hash != nullptr || row_zeros != nullptr;
  if (s->head_dim == 64 && !p.int8) return hip_status(fp8a::launch_fwd_d64(p, block_n, causal != 0, pow2, dump, st));
  return hip_status(fp8a::launch_fwd(p, s->head_dim, block_n, causal != 0, pow2, dump, st));
}

}  // namespace

extern "C" {

int fp8_attn_fwd(const fp8a_shape* s, fp8a_dtype qkv_dtype, const void* q, const void* k, const void* v,
                 const float* q_desc, const float* k_desc, const float* v_desc, float softmax_scale,
                 float p_scale, int32_t kv_order, int32_t block_n, int32_t causal, float* out, float* lse,
                 uint8_t* p_dump, uint64_t* row_hash, uint32_t* row_zeros, int32_t k_sink, void* stream) {
  return fwd_common(s, qkv_dtype, q, k, v, q_desc, k_desc, v_desc, softmax_scale, p_scale, kv_order, block_n,
                    causal, out, lse, p_dump, row_hash, row_zeros, k_sink, stream, false);
}

int fp8_attn_fwd_tile_scaled(const fp8a_shape* s, const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                             const float* q_desc, const float* k_desc, const float* v_desc, float softmax_scale,
                             float p_scale, int32_t kv_order, int32_t block_n, int32_t causal, float* out,
                             float* lse, uint8_t* p_dump, uint64_t* row_hash, uint32_t* row_zeros, int32_t k_sink,
                             void* stream) {
  return fwd_common(s, FP8A_E4M3, q8, k8, v8t, q_desc, k_desc, v_desc, softmax_scale, p_scale, kv_order, block_n,
                    causal, out, lse, p_dump, row_hash, row_zeros, k_sink, stream, true);
}

size_t fp8_attn_head_error_workspace_bytes(const fp8a_shape* s, int64_t nrows) {
  if (check_shape(s) != FP8A_OK || nrows < 1) return 0;
  const int32_t BH = s->batch * s->hq;
  return align_up(static_cast<size_t>(BH) * err_chunks(BH, nrows) * 2 * sizeof(double));
}

int fp8_attn_head_error(const fp8a_shape* s, const float* out, const void* ref, fp8a_dtype ref_dtype,
                        const int32_t* rows, int64_t nrows, double* rel_err, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!out || !ref || !rel_err) return FP8A_ERR_NULL;
  if (ref_dtype != FP8A_F32 && ref_dtype != FP8A_F64) return FP8A_ERR_UNSUPPORTED;
  if (nrows < 1 || (!rows && nrows != s->seqlen)) return FP8A_ERR_SHAPE;
  const size_t need = fp8_attn_head_error_workspace_bytes(s, nrows);
  if (!workspace || workspace_bytes < need) return FP8A_ERR_WORKSPACE;
  fp8a::HeadErrParams p;
  memset(&p, 0, sizeof p);
  p.out = out; p.ref = ref; p.rows = rows; p.rel_err = rel_err;
  p.part = static_cast<double*>(workspace);
  p.nrows = nrows; p.BH = s->batch * s->hq; p.N = s->seqlen; p.D = s->head_dim;
  p.nchunk = err_chunks(p.BH, nrows);
  p.ref_f64 = ref_dtype == FP8A_F64;
  return hip_status(fp8a::launch_head_error(p, static_cast<hipStream_t>(stream)));
}

#ifndef FP8A_SOURCE_SHA256
#define FP8A_SOURCE_SHA256 "unknown"
#endif

const char* fp8_attn_build_info(void) {
  return "source_sha256=" FP8A_SOURCE_SHA256 " arch=gfx950";
}

const char* fp8_attn_strerror(int status) {
  switch (status) {
    case FP8A_OK: return "ok";
    case FP8A_ERR_NULL: return "a required pointer is NULL";
    case FP8A_ERR_SHAPE: return "sizes, strides or alignment not supported";
    case FP8A_ERR_UNSUPPORTED: return "request not implemented (dtype or p_scale)";
    case FP8A_ERR_PARAM: return "scalar parameter out of range";
    case FP8A_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8A_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

}  // extern "C"
