// Host-side launch interface of the attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8a {

struct FwdParams {
  const uint8_t* q8;      // [B,hq,Np,D]
  const uint8_t* k8;      // [B,hkv,Np,D]
  const uint8_t* v8t;     // [B,hkv,D,Np]
  const float* q_desc;
  const float* k_desc;
  const float* v_desc;
  float* out;             // [B,hq,N,D]
  float* lse;             // [B,hq,N] or null
  uint8_t* p_dump;        // [B,hq,N,N] or null
  uint64_t* row_hash;     // [B,hq,N] or null
  uint32_t* row_zeros;    // [B,hq,N] or null
  int32_t B, hq, hkv, N, Np, n_qtiles, kv_order, k_sink;
  int32_t tiles;          // 1: q_desc [B*hq*n_qtiles], k_desc [B*hkv*n_qtiles] per 128-token tile
  int32_t int8;           // 1: q8 / k8 hold int8 codes (exact integer scores)
  float ls2;              // RN32(softmax_scale * log2 e)
  float S;                // static P scale
  float inv_S;            // 1/S when S is a power of two
  uint32_t bad0, bad1;    // binary32 patterns of x whose v_exp_f32 result would flip a code
  float xcheck;           // smaller of the two listed x: blocks whose largest x is below it need no fix-up
  uint32_t rep0, rep1;    // neighbours of the listed x whose v_exp_f32 result is RN32(2^x) of the listed x
};

struct PcastParams {
  const float* q;         // [B,hq,N,D] dense
  const float* k;         // [B,hkv,N,D]
  const float* v;         // [B,hkv,N,D]
  float* out;
  float* lse;
  uint8_t* p_dump;
  uint64_t* row_hash;
  uint32_t* row_zeros;
  int32_t B, hq, hkv, N, block_n, kv_order, causal, k_sink;
  float ls2, S, inv_S;
  uint32_t bad0, bad1;
};

hipError_t launch_fwd(const FwdParams& p, int D, int BC, bool causal, bool pow2, bool dump, hipStream_t st);
// head_dim 64 with E4M3 Q/K on the 32x32x64 instruction (scores bit-identical
// to the zero-padded 16x16x128 form)
hipError_t launch_fwd_d64(const FwdParams& p, int BC, bool causal, bool pow2, bool dump, hipStream_t st);
hipError_t launch_pcast_f32(const PcastParams& p, int D, bool pow2, hipStream_t st);

struct HeadErrParams {
  const float* out;       // [BH, N, D]
  const void* ref;        // [BH, nrows, D] f32 or f64
  const int32_t* rows;    // [nrows] or null
  double* part;           // workspace [BH, nchunk, 2]
  double* rel_err;        // [BH]
  int64_t nrows;
  int32_t BH, N, D, nchunk;
  bool ref_f64;
};

hipError_t launch_head_error(const HeadErrParams& p, hipStream_t st);

}  // namespace fp8a
