// Host-side launch interface of the prologue kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8a {

struct PrepareArgs {
  int32_t B, hq, hkv, N, Np, D;
  bool bf16, rotate, center, prefix, int8;
  int32_t ntile;                 // Q/K scale groups per head: Np/128 with per-tile scales, else 1
  const void *q, *k, *v;
  int64_t qs[3], ks[3], vs[3];   // element strides of (batch, head, token)
  const int8_t* signs;
  float cd;                      // RN32(1/sqrt(D)), folded into the rotated descales
  uint8_t *q8, *k8, *v8t;
  float *q_desc, *k_desc, *v_desc, *k_mean;
  int32_t* status;               // may be null
  uint32_t* amax;                // workspace: B*(hq*ntile + hkv*ntile + hkv)
  double* mean_part;             // workspace: B*hkv*np2*D (CENTER only)
  int32_t n_mean;                // tokens the mean key is taken over (N, or the first tile)
  int32_t np2;                   // chunk count of those tokens rounded up to a power of two
};

hipError_t launch_prepare(const PrepareArgs& a, hipStream_t st);

}  // namespace fp8a
