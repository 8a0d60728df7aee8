// Relative Frobenius output error per (batch, head) for gfx950: the per-head
// metric of the attention-numerics pages (project page: each head's output
// against exact causal attention in binary64; study page, "What do these scores
// mean?": log(1 + relative Frobenius error) per text).  The log and the mean
// over texts are taken by the caller on the B*hq values returned here.
//
// HBM-bound: one streaming pass over O (4 B/element) and the reference (4 or
// 8 B/element).  Sums are binary64; partial sums per chunk are reduced in a
// fixed order, so the result is deterministic.
#include "device_common.hpp"
#include "attn.hpp"

namespace fp8a {

constexpr int kErrThreads = 256;

template <bool REF64>
__global__ __launch_bounds__(kErrThreads) void k_head_err_partial(const HeadErrParams p) {
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int64_t rows_per = (p.nrows + p.nchunk - 1) / p.nchunk;
  const int64_t r0 = chunk * rows_per;
  const int64_t r1 = min(r0 + rows_per, p.nrows);
  double num = 0.0, den = 0.0;
  const int D = p.D;
  for (int64_t e = r0 * D + threadIdx.x; e < r1 * D; e += kErrThreads) {
    const int64_t r = e / D;
    const int cc = static_cast<int>(e % D);
    const int64_t orow = p.rows ? p.rows[r] : r;
    if (orow < 0 || orow >= p.N) continue;   // out-of-range row indices contribute nothing
    const double o = p.out[(static_cast<int64_t>(bh) * p.N + orow) * D + cc];
    const int64_t ri = (static_cast<int64_t>(bh) * p.nrows + r) * D + cc;
    const double rv = REF64 ? static_cast<const double*>(p.ref)[ri] : static_cast<double>(static_cast<const float*>(p.ref)[ri]);
    const double dlt = o - rv;
    num += dlt * dlt;
    den += rv * rv;
  }
  __shared__ double sn[kErrThreads], sd[kErrThreads];
  sn[threadIdx.x] = num;
  sd[threadIdx.x] = den;
  __syncthreads();
  for (int w = kErrThreads / 2; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) {
      sn[threadIdx.x] += sn[threadIdx.x + w];
      sd[threadIdx.x] += sd[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    p.part[(static_cast<int64_t>(bh) * p.nchunk + chunk) * 2] = sn[0];
    p.part[(static_cast<int64_t>(bh) * p.nchunk + chunk) * 2 + 1] = sd[0];
  }
}

__global__ void k_head_err_final(const HeadErrParams p) {
  const int bh = blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= p.BH) return;
  double num = 0.0, den = 0.0;
  for (int c = 0; c < p.nchunk; ++c) {
    num += p.part[(static_cast<int64_t>(bh) * p.nchunk + c) * 2];
    den += p.part[(static_cast<int64_t>(bh) * p.nchunk + c) * 2 + 1];
  }
  p.rel_err[bh] = sqrt(num) / sqrt(den);
}

hipError_t launch_head_error(const HeadErrParams& p, hipStream_t st) {
  const dim3 grid(p.nchunk, p.BH);
  if (p.ref_f64) k_head_err_partial<true><<<grid, dim3(kErrThreads), 0, st>>>(p);
  else k_head_err_partial<false><<<grid, dim3(kErrThreads), 0, st>>>(p);
  k_head_err_final<<<dim3((p.BH + 63) / 64), dim3(64), 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace fp8a
