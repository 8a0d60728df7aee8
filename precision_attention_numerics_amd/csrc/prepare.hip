// Quantisation prologue kernels for gfx950: mean key, per-head amax, fused
// centre + random-sign Walsh-Hadamard + E4M3 quantise, and V quantise into the
// transposed layout the attention core reads.
//
// What is computed follows the attention-numerics project page (second
// section: one max-based scale per (batch, head) for each of Q, K and V, taken
// over all tokens; the same Hadamard on Q and K, never V; mean-key
// subtraction) and the
// study page ("See the vectors and the arithmetic": one maximum-based scale,
// E4M3FN with round-to-nearest-even and saturation at +-448).
//
// All of these kernels are HBM-bound streaming passes.  Rows are handled by
// groups of D/8 consecutive lanes holding 8 channels each, so a wave reads
// whole rows with 16-byte loads; the Hadamard stages within a lane run in
// registers and the cross-lane stages use lane shuffles.  Every binary32
// operation is the one the stage order prescribes, so the codes are bit-exact
// reproducible.
#include "device_common.hpp"
#include "prepare.hpp"

namespace fp8a {

template <typename IT>
__device__ __forceinline__ void load8(const IT* p, float x[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float x[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float x[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}

// Zeroes the scale maxima (n words) and, when given, the status word.
__global__ void k_fill2_u32(uint32_t* __restrict__ p, int64_t n, uint32_t* __restrict__ status) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
  if (i == 0 && status) *status = 0u;
}

// Partial sums of the mean key: each group of D/8 lanes owns one chunk of 64
// tokens of one KV head, 8 channels per lane; tokens are added in increasing
// order in binary64 starting from +0.0.  Chunks in [nchunk, np2) are the
// tree's zero padding.  grid = (ceil(np2 / chunks per block), B*hkv).
template <typename IT, int D>
__global__ __launch_bounds__(256) void k_kmean_partial(const IT* __restrict__ k, int64_t sb, int64_t sh, int64_t sn,
                                                       int32_t hkv, int32_t N, int32_t np2, double* __restrict__ part) {
  constexpr int L = D / 8;
  constexpr int CPB = 256 / L;
  const int32_t li = threadIdx.x % L;
  const int32_t t = blockIdx.x * CPB + threadIdx.x / L;
  const int32_t bg = blockIdx.y;
  if (t >= np2) return;
  const int32_t b = bg / hkv, g = bg % hkv;
  double s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0;
  const int32_t n0 = t * 64;
  const int32_t n1 = min(n0 + 64, N);
  const IT* base = k + b * sb + g * sh + 8 * li;
  int32_t n = n0;
  for (; n + 8 <= n1; n += 8) {
    float x[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r) load8<IT>(base + static_cast<int64_t>(n + r) * sn, x[r]);
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += static_cast<double>(x[r][e]);
  }
  for (; n < n1; ++n) {
    float x[8];
    load8<IT>(base + static_cast<int64_t>(n) * sn, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += static_cast<double>(x[e]);
  }
  double* dst = part + (static_cast<int64_t>(bg) * np2 + t) * D + 8 * li;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = s[e];
}

// Pairwise tree over the np2 chunk partials of each channel (left + right at
// every node, leaves in chunk order), then one binary64 division by N and
// rounding to binary32.  A block handles 8 channels of one KV head with 32
// workers per channel: worker w reduces the aligned subtree of leaves
// [w*Lw, (w+1)*Lw) with a stack (after leaf i the top ctz(i+1) entries are
// folded, which builds exactly that subtree), then the 32 subtree sums are
// combined level by level.  Aligned power-of-two subtrees are nodes of the
// full tree, so the result is the full tree's.  grid = (B*hkv, D/8).
constexpr int kMeanCh = 8;
constexpr int kMeanW = 32;

__global__ __launch_bounds__(kMeanCh * kMeanW) void k_kmean_final(const double* __restrict__ part, int32_t np2,
                                                                  int32_t N, int32_t D, float* __restrict__ mu) {
  // N <= 2^30 gives np2 <= 2^24, so a worker's subtree has at most 2^19
  // leaves and its stack at most 20 entries.
  __shared__ double stack[kMeanCh * kMeanW][24];
  __shared__ double res[kMeanCh][kMeanW];
  const int32_t tid = threadIdx.x, cl = tid % kMeanCh, w = tid / kMeanCh;
  const int32_t c = blockIdx.y * kMeanCh + cl;
  const int32_t bg = blockIdx.x;
  const int32_t W = min(np2, kMeanW);
  const int32_t Lw = np2 / W;
  double v = 0.0;
  if (w < W) {
    const double* col = part + (static_cast<int64_t>(bg) * np2 + static_cast<int64_t>(w) * Lw) * D + c;
    double* st = stack[tid];
    int32_t depth = 0;
    for (int32_t i0 = 0; i0 < Lw; i0 += 8) {
      double xs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[e] = (i0 + e < Lw) ? col[static_cast<int64_t>(i0 + e) * D] : 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (i0 + e < Lw) {
          double x = xs[e];
          for (int32_t f = __builtin_ctz(static_cast<uint32_t>(i0 + e + 1)); f > 0; --f) x = st[--depth] + x;
          st[depth++] = x;
        }
      }
    }
    v = st[0];
  }
  res[cl][w] = v;
  __syncthreads();
  for (int32_t m = W; m > 1; m >>= 1) {
    double x = 0.0;
    if (w < m / 2) x = res[cl][2 * w] + res[cl][2 * w + 1];
    __syncthreads();
    if (w < m / 2) res[cl][w] = x;
    __syncthreads();
  }
  if (w == 0) mu[static_cast<int64_t>(bg) * D + c] = static_cast<float>(res[cl][0] / static_cast<double>(N));
}

// Value of lane (lane ^ M) within a group of 16 lanes (M = 1, 2, 4, 8), by DPP
// (no LDS): quad_perm [1,0,3,2] and [2,3,0,1] for 1 and 2, row_half_mirror
// then quad_perm [3,2,1,0] for 4 (7 - ((i^3) & 7) = (i ^ 4) & 7), row_ror:8
// for 8.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int M>
__device__ __forceinline__ float lane_xor16(float v) {
  if constexpr (M == 1) return dpp_mov<0xB1>(v);
  else if constexpr (M == 2) return dpp_mov<0x4E>(v);
  else if constexpr (M == 4) return dpp_mov<0x1B>(dpp_mov<0x141>(v));
  else return dpp_mov<0x128>(v);
}

// Butterfly stage h = 8*M across the lanes of a row: the lower lane keeps
// x + y, the upper y - x (y = partner's value), written as y + (+-x), which is
// the same binary32 operation.
template <int M>
__device__ __forceinline__ void cross_stage(float x[8], int li) {
  const uint32_t flip = (li & M) ? 0x80000000u : 0u;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = lane_xor16<M>(x[e]);
    x[e] = y + __uint_as_float(__float_as_uint(x[e]) ^ flip);
  }
}

// One row (D channels) held by D/8 lanes, 8 channels per lane: optional
// centring, sign flip and unnormalised Sylvester Walsh-Hadamard transform in
// the stage order h = 1, 2, ..., D/2.
template <int D, bool ROT, bool CENTER>
__device__ __forceinline__ void transform_row(float x[8], int li, const float* __restrict__ mu,
                                              const int8_t* __restrict__ signs) {
  if constexpr (CENTER) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] - mu[8 * li + e];
  }
  if constexpr (ROT) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * static_cast<float>(signs[8 * li + e]);
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if ((i & h) == 0) {
          const float a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
      }
    }
    if constexpr (D / 8 > 1) cross_stage<1>(x, li);
    if constexpr (D / 8 > 2) cross_stage<2>(x, li);
    if constexpr (D / 8 > 4) cross_stage<4>(x, li);
    if constexpr (D / 8 > 8) cross_stage<8>(x, li);
  }
}

constexpr int kPrepThreads = 256;
constexpr int kRowsPerBlock = 256;
constexpr int kRowsInFlight = 4;

// One tensor's share of a prologue pass: the rows of batch*head bh, block bx.
struct RowsJob {
  const void* x;
  int64_t sb, sh, sn;     // element strides of (batch, head, token)
  int32_t H;              // heads of this tensor
  int32_t ntile;          // scale groups per head
  uint32_t* amax;         // per head (ntile == 1) or per 128-token tile
  float* desc;            // descales out (quantise pass)
  uint8_t* codes;         // [B,H,Np,D] codes out (quantise pass)
};

// Max |x| of the transformed rows per head (ntile == 1) or per 128-token tile
// of a head (amax[bh * ntile + tile]) for block (bx, bh): the block's rows are
// tiles 2*bx and 2*bx + 1.
template <typename IT, int D, bool ROT, bool CENTER>
__device__ __forceinline__ void amax_rows(const RowsJob& j, int bh, int bx, int32_t N, const float* __restrict__ mu_all,
                                          const int8_t* __restrict__ signs, int32_t* __restrict__ status) {
  constexpr int L = D / 8;                 // lanes per row
  constexpr int RPI = kPrepThreads / L;    // rows per iteration
  const IT* __restrict__ x = static_cast<const IT*>(j.x);
  const int64_t sb = j.sb, sh = j.sh, sn = j.sn;
  const int32_t H = j.H, ntile = j.ntile;
  uint32_t* __restrict__ amax = j.amax;
  const int b = bh / H, h = bh % H;
  const int li = threadIdx.x % L, rl = threadIdx.x / L;
  const float* mu = CENTER ? mu_all + static_cast<int64_t>(bh) * D : nullptr;
  const IT* base = x + b * sb + h * sh + 8 * li;
  float m = 0.0f, m_hi = 0.0f;   // rows [0, 128) and [128, 256) of the block
  bool bad = false;
  const int n_begin = bx * kRowsPerBlock;
  // kRowsInFlight rows per lane group per step, loaded before any is
  // transformed.  Rows past N are not loaded and not counted; the L lanes of a
  // row share r, so the lane exchanges of a row always run on all its lanes.
  // r0 + u * RPI < kRowsPerBlock always holds (r0 < RPI + 3 * kRowsInFlight * RPI).
  // Rows past N load row N - 1 instead (no branch around the loads, so all
  // of them are in flight together) and are not counted.
  for (int r0 = rl; r0 < kRowsPerBlock; r0 += kRowsInFlight * RPI) {
    float v[kRowsInFlight][8];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int n = min(n_begin + r0 + u * RPI, N - 1);
      load8<IT>(base + static_cast<int64_t>(n) * sn, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int n = n_begin + r0 + u * RPI;
      const bool live = n < N;
#pragma unroll
      for (int e = 0; e < 8; ++e) bad |= live && !__builtin_isfinite(v[u][e]);
      transform_row<D, ROT, CENTER>(v[u], li, mu, signs);
      if (live) {
        float rm = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) rm = __builtin_fmaxf(rm, __builtin_fabsf(v[u][e]));
        if (r0 + u * RPI < kRowsPerBlock / 2) m = __builtin_fmaxf(m, rm);
        else m_hi = __builtin_fmaxf(m_hi, rm);
      }
    }
  }
  if (ntile == 1) m = __builtin_fmaxf(m, m_hi);
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    m = __builtin_fmaxf(m, wave_xor(m, s));
    m_hi = __builtin_fmaxf(m_hi, wave_xor(m_hi, s));
  }
  __shared__ float red[2][kPrepThreads / kWave];
  __shared__ int redbad;
  if (threadIdx.x == 0) redbad = 0;
  __syncthreads();
  if (bad) atomicOr(&redbad, 1);
  if (threadIdx.x % kWave == 0) {
    red[0][threadIdx.x / kWave] = m;
    red[1][threadIdx.x / kWave] = m_hi;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const int half = threadIdx.x;
    float mm = red[half][0];
    for (int w = 1; w < kPrepThreads / kWave; ++w) mm = __builtin_fmaxf(mm, red[half][w]);
    if (ntile == 1) {
      if (half == 0) atomicMax(amax + bh, __float_as_uint(mm));
    } else if (n_begin + half * (kRowsPerBlock / 2) < N) {
      // each tile is written by exactly one block
      atomicMax(amax + static_cast<int64_t>(bh) * ntile + 2 * bx + half, __float_as_uint(mm));
    }
    if (half == 0 && redbad && status) atomicOr(status, 1);
  }
}

// The max pass of Q, K and V in one launch: grid = (ceil(N / 256), B*hq +
// 2*B*hkv); rows of blockIdx.y in [0, B*hq) are Q heads, then K heads
// (centred with the mean key when CENTERK), then V heads (never transformed).
template <typename IT, int D, bool ROT, bool CENTERK>
__global__ __launch_bounds__(kPrepThreads) void k_amax_qkv(const RowsJob q, const RowsJob k, const RowsJob v,
                                                           int32_t B, int32_t N, const float* __restrict__ mu,
                                                           const int8_t* __restrict__ signs,
                                                           int32_t* __restrict__ status) {
  const int y = blockIdx.y, nq = B * q.H, nk = B * k.H;
  if (y < nq) amax_rows<IT, D, ROT, false>(q, y, blockIdx.x, N, nullptr, signs, status);
  else if (y < nq + nk) amax_rows<IT, D, ROT, CENTERK>(k, y - nq, blockIdx.x, N, mu, signs, status);
  else amax_rows<IT, D, false, false>(v, y - nq - nk, blockIdx.x, N, nullptr, nullptr, status);
}

// Running maximum over each head's tile maxima (prefix scales), in place.
// Maxima are non-negative binary32 stored as bits, so unsigned order is their
// order.  One thread per head.
__global__ void k_prefix_max(uint32_t* __restrict__ amax, int32_t nheads, int32_t ntile) {
  const int32_t h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= nheads) return;
  uint32_t* a = amax + static_cast<int64_t>(h) * ntile;
  uint32_t m = 0;
  for (int32_t t = 0; t < ntile; ++t) {
    m = max(m, a[t]);
    a[t] = m;
  }
}

// int8 code: round to nearest even (v_rndne_f32), clamp to +-127, two's
// complement byte; four of them packed little-endian.
__device__ __forceinline__ uint32_t i8_code(float x) {
  const float r = __builtin_fminf(127.0f, __builtin_fmaxf(-127.0f, __builtin_rintf(x)));
  return static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu;
}

__device__ __forceinline__ uint32_t i8_pack4(float a, float b, float c, float d) {
  return i8_code(a) | (i8_code(b) << 8) | (i8_code(c) << 16) | (i8_code(d) << 24);
}

// qmax: the largest code magnitude, 448 for E4M3 and 127 for int8 codes.
__device__ __forceinline__ void scales_from_amax(uint32_t abits, bool rotated, float cd, float& inv, float& desc,
                                                 float qmax = 448.0f) {
  const float A = __uint_as_float(abits);
  if (A == 0.0f) { inv = 1.0f; desc = 1.0f; return; }
  inv = qmax / A;
  desc = A / qmax;
  if (rotated) desc = desc * cd;
}

// Quantise the Q or K rows of block (bx, bh) into [B,H,Np,D] codes; rows in
// [N, Np) are written as 0.  Scales per head (ntile == 1) or per 128-token tile
// (desc[bh * ntile + t]).
template <typename IT, int D, bool ROT, bool CENTER>
__device__ __forceinline__ void quant_rows(const RowsJob& j, int bh, int bx, int32_t N, int32_t Np,
                                           const float* __restrict__ mu_all, const int8_t* __restrict__ signs,
                                           float cd, int32_t int8) {
  const float qmax = int8 ? 127.0f : 448.0f;
  constexpr int L = D / 8;
  constexpr int RPI = kPrepThreads / L;
  const IT* __restrict__ x = static_cast<const IT*>(j.x);
  const int64_t sb = j.sb, sh = j.sh, sn = j.sn;
  const int32_t H = j.H, ntile = j.ntile;
  const uint32_t* __restrict__ amax = j.amax;
  float* __restrict__ desc_out = j.desc;
  uint8_t* __restrict__ codes = j.codes;
  const int b = bh / H, h = bh % H;
  const int li = threadIdx.x % L, rl = threadIdx.x / L;
  const float* mu = CENTER ? mu_all + static_cast<int64_t>(bh) * D : nullptr;
  const int n_begin = bx * kRowsPerBlock;
  // scales of the block's rows [0, 128) and [128, 256)
  float inv, desc, inv_hi, desc_hi;
  if (ntile == 1) {
    scales_from_amax(amax[bh], ROT, cd, inv, desc, qmax);
    inv_hi = inv;
    desc_hi = desc;
    if (bx == 0 && threadIdx.x == 0) desc_out[bh] = desc;
  } else {
    const int64_t t0 = static_cast<int64_t>(bh) * ntile + 2 * bx;
    const bool has_hi = n_begin + kRowsPerBlock / 2 < Np;   // the block's second tile exists
    scales_from_amax(amax[t0], ROT, cd, inv, desc, qmax);
    scales_from_amax(has_hi ? amax[t0 + 1] : 0u, ROT, cd, inv_hi, desc_hi, qmax);
    if (threadIdx.x == 0) desc_out[t0] = desc;
    if (threadIdx.x == 1 && has_hi) desc_out[t0 + 1] = desc_hi;
  }
  const IT* base = x + b * sb + h * sh + 8 * li;
  uint8_t* out = codes + static_cast<int64_t>(bh) * Np * D + 8 * li;
  // kRowsInFlight rows per lane group per step, loaded before any is
  // transformed (the L lanes of a row share r, so its lane exchanges always run
  // on all of them).
  // Rows past N load row N - 1 instead (no branch around the loads) and are
  // written as zero codes.
  for (int r0 = rl; r0 < kRowsPerBlock; r0 += kRowsInFlight * RPI) {
    float v[kRowsInFlight][8];
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int n = min(n_begin + r0 + u * RPI, N - 1);
      load8<IT>(base + static_cast<int64_t>(n) * sn, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kRowsInFlight; ++u) {
      const int n = n_begin + r0 + u * RPI;
      transform_row<D, ROT, CENTER>(v[u], li, mu, signs);
      uint2 w = make_uint2(0u, 0u);
      if (n < N) {
        const float s = (r0 + u * RPI < kRowsPerBlock / 2) ? inv : inv_hi;
        uint32_t lo = 0, hi = 0;
        if (int8) {
          lo = i8_pack4(v[u][0] * s, v[u][1] * s, v[u][2] * s, v[u][3] * s);
          hi = i8_pack4(v[u][4] * s, v[u][5] * s, v[u][6] * s, v[u][7] * s);
        } else {
          lo = e4m3_pack2<false>(v[u][0] * s, v[u][1] * s, lo);
          lo = e4m3_pack2<true>(v[u][2] * s, v[u][3] * s, lo);
          hi = e4m3_pack2<false>(v[u][4] * s, v[u][5] * s, hi);
          hi = e4m3_pack2<true>(v[u][6] * s, v[u][7] * s, hi);
        }
        w = make_uint2(lo, hi);
      }
      // rows in [N, Np) are written as zero codes
      if (n < Np) *reinterpret_cast<uint2*>(out + static_cast<int64_t>(n) * D) = w;
    }
  }
}

// The quantise pass of Q and K in one launch: grid = (ceil(Np / 256), B*hq +
// B*hkv).  Blocks take row ranges and heads in the reverse of the max pass's
// order (K before Q, last rows first): the rows that pass read last are the
// likeliest still to sit in the memory-side cache.
template <typename IT, int D, bool ROT, bool CENTERK>
__global__ __launch_bounds__(kPrepThreads) void k_quant_qk(const RowsJob q, const RowsJob k, int32_t B, int32_t N,
                                                           int32_t Np, const float* __restrict__ mu,
                                                           const int8_t* __restrict__ signs, float cd, int32_t int8) {
  const int bx = gridDim.x - 1 - blockIdx.x;
  const int y = gridDim.y - 1 - blockIdx.y, nq = B * q.H;
  if (y < nq) quant_rows<IT, D, ROT, false>(q, y, bx, N, Np, nullptr, signs, cd, int8);
  else quant_rows<IT, D, ROT, CENTERK>(k, y - nq, bx, N, Np, mu, signs, cd, int8);
}

// Quantise V (never rotated) into the transposed layout [B,Hkv,D,Np]: one block
// per 128 tokens of one head, staged through LDS so both the reads (rows) and
// the writes (channel rows of 128 tokens) are contiguous.
template <typename IT, int D>
__global__ __launch_bounds__(kPrepThreads) void k_quant_vt(const IT* __restrict__ v, int64_t sb, int64_t sh, int64_t sn,
                                                           int32_t H, int32_t N, int32_t Np,
                                                           const uint32_t* __restrict__ amax,
                                                           float* __restrict__ desc_out, uint8_t* __restrict__ v8t) {
  constexpr int L = D / 8;
  constexpr int RPI = kPrepThreads / L;
  constexpr int TOK = 128;
  constexpr int LDSW = TOK + 16;           // padded row of the channel-major tile
  __shared__ __align__(16) uint8_t tile[D * LDSW];
  // reverse of the max pass's order, as in k_quant_rows
  const int bx = gridDim.x - 1 - blockIdx.x;
  const int bh = gridDim.y - 1 - blockIdx.y, b = bh / H, h = bh % H;
  const int li = threadIdx.x % L, rl = threadIdx.x / L;
  float inv, desc;
  scales_from_amax(amax[bh], false, 1.0f, inv, desc);
  if (bx == 0 && threadIdx.x == 0) desc_out[bh] = desc;
  const IT* base = v + b * sb + h * sh + 8 * li;
  const int n0 = bx * TOK;
  for (int r = rl; r < TOK; r += RPI) {
    const int n = n0 + r;
    uint32_t lo = 0, hi = 0;
    if (n < N) {
      float x[8];
      load8<IT>(base + static_cast<int64_t>(n) * sn, x);
      lo = e4m3_pack2<false>(x[0] * inv, x[1] * inv, lo);
      lo = e4m3_pack2<true>(x[2] * inv, x[3] * inv, lo);
      hi = e4m3_pack2<false>(x[4] * inv, x[5] * inv, hi);
      hi = e4m3_pack2<true>(x[6] * inv, x[7] * inv, hi);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[(8 * li + e) * LDSW + r] = static_cast<uint8_t>(lo >> (8 * e));
      tile[(8 * li + 4 + e) * LDSW + r] = static_cast<uint8_t>(hi >> (8 * e));
    }
  }
  __syncthreads();
  uint8_t* out = v8t + static_cast<int64_t>(bh) * D * Np + n0;
  for (int e = threadIdx.x; e < D * (TOK / 16); e += kPrepThreads) {
    const int c = e / (TOK / 16), j = e % (TOK / 16);
    *reinterpret_cast<uint4*>(out + static_cast<int64_t>(c) * Np + 16 * j) =
        *reinterpret_cast<const uint4*>(tile + c * LDSW + 16 * j);
  }
}

// ------------------------------------------------------------------ launch

template <typename IT, int D>
static hipError_t launch_prepare_t(const PrepareArgs& a, hipStream_t st) {
  const dim3 blk(kPrepThreads);
  const int32_t B = a.B, hq = a.hq, hkv = a.hkv, N = a.N, Np = a.Np;
  const int32_t grp = hq / hkv;
  const IT* q = static_cast<const IT*>(a.q);
  const IT* k = static_cast<const IT*>(a.k);
  const IT* v = static_cast<const IT*>(a.v);
  const int32_t nt = a.ntile;
  const int64_t n_amax = static_cast<int64_t>(B) * (hq * nt + hkv * nt + hkv);
  k_fill2_u32<<<dim3(static_cast<unsigned>((n_amax + 255) / 256)), blk, 0, st>>>(
      a.amax, n_amax, reinterpret_cast<uint32_t*>(a.status));
  uint32_t* amax_q = a.amax;
  uint32_t* amax_k = a.amax + static_cast<int64_t>(B) * hq * nt;
  uint32_t* amax_v = amax_k + static_cast<int64_t>(B) * hkv * nt;
  const float* mu = a.k_mean;
  const int i8 = a.int8 ? 1 : 0;
  // mean key first: the K max pass subtracts it
  if (a.center) {
    constexpr int32_t kChunksPerBlock = 256 / (D / 8);
    k_kmean_partial<IT, D><<<dim3((a.np2 + kChunksPerBlock - 1) / kChunksPerBlock, B * hkv), dim3(256), 0, st>>>(
        k, a.ks[0], a.ks[1], a.ks[2], hkv, a.n_mean, a.np2, a.mean_part);
    k_kmean_final<<<dim3(B * hkv, D / kMeanCh), dim3(kMeanCh * kMeanW), 0, st>>>(a.mean_part, a.np2, a.n_mean, D,
                                                                                  a.k_mean);
  }
  const RowsJob jq{q, a.qs[0], a.qs[1], a.qs[2], hq, nt, amax_q, a.q_desc, a.q8};
  const RowsJob jk{k, a.ks[0], a.ks[1], a.ks[2], hkv, nt, amax_k, a.k_desc, a.k8};
  const RowsJob jv{v, a.vs[0], a.vs[1], a.vs[2], hkv, 1, amax_v, a.v_desc, a.v8t};
  const dim3 g_max((N + kRowsPerBlock - 1) / kRowsPerBlock, B * (hq + 2 * hkv));
  const dim3 g_quant((Np + kRowsPerBlock - 1) / kRowsPerBlock, B * (hq + hkv));
  const int8_t* sg = a.rotate ? a.signs : nullptr;
  if (a.rotate && a.center) {
    k_amax_qkv<IT, D, true, true><<<g_max, blk, 0, st>>>(jq, jk, jv, B, N, mu, sg, a.status);
  } else if (a.rotate) {
    k_amax_qkv<IT, D, true, false><<<g_max, blk, 0, st>>>(jq, jk, jv, B, N, mu, sg, a.status);
  } else if (a.center) {
    k_amax_qkv<IT, D, false, true><<<g_max, blk, 0, st>>>(jq, jk, jv, B, N, mu, sg, a.status);
  } else {
    k_amax_qkv<IT, D, false, false><<<g_max, blk, 0, st>>>(jq, jk, jv, B, N, mu, sg, a.status);
  }
  // Q and K tile maxima are contiguous: one running-max launch covers both
  if (a.prefix) k_prefix_max<<<dim3((B * (hq + hkv) + 255) / 256), blk, 0, st>>>(amax_q, B * (hq + hkv), nt);
  if (a.rotate && a.center) {
    k_quant_qk<IT, D, true, true><<<g_quant, blk, 0, st>>>(jq, jk, B, N, Np, mu, sg, a.cd, i8);
  } else if (a.rotate) {
    k_quant_qk<IT, D, true, false><<<g_quant, blk, 0, st>>>(jq, jk, B, N, Np, mu, sg, a.cd, i8);
  } else if (a.center) {
    k_quant_qk<IT, D, false, true><<<g_quant, blk, 0, st>>>(jq, jk, B, N, Np, mu, sg, a.cd, i8);
  } else {
    k_quant_qk<IT, D, false, false><<<g_quant, blk, 0, st>>>(jq, jk, B, N, Np, mu, sg, a.cd, i8);
  }
  k_quant_vt<IT, D><<<dim3(Np / 128, B * hkv), blk, 0, st>>>(v, a.vs[0], a.vs[1], a.vs[2], hkv, N, Np, amax_v, a.v_desc, a.v8t);
  (void)grp;
  return hipGetLastError();
}

hipError_t launch_prepare(const PrepareArgs& a, hipStream_t st) {
  if (a.bf16) {
    if (a.D == 64) return launch_prepare_t<uint16_t, 64>(a, st);
    return launch_prepare_t<uint16_t, 128>(a, st);
  }
  if (a.D == 64) return launch_prepare_t<float, 64>(a, st);
  return launch_prepare_t<float, 128>(a, st);
}

}  // namespace fp8a
