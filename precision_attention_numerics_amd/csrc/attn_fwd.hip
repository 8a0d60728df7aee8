// FP8 (E4M3FN) attention main loop for gfx950.
//
// Semantics (P-Cast summary, Probleemstelling and Methodologie; attention-
// numerics project page, second section): per query row, an online softmax
// over KV blocks of BC keys visited forward (0 -> N) or reverse (N -> 0); the
// probabilities p are multiplied by the static scale S and cast to E4M3 before
// the P.V product; S and the V descale are divided out in the epilogue.
//
// Mapping onto CDNA4:
//  * One workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns QT tiles of 16 rows.  K (row-major) and V (transposed, token axis
//    contiguous) tiles of BC keys are staged in LDS; the next tile is
//    prefetched into registers while the current one is consumed.
//  * S^T = K Q^T with v_mfma_f32_16x16x128_f8f6f4 (the whole head_dim = 128 in
//    one instruction; head_dim 64 is zero-padded).  The K rows of key tile t
//    are permuted so that accumulator lane group g ends up holding keys
//    [g*BC/4, (g+1)*BC/4) of the block for its query: those bytes, once cast,
//    are exactly the B operand of the P.V instruction (O^T = V^T P^T), so P
//    never goes through LDS.
//  * Workgroups are ordered longest-first (causal) and grouped by head per XCD
//    so the K/V of a head stay in one XCD's L2.
#include "device_common.hpp"
#include "attn.hpp"

namespace fp8a {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

__device__ __forceinline__ v8i lds_read32(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
  v8i r;
  r[0] = static_cast<int>(a.x); r[1] = static_cast<int>(a.y); r[2] = static_cast<int>(a.z); r[3] = static_cast<int>(a.w);
  r[4] = static_cast<int>(b.x); r[5] = static_cast<int>(b.y); r[6] = static_cast<int>(b.z); r[7] = static_cast<int>(b.w);
  return r;
}

__device__ __forceinline__ v8i lds_read16_pad(const uint8_t* p) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  v8i r;
  r[0] = static_cast<int>(a.x); r[1] = static_cast<int>(a.y); r[2] = static_cast<int>(a.z); r[3] = static_cast<int>(a.w);
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

__device__ __forceinline__ v4f mfma_f8(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// p = 2^x in binary32.  v_exp_f32 differs from the correctly rounded 2^x in
// the last place for some x; exhaustive checks over every binary32 x in
// [-150, 2^-8] show that for S = 2^k (k = 0..8) only two such x change an E4M3
// code of S*p, and two other x for S = 448.  Those x are recomputed in
// binary64 and rounded once.
__device__ __forceinline__ float exp2_code_exact(float x, uint32_t bad0, uint32_t bad1) {
  float p = __builtin_amdgcn_exp2f(x);
  const uint32_t xb = __float_as_uint(x);
  if (__builtin_expect((xb == bad0) | (xb == bad1), 0)) p = static_cast<float>(exp2(static_cast<double>(x)));
  return p;
}

template <int D, int BC, int QT, bool CAUSAL, bool POW2, bool DUMP>
__global__ __launch_bounds__(kThreads, 2) void k_attn_fwd(const FwdParams p) {
  constexpr int QROWS = kWaves * QT * 16;
  static_assert(QROWS == 128, "query tile must match the 128-token padding");
  constexpr int T = BC / 16;          // 16-key MFMA tiles per block
  constexpr int KPL = BC / 4;         // keys per accumulator lane group
  constexpr int KST = D + 16;         // padded LDS row of the K tile
  constexpr int VST = BC + 16;        // padded LDS row of the V^T tile
  constexpr int KLD = BC * D / 16 / kThreads;  // 16-byte loads per thread
  constexpr int VLD = D * BC / 16 / kThreads;
  static_assert(KLD >= 1 && VLD >= 1, "tile too small for the workgroup");
  __shared__ __align__(16) uint8_t klds[BC * KST];
  __shared__ __align__(16) uint8_t vlds[D * VST];

  // ---- workgroup -> (batch*head, query tile)
  const int BH = p.B * p.hq;
  const int nqt = p.n_qtiles;
  int bh, qtile;
  {
    const int wg = blockIdx.x;
    if (BH % 8 == 0) {
      const int xcd = wg % 8, w = wg / 8, hpx = BH / 8;
      bh = xcd * hpx + w % hpx;
      qtile = nqt - 1 - w / hpx;
    } else {
      bh = wg % BH;
      qtile = nqt - 1 - wg / BH;
    }
  }
  const int b = bh / p.hq, h = bh % p.hq;
  const int g = h / (p.hq / p.hkv);
  const int bg = b * p.hkv + g;
  const int N = p.N, Np = p.Np;
  const int q0 = qtile * QROWS;
  const float c = (p.q_desc[bh] * p.k_desc[bg]) * p.ls2;
  const float vdesc = p.v_desc[bg];

  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int n16 = lane & 15, lg = lane >> 4;

  // ---- Q operand (B of S^T = K Q^T): query row n16, channels [32 lg, 32 lg + 32)
  v8i qop[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int i = q0 + wv * QT * 16 + qt * 16 + n16;
    if (32 * lg < D) {
      const uint8_t* src = p.q8 + (static_cast<int64_t>(bh) * Np + i) * D + 32 * lg;
      const uint4 a = *reinterpret_cast<const uint4*>(src);
      const uint4 bb = *reinterpret_cast<const uint4*>(src + 16);
      qop[qt][0] = a.x; qop[qt][1] = a.y; qop[qt][2] = a.z; qop[qt][3] = a.w;
      qop[qt][4] = bb.x; qop[qt][5] = bb.y; qop[qt][6] = bb.z; qop[qt][7] = bb.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[qt][e] = 0;
    }
  }

  // ---- running state per query tile (replicated over the 4 lane groups)
  float ms[QT], mcp[QT], lsum[QT];
  uint32_t zeros[QT];
  v4f oacc[QT][D / 16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    ms[qt] = -INFINITY; mcp[qt] = -INFINITY; lsum[qt] = 0.0f; zeros[qt] = 0;
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) oacc[qt][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int q_last = min(q0 + QROWS - 1, N - 1);
  const int jmax = CAUSAL ? q_last / BC : (N - 1) / BC;
  const uint8_t* kbase = p.k8 + static_cast<int64_t>(bg) * Np * D;
  const uint8_t* vbase = p.v8t + static_cast<int64_t>(bg) * D * Np;

  uint4 kreg[KLD], vreg[VLD];
  auto gload = [&](int blk) {
    const int j0 = blk * BC;
#pragma unroll
    for (int e = 0; e < KLD; ++e) {
      const int idx = tid + e * kThreads;
      const int row = idx / (D / 16), col = idx % (D / 16);
      kreg[e] = *reinterpret_cast<const uint4*>(kbase + static_cast<int64_t>(j0 + row) * D + 16 * col);
    }
#pragma unroll
    for (int e = 0; e < VLD; ++e) {
      const int idx = tid + e * kThreads;
      const int row = idx / (BC / 16), col = idx % (BC / 16);
      vreg[e] = *reinterpret_cast<const uint4*>(vbase + static_cast<int64_t>(row) * Np + j0 + 16 * col);
    }
  };
  gload(p.kv_order ? jmax : 0);

  for (int it = 0; it <= jmax; ++it) {
    const int blk = p.kv_order ? jmax - it : it;
    const int j0 = blk * BC;
    __syncthreads();  // the previous tile has been consumed by every wave
#pragma unroll
    for (int e = 0; e < KLD; ++e) {
      const int idx = tid + e * kThreads;
      const int row = idx / (D / 16), col = idx % (D / 16);
      *reinterpret_cast<uint4*>(klds + row * KST + 16 * col) = kreg[e];
    }
#pragma unroll
    for (int e = 0; e < VLD; ++e) {
      const int idx = tid + e * kThreads;
      const int row = idx / (BC / 16), col = idx % (BC / 16);
      *reinterpret_cast<uint4*>(vlds + row * VST + 16 * col) = vreg[e];
    }
    __syncthreads();
    if (it < jmax) gload(p.kv_order ? jmax - it - 1 : it + 1);

    // ---- S^T tiles: key tile t, A row m = n16 -> key KPL*(m/4) + 4t + m%4
    v4f sacc[QT][T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int jj = KPL * (n16 >> 2) + 4 * t + (n16 & 3);
      v8i a;
      if (32 * lg < D) {
        a = lds_read32(klds + jj * KST + 32 * lg);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = 0;
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) sacc[qt][t] = mfma_f8(a, qop[qt], v4f{0.0f, 0.0f, 0.0f, 0.0f});
    }

    // ---- online softmax and the P cast; lane holds query n16, keys j0 + KPL*lg + 4t + r
    v8i pop[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int i = q0 + wv * QT * 16 + qt * 16 + n16;
      float bm = -INFINITY;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + KPL * lg + 4 * t + r;
          const bool vis = (j < N) && (!CAUSAL || j <= i);
          bm = __builtin_fmaxf(bm, vis ? sacc[qt][t][r] : -INFINITY);
        }
      bm = __builtin_fmaxf(bm, wave_xor(bm, 16));
      bm = __builtin_fmaxf(bm, wave_xor(bm, 32));
      const float mnew = __builtin_fmaxf(ms[qt], bm);
      const float mc = (mnew == -INFINITY) ? 0.0f : mnew * c;
      const float alpha = (ms[qt] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mcp[qt] - mc);
      lsum[qt] = lsum[qt] * alpha;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct) oacc[qt][ct] *= alpha;
      }
      ms[qt] = mnew;
      mcp[qt] = mc;
      const float nmc = -mc;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + KPL * lg + 4 * t + r;
          const bool vis = (j < N) && (!CAUSAL || j <= i);
          const float x = __builtin_fmaf(sacc[qt][t][r], c, nmc);
          const float pv = exp2_code_exact(x, p.bad0, p.bad1);
          pr[r] = vis ? pv : 0.0f;
          lsum[qt] += pr[r];
        }
        uint32_t w = 0;
        if constexpr (POW2) {
          w = e4m3_pack2_pow2<false>(pr[0], pr[1], p.inv_S, w);
          w = e4m3_pack2_pow2<true>(pr[2], pr[3], p.inv_S, w);
        } else {
          w = e4m3_pack2<false>(pr[0] * p.S, pr[1] * p.S, w);
          w = e4m3_pack2<true>(pr[2] * p.S, pr[3] * p.S, w);
        }
        pop[qt][t] = static_cast<int>(w);
        if constexpr (DUMP) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = j0 + KPL * lg + 4 * t + r;
            const bool vis = (j < N) && (!CAUSAL || j <= i);
            const uint32_t code = (w >> (8 * r)) & 0xFFu;
            if (vis && j >= p.k_sink && code == 0u) ++zeros[qt];
            if (p.p_dump && i < N && j < N)
              p.p_dump[(static_cast<int64_t>(bh) * N + i) * N + j] = static_cast<uint8_t>(code);
          }
        }
      }
#pragma unroll
      for (int t = T; t < 8; ++t) pop[qt][t] = 0;
    }

    // ---- O^T += V^T P^T: A row = channel 16 ct + n16, keys [KPL lg, KPL lg + KPL)
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      const uint8_t* src = vlds + (16 * ct + n16) * VST + KPL * lg;
      const v8i a = (KPL == 32) ? lds_read32(src) : lds_read16_pad(src);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) oacc[qt][ct] = mfma_f8(a, pop[qt], oacc[qt][ct]);
    }
  }

  // ---- epilogue: out = acc * (v_desc / (S * l)); lane holds channels 16 ct + 4 lg + r
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int i = q0 + wv * QT * 16 + qt * 16 + n16;
    float l = lsum[qt];
    l += wave_xor(l, 16);
    l += wave_xor(l, 32);
    const float f = vdesc / (p.S * l);
    if (i < N) {
      float* orow = p.out + (static_cast<int64_t>(bh) * N + i) * D;
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) {
        const v4f o = oacc[qt][ct] * f;
        *reinterpret_cast<float4*>(orow + 16 * ct + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (p.lse && lg == 0) p.lse[static_cast<int64_t>(bh) * N + i] = (mcp[qt] + __log2f(l)) * 0.69314718055994531f;
    }
    if constexpr (DUMP) {
      uint32_t z = zeros[qt];
      z += __shfl_xor(z, 16, kWave);
      z += __shfl_xor(z, 32, kWave);
      if (p.row_zeros && lg == 0 && i < N) p.row_zeros[static_cast<int64_t>(bh) * N + i] = z;
    }
  }
}

// -------------------------------------------------------- P-cast-only path
// Binary32 Q/K/V, only P cast (the "kernel-faithful" simulation of the P-Cast
// summary, Bijdragen item 4).  One thread per query row; the score is an
// ordered binary32 fma chain over the channels.  Not a throughput path.
template <int D, bool POW2>
__global__ __launch_bounds__(64) void k_attn_pcast_f32(const PcastParams p) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int N = p.N;
  if (row >= static_cast<int64_t>(p.B) * p.hq * N) return;
  const int i = static_cast<int>(row % N);
  const int bh = static_cast<int>(row / N);
  const int b = bh / p.hq, h = bh % p.hq, g = h / (p.hq / p.hkv), bg = b * p.hkv + g;
  const float* qr = p.q + (static_cast<int64_t>(bh) * N + i) * D;
  const float* K = p.k + static_cast<int64_t>(bg) * N * D;
  const float* V = p.v + static_cast<int64_t>(bg) * N * D;
  float q[D], acc[D];
#pragma unroll
  for (int cc = 0; cc < D; ++cc) { q[cc] = qr[cc]; acc[cc] = 0.0f; }
  const float c = p.ls2;
  const int nvis = p.causal ? i + 1 : N;
  const int BC = p.block_n;
  const int J = (nvis - 1) / BC;
  float ms = -INFINITY, mcp = -INFINITY, l = 0.0f;
  uint32_t zeros = 0;
  for (int t = 0; t <= J; ++t) {
    const int blk = p.kv_order ? J - t : t;
    const int ja = blk * BC, jb = min((blk + 1) * BC, nvis);
    float bm = -INFINITY;
    for (int j = ja; j < jb; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int cc = 0; cc < D; ++cc) s = __builtin_fmaf(q[cc], K[static_cast<int64_t>(j) * D + cc], s);
      bm = __builtin_fmaxf(bm, s);
    }
    const float mnew = __builtin_fmaxf(ms, bm);
    const float mc = mnew * c;
    const float alpha = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mcp - mc);
    l = l * alpha;
#pragma unroll
    for (int cc = 0; cc < D; ++cc) acc[cc] = acc[cc] * alpha;
    for (int j = ja; j < jb; ++j) {
      float s = 0.0f;
#pragma unroll
      for (int cc = 0; cc < D; ++cc) s = __builtin_fmaf(q[cc], K[static_cast<int64_t>(j) * D + cc], s);
      const float x = __builtin_fmaf(s, c, -mc);
      const float pv = exp2_code_exact(x, p.bad0, p.bad1);
      uint32_t w;
      if constexpr (POW2) w = e4m3_pack2_pow2<false>(pv, 0.0f, p.inv_S, 0u);
      else w = e4m3_pack2<false>(pv * p.S, 0.0f, 0u);
      const uint32_t code = w & 0xFFu;
      const float pt = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(code), 0);
      l = l + pv;
      if (j >= p.k_sink && code == 0u) ++zeros;
      if (p.p_dump) p.p_dump[(static_cast<int64_t>(bh) * N + i) * N + j] = static_cast<uint8_t>(code);
#pragma unroll
      for (int cc = 0; cc < D; ++cc) acc[cc] = acc[cc] + pt * V[static_cast<int64_t>(j) * D + cc];
    }
    ms = mnew;
    mcp = mc;
  }
  const float f = 1.0f / (p.S * l);
  float* o = p.out + (static_cast<int64_t>(bh) * N + i) * D;
#pragma unroll
  for (int cc = 0; cc < D; ++cc) o[cc] = acc[cc] * f;
  if (p.lse) p.lse[static_cast<int64_t>(bh) * N + i] = (mcp + __log2f(l)) * 0.69314718055994531f;
  if (p.row_zeros) p.row_zeros[static_cast<int64_t>(bh) * N + i] = zeros;
}

// ------------------------------------------------------------------ launch

template <int D, int BC, bool CAUSAL, bool POW2, bool DUMP>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.B * p.hq * p.n_qtiles));
  k_attn_fwd<D, BC, 2, CAUSAL, POW2, DUMP><<<grid, dim3(kThreads), 0, st>>>(p);
  return hipGetLastError();
}

template <int D, int BC>
static hipError_t launch_fwd_d(const FwdParams& p, bool causal, bool pow2, bool dump, hipStream_t st) {
  if (causal) {
    if (pow2) return dump ? launch_fwd_t<D, BC, true, true, true>(p, st) : launch_fwd_t<D, BC, true, true, false>(p, st);
    return dump ? launch_fwd_t<D, BC, true, false, true>(p, st) : launch_fwd_t<D, BC, true, false, false>(p, st);
  }
  if (pow2) return dump ? launch_fwd_t<D, BC, false, true, true>(p, st) : launch_fwd_t<D, BC, false, true, false>(p, st);
  return dump ? launch_fwd_t<D, BC, false, false, true>(p, st) : launch_fwd_t<D, BC, false, false, false>(p, st);
}

hipError_t launch_fwd(const FwdParams& p, int D, int BC, bool causal, bool pow2, bool dump, hipStream_t st) {
  if (D == 64) return BC == 64 ? launch_fwd_d<64, 64>(p, causal, pow2, dump, st) : launch_fwd_d<64, 128>(p, causal, pow2, dump, st);
  return BC == 64 ? launch_fwd_d<128, 64>(p, causal, pow2, dump, st) : launch_fwd_d<128, 128>(p, causal, pow2, dump, st);
}

hipError_t launch_pcast_f32(const PcastParams& p, int D, bool pow2, hipStream_t st) {
  const int64_t rows = static_cast<int64_t>(p.B) * p.hq * p.N;
  const dim3 grid(static_cast<unsigned>((rows + 63) / 64));
  if (D == 64) {
    if (pow2) k_attn_pcast_f32<64, true><<<grid, dim3(64), 0, st>>>(p);
    else k_attn_pcast_f32<64, false><<<grid, dim3(64), 0, st>>>(p);
  } else {
    if (pow2) k_attn_pcast_f32<128, true><<<grid, dim3(64), 0, st>>>(p);
    else k_attn_pcast_f32<128, false><<<grid, dim3(64), 0, st>>>(p);
  }
  return hipGetLastError();
}

}  // namespace fp8a
