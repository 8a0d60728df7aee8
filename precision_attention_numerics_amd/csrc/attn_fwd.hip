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
//    owns two tiles of 16 rows.  K (row-major) and V (transposed, token axis
//    contiguous) tiles of BC keys are staged in LDS by buffer-to-LDS DMA into
//    double buffers, the next block's tiles in flight while the current ones
//    are read.
//  * S^T = K Q^T with v_mfma_f32_16x16x128_f8f6f4 (the whole head_dim = 128 in
//    one instruction; head_dim 64 is zero-padded here); int8 Q/K codes use two
//    16x16x64 int8 instructions per key tile.  The K rows of key tile t are
//    permuted so that accumulator lane group g ends up holding keys
//    [g*BC/4, (g+1)*BC/4) of the block for its query: those bytes, once cast,
//    are exactly the B operand of the P.V instruction (O^T = V^T P^T), so P
//    never goes through LDS.
//  * k_attn_fwd_pipe (head_dim 128, blocks of 128: the timed forward) runs the
//    same per-tile arithmetic as k_attn_fwd in a software pipeline across
//    blocks: each step issues Q.K^T of the next block between the chunks of
//    this block's exp/cast half, then P.V of this block between the chunks of
//    the next block's max/fma half.  k_attn_fwd, block by block, serves the
//    P~ dump, row checksum and underflow-count forms and blocks of 64.
//  * Workgroups are ordered longest-first (causal) and grouped by head per XCD
//    so the K/V of a head stay in one XCD's L2.
#include <type_traits>

#include "attn_common.hpp"
#include "attn.hpp"

namespace fp8a {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

__device__ __forceinline__ v8i lds_read16_pad(const uint8_t* p) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  v8i r;
  r[0] = static_cast<int>(a[0]); r[1] = static_cast<int>(a[1]); r[2] = static_cast<int>(a[2]); r[3] = static_cast<int>(a[3]);
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

__device__ __forceinline__ v4f mfma_f8(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

typedef int v4i __attribute__((ext_vector_type(4)));

// 16x16x64 int8 with exact int32 accumulation: A lane l = row l%16, bytes =
// k 16*(l/16) + [0, 16); B likewise by column; D as the 16x16 forms.
__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4i lds_read16_i(const uint8_t* p) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  return v4i{static_cast<int>(a[0]), static_cast<int>(a[1]), static_cast<int>(a[2]), static_cast<int>(a[3])};
}

// p = 2^x in binary32.  v_exp_f32 differs from the correctly rounded 2^x in
// the last place for some x; exhaustive checks over every binary32 x in
// [-150, 2^-8] show that for S = 2^k (k = 0..8) only two such x change an E4M3
// code of S*p, and two other x for S = 448.  Here (the binary32 P-cast path)
// those x are recomputed in binary64 and rounded once; the FP8 main loop
// instead rewrites them to a neighbouring pattern whose v_exp_f32 result is
// that correctly rounded value.
__device__ __forceinline__ float exp2_code_exact(float x, uint32_t bad0, uint32_t bad1) {
  float p = __builtin_amdgcn_exp2f(x);
  const uint32_t xb = __float_as_uint(x);
  if (__builtin_expect((xb == bad0) | (xb == bad1), 0)) p = static_cast<float>(exp2(static_cast<double>(x)));
  return p;
}

// LDS tiles use the unit swizzle swz of attn_common.hpp.  K rows are permuted
// in LDS: key jj of the block (jj = KPL*q + 4t + b, the
// row of MFMA tile t that lane n16 = 4q + b holds) sits at LDS row
// 16t + n16.  V^T rows (channels) are stored in order.  Tiles are filled by
// direct buffer->LDS DMA: one wave instruction writes 64 consecutive units,
// each lane fetching the global chunk that belongs in its unit.

// key (within the block) stored at LDS row r of the K tile
template <int BC>
__device__ __forceinline__ int key_of_row(int r) {
  return (BC / 4) * ((r & 15) >> 2) + 4 * (r >> 4) + (r & 3);
}

// Tile fills by buffer_load ... lds: wave wv issues instructions w = wv*KI + e
// (K) and w = wv*VI + e (V^T); instruction w writes units [64w, 64w + 64) of
// the tile, lane l the unit 64w + l.  The lane's global offsets within a block
// are fixed per (wave, e) and computed once (fill_offsets); each block adds a
// uniform base (fill_issue).  The offset arrays are the kernel's locals
// (KI and VI entries); after inlining they stay in registers.
template <int D, int BC, int WAVES = kWaves>
__device__ __forceinline__ void fill_offsets(int wv, int lane, int Np, uint32_t* koff, uint32_t* voff) {
  constexpr int UK = D / 16, UV = BC / 16;
  constexpr int KI = BC * UK / 64 / WAVES, VI = D * UV / 64 / WAVES;
#pragma unroll
  for (int e = 0; e < KI; ++e) {
    const int u = 64 * (wv * KI + e) + lane;
    const int r = u / UK;
    koff[e] = static_cast<uint32_t>(key_of_row<BC>(r) * D + 16 * ((u % UK) ^ swz<UK>(r & 15)));
  }
#pragma unroll
  for (int e = 0; e < VI; ++e) {
    const int u = 64 * (wv * VI + e) + lane;
    const int r = u / UV;
    voff[e] = static_cast<uint32_t>(r * Np + 16 * ((u % UV) ^ swz<UV>(r & 15)));
  }
}

// K tile [BC rows][D bytes] and V^T tile [D rows][BC bytes] of block blk;
// kbase / vbase are the head's K8 and V8t (head_bytes each).  (The buffer
// resources are built here, from the uniform base pointers.)
template <int D, int BC>
__device__ __forceinline__ void fill_issue(const uint8_t* kbase, const uint8_t* vbase, uint32_t head_bytes, int blk,
                                           int wv, const uint32_t* koff, const uint32_t* voff, uint8_t* kbuf,
                                           uint8_t* vbuf) {
  constexpr int UK = D / 16, UV = BC / 16;
  constexpr int KI = BC * UK / 64 / kWaves, VI = D * UV / 64 / kWaves;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(kbase, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(vbase, head_bytes);
  const uint32_t kblk = static_cast<uint32_t>(blk) * (BC * D);
  const uint32_t vblk = static_cast<uint32_t>(blk) * BC;
#pragma unroll
  for (int e = 0; e < KI; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(kbuf + 1024 * (wv * KI + e)), 16, koff[e], kblk, 0, 0);
#pragma unroll
  for (int e = 0; e < VI; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(vbuf + 1024 * (wv * VI + e)), 16, voff[e], vblk, 0, 0);
}

// Maximum over the four lane groups that hold one query column (lanes l,
// l^16, l^32, l^48): each swap step exchanges halves of a register pair, and
// the max of the pair is the xor-partner combination.
__device__ __forceinline__ float column_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmax_nan(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nan(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float column_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// P = 2^x for the tile's x (in place in s), sum of this lane's P into lpart,
// E4M3 codes of S*P packed in the operand order of the P.V instruction.
// Invisible keys hold x = -inf (NaN when c = 0); MASK maps both to p = 0.
template <int T, bool MASK, bool CAUSAL, bool POW2, bool DUMP>
__device__ __attribute__((always_inline)) inline v8i cast_tile(const v4f (&x)[T], float& lpart, uint32_t& zpart,
                                                               uint64_t& hpart, const int i, const int jb,
                                                               const int N, const FwdParams& p,
                                                               uint8_t* __restrict__ dump_row) {
  v8i out;
  float part[T];
  uint32_t zeros = 0;
  uint64_t hsum = 0;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[r] = __builtin_amdgcn_exp2f(MASK ? __builtin_fmaxf(x[t][r], -INFINITY) : x[t][r]);
    }
    part[t] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
    // both halves of w are written below, so its initial bits are never
    // used; seeding it from a value that is dead by then avoids a move
    uint32_t w = __float_as_uint(pr[0]);
    if constexpr (POW2) {
      w = e4m3_pack2_pow2<false>(pr[0], pr[1], p.inv_S, w);
      w = e4m3_pack2_pow2<true>(pr[2], pr[3], p.inv_S, w);
    } else {
      w = e4m3_pack2<false>(pr[0] * p.S, pr[1] * p.S, w);
      w = e4m3_pack2<true>(pr[2] * p.S, pr[3] * p.S, w);
    }
    out[t] = static_cast<int>(w);
    if constexpr (DUMP) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = jb + 4 * t + r;
        const bool vis = (j < N) && (!CAUSAL || j <= i);
        const uint32_t code = (w >> (8 * r)) & 0xFFu;
        if (vis && j >= p.k_sink && code == 0u) ++zeros;
        if (code != 0u) hsum += static_cast<uint64_t>(code) * key_weight(j);
        if (dump_row && i < N && j < N) dump_row[j] = static_cast<uint8_t>(code);
      }
    }
  }
  // row sum of this lane's keys, pairwise (the order only affects l's rounding)
#pragma unroll
  for (int w = T / 2; w > 0; w >>= 1)
#pragma unroll
    for (int t = 0; t < w; ++t) part[t] = part[t] + part[t + w];
  lpart = part[0];
  zpart = zeros;
  hpart = hsum;
#pragma unroll
  for (int t = T; t < 8; ++t) out[t] = 0;
  return out;
}

// Online-softmax update of one 16-row query tile for one block, first part:
// masking, block max, running max, alpha, l and O rescaled, and s replaced by
// x = fma(s, c, -RN32(m*c)).  The lane holds query i and keys jb + 4t + r
// (t < T, r < 4).  Returns the wave-uniform decision whether some x of the
// tile can be one of the listed exponents (softmax_screen).
template <int D, int T, bool MASK, bool CAUSAL, bool TILES>
__device__ __attribute__((always_inline)) inline bool softmax_front(v4f (&s)[T], const float c, float& ms, float& mcp,
                                                                    float& lsum, v4f (&oacc)[D / 16], const int i,
                                                                    const int jb, const int N, const FwdParams& p) {
  // key jb + k is visible iff k < lim (k = 4t + r): one compare per key
  const int lim = min(N, CAUSAL ? i + 1 : N) - jb;
  if constexpr (MASK) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[t][r] = (4 * t + r < lim) ? s[t][r] : -INFINITY;
  }
  float m4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m4[r] = s[0][r];
#pragma unroll
    for (int t = 1; t < T; ++t) m4[r] = fmax_nan(m4[r], s[t][r]);
  }
  const float bm = column_max(fmax_nan(fmax_nan(m4[0], m4[1]), fmax_nan(m4[2], m4[3])));
  // ms: running max of the raw scores; mcp: running max in scaled units
  // RN32(m * c), 0 while no key has been visible.  With per-tile scales c
  // changes from block to block, so mcp is carried as the max of RN32(bm * c)
  // over the blocks; with one c per row both forms are the same value
  // (rounding is monotone).
  const float mnew = fmax_nan(ms, bm);
  float mc;
  if constexpr (TILES) {
    const float bmc = (bm == -INFINITY) ? -INFINITY : bm * c;
    mc = (mnew == -INFINITY) ? 0.0f : ((ms == -INFINITY) ? bmc : fmax_nan(mcp, bmc));
  } else {
    mc = (mnew == -INFINITY) ? 0.0f : mnew * c;
  }
  const float alpha = (ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mcp - mc);
  lsum = lsum * alpha;
  // Unconditional: alpha is exactly 1 when the max did not move, and a
  // branch here makes the compiler keep two copies of O.
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) oacc[ct] *= alpha;
  ms = mnew;
  mcp = mc;
  const float nmc = -mc;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) s[t][r] = __builtin_fmaf(s[t][r], c, nmc);
  // Every x of this row is at most fma(bm, c, -mc) (the fma is monotone in s
  // for c > 0): the listed x can only occur in blocks holding keys near the
  // running max, and only there is each x screened.
  return __any(__builtin_fmaf(bm, c, nmc) >= p.xcheck);
}

// The exp screen of one tile's x: (xb ^ B0) & (xb ^ B1) is zero whenever xb
// is B0 or B1 (and for the few patterns that agree with B0 or B1 bit by bit,
// which only cost the exact comparison below): one bit-op per x and a min
// over pairs, all in vector registers.  A wave holding a zero replaces each
// listed x by its neighbour pattern, whose v_exp_f32 result is the correctly
// rounded 2^x of the listed x.
template <int T>
__device__ __attribute__((always_inline)) inline void softmax_screen(v4f (&s)[T], const FwdParams& p) {
  uint32_t acc = 0xFFFFFFFFu;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t xb = __float_as_uint(s[t][r]);
      acc = min(acc, (xb ^ p.bad0) & (xb ^ p.bad1));
    }
  if (__builtin_expect(__any(acc == 0u), 0)) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t xb = __float_as_uint(s[t][r]);
        xb = (xb == p.bad0) ? p.rep0 : xb;
        xb = (xb == p.bad1) ? p.rep1 : xb;
        s[t][r] = __uint_as_float(xb);
      }
  }
}

// Last part: p = 2^x, l += sum p, and the E4M3 codes of S*p as the B operand
// of the P.V instruction.
template <int T, bool MASK, bool CAUSAL, bool POW2, bool DUMP>
__device__ __attribute__((always_inline)) inline v8i softmax_back(const v4f (&x)[T], float& lsum, const int i,
                                                                  const int jb, const int N, const FwdParams& p,
                                                                  uint32_t& zeros, uint64_t& hash,
                                                                  uint8_t* __restrict__ dump_row) {
  float lpart;
  uint32_t zpart;
  uint64_t hpart;
  const v8i out = cast_tile<T, MASK, CAUSAL, POW2, DUMP>(x, lpart, zpart, hpart, i, jb, N, p, dump_row);
  lsum = lsum + lpart;
  zeros += zpart;
  hash += hpart;
  return out;
}

// Online-softmax update of one 16-row query tile for one block and the P
// cast (the three parts above in order); s holds the scores on entry and x on
// exit.
template <int D, int T, bool MASK, bool CAUSAL, bool POW2, bool DUMP, bool TILES>
__device__ __attribute__((always_inline)) inline v8i softmax_tile(v4f (&s)[T], const float c, float& ms, float& mcp,
                                                                  float& lsum, v4f (&oacc)[D / 16], const int i,
                                                                  const int jb, const int N, const FwdParams& p,
                                                                  uint32_t& zeros, uint64_t& hash,
                                                                  uint8_t* __restrict__ dump_row) {
  if (softmax_front<D, T, MASK, CAUSAL, TILES>(s, c, ms, mcp, lsum, oacc, i, jb, N, p)) softmax_screen<T>(s, p);
  return softmax_back<T, MASK, CAUSAL, POW2, DUMP>(s, lsum, i, jb, N, p, zeros, hash, dump_row);
}

template <int D, int BC, int QT, bool CAUSAL, bool POW2, bool DUMP, bool TILES, bool I8>
__global__ __launch_bounds__(kThreads, 2) void k_attn_fwd(const FwdParams p) {
  constexpr int QROWS = kWaves * QT * 16;
  static_assert(QROWS == 128, "query tile must match the 128-token padding");
  constexpr int T = BC / 16;          // 16-key MFMA tiles per block
  constexpr int KPL = BC / 4;         // keys per accumulator lane group
  constexpr int UK = D / 16, UV = BC / 16;   // 16-byte units per LDS row of the K and V^T tiles
  constexpr int KBYTES = BC * D;
  static_assert(BC * UK % (64 * kWaves) == 0 && D * UV % (64 * kWaves) == 0, "tile must split into wave DMAs");
  __shared__ __align__(16) uint8_t klds[2 * KBYTES];
  __shared__ __align__(16) uint8_t vlds[2 * KBYTES];

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
  // base-2 logit factor (q_desc * k_desc) * RN32(scale * log2 e): per head, or
  // per block from the query tile's and the block's key tile's descales
  const float qd = TILES ? p.q_desc[static_cast<int64_t>(bh) * nqt + qtile] : p.q_desc[bh];
  const float c_head = TILES ? 0.0f : (qd * p.k_desc[bg]) * p.ls2;
  const float vdesc = p.v_desc[bg];

  // wv is wave-uniform; readfirstlane lets the compiler keep it (and every
  // per-block decision made from it) in scalar registers.
  const int tid = threadIdx.x, lane = tid % kWave, wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n16 = lane & 15, lg = lane >> 4;
  const bool has_k = 32 * lg < D;     // lane groups past head_dim feed zeros (head_dim 64)

  // ---- Q operand (B of S^T = K Q^T): query row n16, channels [32 lg, 32 lg + 32)
  v8i qop[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int i = q0 + wv * QT * 16 + qt * 16 + n16;
    if (has_k) {
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
  // int8 Q operand: query row n16, channels 64 h + [16 lg, 16 lg + 16)
  constexpr int NH8 = D / 64;
  v4i qop8[I8 ? QT : 1][NH8];
  if constexpr (I8) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int h8 = 0; h8 < NH8; ++h8) {
        const int i = q0 + wv * QT * 16 + qt * 16 + n16;
        const uint4 a = *reinterpret_cast<const uint4*>(p.q8 + (static_cast<int64_t>(bh) * Np + i) * D + 64 * h8 + 16 * lg);
        qop8[qt][h8] = v4i{static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w)};
      }
  }

  // ---- per-lane LDS read offsets (tile t / channel tile ct add constants)
  // K: A row m = n16 of tile t -> key KPL*(m/4) + 4t + m%4 = LDS row 16t + n16,
  // channels [32 lg, 32 lg + 32)
  const int kofs0 = 16 * (n16 * UK + ((2 * lg) ^ swz<UK>(n16)));
  const int kofs1 = 16 * (n16 * UK + ((2 * lg + 1) ^ swz<UK>(n16)));
  // int8 K operand: channels 64 h + [16 lg, 16 lg + 16) = unit 4 h + lg
  int kofs8[NH8];
#pragma unroll
  for (int h8 = 0; h8 < NH8; ++h8) kofs8[h8] = 16 * (n16 * UK + ((4 * h8 + lg) ^ swz<UK>(n16)));
  // V^T: A row = channel 16 ct + n16, keys [KPL lg, KPL lg + KPL)
  const int vofs0 = 16 * (n16 * UV + ((KPL == 32 ? 2 * lg : lg) ^ swz<UV>(n16)));
  const int vofs1 = 16 * (n16 * UV + ((2 * lg + 1) ^ swz<UV>(n16)));

  // ---- running state per query tile (replicated over the 4 lane groups)
  float ms[QT], mcp[QT], lsum[QT];
  uint32_t zeros[QT];
  uint64_t hash[QT];
  v4f oacc[QT][D / 16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    ms[qt] = -INFINITY; mcp[qt] = -INFINITY; lsum[qt] = 0.0f; zeros[qt] = 0; hash[qt] = 0;
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) oacc[qt][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int q_last = min(q0 + QROWS - 1, N - 1);
  const int jmax = CAUSAL ? q_last / BC : (N - 1) / BC;
  const uint8_t* kbase = p.k8 + static_cast<int64_t>(bg) * Np * D;
  const uint8_t* vbase = p.v8t + static_cast<int64_t>(bg) * D * Np;
  const uint32_t head_bytes = static_cast<uint32_t>(Np) * D;
  const int wrow0 = q0 + wv * QT * 16;
  uint32_t koff[BC * D / 16 / 64 / kWaves], voff[D * BC / 16 / 64 / kWaves];
  fill_offsets<D, BC>(wv, lane, Np, koff, voff);

  fill_issue<D, BC>(kbase, vbase, head_bytes, p.kv_order ? jmax : 0, wv, koff, voff, klds, vlds);

  for (int it = 0; it <= jmax; ++it) {
    const int blk = p.kv_order ? jmax - it : it;
    const int j0 = blk * BC;
    const int cur = (it & 1) * KBYTES;
    // This wave's DMA into the current buffers has landed; the barrier makes
    // every wave's share visible and ends all reads of the other buffers.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (it < jmax)
      fill_issue<D, BC>(kbase, vbase, head_bytes, p.kv_order ? jmax - it - 1 : it + 1, wv, koff, voff,
                        klds + (KBYTES - cur),
                        vlds + (KBYTES - cur));
    const uint8_t* kt = klds + cur;
    const uint8_t* vt = vlds + cur;
    const float c = TILES ? (qd * p.k_desc[static_cast<int64_t>(bg) * nqt + (j0 >> 7)]) * p.ls2 : c_head;

    // ---- S^T = K Q^T for both 16-row query tiles from one LDS read of each K
    // tile, then per query tile the online softmax and the P cast; the lane
    // ends up holding query n16 and keys j0 + KPL*lg + 4t + r.
    const bool need_mask = (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > wrow0);
    v8i pop[QT];
    v4f sall[QT][T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if constexpr (I8) {
        // exact int32 scores, converted once (|s| <= 127^2 * 128 < 2^24)
        v4i a8[NH8];
#pragma unroll
        for (int h8 = 0; h8 < NH8; ++h8) a8[h8] = lds_read16_i(kt + kofs8[h8] + t * 256 * UK);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          v4i acc = v4i{0, 0, 0, 0};
#pragma unroll
          for (int h8 = 0; h8 < NH8; ++h8) acc = mfma_i8(a8[h8], qop8[qt][h8], acc);
          sall[qt][t] = v4f{static_cast<float>(acc[0]), static_cast<float>(acc[1]), static_cast<float>(acc[2]),
                            static_cast<float>(acc[3])};
        }
      } else {
        v8i a;
        if (has_k) {
          a = lds_read_pair(kt + kofs0 + t * 256 * UK, kt + kofs1 + t * 256 * UK);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = 0;
        }
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) sall[qt][t] = mfma_f8(a, qop[qt], v4f{0.0f, 0.0f, 0.0f, 0.0f});
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      v4f (&sacc)[T] = sall[qt];
      const int i = wrow0 + qt * 16 + n16;
      uint8_t* drow = nullptr;
      if constexpr (DUMP) drow = p.p_dump ? p.p_dump + (static_cast<int64_t>(bh) * N + i) * N : nullptr;
      if (DUMP || need_mask)
        pop[qt] = softmax_tile<D, T, true, CAUSAL, POW2, DUMP, TILES>(sacc, c, ms[qt], mcp[qt], lsum[qt], oacc[qt], i,
                                                              j0 + KPL * lg, N, p, zeros[qt], hash[qt], drow);
      else
        pop[qt] = softmax_tile<D, T, false, CAUSAL, POW2, DUMP, TILES>(sacc, c, ms[qt], mcp[qt], lsum[qt], oacc[qt], i,
                                                               j0 + KPL * lg, N, p, zeros[qt], hash[qt], drow);
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      v8i a;
      if constexpr (KPL == 32) {
        a = lds_read_pair(vt + vofs0 + ct * 256 * UV, vt + vofs1 + ct * 256 * UV);
      } else {
        a = lds_read16_pad(vt + vofs0 + ct * 256 * UV);
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) oacc[qt][ct] = mfma_f8(a, pop[qt], oacc[qt][ct]);
    }
  }

  // ---- epilogue: out = acc * (v_desc / (S * l)); lane holds channels 16 ct + 4 lg + r
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int i = q0 + wv * QT * 16 + qt * 16 + n16;
    const float l = column_sum(lsum[qt]);
    const float f = vdesc / (p.S * l);
    if (i < N) {
      float* orow = p.out + (static_cast<int64_t>(bh) * N + i) * D;
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) {
        const v4f o = oacc[qt][ct] * f;
        store4_stream(orow + 16 * ct + 4 * lg, o[0], o[1], o[2], o[3]);
      }
      if (p.lse && lg == 0) p.lse[static_cast<int64_t>(bh) * N + i] = (mcp[qt] + __log2f(l)) * 0.69314718055994531f;
    }
    if constexpr (DUMP) {
      uint32_t z = zeros[qt];
      z += __shfl_xor(z, 16, kWave);
      z += __shfl_xor(z, 32, kWave);
      if (p.row_zeros && lg == 0 && i < N) p.row_zeros[static_cast<int64_t>(bh) * N + i] = z;
      unsigned long long hs = hash[qt];
      hs += __shfl_xor(hs, 16, kWave);
      hs += __shfl_xor(hs, 32, kWave);
      if (p.row_hash && lg == 0 && i < N) p.row_hash[static_cast<int64_t>(bh) * N + i] = hs;
    }
  }
}

// ------------------------------------------------ software-pipelined loop
// The same computation as k_attn_fwd for head_dim 128, KV blocks of 128 keys,
// E4M3 scores and no per-key outputs (P dump, checksums, underflow counts).
// Each query tile goes through the same operations on the same values in the
// same order as there, so the outputs are bit-identical; only the issue order
// changes.  The loop is pipelined across blocks: step n issues
//   run 1: Q.K^T of block n+1 for both 16-row tiles (one LDS read of each K
//          tile serves both), each pair of matrix instructions followed by the
//          exp / row-sum / E4M3-cast work of block n on the same key tile
//          (the scores' registers are consumed as the new scores arrive);
//   run 2: P.V of block n for both tiles (one LDS read of each V^T tile),
//          each O tile rescaled by block n's alpha just before its matrix
//          instruction, followed by the max / fma work of block n+1.
// The vector work issues while the matrix unit executes the wave's own
// preceding instructions.  LDS holds K of block n+1 and V^T of block n.
namespace pipe {

constexpr int D = 128, BC = 128, T = 8, UK = 8, UV = 8, KBYTES = BC * D;
// DMA instructions per wave for one K or V^T tile, with W waves per workgroup
template <int W>
constexpr int KI = BC * UK / 64 / W;
template <int W>
constexpr int VI = D * UV / 64 / W;

template <int W>
__device__ __forceinline__ void fill_k(const __amdgpu_buffer_rsrc_t krs, int blk, int wv, const uint32_t* koff,
                                       uint8_t* kbuf) {
  const uint32_t kblk = static_cast<uint32_t>(blk) * (BC * D);
#pragma unroll
  for (int e = 0; e < KI<W>; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)(kbuf + 1024 * (wv * KI<W> + e)), 16, koff[e], kblk, 0,
                                             0);
}

template <int W>
__device__ __forceinline__ void fill_v(const __amdgpu_buffer_rsrc_t vrs, int blk, int wv, const uint32_t* voff,
                                       uint8_t* vbuf) {
  const uint32_t vblk = static_cast<uint32_t>(blk) * BC;
#pragma unroll
  for (int e = 0; e < VI<W>; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)(vbuf + 1024 * (wv * VI<W> + e)), 16, voff[e], vblk, 0,
                                             0);
}

// Per-tile running state.
struct Tile {
  v8i q;            // Q operand (B of S^T = K Q^T)
  v4f s[T];         // scores, then x
  v8i pop;          // E4M3 codes of S*p, B operand of the P.V instruction
  v4f o[D / 16];    // O^T accumulator
  float ms, mcp, lsum;
  float alpha;      // rescale factor of O for the block whose P.V comes next
  int i;            // query row of the lane
};

// Q operand of query row i (channels [32 lg, 32 lg + 32)) and empty state.
__device__ __forceinline__ void init_tile(Tile& X, const uint8_t* q8, int bh, int Np, int i, int lg) {
  X.i = i;
  const uint8_t* src = q8 + (static_cast<int64_t>(bh) * Np + i) * D + 32 * lg;
  const uint4 a = *reinterpret_cast<const uint4*>(src);
  const uint4 bb = *reinterpret_cast<const uint4*>(src + 16);
  X.q[0] = a.x; X.q[1] = a.y; X.q[2] = a.z; X.q[3] = a.w;
  X.q[4] = bb.x; X.q[5] = bb.y; X.q[6] = bb.z; X.q[7] = bb.w;
  X.ms = -INFINITY; X.mcp = -INFINITY; X.lsum = 0.0f; X.alpha = 0.0f;
#pragma unroll
  for (int t = 0; t < T; ++t) X.pop[t] = 0;
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) X.o[ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
}

// S^T of key tile t (operand a, read from LDS) for the NT query tiles of the
// wave.  E4M3 codes: one 16x16x128 instruction per query tile.  Int8 codes:
// two 16x16x64 instructions; each operand's 32 channels per lane (channels
// [32 lg, 32 lg + 32)) are split into the same two 16-byte halves on both
// sides, so the pair sums every channel once, and the int32 sum is exact
// (|s| <= 127^2 * 128 < 2^24).  It is kept as its bit pattern in s until the
// softmax front converts it (front_step, I8).
template <bool I8, int NT>
__device__ __forceinline__ void qk_tiles(const v8i a, Tile (&X)[NT], int t) {
  if constexpr (I8) {
    const v4i alo = v4i{a[0], a[1], a[2], a[3]}, ahi = v4i{a[4], a[5], a[6], a[7]};
    v4i acc[NT];
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k] = mfma_i8(alo, v4i{X[k].q[0], X[k].q[1], X[k].q[2], X[k].q[3]}, v4i{0, 0, 0, 0});
#pragma unroll
    for (int k = 0; k < NT; ++k) acc[k] = mfma_i8(ahi, v4i{X[k].q[4], X[k].q[5], X[k].q[6], X[k].q[7]}, acc[k]);
#pragma unroll
    for (int k = 0; k < NT; ++k) X[k].s[t] = __builtin_bit_cast(v4f, acc[k]);
  } else {
#pragma unroll
    for (int k = 0; k < NT; ++k) X[k].s[t] = mfma_f8(a, X[k].q, v4f{0.0f, 0.0f, 0.0f, 0.0f});
  }
}

// Int8 scores of key tile t, held as int32 bit patterns, to binary32 (exact).
__device__ __attribute__((always_inline)) inline void scores_to_f32(Tile& X, int t) {
  const v4i v = __builtin_bit_cast(v4i, X.s[t]);
  X.s[t] = v4f{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
               static_cast<float>(v[3])};
}

// Epilogue of one tile: out = acc * (v_desc / (S * l)); the lane holds
// channels 16 ct + 4 lg + r of its query row.
__device__ __forceinline__ void store_tile(const Tile& X, const FwdParams& p, int bh, int N, float vdesc, int lg) {
  const int i = X.i;
  const float l = column_sum(X.lsum);
  const float f = vdesc / (p.S * l);
  if (i < N) {
    float* orow = p.out + (static_cast<int64_t>(bh) * N + i) * D;
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      const v4f o = X.o[ct] * f;
      store4_stream(orow + 16 * ct + 4 * lg, o[0], o[1], o[2], o[3]);
    }
    if (p.lse && lg == 0) p.lse[static_cast<int64_t>(bh) * N + i] = (X.mcp + __log2f(l)) * 0.69314718055994531f;
  }
}

// Compile-time loop: f(integral_constant<int, I>) for I = B..E-1.
template <int I, int E, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  if constexpr (I < E) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, E>(f);
  }
}

// Keeps a value computed at this point of the instruction stream: an empty
// register constraint, so code motion before instruction selection cannot sink
// the computation past the scheduling fence that follows its chunk.  (Device
// pass only; the host pass never sees AMDGPU register constraints.)
template <typename V>
__device__ __attribute__((always_inline)) inline void pin(V& v) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(v));
#endif
}

// State of one tile's softmax between its chunks.
struct Front {
  float m[4];       // per-lane maxima over the key tiles, per accumulator register r
  float v;          // lane maximum, then the block max bm of the row
  float mnew, mc, nmc;
  float alpha;      // the block's alpha (applied to O before its P.V)
  bool gate;
};

// The first part of the online-softmax update (softmax_front) cut into eight
// chunks, each issued after one pair of matrix instructions.  Same operations
// on the same values as softmax_front (the max is exact in any order), so the
// results are bit-identical; O is rescaled separately (rescale_o), right
// before the block's P.V instruction of each O tile.
//   0-2: block max over the key tiles;  3-4: across the lane groups, new
//   running max;  5: alpha, l rescaled;  4-7: x = fma(s, c, -mc);  7: gate of
//   the exp screen.
// FIRST: the first block visited.  Every row has a visible key in it (the
// diagonal block holds key 128*qtile, block 0 holds key 0), so after it the
// running max is finite and the -inf cases of mc and alpha cannot occur.
// I8: the scores arrive as int32 bit patterns and are converted chunk by chunk
// before the max reads them (all at once where the block is masked).
template <int K, bool MASK, bool CAUSAL, bool TILES, bool FIRST = true, bool I8 = false>
__device__ __attribute__((always_inline)) inline void front_step(Front& f, Tile& X, const float c, const int jb,
                                                                 const int N, const FwdParams& p) {
  if constexpr (I8) {
    if constexpr (K == 0) {
      constexpr int last = MASK ? T : 3;
#pragma unroll
      for (int t = 0; t < last; ++t) scores_to_f32(X, t);
    } else if constexpr (!MASK && K == 1) {
      scores_to_f32(X, 3);
      scores_to_f32(X, 4);
    } else if constexpr (!MASK && K == 2) {
      scores_to_f32(X, 5);
      scores_to_f32(X, 6);
    } else if constexpr (!MASK && K == 3) {
      scores_to_f32(X, 7);
    }
  }
  if constexpr (K == 0) {
    if constexpr (MASK) {
      const int lim = min(N, CAUSAL ? X.i + 1 : N) - jb;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) X.s[t][r] = (4 * t + r < lim) ? X.s[t][r] : -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f.m[r] = fmax_nan(fmax_nan(X.s[0][r], X.s[1][r]), X.s[2][r]);
      pin(f.m[r]);
    }
  } else if constexpr (K == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f.m[r] = fmax_nan(fmax_nan(f.m[r], X.s[3][r]), X.s[4][r]);
      pin(f.m[r]);
    }
  } else if constexpr (K == 2) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f.m[r] = fmax_nan(fmax_nan(f.m[r], X.s[5][r]), X.s[6][r]);
      pin(f.m[r]);
    }
  } else if constexpr (K == 3) {
#pragma unroll
    for (int r = 0; r < 4; ++r) f.m[r] = fmax_nan(f.m[r], X.s[7][r]);
    const float v = fmax_nan(fmax_nan(f.m[0], f.m[1]), fmax_nan(f.m[2], f.m[3]));
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    f.v = fmax_nan(__uint_as_float(a[0]), __uint_as_float(a[1]));
    pin(f.v);
  } else if constexpr (K == 4) {
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(f.v), __float_as_uint(f.v), false, false);
    const float bm = fmax_nan(__uint_as_float(b[0]), __uint_as_float(b[1]));
    f.v = bm;
    f.mnew = fmax_nan(X.ms, bm);
    if constexpr (!FIRST) {
      f.mc = TILES ? fmax_nan(X.mcp, bm * c) : f.mnew * c;
    } else if constexpr (TILES) {
      const float bmc = (bm == -INFINITY) ? -INFINITY : bm * c;
      f.mc = (f.mnew == -INFINITY) ? 0.0f : ((X.ms == -INFINITY) ? bmc : fmax_nan(X.mcp, bmc));
    } else {
      f.mc = (f.mnew == -INFINITY) ? 0.0f : f.mnew * c;
    }
    f.nmc = -f.mc;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) X.s[t][r] = __builtin_fmaf(X.s[t][r], c, f.nmc);
      pin(X.s[t]);
    }
  } else if constexpr (K == 5) {
    f.alpha = (FIRST && X.ms == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(X.mcp - f.mc);
    X.lsum = X.lsum * f.alpha;
    X.ms = f.mnew;
    X.mcp = f.mc;
    pin(X.lsum);
    pin(f.alpha);
#pragma unroll
    for (int t = 2; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) X.s[t][r] = __builtin_fmaf(X.s[t][r], c, f.nmc);
      pin(X.s[t]);
    }
  } else if constexpr (K == 6) {
#pragma unroll
    for (int t = 4; t < 6; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) X.s[t][r] = __builtin_fmaf(X.s[t][r], c, f.nmc);
      pin(X.s[t]);
    }
  } else {
#pragma unroll
    for (int t = 6; t < 8; ++t) {
#pragma unroll
      for (int r = 0; r < 4; ++r) X.s[t][r] = __builtin_fmaf(X.s[t][r], c, f.nmc);
      pin(X.s[t]);
    }
    f.gate = __any(__builtin_fmaf(f.v, c, f.nmc) >= p.xcheck);
  }
}

// O tile ct of one query tile rescaled by the alpha of the block whose P.V
// comes next (exactly 1 when the max did not move, 0 before the first block).
__device__ __attribute__((always_inline)) inline void rescale_o(Tile& X, int ct) {
  X.o[ct] *= X.alpha;
  pin(X.o[ct]);
}

// The whole O of a tile rescaled, skipped when alpha is 1 in every row of the
// tile (no row's max moved: multiplying by 1 changes no bit).
__device__ __attribute__((always_inline)) inline void rescale_o_if_moved(Tile& X) {
  if (__any(X.alpha != 1.0f)) {
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) X.o[ct] *= X.alpha;
  }
}

// The last part (softmax_back) cut into eight chunks: chunk t takes p = 2^x
// and the codes of key tile t; the lane's row sum is added in cast_tile's
// pairwise order.
template <int K, bool MASK, bool POW2>
__device__ __attribute__((always_inline)) inline void back_step(float (&part)[T], Tile& X, const FwdParams& p) {
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(MASK ? __builtin_fmaxf(X.s[K][r], -INFINITY) : X.s[K][r]);
  part[K] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
  // both halves of w are written below; its initial bits are the previous
  // block's codes of this key tile (dead by now: that P.V has been issued), so
  // the loop keeps the codes in one register and no copy is needed
  uint32_t w = static_cast<uint32_t>(X.pop[K]);
  if constexpr (POW2) {
    w = e4m3_pack2_pow2<false>(pr[0], pr[1], p.inv_S, w);
    w = e4m3_pack2_pow2<true>(pr[2], pr[3], p.inv_S, w);
  } else {
    w = e4m3_pack2<false>(pr[0] * p.S, pr[1] * p.S, w);
    w = e4m3_pack2<true>(pr[2] * p.S, pr[3] * p.S, w);
  }
  pin(w);
  X.pop[K] = static_cast<int>(w);
  if constexpr (K >= 4) part[K - 4] = part[K - 4] + part[K];
  pin(part[K >= 4 ? K - 4 : K]);
  if constexpr (K == 7) {
    part[0] = part[0] + part[2];
    part[1] = part[1] + part[3];
    part[0] = part[0] + part[1];
    X.lsum = X.lsum + part[0];
    pin(X.lsum);
  }
}

}  // namespace pipe

// NT query tiles of 16 rows per wave and W = 8 / NT waves: a workgroup covers
// one 128-row query tile either way.  With NT = 2 two waves share a SIMD (256
// registers each) and each K/V operand read from LDS feeds two matrix
// instructions; with NT = 1 four waves share a SIMD (128 registers each), so
// more waves interleave their vector work, for twice the LDS reads per row.
// I8: Q and K hold int8 codes (exact integer scores on the 16x16x64 int8
// instruction, qk_tiles); P and V stay E4M3.
template <bool CAUSAL, bool POW2, bool TILES, int NT, bool I8>
__global__ __launch_bounds__(64 * 8 / NT, 4 / NT) void k_attn_fwd_pipe(const FwdParams p) {
  using namespace pipe;
  constexpr int W = 8 / NT;
  constexpr int QROWS = 128;
  constexpr int KPL = BC / 4;
  __shared__ __align__(16) uint8_t klds[2 * KBYTES];
  __shared__ __align__(16) uint8_t vlds[2 * KBYTES];

  // ---- workgroup -> (batch*head, query tile), as k_attn_fwd
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
  const float qd = TILES ? p.q_desc[static_cast<int64_t>(bh) * nqt + qtile] : p.q_desc[bh];
  const float c_head = TILES ? 0.0f : (qd * p.k_desc[bg]) * p.ls2;
  const float vdesc = p.v_desc[bg];

  const int tid = threadIdx.x, lane = tid % kWave, wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n16 = lane & 15, lg = lane >> 4;
  const int wrow0 = q0 + wv * 16 * NT;

  Tile X[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) init_tile(X[k], p.q8, bh, Np, wrow0 + 16 * k + n16, lg);
  const int kofs0 = 16 * (n16 * UK + ((2 * lg) ^ swz<UK>(n16)));
  const int kofs1 = 16 * (n16 * UK + ((2 * lg + 1) ^ swz<UK>(n16)));
  const int vofs0 = 16 * (n16 * UV + ((2 * lg) ^ swz<UV>(n16)));
  const int vofs1 = 16 * (n16 * UV + ((2 * lg + 1) ^ swz<UV>(n16)));

  const int q_last = min(q0 + QROWS - 1, N - 1);
  const int J = CAUSAL ? q_last / BC : (N - 1) / BC;
  const uint32_t head_bytes = static_cast<uint32_t>(Np) * D;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(p.k8 + static_cast<int64_t>(bg) * Np * D, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(p.v8t + static_cast<int64_t>(bg) * D * Np, head_bytes);
  uint32_t koff[KI<W>], voff[VI<W>];
  fill_offsets<D, BC, W>(wv, lane, Np, koff, voff);

  // block visited at step it, its logit factor and whether the wave must mask it
  auto blk_of = [&](int it) { return p.kv_order ? J - it : it; };
  auto c_of = [&](int blk) {
    return TILES ? (qd * p.k_desc[static_cast<int64_t>(bg) * nqt + blk]) * p.ls2 : c_head;
  };
  auto masked = [&](int blk) {
    const int j0 = blk * BC;
    return (j0 + BC > N) || (CAUSAL && j0 + BC - 1 > wrow0);
  };
  using yes = std::true_type;
  using no = std::false_type;
  // Non-interleaved forms (first and last step).
  auto front_all = [&](Tile& X, Front& f, int blk, auto maskc) __attribute__((always_inline)) {
    constexpr bool M = decltype(maskc)::value;
    const float c = c_of(blk);
    const int jb = blk * BC + KPL * lg;
    static_for<0, T>([&](auto kc) __attribute__((always_inline)) {
      front_step<decltype(kc)::value, M, CAUSAL, TILES, true, I8>(f, X, c, jb, N, p);
    });
    X.alpha = f.alpha;
    if (f.gate) softmax_screen<T>(X.s, p);
  };
  auto back_all = [&](Tile& X, auto maskc) __attribute__((always_inline)) {
    constexpr bool M = decltype(maskc)::value;
    float part[T];
    static_for<0, T>([&](auto kc) __attribute__((always_inline)) {
      back_step<decltype(kc)::value, M, POW2>(part, X, p);
    });
  };
  auto front_first = [&](int blk) __attribute__((always_inline)) {
    Front f[NT];
    if (masked(blk)) {
#pragma unroll
      for (int k = 0; k < NT; ++k) front_all(X[k], f[k], blk, yes{});
    } else {
#pragma unroll
      for (int k = 0; k < NT; ++k) front_all(X[k], f[k], blk, no{});
    }
  };

  // ---- first block: K tile, Q.K^T of both tiles (one K read serves both),
  // the front of both softmaxes
  fill_k<W>(krs, blk_of(0), wv, koff, klds);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (J >= 1) fill_k<W>(krs, blk_of(1), wv, koff, klds + KBYTES);
  fill_v<W>(vrs, blk_of(0), wv, voff, vlds);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    qk_tiles<I8>(lds_read_pair(klds + kofs0 + t * 256 * UK, klds + kofs1 + t * 256 * UK), X, t);
  }
  front_first(blk_of(0));

  // ---- step it = 0 .. J-1: back of block it's softmax under Q.K^T of block
  // it+1, then P.V of block it under the front of block it+1's softmax.  MB /
  // MF: block it / it+1 is the one block that needs masking (the diagonal
  // block, or the block holding key N-1); it is always first or last in the
  // visit order, so only the first or the last step instantiates a masked form.
  auto step = [&](int it, auto mask_back, auto mask_front) __attribute__((always_inline)) {
    constexpr bool MB = decltype(mask_back)::value, MF = decltype(mask_front)::value;
    // K of block it+1 and V^T of block it have landed (every wave's share,
    // after the barrier), and every wave is done with the buffers refilled here
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (it + 2 <= J) fill_k<W>(krs, blk_of(it + 2), wv, koff, klds + (it & 1) * KBYTES);
    fill_v<W>(vrs, blk_of(it + 1), wv, voff, vlds + ((it + 1) & 1) * KBYTES);
    // O by block it's alpha before its P.V below (the previous P.V has completed)
#pragma unroll
    for (int k = 0; k < NT; ++k) rescale_o_if_moved(X[k]);
    const uint8_t* kt = klds + ((it + 1) & 1) * KBYTES;
    const uint8_t* vt = vlds + (it & 1) * KBYTES;
    const int bn = blk_of(it + 1);
    const float cn = c_of(bn);
    const int jbn = bn * BC + KPL * lg;
    // Pairs n = 0..15 of matrix instructions, both tiles sharing operand n:
    //   0-7  Q.K^T of key tile n for block it+1, after the back chunk n of
    //        block it's softmax (which frees the x registers the scores land in)
    //   8-15 P.V of V^T tile n-8 for block it (O tile rescaled first), then the
    //        front chunk n-8 of block it+1's softmax
    // Operand n is read from LDS two pairs ahead into ops[n % 3]; a scheduling
    // fence keeps each pair with its vector chunk.
    auto read_op = [&](auto nc) __attribute__((always_inline)) {
      constexpr int n = decltype(nc)::value;
      if constexpr (n < 8) return lds_read_pair(kt + kofs0 + n * 256 * UK, kt + kofs1 + n * 256 * UK);
      else return lds_read_pair(vt + vofs0 + (n - 8) * 256 * UV, vt + vofs1 + (n - 8) * 256 * UV);
    };
    v8i ops[3];
    Front f[NT];
    float part[NT][T];
    ops[0] = read_op(std::integral_constant<int, 0>{});
    ops[1] = read_op(std::integral_constant<int, 1>{});
    static_for<0, 16>([&](auto nc) __attribute__((always_inline)) {
      constexpr int n = decltype(nc)::value;
      constexpr int j = n % 8;
      if constexpr (n + 2 < 16) ops[(n + 2) % 3] = read_op(std::integral_constant<int, n + 2>{});
      if constexpr (n < 8) {
#pragma unroll
        for (int k = 0; k < NT; ++k) back_step<j, MB, POW2>(part[k], X[k], p);
        qk_tiles<I8>(ops[n % 3], X, j);
      } else {
#pragma unroll
        for (int k = 0; k < NT; ++k) X[k].o[j] = mfma_f8(ops[n % 3], X[k].pop, X[k].o[j]);
#pragma unroll
        for (int k = 0; k < NT; ++k) front_step<j, MF, CAUSAL, TILES, false, I8>(f[k], X[k], cn, jbn, N, p);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int k = 0; k < NT; ++k) X[k].alpha = f[k].alpha;
#pragma unroll
    for (int k = 0; k < NT; ++k)
      if (f[k].gate) softmax_screen<T>(X[k].s, p);
  };
  const bool first_masked = masked(blk_of(0));
  const bool last_masked = J >= 1 && masked(blk_of(J));
  int it = 0;
  if (J >= 1 && first_masked) {
    step(0, yes{}, no{});
    it = 1;
  }
  const int fast_end = last_masked ? J - 2 : J - 1;
  for (; it <= fast_end; ++it) step(it, no{}, no{});
  if (last_masked && it == J - 1) step(J - 1, no{}, yes{});

  // ---- last block: back of its softmax, P.V of both tiles
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (masked(blk_of(J))) {
#pragma unroll
    for (int k = 0; k < NT; ++k) back_all(X[k], yes{});
  } else {
#pragma unroll
    for (int k = 0; k < NT; ++k) back_all(X[k], no{});
  }
  {
    const uint8_t* vt = vlds + (J & 1) * KBYTES;
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct) {
      const v8i a = lds_read_pair(vt + vofs0 + ct * 256 * UV, vt + vofs1 + ct * 256 * UV);
#pragma unroll
      for (int k = 0; k < NT; ++k) rescale_o(X[k], ct);
#pragma unroll
      for (int k = 0; k < NT; ++k) X[k].o[ct] = mfma_f8(a, X[k].pop, X[k].o[ct]);
    }
  }

  // ---- epilogue
#pragma unroll
  for (int k = 0; k < NT; ++k) store_tile(X[k], p, bh, N, vdesc, lg);
}

// -------------------------------------------------------- P-cast-only path
// Binary32 Q/K/V, only P cast (the P-Cast summary's simulation that follows
// the kernel step by step, Bijdragen item 4).  One thread per query row; the score is an
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
  uint64_t hash = 0;
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
      if (code != 0u) hash += static_cast<uint64_t>(code) * key_weight(j);
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
  if (p.row_hash) p.row_hash[static_cast<int64_t>(bh) * N + i] = hash;
}

// ------------------------------------------------------------------ launch

// Query tiles per wave of the pipelined kernel: two (two waves per SIMD).  One
// tile per wave (four waves per SIMD, 128 registers each) passes the same
// parity tests but measured 4% slower on the 32k workload: the doubled LDS
// operand reads and per-step work per row outweigh the extra waves.
constexpr int kPipeTiles = 2;

template <int D, int BC, bool CAUSAL, bool POW2, bool DUMP>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(p.B * p.hq * p.n_qtiles));
  if constexpr (D == 128 && BC == 128 && !DUMP) {
    constexpr int NT = kPipeTiles;
    const dim3 block(64 * 8 / NT);
    if (p.int8) k_attn_fwd_pipe<CAUSAL, POW2, false, NT, true><<<grid, block, 0, st>>>(p);
    else if (p.tiles) k_attn_fwd_pipe<CAUSAL, POW2, true, NT, false><<<grid, block, 0, st>>>(p);
    else k_attn_fwd_pipe<CAUSAL, POW2, false, NT, false><<<grid, block, 0, st>>>(p);
    return hipGetLastError();
  }
  if (p.tiles) k_attn_fwd<D, BC, 2, CAUSAL, POW2, DUMP, true, false><<<grid, dim3(kThreads), 0, st>>>(p);
  else if (p.int8) k_attn_fwd<D, BC, 2, CAUSAL, POW2, DUMP, false, true><<<grid, dim3(kThreads), 0, st>>>(p);
  else k_attn_fwd<D, BC, 2, CAUSAL, POW2, DUMP, false, false><<<grid, dim3(kThreads), 0, st>>>(p);
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
