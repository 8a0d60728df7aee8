// Device helpers shared by the attention main-loop kernels (16x16 and 32x32
// matrix-instruction forms).
#pragma once
#include "device_common.hpp"

namespace fp8a {

// 16-byte register type (a clang vector, so private arrays of it stay in
// registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS tiles are stored in 16-byte units; unit u of LDS row r sits at
// position u ^ swz(r mod 16) of its row.  Every operand read has the same
// shape: the 16 lanes of a lane group read LDS rows 16*tile + n16, so the
// swizzle depends on n16 alone and each tile is read at a constant offset from
// one per-lane base.  For 128-byte rows the swizzle (n0^n3, n1, n2) was chosen
// by measuring ds_read_b128 throughput on gfx950 (full rate, like a linear
// read); for 64-byte rows no 2-bit XOR swizzle reaches full rate and
// (n0^n3, n1^n2) is among the best measured.
template <int U>
__device__ __forceinline__ int swz(int n) {
  if constexpr (U == 8) return ((n ^ (n >> 3)) & 1) | (n & 6);
  else return ((n ^ (n >> 3)) & 1) | ((((n >> 1) ^ (n >> 2)) & 1) << 1);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over one head's bytes (raw buffer: stride 0, byte offsets;
// loads past num_records return zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

__device__ __forceinline__ v8i lds_read_pair(const uint8_t* p0, const uint8_t* p1) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p0);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p1);
  v8i r;
  r[0] = static_cast<int>(a[0]); r[1] = static_cast<int>(a[1]); r[2] = static_cast<int>(a[2]); r[3] = static_cast<int>(a[3]);
  r[4] = static_cast<int>(b[0]); r[5] = static_cast<int>(b[1]); r[6] = static_cast<int>(b[2]); r[7] = static_cast<int>(b[3]);
  return r;
}

// Weight of key j in the P~ row checksum: splitmix64's (j+1)-th output from
// seed 0 (Steele, Lea and Flood, OOPSLA 2014), made odd so that every code
// change moves the sum.
__device__ __forceinline__ uint64_t key_weight(int j) {
  uint64_t z = static_cast<uint64_t>(j + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (z ^ (z >> 31)) | 1ull;
}

// Maximum that propagates NaN (v_maximum3_f32 on gfx950; unlike fmaxf it
// needs no quieting of its inputs).  Scores are finite or -inf here.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

}  // namespace fp8a
