// Device helpers shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8a {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Output rows are written once and never read back by the kernel: streaming
// (non-temporal) stores keep them from displacing K/V lines in the caches.
// Used where a wave's store covers 64 contiguous bytes of a row; with 32-byte
// pieces (the head_dim 64 kernel) they measured slower than plain stores.
__device__ __forceinline__ void store4_stream(float* dst, float a, float b, float c, float d) {
  __builtin_nontemporal_store(v4f{a, b, c, d}, reinterpret_cast<v4f*>(dst));
}
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Largest finite E4M3FN magnitude.
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// E4M3FN code of x with round-to-nearest-even and saturation.  The hardware
// convert rounds to nearest-even but returns NaN above 464, so the operand is
// clamped to +-448 first (values in (448, 464] round to 448 either way).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old) {
  a = __builtin_fminf(__builtin_fmaxf(a, -kE4M3Max), kE4M3Max);
  b = __builtin_fminf(__builtin_fmaxf(b, -kE4M3Max), kE4M3Max);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HI));
}

// Two codes of E4M3(a * 2^k), E4M3(b * 2^k) packed into the low or high half
// of `old`: the scaled convert divides by its scale operand (here 2^-k)
// without an intermediate rounding.  Callers guarantee |a|, |b| * 2^k < 464.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pack2_pow2(float a, float b, float inv_scale, uint32_t old) {
  union { uint32_t u; v2s s; } cv;
  cv.u = old;
  cv.s = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(cv.s, a, b, inv_scale, HI);
  return cv.u;
}

__device__ __forceinline__ float e4m3_decode_byte(uint32_t word, int byte_sel) {
  switch (byte_sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), 3);
  }
}

template <typename T>
__device__ __forceinline__ T wave_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

}  // namespace fp8a
