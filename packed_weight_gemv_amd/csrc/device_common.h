// Device helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pwg {
namespace dev {

constexpr int kWave = 64;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dot4(unsigned a, unsigned b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// ---------------------------------------------------------------------------
// int8-table activation limbs for the VALU projection (v_dot4_i32_i8), one
// exponent per 16-element chunk: X = rint(h * 2^(38 - e)) with max|h| < 2^e
// over the chunk (|X| <= 2^38), written as kI8Limbs balanced base-256 digits
// in [-128, 127].  The rounding of h is at most 2^(e - 39) per element.  For
// each 16-element chunk the LDS holds kI8Limbs * 4 dwords: dword 4 l + g =
// digit l of elements 4g .. 4g + 3 (byte i = element 4g + i), matching the
// byte order of the int8 table row; the chunk exponents (38 - e) follow the
// limb planes as ints.
// ---------------------------------------------------------------------------
constexpr int kI8Limbs = 5;
constexpr int kI8FixedBits = 38;
constexpr int kI8ChunkDwords = 4 * kI8Limbs;

// Maximum over the 4 consecutive lanes 4q..4q+3 (one chunk's groups).
__device__ __forceinline__ float max4(float m) {
  m = fmaxf(m, __shfl_xor(m, 1, kWave));
  return fmaxf(m, __shfl_xor(m, 2, kWave));
}

// Group g of four elements (lane-consecutive groups 4c .. 4c + 3 form chunk
// c and must be converted by active lanes together).
__device__ __forceinline__ void i8_convert_group(const float4 v, int g, unsigned* lds, int* lds_e) {
  const float m = max4(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  const int e = m > 0.f ? __builtin_amdgcn_frexp_expf(m) : 0;  // m < 2^e
  const int E = kI8FixedBits - e;
  const float hv[4] = {v.x, v.y, v.z, v.w};
  unsigned dw[kI8Limbs];
#pragma unroll
  for (int l = 0; l < kI8Limbs; ++l) dw[l] = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // |h * 2^E| < 2^38 is an exact float32; its rounding converts exactly
    long long X = static_cast<long long>(rintf(ldexpf(hv[i], E)));
#pragma unroll
    for (int l = 0; l < kI8Limbs; ++l) {
      const int d = l < kI8Limbs - 1 ? static_cast<int>(((X + 128) & 255) - 128) : static_cast<int>(X);
      X = (X - d) >> 8;
      dw[l] |= (static_cast<unsigned>(d) & 255u) << (8 * i);
    }
  }
  unsigned* dst = lds + (g >> 2) * kI8ChunkDwords + (g & 3);
#pragma unroll
  for (int l = 0; l < kI8Limbs; ++l) dst[4 * l] = dw[l];
  if ((g & 3) == 0) lds_e[g >> 2] = E;
}

// Converts h (cols values, cols % 64 == 0) into the limb planes and chunk
// exponents; all threads of the block take part (blockDim.x a multiple of
// 64), then the block synchronises.
__device__ __forceinline__ void i8_prepare_x(const float* __restrict__ h, int cols, unsigned* lds, int* lds_e) {
  const int ngroups = cols >> 2;
  const float4* h4 = reinterpret_cast<const float4*>(h);
  for (int base = 0; base < ngroups; base += blockDim.x) {  // uniform trip count
    const int g = base + static_cast<int>(threadIdx.x);
    const float4 v = g < ngroups ? h4[g] : make_float4(0.f, 0.f, 0.f, 0.f);
    // groups past the end form whole chunks past the end (ngroups % 16 == 0)
    if (g < ngroups) i8_convert_group(v, g, lds, lds_e);
  }
  __syncthreads();
}

// Sum over aligned groups of T lanes (T a power of two <= 64); every lane of
// a group ends with the group's sum.  The order of additions is fixed, so
// results are reproducible bit for bit.
template <int T>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = T / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Orderable 64-bit key of (value, index): larger value wins, then the lower
// index.  NaN maps to the smallest key.
__device__ __forceinline__ unsigned long long argmax_key(float v, unsigned idx) {
  unsigned b = __float_as_uint(v);
  if (v != v) return 0ull;
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<unsigned long long>(b) << 32) | (0xFFFFFFFFu - idx);
}
__device__ __forceinline__ unsigned argmax_key_index(unsigned long long k) {
  return 0xFFFFFFFFu - static_cast<unsigned>(k & 0xFFFFFFFFull);
}

}  // namespace dev
}  // namespace pwg
