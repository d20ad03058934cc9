// Device helpers shared by the gfx950 kernels.
//
// Both GEMVs form their dot products exactly in integers with the packed
// dot-product instructions of CDNA4 (v_dot8_i32_i4 for ternary weights,
// v_dot4_i32_i8 for int8 tables).  The float32 activation vector is turned
// once per workgroup into fixed-point integers with one power-of-two exponent
// per chunk (23 significant bits including sign, relative to the chunk's
// max|x|), split into signed digits ("limbs"), and the digit planes are
// written to LDS in the order the weight lanes expect.  Each wave then keeps the limbs of its
// own K-slice in VGPRs for every row it streams, so activations are read
// from LDS once per wave, not once per row.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pwg {
namespace dev {

constexpr int kWave = 64;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int dot8(unsigned a, unsigned b, int c) {
  return __builtin_amdgcn_sdot8(static_cast<int>(a), static_cast<int>(b), c, false);
}
__device__ __forceinline__ int dot4(unsigned a, unsigned b, int c) {
  return __builtin_amdgcn_sdot4(static_cast<int>(a), static_cast<int>(b), c, false);
}

// Byte l of four 24-bit values a, b, c, d gathered into one dword per l:
// T[l] = a.byte(l) | b.byte(l) << 8 | c.byte(l) << 16 | d.byte(l) << 24.
// v_perm_b32 selects bytes from {src0, src1} (selector 0-3: src1, 4-7: src0,
// 0x0C: zero).
__device__ __forceinline__ void gather_bytes4(unsigned a, unsigned b, unsigned c, unsigned d, unsigned T[3]) {
  const unsigned p_ab = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
  const unsigned q_ab = __builtin_amdgcn_perm(b, a, 0x0C0C0602u);  // a2 b2 0  0
  const unsigned p_cd = __builtin_amdgcn_perm(d, c, 0x05010400u);
  const unsigned q_cd = __builtin_amdgcn_perm(d, c, 0x0C0C0602u);
  T[0] = __builtin_amdgcn_perm(p_cd, p_ab, 0x05040100u);  // a0 b0 c0 d0
  T[1] = __builtin_amdgcn_perm(p_cd, p_ab, 0x07060302u);  // a1 b1 c1 d1
  T[2] = __builtin_amdgcn_perm(q_cd, q_ab, 0x05040100u);  // a2 b2 c2 d2
}

// Exponent E with m * 2^E < 2^bits (frexp: m = f * 2^e, f in [0.5, 1)).
__device__ __forceinline__ int fixed_exponent(float maxabs, int bits) {
  return bits - __builtin_amdgcn_frexp_expf(maxabs);
}

// Maximum over the 4 consecutive lanes 4q..4q+3 (one chunk's groups).
__device__ __forceinline__ float max4(float m) {
  m = fmaxf(m, __shfl_xor(m, 1, kWave));
  return fmaxf(m, __shfl_xor(m, 2, kWave));
}

// Round x * 2^E to the nearest integer v (ties to even) and return
// v + bias as an unsigned 24-bit value.  Requires |x * 2^E| <= 2^22.
// Adding 1.5 * 2^23 in float32 puts the sum in [2^23, 2^24], where the ulp is
// 1, so the float addition itself performs the rounding; the integer
// subtraction then swaps that offset for `bias`.
__device__ __forceinline__ unsigned biased_fixed(float x, int E, unsigned bias) {
  const float t = ldexpf(x, E) + 12582912.0f;
  return static_cast<unsigned>(t) - (0xC00000u - bias);
}

// Fixed-point precision: |x_fixed| <= 2^22 relative to the chunk's max|x|.
constexpr int kFixedBits = 22;

// ---------------------------------------------------------------------------
// Ternary (T2) activation limbs, one exponent per 64-element chunk.
// x_fixed = rne(x * 2^E_c) with |x_fixed| <= 2^22, written as six signed
// base-16 digits d_0..d_5 in [-8, 7]: x_fixed = sum_l d_l 16^l.  With
// u = x_fixed + 0x888888 in [0, 2^24), digit l is nibble l of u minus 8, i.e.
// nibble l of (u ^ 0x888888) read as a signed 4-bit value.
//
// For each 16-element group of x the LDS holds 12 dwords:
//   [0..5]  lo limbs: nibble n of limb l = d_l of element e(n) = {0,8,2,10,4,12,6,14}[n]
//   [6..11] hi limbs: the same for element e(n) + 1
// matching the T2 word: (word << 2) & 0xCCCCCCCC has 4*w[e(n)] in nibble n and
// word & 0xCCCCCCCC has 4*w[e(n)+1] in nibble n.  Groups of one 64-element
// chunk are contiguous; chunks are kT2ChunkDwords apart (48 + 4 pad, which
// keeps 16 lanes' 16-byte LDS reads on distinct banks).  The chunk exponents
// follow the limb planes as ints.
// ---------------------------------------------------------------------------
constexpr int kT2ChunkDwords = 52;
constexpr unsigned kT2Bias = 0x888888u;

__device__ __forceinline__ void t2_limbs_from_u(const unsigned u[16], unsigned out[12]) {
  unsigned Ta[3], Tb[3];
#pragma unroll
  for (int half = 0; half < 2; ++half) {  // half 0: even elements (lo), 1: odd (hi)
    gather_bytes4(u[0 + half], u[2 + half], u[4 + half], u[6 + half], Ta);
    gather_bytes4(u[8 + half], u[10 + half], u[12 + half], u[14 + half], Tb);
#pragma unroll
    for (int lp = 0; lp < 3; ++lp) {
      const unsigned even = (Ta[lp] & 0x0F0F0F0Fu) | ((Tb[lp] << 4) & 0xF0F0F0F0u);
      const unsigned odd = ((Ta[lp] >> 4) & 0x0F0F0F0Fu) | (Tb[lp] & 0xF0F0F0F0u);
      out[6 * half + 2 * lp] = even ^ 0x88888888u;
      out[6 * half + 2 * lp + 1] = odd ^ 0x88888888u;
    }
  }
}

// Activation registers of a thread: up to G groups of 16 floats.  Loading
// them is split from converting them so that a caller can issue the loads
// early (they head the memory queue) and convert later.
template <int G>
struct T2XRegs {
  float4 v[G][4];
};

// Loads groups g = t + i * nt (i < G) of x, where t = threadIdx.x - first and
// nt = blockDim.x - first (threads below `first` load nothing).
template <int G>
__device__ __forceinline__ void t2_x_load(const float* __restrict__ x, int cols, T2XRegs<G>& xr, int first = 0) {
  const int ngroups = cols >> 4;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  const int t = static_cast<int>(threadIdx.x) - first, nt = static_cast<int>(blockDim.x) - first;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int g = t + i * nt;
    if (t >= 0 && g < ngroups) {
#pragma unroll
      for (int q = 0; q < 4; ++q) xr.v[i][q] = x4[4 * g + q];
    }
  }
}

// Converts the loaded groups into the T2 limb planes in lds and the per-chunk
// exponents in lds_e, then synchronises the block.  blockDim.x and `first`
// must be multiples of 64 (a chunk's four groups then sit in four consecutive
// lanes of one wave, active together) and G * (blockDim.x - first) must cover
// cols / 16.
template <int G>
__device__ __forceinline__ void t2_x_convert(const T2XRegs<G>& xr, int cols, unsigned* lds, int* lds_e, int first = 0) {
  const int ngroups = cols >> 4;
  const int t = static_cast<int>(threadIdx.x) - first, nt = static_cast<int>(blockDim.x) - first;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int g = t + i * nt;
    if (t >= 0 && g < ngroups) {
      const float4* v = xr.v[i];
      float m = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[q].x), fabsf(v[q].y)), fmaxf(fabsf(v[q].z), fabsf(v[q].w))));
      const int E = fixed_exponent(max4(m), kFixedBits);
      unsigned u[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u[4 * q + 0] = biased_fixed(v[q].x, E, kT2Bias);
        u[4 * q + 1] = biased_fixed(v[q].y, E, kT2Bias);
        u[4 * q + 2] = biased_fixed(v[q].z, E, kT2Bias);
        u[4 * q + 3] = biased_fixed(v[q].w, E, kT2Bias);
      }
      unsigned out[12];
      t2_limbs_from_u(u, out);
      u32x4* dst = reinterpret_cast<u32x4*>(lds + (g >> 2) * kT2ChunkDwords + (g & 3) * 12);
      dst[0] = u32x4{out[0], out[1], out[2], out[3]};
      dst[1] = u32x4{out[4], out[5], out[6], out[7]};
      dst[2] = u32x4{out[8], out[9], out[10], out[11]};
      if ((g & 3) == 0) lds_e[g >> 2] = E;
    }
  }
  __syncthreads();
}

// Converts groups g = t, t + nt, t + 2 nt, ... of x (float32, any address
// space) into limb planes and chunk exponents (any address space).  No block
// synchronisation.  A chunk's four groups must be converted by four
// consecutive lanes that are active together: t and nt are multiples of 4
// apart within a wave (nt a multiple of 64 and t the lane-linear index).
__device__ __forceinline__ void t2_convert_groups(const float* xs, int cols, unsigned* planes, int* plane_e, int t,
                                                  int nt) {
  const int ngroups = cols >> 4;
  for (int base = 0; base < ngroups; base += nt) {
    const int g = base + t;
    if (g < ngroups) {
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = reinterpret_cast<const float4*>(xs)[4 * g + q];
      float m = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[q].x), fabsf(v[q].y)), fmaxf(fabsf(v[q].z), fabsf(v[q].w))));
      const int E = fixed_exponent(max4(m), kFixedBits);
      unsigned u[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u[4 * q + 0] = biased_fixed(v[q].x, E, kT2Bias);
        u[4 * q + 1] = biased_fixed(v[q].y, E, kT2Bias);
        u[4 * q + 2] = biased_fixed(v[q].z, E, kT2Bias);
        u[4 * q + 3] = biased_fixed(v[q].w, E, kT2Bias);
      }
      unsigned out[12];
      t2_limbs_from_u(u, out);
      u32x4* dst = reinterpret_cast<u32x4*>(planes + (g >> 2) * kT2ChunkDwords + (g & 3) * 12);
      dst[0] = u32x4{out[0], out[1], out[2], out[3]};
      dst[1] = u32x4{out[4], out[5], out[6], out[7]};
      dst[2] = u32x4{out[8], out[9], out[10], out[11]};
      if ((g & 3) == 0) plane_e[g >> 2] = E;
    }
  }
}

// Converts activations staged raw (float32) in LDS into limb planes; all
// threads of the block take part, then the block synchronises.
__device__ __forceinline__ void t2_convert_staged(const float* xs, int cols, unsigned* lds, int* lds_e) {
  t2_convert_groups(xs, cols, lds, lds_e, static_cast<int>(threadIdx.x), static_cast<int>(blockDim.x));
  __syncthreads();
}

// Load + convert in one go, for any cols (loops over groups).
__device__ __forceinline__ void t2_prepare_x(const float* __restrict__ x, int cols, unsigned* lds, int* lds_e) {
  const int ngroups = cols >> 4;
  for (int base = 0; base < ngroups; base += blockDim.x) {
    T2XRegs<1> xr;
    const int g = base + threadIdx.x;
    if (g < ngroups) {
      const float4* x4 = reinterpret_cast<const float4*>(x);
#pragma unroll
      for (int q = 0; q < 4; ++q) xr.v[0][q] = x4[4 * g + q];
      const float4* v = xr.v[0];
      float m = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[q].x), fabsf(v[q].y)), fmaxf(fabsf(v[q].z), fabsf(v[q].w))));
      const int E = fixed_exponent(max4(m), kFixedBits);
      unsigned u[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u[4 * q + 0] = biased_fixed(v[q].x, E, kT2Bias);
        u[4 * q + 1] = biased_fixed(v[q].y, E, kT2Bias);
        u[4 * q + 2] = biased_fixed(v[q].z, E, kT2Bias);
        u[4 * q + 3] = biased_fixed(v[q].w, E, kT2Bias);
      }
      unsigned out[12];
      t2_limbs_from_u(u, out);
      u32x4* dst = reinterpret_cast<u32x4*>(lds + (g >> 2) * kT2ChunkDwords + (g & 3) * 12);
      dst[0] = u32x4{out[0], out[1], out[2], out[3]};
      dst[1] = u32x4{out[4], out[5], out[6], out[7]};
      dst[2] = u32x4{out[8], out[9], out[10], out[11]};
      if ((g & 3) == 0) lds_e[g >> 2] = E;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// int8-table activation limbs, one exponent per 16-element chunk:
// x_fixed = rne(h * 2^E_c), |x_fixed| <= 2^22, three signed base-256 digits in
// [-128, 127] (u = x_fixed + 0x808080, digit l = byte l of u ^ 0x80).  For each
// 16-element chunk the LDS holds 12 dwords: dword 3*g + l = digit l of
// elements 4g..4g+3 (byte i = element 4g+i), matching the byte order of the
// int8 table row.  Chunks are 12 dwords apart (conflict-free for 16-byte reads
// of 16 consecutive lanes); the chunk exponents follow as ints.
// ---------------------------------------------------------------------------
constexpr int kI8ChunkDwords = 12;
constexpr unsigned kI8Bias = 0x808080u;

template <int G>
struct I8XRegs {
  float4 v[G];
};

template <int G>
__device__ __forceinline__ void i8_x_load(const float* __restrict__ h, int cols, I8XRegs<G>& xr, int first = 0) {
  const int ngroups = cols >> 2;  // groups of 4 elements
  const float4* h4 = reinterpret_cast<const float4*>(h);
  const int t = static_cast<int>(threadIdx.x) - first, nt = static_cast<int>(blockDim.x) - first;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int g = t + i * nt;
    if (t >= 0 && g < ngroups) xr.v[i] = h4[g];
  }
}

__device__ __forceinline__ void i8_convert_group(const float4 v, int g, unsigned* lds, int* lds_e) {
  const float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  const int E = fixed_exponent(max4(m), kFixedBits);
  unsigned T[3];
  gather_bytes4(biased_fixed(v.x, E, kI8Bias), biased_fixed(v.y, E, kI8Bias), biased_fixed(v.z, E, kI8Bias),
                biased_fixed(v.w, E, kI8Bias), T);
  unsigned* dst = lds + (g >> 2) * kI8ChunkDwords + (g & 3) * 3;
  dst[0] = T[0] ^ 0x80808080u;
  dst[1] = T[1] ^ 0x80808080u;
  dst[2] = T[2] ^ 0x80808080u;
  if ((g & 3) == 0) lds_e[g >> 2] = E;
}

template <int G>
__device__ __forceinline__ void i8_x_convert(const I8XRegs<G>& xr, int cols, unsigned* lds, int* lds_e, int first = 0) {
  const int ngroups = cols >> 2;
  const int t = static_cast<int>(threadIdx.x) - first, nt = static_cast<int>(blockDim.x) - first;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int g = t + i * nt;
    if (t >= 0 && g < ngroups) i8_convert_group(xr.v[i], g, lds, lds_e);
  }
  __syncthreads();
}

// Converts groups g = t, t + nt, ... of h (any address space) into int8
// limb planes; a wave-uniform trip count, no block synchronisation (same
// lane requirements as t2_convert_groups).
__device__ __forceinline__ void i8_convert_groups(const float* h, int cols, unsigned* planes, int* plane_e, int t,
                                                  int nt) {
  const int ngroups = cols >> 2;
  const float4* h4 = reinterpret_cast<const float4*>(h);
  for (int base = 0; base < ngroups; base += nt) {
    const int g = base + t;
    if (g < ngroups) i8_convert_group(h4[g], g, planes, plane_e);
  }
}

__device__ __forceinline__ void i8_prepare_x(const float* __restrict__ h, int cols, unsigned* lds, int* lds_e) {
  i8_convert_groups(h, cols, lds, lds_e, static_cast<int>(threadIdx.x), static_cast<int>(blockDim.x));
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
