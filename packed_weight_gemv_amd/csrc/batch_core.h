// Matrix-core pieces shared by the per-call small-batch kernels and the
// batched decode step (page "The Neutrino Engine", section "The 0.6B model
// does not get to decide": a draft of several tokens is scored in one batched
// pass, so every weight is read once for all of them).
//
// Operands.  Each vector's input is rounded per 256-value section (int8
// tables) or 1,024-value block (ternary levels) to fixed point,
// X = rint(x * 2^(30 - e)) with max|x| < 2^e in the section or block
// (|X| <= 2^30, a rounding of at most 2^(e - 31) per value), and X is
// written as four balanced base-256 digits (int8).  Four vectors share the
// 16 columns of one v_mfma_i32_16x16x64_i8 B operand: column 4 j + d holds
// digit d of vector j of the group.  The instructions of a section or block
// sum exactly in int32 (|sum| <= 2^23); one fused multiply-add by the
// column's power of two per section or block moves the sum into a float32
// accumulator.
//
// Operand area of one input (per 64-value K-step m and group G of four
// vectors, 1 KiB: 64 lanes x 16 bytes) and the section exponents
// [section][vector].  A compute pass reads it in slices of kSliceSteps
// K-steps, staged into LDS.
#pragma once
#include "device_common.h"

namespace pwg {
namespace bcore {

using namespace dev;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) unsigned g_u32;
typedef __attribute__((address_space(1))) float g_float;
typedef const __attribute__((address_space(4))) float c_float;

constexpr int kW = 8;                 // waves: wave 0 stages operand slices, waves 1..7 compute
constexpr int kCW = kW - 1;
constexpr int kThreads = kW * 64;
constexpr int kSliceSteps = 16;       // K-steps (64 values each) per staged slice
constexpr int kStepBytes = 1024;      // one group's B operand of one K-step: 64 lanes x 16 bytes
constexpr int kLoads = 4;             // tile loads per register group (two groups per compute wave)
constexpr unsigned long long kSpinLimit = 50000000ull;  // 0.5 s of the 100 MHz real-time counter
static_assert(kSliceSteps % 8 == 0, "a slice holds whole pairs of sections");

template <int NG>
struct SliceShape {
  static constexpr int kB = 4 * NG;                                  // vectors
  static constexpr int kOps = kSliceSteps * NG * kStepBytes;          // digits of one slice
  static constexpr int kExpBytes = (kSliceSteps / 4) * kB * 4;        // its sections' exponents
  static constexpr int kBytes = kOps + kExpBytes;
};

// Operand bytes of one input of `cols` values per vector (digits, then the
// exponents), 256-byte aligned.
__host__ __device__ constexpr size_t operand_digit_bytes(int64_t cols, int batch) {
  return static_cast<size_t>(cols / 64) * (batch / 4) * kStepBytes;
}
__host__ __device__ constexpr size_t operand_bytes(int64_t cols, int batch) {
  return (operand_digit_bytes(cols, batch) + static_cast<size_t>(cols / 256) * batch * 4 + 255) / 256 * 256;
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uni(T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)));
  return reinterpret_cast<T*>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// LDS flag store that does not wait for this wave's outstanding copies into
// LDS first (the compiler would; the flags are never a copy's destination).
__device__ __forceinline__ void lds_publish(int* p, int v) {
  const unsigned addr = static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) int*)p));
  asm volatile("s_waitcnt lgkmcnt(0)\n\tds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ int lds_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

constexpr int kDigits = 4;       // balanced base-256 digits per value
constexpr int kFixedBits = 30;   // |X| <= 2^30

// Balanced base-256 digits of the fixed-point values of xv (exponent e of the
// section): dw[d] byte i = digit d of value i.  |xv * 2^(30 - e)| < 2^30 is
// an exact float32, so the rounding to an integer is the only one.
__device__ __forceinline__ void section_digits(const float (&xv)[4], int e, unsigned (&dw)[kDigits]) {
#pragma unroll
  for (int d = 0; d < kDigits; ++d) dw[d] = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int X = static_cast<int>(rintf(ldexpf(xv[i], kFixedBits - e)));
#pragma unroll
    for (int d = 0; d < kDigits; ++d) {
      const int dg = d < kDigits - 1 ? ((X + 128) & 255) - 128 : X;
      X = (X - dg) >> 8;
      dw[d] |= (static_cast<unsigned>(dg) & 255u) << (8 * i);
    }
  }
}

__device__ __forceinline__ int section_exponent(float amax) {
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  return amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 0;  // amax < 2^e
}

// int8 tables: one wave converts section `sec` of vector b (xb = that
// vector's values); lane t owns values 4 t .. 4 t + 3, which go to K-step
// m = 4 sec + t / 16 (lane group g = (t % 16) / 4, byte 4 (t % 4) of its 16).
__device__ __forceinline__ void convert_int8_section(const float* xb, int sec, int b, int ngroups,
                                                     unsigned char* ops, int* exps, unsigned lane) {
  const float4 v = reinterpret_cast<const float4*>(xb + 256 * sec)[lane];
  const int e = section_exponent(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  const float xv[4] = {v.x, v.y, v.z, v.w};
  unsigned dw[kDigits];
  section_digits(xv, e, dw);
  const int m = 4 * sec + static_cast<int>(lane >> 4), g = static_cast<int>((lane & 15u) >> 2);
  const int j0 = 4 * static_cast<int>(lane & 3u);
  const int G = b >> 2, n0 = 4 * (b & 3);
  unsigned char* base = ops + (static_cast<size_t>(m) * ngroups + G) * kStepBytes + (16 * g + n0) * 16 + j0;
#pragma unroll
  for (int d = 0; d < kDigits; ++d) *(g_u32*)(base + d * 16) = dw[d];
  if (lane == 0) exps[sec * 4 * ngroups + b] = e - kFixedBits;
}

// Ternary levels: the same digits with one exponent per 1,024-value block
// (four sections: the integer sums of a whole block stay exact, |sum| <=
// 2^17, so the kernel converts them to float once per block), stored in the
// K order in which the tile unpack below hands the weights to the
// instruction.  A 1 KiB ternary tile holds 256 values of each of its 16 rows
// (one section); lane (g, i) holds weights 64 g .. 64 g + 63, as four T2
// words.  The unpack gives MFMA j (j = 0..3) word j; its byte k = 4 s + b is
// weight 16 j + m(s, b) of the lane's 64, m(s, b) = 8 (s / 2) + 2 b + s % 2
// (the T2 bit order).  For each section of block `blk` of vector b, lane t
// of the wave converts B bytes 4 s .. 4 s + 3 of lane group g = t / 16 for
// MFMA j = (t / 4) % 4, s = t % 4; every section of the block records the
// block's exponent.
__device__ __forceinline__ void convert_ternary_block(const float* xb, int blk, int b, int ngroups,
                                                      unsigned char* ops, int* exps, unsigned lane) {
  const int t = static_cast<int>(lane);
  const int g = t >> 4, j = (t >> 2) & 3, sq = t & 3;
  float xv[4][4];
  float amax = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* xs = xb + 256 * (4 * blk + q) + 64 * g + 16 * j + 8 * (sq >> 1) + (sq & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[q][i] = xs[2 * i];
      amax = fmaxf(amax, fabsf(xv[q][i]));
    }
  }
  const int e = section_exponent(amax);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int sec = 4 * blk + q;
    unsigned dw[kDigits];
    section_digits(xv[q], e, dw);
    const int m = 4 * sec + j, G = b >> 2, n0 = 4 * (b & 3);
    unsigned char* base = ops + (static_cast<size_t>(m) * ngroups + G) * kStepBytes + (16 * g + n0) * 16 + 4 * sq;
#pragma unroll
    for (int d = 0; d < kDigits; ++d) *(g_u32*)(base + d * 16) = dw[d];
    if (t == 0) exps[sec * 4 * ngroups + b] = e - kFixedBits;
  }
}

// int8 A operand of MFMA j of a ternary tile slice (the lane's T2 word j):
// byte b of dword s is the code at bits 8 b + 2 s, mapped 0 -> 0, 1 -> 1,
// 3 -> -1 by a byte lookup.
__device__ __forceinline__ void t2_unpack_i8(unsigned w, int (&a)[4]) {
#pragma unroll
  for (int sq = 0; sq < 4; ++sq)
    a[sq] = static_cast<int>(__builtin_amdgcn_perm(0u, 0xFF000100u, (w >> (2 * sq)) & 0x03030303u));
}

// The 16 row scales of row block rb (clamped to the last row) through scalar
// loads; returns those of rows 4 g + i.
__device__ __forceinline__ v4f block_scales(const float* scale, int rb, int rows, unsigned g) {
  c_float* s = (c_float*)scale;
  float r[16];
  const int base = rb * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = s[base + i < rows ? base + i : rows - 1];
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r[i])));
  v4f out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = g == 0 ? r[i] : g == 1 ? r[4 + i] : g == 2 ? r[8 + i] : r[12 + i];
  return out;
}

// Arithmetic of one compute wave over kR row blocks and NG groups of four
// vectors.  kTernary: a tile load is one 256-value section of a T2 tile
// (four K-steps, unpacked in registers); otherwise one int8 K-step.
template <int NG, bool kTernary>
struct Compute {
  static constexpr int kR = kTernary ? 1 : 2;  // ternary: 1, so that the unpacked operands stay in registers
  static constexpr int kStepsPerLoad = kTernary ? 4 : 1;
  static constexpr int kSecSteps = kTernary ? 16 : 4;  // K-steps per exponent (ternary: a 1,024-value block)
  static constexpr int kB = 4 * NG;
  static constexpr int kOps = SliceShape<NG>::kOps;
  unsigned lane, g;
  int vec_in_group, digit;

  __device__ __forceinline__ explicit Compute(unsigned l) : lane(l), g(l >> 4) {
    const unsigned n = l & 15u;
    vec_in_group = static_cast<int>(n >> 2);
    digit = static_cast<int>(n & 3u);
  }

  // End of a 256-value section of the slice in `buf`: the exact sums scaled
  // by this column's exponent, 2^(e + 8 d) for digit column d.
  // float(sum) * 2^(e + 8 d) is exact (|sum| < 2^24), so the fused
  // multiply-add rounds once, as an add of the scaled sum would.
  __device__ __forceinline__ void section_end(const unsigned char* buf, int sec_in_slice, v4i (&iacc)[kR][NG],
                                              v4f (&facc)[kR][NG]) const {
    const int* ex = reinterpret_cast<const int*>(buf + kOps) + sec_in_slice * kB;
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      const float sc = ldexpf(1.0f, ex[4 * G + vec_in_group] + 8 * digit);
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        facc[r][G].x = fmaf(static_cast<float>(iacc[r][G].x), sc, facc[r][G].x);
        facc[r][G].y = fmaf(static_cast<float>(iacc[r][G].y), sc, facc[r][G].y);
        facc[r][G].z = fmaf(static_cast<float>(iacc[r][G].z), sc, facc[r][G].z);
        facc[r][G].w = fmaf(static_cast<float>(iacc[r][G].w), sc, facc[r][G].w);
        iacc[r][G] = v4i{0, 0, 0, 0};
      }
    }
  }

  // B operands of K-step s_in (slice-relative) of every group.
  __device__ __forceinline__ void read_b(const unsigned char* buf, int s_in, v4i (&B)[NG]) const {
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + (s_in * NG + G) * kStepBytes + lane * 16);
      B[G] = v4i{static_cast<int>(bv.x), static_cast<int>(bv.y), static_cast<int>(bv.z), static_cast<int>(bv.w)};
    }
  }

  // One register group: tile loads load0 .. load0 + kLoads - 1 of every row
  // block, kLoads x kStepsPerLoad K-steps.  Each K-step's B operands are read
  // from LDS one K-step ahead of its instructions; one K-step's A operands
  // live at a time (no hoisting of later unpacks above the barrier).
  __device__ __forceinline__ void group(const u32x4 (&x)[kLoads][kR], const unsigned char* buf, int load0,
                                        v4f (&facc)[kR][NG]) const {
    constexpr int kSteps = kLoads * kStepsPerLoad;
    const int st0 = (load0 * kStepsPerLoad) % kSliceSteps;  // first K-step of the group in the slice
    v4i iacc[kR][NG];
#pragma unroll
    for (int r = 0; r < kR; ++r)
#pragma unroll
      for (int G = 0; G < NG; ++G) iacc[r][G] = v4i{0, 0, 0, 0};
    v4i Bc[NG], Bn[NG];
    read_b(buf, st0, Bc);
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      const int u = i / kStepsPerLoad, j = i % kStepsPerLoad;
      v4i A[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if (kTernary) {
          // a ternary tile is one section: 4 K-steps from the lane's 4 words
          const unsigned w = j == 0 ? x[u][r].x : j == 1 ? x[u][r].y : j == 2 ? x[u][r].z : x[u][r].w;
          int a[4];
          t2_unpack_i8(w, a);
          A[r] = v4i{a[0], a[1], a[2], a[3]};
        } else {
          A[r] = v4i{static_cast<int>(x[u][r].x), static_cast<int>(x[u][r].y), static_cast<int>(x[u][r].z),
                     static_cast<int>(x[u][r].w)};
        }
      }
      if (i + 1 < kSteps) read_b(buf, st0 + i + 1, Bn);
#pragma unroll
      for (int G = 0; G < NG; ++G)
#pragma unroll
        for (int r = 0; r < kR; ++r) iacc[r][G] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[r], Bc[G], iacc[r][G], 0, 0, 0);
      // int8: the sums of one section (4 K-steps); ternary: of one block (16)
      if (i % kSecSteps == kSecSteps - 1) section_end(buf, (st0 + i) / 4, iacc, facc);
#pragma unroll
      for (int G = 0; G < NG; ++G) Bc[G] = Bn[G];
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Results of slot r (row block rb): the four columns of each vector summed
  // (quad DPP), times the row scale; lanes 4 j of the quad hold vector
  // 4 G + j's values of rows 4 g .. 4 g + 3.  Written to out[b][row] when out
  // is set; int8 tables also track each vector's (max, lowest row).
  __device__ __forceinline__ void finish(const v4f (&facc)[kR][NG], int r, int rb, const float* scale, int rows,
                                         float* out, float (&best)[NG], unsigned (&bidx)[NG]) const {
    const v4f sc = block_scales(scale, rb, rows, g);
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      v4f a = facc[r][G];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = a[i];
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
        a[i] = v * sc[i];
      }
      if (digit == 0) {
        const int b = 4 * G + vec_in_group;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rb * 16 + 4 * static_cast<int>(g) + i;
          if (row < rows) {
            if (out) ((g_float*)out)[static_cast<size_t>(b) * rows + row] = a[i];
            if (!kTernary && a[i] > best[G]) {  // a lane's rows ascend: ties keep the lower row
              best[G] = a[i];
              bidx[G] = static_cast<unsigned>(row);
            }
          }
        }
      }
    }
  }

  // Per vector: the max key over the four lane groups, into keys[vector]
  // (lanes 0..15 of digit 0 write).
  __device__ __forceinline__ void wave_keys(const float (&best)[NG], const unsigned (&bidx)[NG],
                                            unsigned long long* keys) const {
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      unsigned long long key = (digit == 0 && bidx[G] != 0xFFFFFFFFu) ? argmax_key(best[G], bidx[G]) : 0ull;
      unsigned long long o = __shfl_xor(key, 16, kWave);
      key = o > key ? o : key;
      o = __shfl_xor(key, 32, kWave);
      key = o > key ? o : key;
      if (lane < 16 && digit == 0) keys[4 * G + vec_in_group] = key;
    }
  }
};

}  // namespace bcore
}  // namespace pwg
