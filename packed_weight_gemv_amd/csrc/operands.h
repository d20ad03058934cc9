// Activation operands of the matrix-core GEMVs (shared by the stream step and
// the per-call batch-1 kernels).
//
// Ternary weights run on v_mfma_scale_f32_16x16x128_f8f6f4 with A in FP4
// (the masked T2 words: +2 / -2 / 0) and B in FP8 e4m3.  Each 32-value block
// of x that one E8M0 block scale covers is written as kSplits e4m3 pieces per
// value, each piece with its own exponent per value:
//     s_j = 2^(e - 8 - 4 j),  q_j = RNE_e4m3(r_j / s_j) or 0,  r_{j+1} = r_j - q_j s_j,
// r_0 = x, max|x| < 2^e over the block.  B column j carries piece j.
//
// The instruction does not add its 128 products as float32 numbers: on
// gfx950 it sums each group of 8 consecutive K values aligned to the group's
// largest product, and bits more than 13 binary places below that product's
// leading bit are dropped (measured: 256 + 2^-5 keeps the small term, 256 +
// 2^-6 loses it); the group sums then add at float32 precision.  So a piece
// is only taken where it lies within that window: in every split, a value
// whose residual is below 2^-8 of the largest residual among its 8 group
// mates gets piece 0 and keeps its residual for a later split, when the large
// residuals have shrunk.  Every nonzero piece then has its lowest bit at most
// 13 places below the group's largest product, every product is summed
// exactly, and a row sum is exact products rounded in float32.  Representation:
// |r_j / s_j| < 2^8 stays inside e4m3's range; a value taken in every split
// keeps four more significant bits per split (exact when its group is within
// 2^8 of it), a deferred one enters once its group's residuals have shrunk to
// within 2^8 of it, so |x - sum_j q_j s_j| <= 2^(e - 30) for every value
// (and 2^-24 |x| for values within 2^8 of their group maximum).
//
// int8 tables run on v_mfma_i32_16x16x64_i8: B column d holds balanced
// base-256 digit d of X = rint(h * 2^(46 - e)) (e: exponent of the 256-value
// section maximum, |X| <= 2^46); the digit sums of a section are exact in
// int32 and each moves into float32 with its power of two.  The rounding of h
// is at most 2^(e - 47) per value.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pwg {
namespace ops {

constexpr int kSplits = 6;              // e4m3 pieces per activation value
constexpr int kInt8Digits = 6;          // base-256 digits of h per value
constexpr int kInt8FixedBits = 46;      // |X| <= 2^46

// One 16 x 16 x 128 instruction's B operand: 4 lane groups x kSplits columns
// x 32 bytes (32 e4m3 values per lane).
constexpr int kTernaryMfmaBytes = 4 * kSplits * 32;
// One 16 x 16 x 64 int8 instruction's B operand: 4 lane groups x 6 digit
// columns x 16 bytes.
constexpr int kInt8MfmaBytes = 4 * kInt8Digits * 16;
constexpr int kSectionMfmas = 4;        // int8 instructions per exponent section (256 values)

// Ternary operand region for `cols` values (cols a multiple of 64; the last
// 256-value tile may be partial, its missing values are zero): the B bytes of
// every instruction, then the B scale dwords (per group of 4 instructions,
// one per lane: byte m % 4 for instruction m), then the A scale dwords (per
// group of 4 instructions, one per lane group).
__host__ __device__ constexpr size_t ternary_mfmas(int64_t cols) { return static_cast<size_t>((cols + 255) / 256) * 2; }
// The same layout for any instruction count (both weight formats).
__host__ __device__ constexpr size_t operand_quads(size_t mfmas) { return (mfmas + 3) / 4; }
__host__ __device__ constexpr size_t operand_bsc_off(size_t mfmas) { return mfmas * kTernaryMfmaBytes; }
__host__ __device__ constexpr size_t operand_asc_off(size_t mfmas) { return operand_bsc_off(mfmas) + operand_quads(mfmas) * 256; }
__host__ __device__ constexpr size_t operand_region_bytes(size_t mfmas) {
  return (operand_asc_off(mfmas) + operand_quads(mfmas) * 16 + 15) / 16 * 16;
}
__host__ __device__ constexpr size_t ternary_quads(int64_t cols) { return operand_quads(ternary_mfmas(cols)); }
__host__ __device__ constexpr size_t ternary_bsc_off(int64_t cols) { return operand_bsc_off(ternary_mfmas(cols)); }
__host__ __device__ constexpr size_t ternary_asc_off(int64_t cols) { return operand_asc_off(ternary_mfmas(cols)); }
__host__ __device__ constexpr size_t ternary_region_bytes(int64_t cols) { return operand_region_bytes(ternary_mfmas(cols)); }

// Base-3 weights (five per byte, base-3 digits w + 1, first weight least
// significant), arranged in 30-weight groups of 6 bytes, 8 groups to a
// 768-byte tile window: lane (i, g) of window t holds group 8 t + g (the A
// operand of instruction 2 t, lane group g) and group 8 t + 4 + g
// (instruction 2 t + 1).  A lane group's 32 K values are the group's 30
// weights in order and two zeros.
constexpr int kB3GroupWeights = 30;
constexpr int kB3TileBytes = 768;
__host__ __device__ constexpr int64_t b3_row_bytes(int64_t cols) { return (cols + 4) / 5; }
__host__ __device__ constexpr int64_t b3_windows(int64_t cols) { return ((b3_row_bytes(cols) + 5) / 6 + 7) / 8; }
__host__ __device__ constexpr size_t b3_mfmas(int64_t cols) { return static_cast<size_t>(b3_windows(cols)) * 2; }
// int8 (h) region: B digits of every instruction, then one int32 exponent per section.
__host__ __device__ constexpr size_t int8_exp_off(int64_t hidden) { return static_cast<size_t>(hidden / 64) * kInt8MfmaBytes; }
__host__ __device__ constexpr size_t int8_region_bytes(int64_t hidden) {
  return (int8_exp_off(hidden) + static_cast<size_t>((hidden / 64 + kSectionMfmas - 1) / kSectionMfmas) * 4 + 15) / 16 * 16;
}

// B entry of lane (column n, lane group g) inside one instruction's bytes.
// A column >= kSplits reads column n % kSplits (its scale is 2^-127 and the
// kernel drops that column's sums).
__host__ __device__ constexpr unsigned ternary_b_entry(unsigned n, unsigned g) {
  return (kSplits * g + n % kSplits) * 32u;
}
__host__ __device__ constexpr unsigned int8_b_entry(unsigned n, unsigned g) {
  return (kInt8Digits * g + n % kInt8Digits) * 16u;
}

// Inside a 32-weight K block, the masked T2 words hand the instruction the
// weights in this order: A nibble p (p = 8 dd + p', dd the dword) is weight
// 16 (dd / 2) + 8 (p' % 2) + 2 (p' / 2) + 1 - dd % 2 of the block.  The 16
// nibbles p = 16 h + j (h = 0, 1) are weights 16 h + lambda(j).
__host__ __device__ constexpr int lambda16(int j) { return 8 * (j & 1) + 2 * ((j >> 1) & 3) + 1 - ((j >> 3) & 1); }

// E8M0 scale bytes of one 32-value block with exponent e: B column j gets
// 2^(e - 8 - 4 j), A gets 2^-1 (its FP4 nibbles hold 2 w).  Where column
// kSplits - 1 would fall below 2^-127 the common factor 2^ashift moves to A.
__device__ __forceinline__ int split_ashift(int e) { return e + 99 < 0 ? e + 99 : 0; }
__device__ __forceinline__ unsigned split_b_scale(int e, int j) {
  return static_cast<unsigned>(119 + e - 4 * j - split_ashift(e));
}
__device__ __forceinline__ unsigned split_a_scale(int e) { return static_cast<unsigned>(126 + split_ashift(e)); }

typedef short v2s16 __attribute__((ext_vector_type(2)));
typedef float v2f32 __attribute__((ext_vector_type(2)));
constexpr int kDeferBits = 8;  // a residual below 2^-8 of its group's largest waits for a later split

// Splits the 8 values of one summation group of the instruction (r[j]: K
// value j of the group) into out[s][d]: bytes 4 d .. 4 d + 3 of piece s,
// e4m3 codes in operand order.  Piece s holds the residual at scale
// 2^(e - 8 - 4 s).  The residuals are kept in units of the first piece's
// scale (one exact power-of-two scaling per value: the kept residuals stay
// far above float32's normal range), so that each piece needs no per-value
// scaling: the gfx950 scaled conversion divides by 2^-4s on the way to e4m3,
// and one fused multiply-add by 2^-4s takes the piece back off, exactly.
// r is consumed.
__device__ __forceinline__ void fp8_splits8(float (&r)[8], int e, unsigned (&out)[kSplits][2]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = ldexpf(r[j], 8 - e);
#pragma unroll
  for (int s = 0; s < kSplits; ++s) {
    const float down = __builtin_bit_cast(float, static_cast<unsigned>(127 - 4 * s) << 23);  // 2^-4s
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(r[j]));
    const float thr = ldexpf(m, -kDeferBits);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float rv = r[4 * d + q];
        v[q] = fabsf(rv) >= thr ? rv : 0.f;
      }
      v2s16 w2 = {0, 0};
      w2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w2, v[0], v[1], down, false);
      w2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w2, v[2], v[3], down, true);
      const unsigned w = __builtin_bit_cast(unsigned, w2);
      out[s][d] = w;
      if (s + 1 < kSplits) {
        // the piece's value, exactly; the residual is exact in float32
        const v2f32 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
        const v2f32 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
        r[4 * d + 0] = fmaf(-lo.x, down, r[4 * d + 0]);
        r[4 * d + 1] = fmaf(-lo.y, down, r[4 * d + 1]);
        r[4 * d + 2] = fmaf(-hi.x, down, r[4 * d + 2]);
        r[4 * d + 3] = fmaf(-hi.y, down, r[4 * d + 3]);
      }
    }
  }
}

// The same for 16 values (two summation groups, which split independently).
__device__ __forceinline__ void fp8_splits16(float (&r)[16], int e, unsigned (&out)[kSplits][4]) {
#pragma unroll
  for (int G = 0; G < 2; ++G) {
    float g8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) g8[j] = r[8 * G + j];
    unsigned o[kSplits][2];
    fp8_splits8(g8, e, o);
#pragma unroll
    for (int s = 0; s < kSplits; ++s) {
      out[s][2 * G] = o[s][0];
      out[s][2 * G + 1] = o[s][1];
    }
  }
}

// Block exponent: max|x| < 2^e (0 for an all-zero block).
__device__ __forceinline__ int block_exponent(float amax) {
  return amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 0;
}

// Writes 16 values in K order (r[j] multiplies K value 16 h + j of A lane
// group ga of instruction m; e = the exponent of that lane group's whole
// 32-value block) into the operand region `b` (any address space, aligned to
// 16): B lane group 2 (ga % 2) + h at byte 16 (ga / 2).  Half 0 also writes
// the block's scale bytes (columns >= kSplits: 0, i.e. 2^-127).  r is
// consumed.
__device__ __forceinline__ void write_operand_half(unsigned char* b, size_t bsc_off, size_t asc_off, int m, int ga,
                                                   int h, float (&r)[16], int e) {
  unsigned q[kSplits][4];
  fp8_splits16(r, e, q);
  const unsigned g = 2u * static_cast<unsigned>(ga & 1) + static_cast<unsigned>(h);
  unsigned char* base = b + static_cast<size_t>(m) * kTernaryMfmaBytes + 16 * (ga >> 1);
#pragma unroll
  for (int s = 0; s < kSplits; ++s)
    *reinterpret_cast<uint4*>(base + ternary_b_entry(static_cast<unsigned>(s), g)) = make_uint4(q[s][0], q[s][1], q[s][2], q[s][3]);
  if (h == 0) {
    unsigned char* sb = b + bsc_off + static_cast<size_t>(m >> 2) * 256 + (m & 3);
#pragma unroll
    for (int n = 0; n < 16; ++n) sb[4 * (16 * ga + n)] = n < kSplits ? static_cast<unsigned char>(split_b_scale(e, n)) : 0;
    b[asc_off + static_cast<size_t>(m >> 2) * 16 + 4 * ga + (m & 3)] = static_cast<unsigned char>(split_a_scale(e));
  }
}

// One summation group of the same: r[j] multiplies K value 16 h + 8 G + j
// of A lane group ga of instruction m; the 8 bytes of each piece go to byte
// 16 (ga / 2) + 8 G of B lane group 2 (ga % 2) + h.  Quarter (h, G) = (0, 0)
// also writes the block's scale bytes.
__device__ __forceinline__ void write_operand_quarter(unsigned char* b, size_t bsc_off, size_t asc_off, int m, int ga,
                                                      int h, int G, float (&r)[8], int e) {
  unsigned q[kSplits][2];
  fp8_splits8(r, e, q);
  const unsigned g = 2u * static_cast<unsigned>(ga & 1) + static_cast<unsigned>(h);
  unsigned char* base = b + static_cast<size_t>(m) * kTernaryMfmaBytes + 16 * (ga >> 1) + 8 * G;
#pragma unroll
  for (int s = 0; s < kSplits; ++s)
    *reinterpret_cast<uint2*>(base + ternary_b_entry(static_cast<unsigned>(s), g)) = make_uint2(q[s][0], q[s][1]);
  if (h == 0 && G == 0) {
    unsigned char* sb = b + bsc_off + static_cast<size_t>(m >> 2) * 256 + (m & 3);
#pragma unroll
    for (int n = 0; n < 16; ++n) sb[4 * (16 * ga + n)] = n < kSplits ? static_cast<unsigned char>(split_b_scale(e, n)) : 0;
    b[asc_off + static_cast<size_t>(m >> 2) * 16 + 4 * ga + (m & 3)] = static_cast<unsigned char>(split_a_scale(e));
  }
}

// a where the mask bits are set, b elsewhere (v_bfi_b32).  Written as an
// instruction: a choice between two elements of one array would otherwise be
// folded into a computed index, which moves the array to scratch memory.
__device__ __forceinline__ float pick(unsigned mask, float a, float b) {
  float out;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(out) : "v"(mask), "v"(a), "v"(b));
  return out;
}

// Quarter (h, G) of 32-value T2 block beta: xs = the half's 16 values
// (x[32 beta + 16 h + i]); in K order the group holds xs[lambda16(8 G + j)].
__device__ __forceinline__ void write_ternary_quarter(unsigned char* b, size_t bsc_off, size_t asc_off, int beta, int h,
                                                      int G, const float (&xs)[16], int e) {
  const unsigned first = G ? 0u : ~0u;
  float r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = pick(first, xs[lambda16(j)], xs[lambda16(8 + j)]);
  write_operand_quarter(b, bsc_off, asc_off, 2 * (beta >> 3) + (beta & 1), (beta & 7) >> 1, h, G, r, e);
}

// Quarter (h, G) of base-3 group q: r[j] = x[30 q + 16 h + 8 G + j] (zero
// past the group's 30 values or past cols).
__device__ __forceinline__ void write_b3_quarter(unsigned char* b, size_t bsc_off, size_t asc_off, int q, int h, int G,
                                                 float (&r)[8], int e) {
  write_operand_quarter(b, bsc_off, asc_off, 2 * (q >> 3) + ((q >> 2) & 1), q & 3, h, G, r, e);
}

// Converts half h of 32-value block `beta` of a ternary input (values at
// xs[0..15] = x[32 beta + 16 h .. + 15], absent values zero; e = the whole
// block's exponent) into the operand region `b` (any address space, aligned
// to 16): the 16 values go to B lane group 2 (ga % 2) + h at byte 16 (ga / 2)
// of instruction m, where m = 2 (beta / 8) + beta % 2 and ga = (beta % 8) / 2
// is the A lane group whose weights they multiply.  Half 0 also writes the
// block's scale bytes (columns >= kSplits: 0, i.e. 2^-127).
__device__ __forceinline__ void write_ternary_half(unsigned char* b, size_t bsc_off, size_t asc_off, int beta, int h,
                                                   const float (&xs)[16], int e) {
  float r[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) r[j] = xs[lambda16(j)];
  write_operand_half(b, bsc_off, asc_off, 2 * (beta >> 3) + (beta & 1), (beta & 7) >> 1, h, r, e);
}

// Converts half h of base-3 group q (xs[i] = x[30 q + 16 h + i] for
// 16 h + i < 30, else zero; e = the group's exponent): the group is A lane
// group q % 4 of instruction 2 (q / 8) + (q / 4) % 2.
__device__ __forceinline__ void write_b3_half(unsigned char* b, size_t bsc_off, size_t asc_off, int q, int h,
                                              float (&xs)[16], int e) {
  write_operand_half(b, bsc_off, asc_off, 2 * (q >> 3) + ((q >> 2) & 1), q & 3, h, xs, e);
}

// Balanced base-256 digits of X = rint(h * 2^(46 - e)) for four values:
// dw[d] byte i = digit d of value i.  Exact: |h * 2^(46 - e)| < 2^46 is a
// float32 whose rounding to an integer converts exactly to 64 bits.
__device__ __forceinline__ void int8_digits4(const float (&hv)[4], int e, unsigned (&dw)[kInt8Digits]) {
#pragma unroll
  for (int d = 0; d < kInt8Digits; ++d) dw[d] = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    long long X = static_cast<long long>(rintf(ldexpf(hv[i], kInt8FixedBits - e)));
#pragma unroll
    for (int d = 0; d < kInt8Digits; ++d) {
      const int dg = d < kInt8Digits - 1 ? static_cast<int>(((X + 128) & 255) - 128) : static_cast<int>(X);
      X = (X - dg) >> 8;
      dw[d] |= (static_cast<unsigned>(dg) & 255u) << (8 * i);
    }
  }
}

// ----------------------------------------------------------------- tiles
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// A operands of one ternary tile slice: FP4 nibbles +2 / -2 / 0 of the 64
// weights in this lane's 16 bytes (two instructions' worth).
__device__ __forceinline__ void ternary_unpack(const u32x4_t v, v8i& a0, v8i& a1) {
  constexpr unsigned kMask = 0xCCCCCCCCu;
  a0 = v8i{static_cast<int>(v.x & kMask), static_cast<int>((v.x << 2) & kMask), static_cast<int>(v.y & kMask),
           static_cast<int>((v.y << 2) & kMask), 0, 0, 0, 0};
  a1 = v8i{static_cast<int>(v.z & kMask), static_cast<int>((v.z << 2) & kMask), static_cast<int>(v.w & kMask),
           static_cast<int>((v.w << 2) & kMask), 0, 0, 0, 0};
}

// FP4 nibbles of one base-3 byte: weight i (digit d_i of the byte) at bits
// 4 i .. 4 i + 3 as +2 (0b0100, w = +1), -2 (0b1100, w = -1) or 0; the
// bytes 243..255 (never written by the packer) decode to zero weights.
__host__ __device__ constexpr unsigned b3_nibbles(unsigned byte) {
  unsigned out = 0, v = byte;
  for (int i = 0; i < 5; ++i) {
    const unsigned d = v % 3;
    v /= 3;
    out |= (d == 2 ? 0x4u : d == 0 ? 0xCu : 0u) << (4 * i);
  }
  return byte < 243 ? out : 0u;
}

// A operands of one base-3 lane slice (12 bytes: group g, then group g + 4
// of the window) through the 256-entry nibble table `lut` in LDS: each
// group's six 20-bit table entries fill nibbles 0..29 of four dwords.
__device__ __forceinline__ void b3_group(const unsigned* lut, unsigned b0, unsigned b1, unsigned b2, unsigned b3,
                                         unsigned b4, unsigned b5, v8i& a) {
  const unsigned l0 = lut[b0], l1 = lut[b1], l2 = lut[b2], l3 = lut[b3], l4 = lut[b4], l5 = lut[b5];
  a = v8i{static_cast<int>(l0 | (l1 << 20)), static_cast<int>((l1 >> 12) | (l2 << 8) | (l3 << 28)),
          static_cast<int>((l3 >> 4) | (l4 << 16)), static_cast<int>((l4 >> 16) | (l5 << 4)), 0, 0, 0, 0};
}
__device__ __forceinline__ void b3_unpack(const unsigned* lut, unsigned v0, unsigned v1, unsigned v2, v8i& a0, v8i& a1) {
  b3_group(lut, v0 & 255u, (v0 >> 8) & 255u, (v0 >> 16) & 255u, v0 >> 24, v1 & 255u, (v1 >> 8) & 255u, a0);
  b3_group(lut, (v1 >> 16) & 255u, v1 >> 24, v2 & 255u, (v2 >> 8) & 255u, (v2 >> 16) & 255u, v2 >> 24, a1);
}

// Sum over the 16 lanes of a DPP row (one lane group: the columns of one
// row of the instruction's result); every lane ends with the same total.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // mirror
  return v;
}

// The 16 row scales of row block blk (rows 16 blk .. 16 blk + 15, clamped to
// rows - 1) through scalar loads (they count on the scalar memory counter, so
// waiting for them never waits for weight loads); returns the scales of rows
// 4 g + i.
__device__ __forceinline__ v4f block_scales(const float* scale, long blk, long rows, unsigned g) {
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* s = (cfloat*)scale;
  float r[16];
  const long base = blk * 16;
  if (base + 16 <= rows) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = s[base + i];
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = s[base + i < rows ? base + i : rows - 1];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r[i])));
  v4f out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = g == 0 ? r[i] : g == 1 ? r[4 + i] : g == 2 ? r[8 + i] : r[12 + i];
  return out;
}

}  // namespace ops
}  // namespace pwg
