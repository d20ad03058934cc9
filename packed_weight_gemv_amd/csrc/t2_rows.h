// Row engine of the ternary GEMV for rows of >= 4096 weights (64 lanes per
// row), shared by the standalone kernel and the persistent step kernel.
//
// Per lane and 64-weight chunk: 4 words of T2 are unpacked with one AND (hi
// pairs, nibble = 4*w) and one shift + AND (lo pairs) and multiplied against
// six 4-bit limb planes of the chunk's fixed-point activations with 48
// v_dot8_i32_i4.  The six limb accumulators are never reset between rows:
// their weighted combination is taken modulo 2^32 after every row and the
// row's exact sum is the difference to the previous combination (every row
// sum fits in 31 bits, so the wrap-around cancels).  Tiles of U rows are then
// reduced over the 64 lanes together: v_permlane32_swap and v_permlane16_swap
// fold the U partial vectors into one register holding each row in a 16-lane
// row of the wave, and four DPP steps finish the sums.
#pragma once
#include "device_common.h"

namespace pwg {
namespace dev {

// acc[l] += 4 * sum over the chunk's 64 weights of w * digit_l(x).
__device__ __forceinline__ void t2_chunk_dot(const u32x4 wv, const unsigned* X, int acc[6]) {
  const unsigned wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned hi = wd[j] & 0xCCCCCCCCu;
    const unsigned lo = (wd[j] << 2) & 0xCCCCCCCCu;
#pragma unroll
    for (int l = 0; l < 6; ++l) {
      acc[l] = dot8(lo, X[12 * j + l], acc[l]);
      acc[l] = dot8(hi, X[12 * j + 6 + l], acc[l]);
    }
  }
}

// sum_l acc[l] * 16^l modulo 2^32.
__device__ __forceinline__ unsigned combine_limbs6(const int acc[6]) {
  unsigned v = static_cast<unsigned>(acc[5]);
#pragma unroll
  for (int l = 4; l >= 0; --l) v = v * 16u + static_cast<unsigned>(acc[l]);
  return v;
}

template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false);
  return v + __int_as_float(moved);
}

// Sums over the 16 lanes of each row of the wave; every lane gets its row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  return v;
}

// v_permlane32_swap: a = [a lanes 0-31, b lanes 0-31], b = [a lanes 32-63, b lanes 32-63].
// (The pair's elements are copied to integers before reinterpretation: a
// bit_cast of the second element directly has been seen to yield the first.)
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __uint_as_float(r0);
  b = __uint_as_float(r1);
}
// v_permlane16_swap: a = [a row 0, b row 0, a row 2, b row 2],
//                    b = [a row 1, b row 1, a row 3, b row 3] (rows of 16 lanes).
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __uint_as_float(r0);
  b = __uint_as_float(r1);
}

// Reduces U (1, 2 or 4) per-lane partials over the wave.  Afterwards 16-lane
// row q of the wave (lanes 16q..16q+15) holds the total of tile row
// row_of<U>(q).  The order of additions is fixed: results are reproducible.
template <int U>
__device__ __forceinline__ float tile_reduce(float (&p)[U]) {
  if constexpr (U == 4) {
    swap32(p[0], p[1]);
    swap32(p[2], p[3]);
    float a = p[0] + p[1];  // lanes 0-31: row 0 halves, 32-63: row 1 halves
    float b = p[2] + p[3];  // row 2 | row 3
    swap16(a, b);
    return row16_sum(a + b);  // rows of the wave: tile rows 0, 2, 1, 3
  } else if constexpr (U == 2) {
    swap32(p[0], p[1]);
    float a = p[0] + p[1];  // row 0 | row 1
    float b = a;
    swap16(a, b);
    return row16_sum(a + b);  // tile rows 0, 0, 1, 1
  } else {
    float a = p[0], b = p[0];
    swap32(a, b);
    float c = a + b, d = c;
    swap16(c, d);
    return row16_sum(c + d);  // tile row 0 everywhere
  }
}

template <int U>
__device__ __forceinline__ int row_of(int q) {
  if constexpr (U == 4) return (q == 0) ? 0 : (q == 1) ? 2 : (q == 2) ? 1 : 3;
  else if constexpr (U == 2) return q >> 1;
  else return 0;
}

// Per-lane state of one level: activation limbs of the lane's C chunks, the
// chunks' scale exponents, and the running limb totals.
template <int C>
struct T2Lane {
  unsigned X[C][48];
  int Ec[C];  // -(E_c + 2)
  int acc[C][6];
  unsigned prev[C];
};

// Loads the lane's limbs for chunks lane, lane+64, ... from the LDS planes
// written by t2_prepare_x; chunks past the row are zero.
template <int C>
__device__ __forceinline__ void t2_lane_init(T2Lane<C>& st, const unsigned* lds, const int* lds_e, int nchunks,
                                             unsigned lane) {
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const unsigned chunk = lane + 64u * c;
    const bool ok = chunk < static_cast<unsigned>(nchunks);
    st.Ec[c] = ok ? -(lds_e[chunk] + 2) : 0;
    const u32x4* src = reinterpret_cast<const u32x4*>(lds + (ok ? chunk : 0u) * kT2ChunkDwords);
#pragma unroll
    for (int q = 0; q < 12; ++q) {
      const u32x4 v = ok ? src[q] : u32x4{0u, 0u, 0u, 0u};
      st.X[c][4 * q] = v.x; st.X[c][4 * q + 1] = v.y; st.X[c][4 * q + 2] = v.z; st.X[c][4 * q + 3] = v.w;
    }
#pragma unroll
    for (int l = 0; l < 6; ++l) st.acc[c][l] = 0;
    st.prev[c] = 0u;
  }
}

template <int C, int U>
struct T2Tile {
  u32x4 w[U][C];
  float s;  // scale of the tile row this lane stores (row_of<U>(lane >> 4))
};

// Issues the loads of tile rows [r, r + U) (rows >= r1 are not loaded).
// `r` and `r1` are wave-uniform, so the row tests are scalar branches.
template <int C, int U>
__device__ __forceinline__ void t2_tile_load(const u32x4* __restrict__ w, const float* __restrict__ scale, int nchunks,
                                             long r, long r1, unsigned lane, T2Tile<C, U>& t) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (r + u < r1) {
      const u32x4* row = w + (r + u) * static_cast<long>(nchunks);
#pragma unroll
      for (int c = 0; c < C; ++c) {
        unsigned chunk = lane + 64u * c;
        if (C > 1 || nchunks < 64) chunk = chunk < static_cast<unsigned>(nchunks) ? chunk : static_cast<unsigned>(nchunks - 1);
        t.w[u][c] = __builtin_nontemporal_load(row + chunk);
      }
    }
  }
  const long rs = r + row_of<U>(static_cast<int>(lane >> 4));
  t.s = rs < r1 ? scale[rs] : 0.f;
}

// Computes tile rows [r, r + U) and returns, per lane, the finished value of
// tile row row_of<U>(lane >> 4) (already multiplied by its row scale).
template <int C, int U>
__device__ __forceinline__ float t2_tile_compute(T2Lane<C>& st, const T2Tile<C, U>& t, long r, long r1) {
  float p[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    p[u] = 0.f;
    if (r + u < r1) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        t2_chunk_dot(t.w[u][c], st.X[c], st.acc[c]);
        const unsigned comb = combine_limbs6(st.acc[c]);
        const int v = static_cast<int>(comb - st.prev[c]);
        st.prev[c] = comb;
        p[u] += ldexpf(static_cast<float>(v), st.Ec[c]);
      }
    }
  }
  return t.s * tile_reduce<U>(p);
}

}  // namespace dev
}  // namespace pwg
