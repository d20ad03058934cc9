// Batch-1 ternary GEMV on gfx950: y[r] = s[r] * sum_k W[r,k] x[k].
//
// Page "The Neutrino Engine", section "A 104 microsecond floor inside a 694
// microsecond step": at batch one every weight serves one multiply-accumulate
// per token, so the kernel is a pure weight stream; section "The file is not
// the traffic": ternary weights with row scales, read in place.
//
// Mapping (wave64):
//  * a row is cut into 64-weight chunks (16 bytes of T2 = one 128-bit load);
//    T lanes share a row (T = 64 for rows of >= 4096 weights) and lane `slot`
//    owns chunks slot, slot+T, ..., so every load instruction of a wave reads
//    T*16 contiguous bytes of one row (64 lanes -> 1 KiB, fully coalesced);
//  * each wave owns a contiguous range of row groups and software-pipelines
//    U row groups: the next U groups' loads are in flight while the current
//    ones are reduced (non-temporal loads: weights are used once);
//  * the activation limbs of a lane's chunks stay in VGPRs for all rows.
// Per 64 weights a lane spends 4 AND/shift pairs to unpack and 48 v_dot8
// (6 limbs x 8 nibble lanes x 2 halves); per row it combines the six limb
// accumulators with shifts, converts once to float and reduces over T lanes.
#include "device_common.h"
#include "pwg_internal.h"
#include "t2_rows.h"

namespace pwg {
namespace {

using namespace dev;

// Rows narrower than 64 chunks: T lanes (a power of two) share a row and a
// wave works on 64 / T rows at a time.
template <int T, int C, int U, int WPB>
__global__ __launch_bounds__(WPB * 64) void ternary_gemv_kernel(const u32x4* __restrict__ w,
                                                                 const float* __restrict__ scale, int rows,
                                                                 int cols, const float* __restrict__ x,
                                                                 float* __restrict__ y) {
  extern __shared__ __align__(16) unsigned lds[];
  const int nchunks = cols >> 6;
  int* lds_e = reinterpret_cast<int*>(lds + nchunks * kT2ChunkDwords);
  t2_prepare_x(x, cols, lds, lds_e);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane & (T - 1), ri = lane / T;
  constexpr int RW = 64 / T;

  unsigned X[C][48];
  int Ec[C];  // -(E_c + 2): undoes the chunk's 2^E_c and the 4 of the weight nibbles
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int chunk = slot + T * c;
    Ec[c] = chunk < nchunks ? -(lds_e[chunk] + 2) : 0;
    if (chunk < nchunks) {
      const u32x4* src = reinterpret_cast<const u32x4*>(lds + chunk * kT2ChunkDwords);
#pragma unroll
      for (int q = 0; q < 12; ++q) {
        const u32x4 v = src[q];
        X[c][4 * q + 0] = v.x; X[c][4 * q + 1] = v.y; X[c][4 * q + 2] = v.z; X[c][4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 48; ++q) X[c][q] = 0u;
    }
  }

  const long groups = (static_cast<long>(rows) + RW - 1) / RW;
  const long gw = static_cast<long>(blockIdx.x) * WPB + wave, nw = static_cast<long>(gridDim.x) * WPB;
  const long g0 = gw * groups / nw, g1 = (gw + 1) * groups / nw;

  auto load = [&](long g, u32x4 (&Wv)[U][C], float (&sv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long r = (g + u) * RW + ri;
      const bool valid = (g + u < g1) && r < rows;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int chunk = slot + T * c;
        Wv[u][c] = (valid && chunk < nchunks) ? __builtin_nontemporal_load(w + r * nchunks + chunk) : u32x4{0u, 0u, 0u, 0u};
      }
      sv[u] = valid ? scale[r] : 0.f;
    }
  };
  auto compute = [&](long g, const u32x4 (&Wv)[U][C], const float (&sv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        int acc[6] = {0, 0, 0, 0, 0, 0};
        t2_chunk_dot(Wv[u][c], X[c], acc);
        part += ldexpf(static_cast<float>(static_cast<int>(combine_limbs6(acc))), Ec[c]);
      }
      const float total = group_sum<T>(part);
      const long r = (g + u) * RW + ri;
      if (slot == 0 && (g + u < g1) && r < rows) y[r] = sv[u] * total;
    }
  };

  u32x4 A[U][C], B[U][C];
  float sA[U], sB[U];
  long g = g0;
  if (g < g1) load(g, A, sA);
  while (g < g1) {
    const long gn = g + U;
    if (gn < g1) load(gn, B, sB);
    compute(g, A, sA);
    g = gn;
    if (g >= g1) break;
    const long gnn = g + U;
    if (gnn < g1) load(gnn, A, sA);
    compute(g, B, sB);
    g = gnn;
  }
}

// Rows of 64 or more chunks: the whole wave works on one row at a time, in
// tiles of U rows with NB tiles in flight (see t2_rows.h).  G > 0: the
// activation loads are issued before the first weight tiles; G == 0: the
// activation is prepared after priming (widest rows, to save registers).
template <int C, int U, int NB, int WPB, int G>
__global__ __launch_bounds__(WPB * 64) void t2_rows_kernel(const u32x4* __restrict__ w,
                                                           const float* __restrict__ scale, int rows, int cols,
                                                           const float* __restrict__ x, float* __restrict__ y) {
  extern __shared__ __align__(16) unsigned lds[];
  const int nchunks = cols >> 6;
  int* lds_e = reinterpret_cast<int*>(lds + nchunks * kT2ChunkDwords);
  const unsigned lane = threadIdx.x & 63u;
  const unsigned wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long gw = static_cast<long>(blockIdx.x) * WPB + wave, nw = static_cast<long>(gridDim.x) * WPB;
  const long r0 = gw * rows / nw, r1 = (gw + 1) * rows / nw;

  T2XRegs<(G > 0 ? G : 1)> xr;
  if constexpr (G > 0) t2_x_load<G>(x, cols, xr);
  T2Tile<C, U> tiles[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    if (r0 + b * U < r1) t2_tile_load<C, U>(w, scale, nchunks, r0 + b * U, r1, lane, tiles[b]);
  if constexpr (G > 0) t2_x_convert<G>(xr, cols, lds, lds_e);
  else t2_prepare_x(x, cols, lds, lds_e);
  T2Lane<C> st;
  t2_lane_init<C>(st, lds, lds_e, nchunks, lane);

  for (long r = r0; r < r1; r += NB * U) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const long rb = r + b * U;
      if (rb < r1) {
        const float v = t2_tile_compute<C, U>(st, tiles[b], rb, r1);
        const long row = rb + row_of<U>(static_cast<int>(lane >> 4));
        if ((lane & (64u / U - 1u)) == 0u && row < r1) y[row] = v;
        if (rb + NB * U < r1) t2_tile_load<C, U>(w, scale, nchunks, rb + NB * U, r1, lane, tiles[b]);
      }
    }
  }
}

struct Instance {
  const void* fn;
  int wpb;
  int rows_per_group;
  int max_active;  // resident workgroups per CU (0 = not queried yet)
};

template <int T, int C, int U, int WPB>
Instance make() {
  return Instance{reinterpret_cast<const void*>(&ternary_gemv_kernel<T, C, U, WPB>), WPB, 64 / T, 0};
}

template <int C, int U, int NB, int WPB, int G>
Instance make_rows() {
  return Instance{reinterpret_cast<const void*>(&t2_rows_kernel<C, U, NB, WPB, G>), WPB, 1, 0};
}

// Smallest lane count T (power of two) whose C chunks cover the row.
Instance* pick(int cols) {
  static Instance t1 = make<1, 1, 4, 16>(), t2 = make<2, 1, 4, 16>(), t4 = make<4, 1, 4, 16>(),
                  t8 = make<8, 1, 4, 16>(), t16 = make<16, 1, 4, 16>(), t32 = make<32, 1, 4, 16>(),
                  t64 = make_rows<1, 4, 2, 16, 1>(), c2 = make_rows<2, 2, 2, 8, 1>(), c3 = make_rows<3, 1, 2, 8, 2>(),
                  c4 = make_rows<4, 1, 2, 4, 0>();
  const int nchunks = cols / 64;
  if (nchunks <= 1) return &t1;
  if (nchunks <= 2) return &t2;
  if (nchunks <= 4) return &t4;
  if (nchunks <= 8) return &t8;
  if (nchunks <= 16) return &t16;
  if (nchunks <= 32) return &t32;
  if (nchunks <= 64) return &t64;
  if (nchunks <= 128) return &c2;
  if (nchunks <= 192) return &c3;
  return &c4;
}

int device_cus() {
  static int cus = -1;
  if (cus < 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
  }
  return cus;
}

}  // namespace

size_t t2_lds_bytes(int64_t cols) { return static_cast<size_t>(cols / 64) * (kT2ChunkDwords + 1) * 4; }

int launch_ternary_gemv(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
                        float* y, void* stream) {
  if (batch > 1) return launch_ternary_gemv_batch(w, s, rows, cols, x, batch, y, stream);
  Instance* in = pick(static_cast<int>(cols));
  const size_t lds = t2_lds_bytes(cols);
  if (in->max_active == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, in->fn, in->wpb * 64, lds) != hipSuccess || n < 1) n = 1;
    in->max_active = n;
  }
  const long groups = (rows + in->rows_per_group - 1) / in->rows_per_group;
  const long want = (groups + in->wpb - 1) / in->wpb;  // at least one row group per wave
  const long cap = static_cast<long>(device_cus()) * in->max_active;
  const unsigned grid = static_cast<unsigned>(want < cap ? want : cap);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int b = 0; b < batch; ++b) {
    void* args[] = {const_cast<void**>(&w), const_cast<float**>(&s), nullptr, nullptr, nullptr, nullptr};
    const u32x4* wp = static_cast<const u32x4*>(w);
    int r32 = static_cast<int>(rows), c32 = static_cast<int>(cols);
    const float* xb = x + static_cast<size_t>(b) * cols;
    float* yb = y + static_cast<size_t>(b) * rows;
    args[0] = &wp;
    args[1] = const_cast<float**>(&s);
    args[2] = &r32;
    args[3] = &c32;
    args[4] = &xb;
    args[5] = &yb;
    const hipError_t e = hipLaunchKernel(in->fn, dim3(grid), dim3(in->wpb * 64), args, lds, st);
    if (e != hipSuccess) return fail(PWG_ERR_HIP, "ternary_gemv launch: %s", hipGetErrorString(e));
  }
  return PWG_OK;
}

}  // namespace pwg
