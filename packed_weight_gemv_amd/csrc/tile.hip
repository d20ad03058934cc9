// Load-time arrangement of a row-major byte matrix (a T2 blob, cols / 4
// bytes per row, or an int8 table, cols bytes per row) into 16-row x 64-byte
// tiles for the matrix-core step, and of a base-3 blob into 768-byte
// windows of 30-weight groups for the base-3 GEMV.
//
// Page "The Neutrino Engine", section "The same weights take four execution
// paths": the loader arranges the same stored values for each device at load
// time.  Here one 1 KiB tile is what one wave load instruction reads: lane
// L = 16 q + i gets row i of the 16-row block, bytes 16 q .. 16 q + 15 of the
// tile's 64-byte column window, which is the operand layout of the 16 x 16
// MFMA instructions (lane = matrix row + 16 x K-group).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "operands.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

using dev::u32x4;

// One thread per 16-byte unit of the tiled output; rows past the end are zero.
__global__ __launch_bounds__(256) void tile_rows_kernel(const u32x4* __restrict__ src, int64_t rows,
                                                        int64_t row_bytes, u32x4* __restrict__ dst,
                                                        int64_t n_units) {
  const int64_t tiles_per_row = row_bytes / 64;
  const int64_t units_per_row = row_bytes / 16;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < n_units;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t tile = u >> 6;
    const int lane = static_cast<int>(u & 63);
    const int64_t rb = tile / tiles_per_row, tc = tile - rb * tiles_per_row;
    const int64_t r = rb * 16 + (lane & 15);
    const int64_t c16 = tc * 4 + (lane >> 4);  // 16-byte unit within the row
    dst[u] = r < rows ? src[r * units_per_row + c16] : u32x4{0u, 0u, 0u, 0u};
  }
}

// Base-3 device arrangement: one thread per 12-byte lane unit (lane L =
// 16 g + i of window tile (rb, t): groups 8 t + g and 8 t + 4 + g of row
// 16 rb + i, 6 stored bytes each); bytes past the row or the matrix are the
// zero-weight byte 121.
__global__ __launch_bounds__(256) void tile_b3_kernel(const unsigned char* __restrict__ src, int64_t rows,
                                                      int64_t row_bytes, int64_t windows, unsigned* __restrict__ dst,
                                                      int64_t n_units) {
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < n_units;
       u += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t tile = u >> 6;
    const int lane = static_cast<int>(u & 63);
    const int64_t rb = tile / windows, t = tile - rb * windows;
    const int64_t r = rb * 16 + (lane & 15);
    const int g = lane >> 4;
    unsigned w[3] = {0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < 12; ++b) {
      const int64_t m = 6 * (8 * t + 4 * (b / 6) + g) + b % 6;  // stored byte of row r
      const unsigned v = r < rows && m < row_bytes ? src[r * row_bytes + m] : 121u;
      w[b >> 2] |= v << (8 * (b & 3));
    }
    dst[3 * u] = w[0];
    dst[3 * u + 1] = w[1];
    dst[3 * u + 2] = w[2];
  }
}

}  // namespace

size_t b3_tiled_bytes(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || cols > PWG_MAX_COLS) return 0;
  return static_cast<size_t>((rows + 15) / 16) * static_cast<size_t>(ops::b3_windows(cols)) * ops::kB3TileBytes;
}

int launch_tile_b3(const void* src, int64_t rows, int64_t cols, void* dst, void* stream) {
  const int64_t n_units = static_cast<int64_t>(b3_tiled_bytes(rows, cols) / 12);
  const int64_t blocks = std::min<int64_t>((n_units + 255) / 256, 65536);
  hipLaunchKernelGGL(tile_b3_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const unsigned char*>(src), rows,
                     ops::b3_row_bytes(cols), ops::b3_windows(cols), static_cast<unsigned*>(dst), n_units);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "tile_b3 launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

size_t tiled_bytes(int64_t rows, int64_t row_bytes) {
  if (rows < 1 || row_bytes < 64 || row_bytes % 64 != 0) return 0;
  return static_cast<size_t>((rows + 15) / 16) * 16 * static_cast<size_t>(row_bytes);
}

int launch_tile_rows(const void* src, int64_t rows, int64_t row_bytes, void* dst, void* stream) {
  const int64_t n_units = static_cast<int64_t>(tiled_bytes(rows, row_bytes) / 16);
  const int64_t blocks = std::min<int64_t>((n_units + 255) / 256, 65536);
  hipLaunchKernelGGL(tile_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), rows, row_bytes,
                     static_cast<u32x4*>(dst), n_units);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "tile_rows launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

}  // namespace pwg
