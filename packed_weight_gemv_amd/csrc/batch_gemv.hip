// Small-batch ternary GEMV and int8 output projection + argmax: the weights
// stream once for all B activation vectors.
//
// Page "The Neutrino Engine", section "The 0.6B model does not get to
// decide": the large model scores a draft of one to seven tokens in a single
// batched forward pass, so its weights are read once per verify step rather
// than once per token.  Y[b, r] = s_r * sum_k W_rk X[b, k] for b < B, and for
// the output projection the argmax of every column b.
//
// A workgroup owns a contiguous block of rows.  The B vectors are taken in
// groups of BG whose limb planes (the fixed-point digits of t2/i8 GEMV, one
// exponent per chunk) fit in LDS; a group's planes are converted once per
// workgroup.  Each wave walks 4-row tiles of the block: the tile's weights
// are loaded into registers once per group, and for every vector of the
// group each lane reads its limbs from LDS once and applies them to the four
// rows (two for rows of more than 8,192 columns), so LDS traffic per weight
// byte is a quarter (a half) of a one-row kernel's.
// Later groups read the block's weights again, normally from the caches (a
// block is at most a few hundred KiB), so HBM sees each weight about once.
// Row sums are exact in integers as in the batch-1 kernels; results are
// identical to the batch-1 path vector by vector.
#include "device_common.h"
#include "pwg_internal.h"
#include "t2_rows.h"

namespace pwg {
namespace {

using namespace dev;

constexpr int kBatchWaves = 8;
constexpr int kBatchThreads = kBatchWaves * 64;

// Dwords of one vector's planes (limbs, then one exponent per chunk), padded
// to 16 bytes.
__host__ __device__ constexpr int t2_plane_dwords(int cols) { return ((cols / 64) * (kT2ChunkDwords + 1) + 3) & ~3; }
__host__ __device__ constexpr int i8_plane_dwords(int cols) { return ((cols / 16) * (kI8ChunkDwords + 1) + 3) & ~3; }

__device__ __forceinline__ void block_rows(long rows, long& R0, long& R1) {
  R0 = static_cast<long>(blockIdx.x) * rows / gridDim.x;
  R1 = static_cast<long>(blockIdx.x + 1) * rows / gridDim.x;
}

template <int C, int BG, int U>
__global__ __launch_bounds__(kBatchThreads) void t2_batch_kernel(const u32x4* __restrict__ w,
                                                                 const float* __restrict__ scale, int rows, int cols,
                                                                 const float* __restrict__ x, int batch,
                                                                 float* __restrict__ y) {
  extern __shared__ __align__(16) unsigned lds[];
  const int nchunks = cols >> 6;
  const int pdw = t2_plane_dwords(cols);
  const unsigned lane = threadIdx.x & 63u;
  const unsigned wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  long R0, R1;
  block_rows(rows, R0, R1);
  const int ntiles = static_cast<int>((R1 - R0 + U - 1) / U);

  for (int g0 = 0; g0 < batch; g0 += BG) {
    const int nb = batch - g0 < BG ? batch - g0 : BG;
    for (int bb = 0; bb < nb; ++bb) {
      unsigned* planes = lds + bb * pdw;
      t2_convert_groups(x + static_cast<size_t>(g0 + bb) * cols, cols, planes,
                        reinterpret_cast<int*>(planes + nchunks * kT2ChunkDwords), static_cast<int>(threadIdx.x),
                        static_cast<int>(blockDim.x));
    }
    __syncthreads();
    for (int t = static_cast<int>(wave); t < ntiles; t += kBatchWaves) {
      const long r = R0 + static_cast<long>(U) * t;
      u32x4 wt[U][C];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const unsigned chunk = lane + 64u * c;
          wt[u][c] = (r + u < R1 && chunk < static_cast<unsigned>(nchunks)) ? w[(r + u) * nchunks + chunk]
                                                                             : u32x4{0u, 0u, 0u, 0u};
        }
      }
      const long rs = r + row_of<U>(static_cast<int>(lane >> 4));
      const float sc = rs < R1 ? scale[rs] : 0.f;
#pragma unroll
      for (int bb = 0; bb < BG; ++bb) {
        if (bb < nb) {
          const unsigned* planes = lds + bb * pdw;
          const int* pe = reinterpret_cast<const int*>(planes + nchunks * kT2ChunkDwords);
          float p[U];
#pragma unroll
          for (int u = 0; u < U; ++u) p[u] = 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) {
            const unsigned chunk = lane + 64u * c;
            const bool ok = chunk < static_cast<unsigned>(nchunks);
            unsigned X[48];
            const u32x4* src = reinterpret_cast<const u32x4*>(planes + (ok ? chunk : 0u) * kT2ChunkDwords);
#pragma unroll
            for (int q = 0; q < 12; ++q) {
              const u32x4 v = ok ? src[q] : u32x4{0u, 0u, 0u, 0u};
              X[4 * q] = v.x; X[4 * q + 1] = v.y; X[4 * q + 2] = v.z; X[4 * q + 3] = v.w;
            }
            const int Ec = ok ? -(pe[chunk] + 2) : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
              int acc[6] = {0, 0, 0, 0, 0, 0};
              t2_chunk_dot(wt[u][c], X, acc);
              p[u] += ldexpf(static_cast<float>(static_cast<int>(combine_limbs6(acc))), Ec);
            }
          }
          const float total = tile_reduce<U>(p);
          if ((lane & (64u / U - 1u)) == 0u && rs < R1) y[static_cast<size_t>(g0 + bb) * rows + rs] = sc * total;
        }
      }
    }
    __syncthreads();  // the planes are rewritten for the next group
  }
}

template <int C, int BG, int U>
__global__ __launch_bounds__(kBatchThreads) void i8_batch_kernel(const u32x4* __restrict__ table,
                                                                 const float* __restrict__ scale, int rows, int cols,
                                                                 const float* __restrict__ h, int batch,
                                                                 float* __restrict__ logits, size_t nparts,
                                                                 unsigned long long* __restrict__ partials) {
  extern __shared__ __align__(16) unsigned lds[];
  __shared__ unsigned long long wkeys[kBatchWaves][BG];
  const int nchunks = cols >> 4;  // 16 int8 per 128-bit chunk
  const int pdw = i8_plane_dwords(cols);
  const unsigned lane = threadIdx.x & 63u;
  const unsigned wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  long R0, R1;
  block_rows(rows, R0, R1);
  const int ntiles = static_cast<int>((R1 - R0 + U - 1) / U);

  for (int g0 = 0; g0 < batch; g0 += BG) {
    const int nb = batch - g0 < BG ? batch - g0 : BG;
    for (int bb = 0; bb < nb; ++bb) {
      unsigned* planes = lds + bb * pdw;
      i8_convert_groups(h + static_cast<size_t>(g0 + bb) * cols, cols, planes,
                        reinterpret_cast<int*>(planes + nchunks * kI8ChunkDwords), static_cast<int>(threadIdx.x),
                        static_cast<int>(blockDim.x));
    }
    __syncthreads();
    float best[BG];
    unsigned best_idx[BG];
#pragma unroll
    for (int bb = 0; bb < BG; ++bb) {
      best[bb] = -__builtin_inff();
      best_idx[bb] = 0xFFFFFFFFu;
    }
    for (int t = static_cast<int>(wave); t < ntiles; t += kBatchWaves) {
      const long r = R0 + static_cast<long>(U) * t;
      u32x4 q[U][C];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const unsigned chunk = lane + 64u * c;
          q[u][c] = (r + u < R1 && chunk < static_cast<unsigned>(nchunks)) ? table[(r + u) * nchunks + chunk]
                                                                            : u32x4{0u, 0u, 0u, 0u};
        }
      }
      const long rs = r + row_of<U>(static_cast<int>(lane >> 4));
      const float sc = rs < R1 ? scale[rs] : 0.f;
#pragma unroll
      for (int bb = 0; bb < BG; ++bb) {
        if (bb < nb) {
          const unsigned* planes = lds + bb * pdw;
          const int* pe = reinterpret_cast<const int*>(planes + nchunks * kI8ChunkDwords);
          float p[U];
#pragma unroll
          for (int u = 0; u < U; ++u) p[u] = 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) {
            const unsigned chunk = lane + 64u * c;
            const bool ok = chunk < static_cast<unsigned>(nchunks);
            unsigned H[12];
            const u32x4* src = reinterpret_cast<const u32x4*>(planes + (ok ? chunk : 0u) * kI8ChunkDwords);
#pragma unroll
            for (int qq = 0; qq < 3; ++qq) {
              const u32x4 v = ok ? src[qq] : u32x4{0u, 0u, 0u, 0u};
              H[4 * qq] = v.x; H[4 * qq + 1] = v.y; H[4 * qq + 2] = v.z; H[4 * qq + 3] = v.w;
            }
            const int Ec = ok ? -pe[chunk] : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
              int a0 = 0, a1 = 0, a2 = 0;
              const unsigned qd[4] = {q[u][c].x, q[u][c].y, q[u][c].z, q[u][c].w};
#pragma unroll
              for (int gg = 0; gg < 4; ++gg) {
                a0 = dot4(qd[gg], H[3 * gg + 0], a0);
                a1 = dot4(qd[gg], H[3 * gg + 1], a1);
                a2 = dot4(qd[gg], H[3 * gg + 2], a2);
              }
              // each limb sum is exact in float32 (|a| <= 16*127*128 < 2^24); the shifts are exact
              const float pc = fmaf(static_cast<float>(a2), 65536.0f, fmaf(static_cast<float>(a1), 256.0f, static_cast<float>(a0)));
              p[u] += ldexpf(pc, Ec);
            }
          }
          const float total = tile_reduce<U>(p);
          if ((lane & (64u / U - 1u)) == 0u && rs < R1) {
            const float logit = sc * total;
            if (logits) logits[static_cast<size_t>(g0 + bb) * rows + rs] = logit;
            if (logit > best[bb]) {  // rows of one lane ascend: ties keep the lower index
              best[bb] = logit;
              best_idx[bb] = static_cast<unsigned>(rs);
            }
          }
        }
      }
    }
    // workgroup (max, lowest index) of every vector of the group
#pragma unroll
    for (int bb = 0; bb < BG; ++bb) {
      unsigned long long key = best_idx[bb] == 0xFFFFFFFFu ? 0ull : argmax_key(best[bb], best_idx[bb]);
      for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(key, off, kWave);
        key = o > key ? o : key;
      }
      if (lane == 0) wkeys[wave][bb] = key;
    }
    __syncthreads();
    if (threadIdx.x < static_cast<unsigned>(nb)) {
      unsigned long long m = 0ull;
      for (int i = 0; i < kBatchWaves; ++i) m = wkeys[i][threadIdx.x] > m ? wkeys[i][threadIdx.x] : m;
      partials[static_cast<size_t>(g0 + threadIdx.x) * nparts + blockIdx.x] = m;
    }
    __syncthreads();  // the planes and keys are rewritten for the next group
  }
}

// Stage 2 for every vector: block b reduces vector b's keys.
__global__ __launch_bounds__(256) void argmax_reduce_batch_kernel(const unsigned long long* __restrict__ partials,
                                                                  int n, size_t nparts, int32_t* __restrict__ token) {
  const unsigned long long* pb = partials + static_cast<size_t>(blockIdx.x) * nparts;
  unsigned long long k = 0ull;
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + static_cast<int>(threadIdx.x);
    if (i < n) k = pb[i] > k ? pb[i] : k;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(k, off, kWave);
    k = o > k ? o : k;
  }
  __shared__ unsigned long long wk[4];
  if ((threadIdx.x & 63) == 0) wk[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = wk[0];
    for (int i = 1; i < 4; ++i) m = wk[i] > m ? wk[i] : m;
    token[blockIdx.x] = static_cast<int32_t>(argmax_key_index(m));
  }
}

struct BatchInstance {
  const void* fn;
  int bg;          // vectors per group
  size_t lds;      // bytes of LDS for a given cols (set at launch)
  int max_active;  // workgroups per CU at that LDS size (0: not queried)
  int cols;
};

int device_cus() {
  static int cus = -1;
  if (cus < 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
  }
  return cus;
}

int occupancy(BatchInstance& in, size_t lds, int cols) {
  if (in.max_active == 0 || in.cols != cols) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, in.fn, kBatchThreads, lds) != hipSuccess || n < 1) n = 1;
    in.max_active = n;
    in.cols = cols;
  }
  return in.max_active;
}

// Grid: enough workgroups to fill the chip, each with at least 8 row tiles.
unsigned batch_grid(int64_t rows, int per_cu, size_t cap) {
  const long want = (rows + 31) / 32;
  long g = static_cast<long>(device_cus()) * per_cu;
  if (g > want) g = want;
  if (g < 1) g = 1;
  if (static_cast<size_t>(g) > cap) g = static_cast<long>(cap);
  return static_cast<unsigned>(g);
}

}  // namespace

int launch_ternary_gemv_batch(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
                              float* y, void* stream) {
  // groups of vectors whose planes fit in 160 KiB of LDS
  static BatchInstance c1 = {reinterpret_cast<const void*>(&t2_batch_kernel<1, 4, 4>), 4, 0, 0, 0};
  static BatchInstance c2 = {reinterpret_cast<const void*>(&t2_batch_kernel<2, 4, 4>), 4, 0, 0, 0};
  static BatchInstance c3 = {reinterpret_cast<const void*>(&t2_batch_kernel<3, 2, 2>), 2, 0, 0, 0};
  static BatchInstance c4 = {reinterpret_cast<const void*>(&t2_batch_kernel<4, 2, 1>), 2, 0, 0, 0};
  const int c = static_cast<int>((cols / 64 + 63) / 64);  // cols <= PWG_MAX_COLS: c <= 4
  BatchInstance& in = c == 1 ? c1 : c == 2 ? c2 : c == 3 ? c3 : c4;
  const size_t lds = static_cast<size_t>(in.bg) * t2_plane_dwords(static_cast<int>(cols)) * 4;
  const unsigned grid = batch_grid(rows, occupancy(in, lds, static_cast<int>(cols)), static_cast<size_t>(rows));
  const u32x4* wp = static_cast<const u32x4*>(w);
  int r32 = static_cast<int>(rows), c32 = static_cast<int>(cols), b32 = batch;
  void* args[] = {&wp, const_cast<float**>(&s), &r32, &c32, const_cast<float**>(&x), &b32, &y};
  const hipError_t e =
      hipLaunchKernel(in.fn, dim3(grid), dim3(kBatchThreads), args, lds, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "ternary_gemv (batch) launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

int launch_argmax_reduce_batch(const unsigned long long* partials, int n, size_t nparts, int32_t batch, int32_t* token,
                               void* stream) {
  void* args[] = {const_cast<unsigned long long**>(&partials), &n, &nparts, &token};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&argmax_reduce_batch_kernel), dim3(batch), dim3(256),
                                       args, 0, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "argmax_reduce (batch) launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

int launch_int8_gemv_argmax_batch(const int8_t* table, const float* s, int64_t rows, int64_t cols, const float* h,
                                  int32_t batch, void* ws, int32_t* token, float* logits, void* stream) {
  static BatchInstance c1 = {reinterpret_cast<const void*>(&i8_batch_kernel<1, 4, 4>), 4, 0, 0, 0};
  static BatchInstance c2 = {reinterpret_cast<const void*>(&i8_batch_kernel<2, 4, 4>), 4, 0, 0, 0};
  static BatchInstance c4 = {reinterpret_cast<const void*>(&i8_batch_kernel<4, 4, 4>), 4, 0, 0, 0};
  static BatchInstance c8 = {reinterpret_cast<const void*>(&i8_batch_kernel<8, 2, 2>), 2, 0, 0, 0};
  const int c = static_cast<int>((cols / 16 + 63) / 64);  // cols <= kMaxInt8Cols: c <= 8
  BatchInstance& in = c == 1 ? c1 : c == 2 ? c2 : c <= 4 ? c4 : c8;
  const size_t lds = static_cast<size_t>(in.bg) * i8_plane_dwords(static_cast<int>(cols)) * 4;
  const size_t nparts = int8_partials(rows);
  const unsigned grid = batch_grid(rows, occupancy(in, lds, static_cast<int>(cols)), nparts);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const u32x4* tp = reinterpret_cast<const u32x4*>(table);
  unsigned long long* parts = static_cast<unsigned long long*>(ws);
  int r32 = static_cast<int>(rows), c32 = static_cast<int>(cols), b32 = batch;
  size_t np = nparts;
  void* args[] = {&tp, const_cast<float**>(&s), &r32, &c32, const_cast<float**>(&h), &b32, &logits, &np, &parts};
  hipError_t e = hipLaunchKernel(in.fn, dim3(grid), dim3(kBatchThreads), args, lds, st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "int8_gemv_argmax (batch) launch: %s", hipGetErrorString(e));
  return launch_argmax_reduce_batch(parts, static_cast<int>(grid), np, batch, token, stream);
}

}  // namespace pwg
