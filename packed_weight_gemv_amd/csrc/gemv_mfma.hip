// Batch-1 ternary GEMV on the CDNA4 matrix cores, one call per matrix:
// y[r] = s[r] * sum_k W[r,k] x[k].
//
// Page "The Neutrino Engine", section "A 104 microsecond floor inside a 694
// microsecond step": at batch one every weight serves one multiply-accumulate
// per token, so the kernel is a pure weight stream; section "The file is not
// the traffic": ternary weights with row scales, read in place.
//
// Arithmetic (operands.h): every workgroup first writes x into LDS as the B
// operands of v_mfma_scale_f32_16x16x128_f8f6f4 (six e4m3 pieces per value
// that sum to x exactly, E8M0 scales per 32-value block); the weights are the
// A operands, a T2 word masked into FP4 nibbles +2 / -2 / 0 with three VALU
// operations.  Products are exact and the instruction adds in float32.
//
// Work: 16-row blocks, contiguous ranges per wave (every wave of the grid
// takes about the same number).  A block is cols / 256 tiles of 16 rows x 64
// bytes; one wave load instruction moves one tile (lane 16 q + i: row i,
// bytes 64 t + 16 q .. + 15), from the tiled arrangement (one contiguous KiB)
// or straight from the row-major blob (16 pieces of 64 bytes).  Each wave
// keeps two groups of kG tile loads in flight: one group's loads are issued
// before the other group is multiplied.
#include "device_common.h"
#include "operands.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

using namespace dev;
using ops::v4f;
using ops::v8i;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kG = 4;  // tile loads per register group (two groups in flight per wave)

typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) f32x4 cg_f32x4;
typedef __attribute__((address_space(1))) float g_float;
typedef __attribute__((address_space(1))) f32x4 g_f32x4;

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Writes the operands of x (cols values, cols % 64 == 0) into the LDS region
// `ops_lds`: thread (beta, h) converts half h of 32-value block beta; blocks
// past cols (the rest of the last 256-value tile) are zero.  All threads of
// the workgroup take part (uniform trip count: the half-block partners
// exchange their maxima with a lane shuffle).
__device__ __forceinline__ void convert_x(const float* __restrict__ x, int cols, unsigned char* ops_lds) {
  const int T = (cols + 255) >> 8;
  const int nhalf = T * 16;
  const size_t bsc_off = ops::ternary_bsc_off(cols), asc_off = ops::ternary_asc_off(cols);
  for (int t0 = 0; t0 < nhalf; t0 += kThreads) {
    const int tid = t0 + static_cast<int>(threadIdx.x);
    const int beta = tid >> 1, h = tid & 1, k0 = 32 * beta + 16 * h;
    float xs[16];
    float amax = 0.f;
    const bool in = tid < nhalf && k0 < cols;  // cols % 16 == 0: a half is all in or all out
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = in ? ((cg_f32x4*)(x + k0))[q] : f32x4{0.f, 0.f, 0.f, 0.f};
      xs[4 * q] = v.x; xs[4 * q + 1] = v.y; xs[4 * q + 2] = v.z; xs[4 * q + 3] = v.w;
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    if (tid < nhalf) ops::write_ternary_half(ops_lds, bsc_off, asc_off, beta, h, xs, ops::block_exponent(amax));
  }
  __syncthreads();
}

template <bool kTiled>
__global__ __launch_bounds__(kThreads) void t2_mfma_gemv_kernel(const unsigned char* __restrict__ w,
                                                                 const float* __restrict__ scale, int rows, int cols,
                                                                 const float* __restrict__ x, float* __restrict__ y) {
  extern __shared__ __align__(16) unsigned char smem[];
  convert_x(x, cols, smem);

  const unsigned lane = threadIdx.x & 63u, n = lane & 15u, g = lane >> 4;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const int T = (cols + 255) >> 8;
  const int row_bytes = cols >> 2;
  const int bsc_off = static_cast<int>(ops::ternary_bsc_off(cols)), asc_off = static_cast<int>(ops::ternary_asc_off(cols));
  const long nb = (static_cast<long>(rows) + 15) / 16;
  const long gw = static_cast<long>(blockIdx.x) * kWaves + wave, nw = static_cast<long>(gridDim.x) * kWaves;
  const long b0 = gw * nb / nw, b1 = (gw + 1) * nb / nw;
  const unsigned tboff = ops::ternary_b_entry(n, g);

  // tile (blk, t) of this lane; tiles past the matrix read as zero
  auto load = [&](long blk, int t) -> u32x4 {
    if (kTiled) return __builtin_nontemporal_load((g_u32x4*)(w + (static_cast<size_t>(blk) * T + t) * 1024u + 16u * lane));
    const long r = blk * 16 + n;
    const int off = 64 * t + 16 * static_cast<int>(g);
    if (r >= rows || off >= row_bytes) return u32x4{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load((g_u32x4*)(w + static_cast<size_t>(r) * row_bytes + off));
  };

  long lblk = b0, cblk = b0;
  int lt = 0, ct = 0;
  auto load_group = [&](u32x4 (&r)[kG]) {
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      if (lblk < b1) r[j] = load(lblk, lt);
      if (++lt == T) {
        lt = 0;
        ++lblk;
      }
    }
  };
  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto finish = [&]() {
    const v4f sc = ops::block_scales(scale, cblk, rows, g);
    v4f a = acc0 + acc1;  // rows 4 g + i, column n
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = ops::row16_sum(n < static_cast<unsigned>(ops::kSplits) ? a[i] : 0.f) * sc[i];
    const long r0 = cblk * 16 + 4 * g;
    if (n == 0) {
      if (r0 + 3 < rows) {
        *(g_f32x4*)(y + r0) = f32x4{a[0], a[1], a[2], a[3]};
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r0 + i < rows) ((g_float*)y)[r0 + i] = a[i];
      }
    }
    acc0 = v4f{0.f, 0.f, 0.f, 0.f};
    acc1 = v4f{0.f, 0.f, 0.f, 0.f};
  };
  auto compute_group = [&](const u32x4 (&r)[kG]) {
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      if (cblk < b1) {
        v8i a0, a1;
        ops::ternary_unpack(r[j], a0, a1);
        const unsigned char* bp = smem + static_cast<size_t>(2 * ct) * ops::kTernaryMfmaBytes + tboff;
        const u32x4 b0l = *reinterpret_cast<const u32x4*>(bp), b0h = *reinterpret_cast<const u32x4*>(bp + 16);
        const u32x4 b1l = *reinterpret_cast<const u32x4*>(bp + ops::kTernaryMfmaBytes);
        const u32x4 b1h = *reinterpret_cast<const u32x4*>(bp + ops::kTernaryMfmaBytes + 16);
        const int sb = *reinterpret_cast<const int*>(smem + bsc_off + (ct >> 1) * 256 + 4 * lane);
        const int sa = *reinterpret_cast<const int*>(smem + asc_off + (ct >> 1) * 16 + 4 * g);
        const v8i B0 = {static_cast<int>(b0l.x), static_cast<int>(b0l.y), static_cast<int>(b0l.z), static_cast<int>(b0l.w),
                        static_cast<int>(b0h.x), static_cast<int>(b0h.y), static_cast<int>(b0h.z), static_cast<int>(b0h.w)};
        const v8i B1 = {static_cast<int>(b1l.x), static_cast<int>(b1l.y), static_cast<int>(b1l.z), static_cast<int>(b1l.w),
                        static_cast<int>(b1h.x), static_cast<int>(b1h.y), static_cast<int>(b1h.z), static_cast<int>(b1h.w)};
        if (ct & 1) {  // instructions 2 ct, 2 ct + 1: scale bytes 2 and 3 of their quad's dwords
          acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, B0, acc0, 4, 0, 2, sa, 2, sb);
          acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, B1, acc1, 4, 0, 3, sa, 3, sb);
        } else {
          acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, B0, acc0, 4, 0, 0, sa, 0, sb);
          acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, B1, acc1, 4, 0, 1, sa, 1, sb);
        }
        // operands live past the instructions: no destination shares their registers
        asm volatile("" ::"v"(a0), "v"(a1), "v"(B0), "v"(B1));
        if (++ct == T) {
          finish();
          ct = 0;
          ++cblk;
        }
      }
    }
  };

  u32x4 ra[kG], rb[kG];
  load_group(ra);
  while (cblk < b1) {
    load_group(rb);
    compute_group(ra);
    load_group(ra);
    compute_group(rb);
  }
}

struct Instance {
  const void* fn;
  int max_active;  // resident workgroups per CU for the LDS of the last query
  size_t lds;
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

int launch(Instance& in, const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
           float* y, void* stream) {
  const size_t lds = ops::ternary_region_bytes(cols);
  if (in.max_active == 0 || in.lds != lds) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, in.fn, kThreads, lds) != hipSuccess || n < 1) n = 1;
    in.max_active = n;
    in.lds = lds;
  }
  const long nb = (rows + 15) / 16;
  const long cap = static_cast<long>(device_cus()) * in.max_active;
  const unsigned grid = static_cast<unsigned>(nb < cap ? nb : cap);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int r32 = static_cast<int>(rows), c32 = static_cast<int>(cols);
  const unsigned char* wp = static_cast<const unsigned char*>(w);
  for (int b = 0; b < batch; ++b) {
    const float* xb = x + static_cast<size_t>(b) * cols;
    float* yb = y + static_cast<size_t>(b) * rows;
    void* args[] = {&wp, const_cast<float**>(&s), &r32, &c32, &xb, &yb};
    const hipError_t e = hipLaunchKernel(in.fn, dim3(grid), dim3(kThreads), args, lds, st);
    if (e != hipSuccess) return fail(PWG_ERR_HIP, "ternary GEMV launch: %s", hipGetErrorString(e));
  }
  return PWG_OK;
}

}  // namespace

// Row-major T2 blob; batch > 1 runs one pass per vector.
int launch_ternary_gemv(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
                        float* y, void* stream) {
  static Instance rowmajor{reinterpret_cast<const void*>(&t2_mfma_gemv_kernel<false>), 0, 0};
  return launch(rowmajor, w, s, rows, cols, x, batch, y, stream);
}

// Tiled T2 (cols % 256 == 0), batch 1.
int launch_ternary_gemv_tiled1(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, float* y,
                               void* stream) {
  static Instance tiled{reinterpret_cast<const void*>(&t2_mfma_gemv_kernel<true>), 0, 0};
  return launch(tiled, w, s, rows, cols, x, 1, y, stream);
}

}  // namespace pwg
