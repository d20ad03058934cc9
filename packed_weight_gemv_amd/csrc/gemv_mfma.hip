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
// Work: each workgroup (8 waves, one per CU) takes a contiguous range of
// 16-row blocks, in batches that its LDS partial slots hold.  Every block's
// K range is cut into KW chunks (KW = the largest power of two <= 8 that is
// at most the block's tiles) and the 8 waves take one chunk of 8 / KW blocks
// each at a time, so all waves stream even when the matrix has few rows.  A
// chunk's partial 16 x 16 result goes to an LDS slot; at the end of a batch
// one wave per block adds its KW partials in a fixed order (results do not
// depend on timing), sums the piece columns, scales and stores.  A tile is
// 16 rows x 64 bytes; one wave load instruction moves one tile (lane 16 q + i:
// row i, bytes 64 t + 16 q .. + 15), from the tiled arrangement (one
// contiguous KiB) or straight from the row-major blob (16 pieces of 64 bytes).
// Each wave keeps two groups of kG tile loads in flight across chunk and
// batch boundaries; the first group is issued before x is converted.
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

constexpr int kMaxSlots = 96;                  // LDS partial slots (1 KiB each)
constexpr size_t kLdsBudget = 160 * 1024;

// Position of a wave in its sequence of tiles: batch b, block j of the
// batch, tile t of the wave's chunk [t0, t1).  b == nbatch: done.
struct Seq {
  int b, j, t;
};

template <bool kTiled>
__global__ __launch_bounds__(kThreads) void t2_mfma_gemv_kernel(const unsigned char* __restrict__ w,
                                                                 const float* __restrict__ scale, int rows, int cols,
                                                                 const float* __restrict__ x, float* __restrict__ y,
                                                                 int kw, int nbb) {
  extern __shared__ __align__(16) unsigned char smem[];
  const unsigned lane = threadIdx.x & 63u, n = lane & 15u, g = lane >> 4;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const int T = (cols + 255) >> 8;
  const int row_bytes = cols >> 2;
  const size_t region = ops::ternary_region_bytes(cols);
  unsigned char* slots = smem + region;
  const int bsc_off = static_cast<int>(ops::ternary_bsc_off(cols)), asc_off = static_cast<int>(ops::ternary_asc_off(cols));
  const long nb = (static_cast<long>(rows) + 15) / 16;
  const long bw0 = static_cast<long>(blockIdx.x) * nb / gridDim.x, bw1 = (static_cast<long>(blockIdx.x) + 1) * nb / gridDim.x;
  const int nblk = static_cast<int>(bw1 - bw0);
  const int nbatch = (nblk + nbb - 1) / nbb;
  const int P = kWaves / kw;                // blocks in progress at a time
  const int c = wave % kw, s0 = wave / kw;  // this wave's chunk and first block slot
  const int t0 = c * T / kw, t1 = (c + 1) * T / kw;
  const unsigned tboff = ops::ternary_b_entry(n, g);
  auto blocks_in = [&](int b) { return min(nbb, nblk - b * nbb); };
  auto norm = [&](Seq& q) {
    while (q.b < nbatch) {
      if (q.j < blocks_in(q.b) && q.t < t1) return;
      if (q.t >= t1) {
        q.j += P;
        q.t = t0;
      }
      if (q.j >= blocks_in(q.b)) {
        ++q.b;
        q.j = s0;
        q.t = t0;
      }
    }
  };
  auto block_of = [&](const Seq& q) { return bw0 + static_cast<long>(q.b) * nbb + q.j; };

  // tile (blk, t) of this lane; tiles past the matrix read as zero
  auto load = [&](long blk, int t) -> u32x4 {
    if (kTiled) return __builtin_nontemporal_load((g_u32x4*)(w + (static_cast<size_t>(blk) * T + t) * 1024u + 16u * lane));
    const long r = blk * 16 + n;
    const int off = 64 * t + 16 * static_cast<int>(g);
    if (r >= rows || off >= row_bytes) return u32x4{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load((g_u32x4*)(w + static_cast<size_t>(r) * row_bytes + off));
  };
  Seq ld{0, s0, t0}, cs{0, s0, t0};
  norm(ld);
  norm(cs);
  auto load_group = [&](u32x4 (&r)[kG]) {
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      if (ld.b < nbatch) {
        r[j] = load(block_of(ld), ld.t);
        ++ld.t;
        norm(ld);
      }
    }
  };
  u32x4 ra[kG], rb[kG];
  load_group(ra);  // the first loads do not wait for x
  convert_x(x, cols, smem);

  // End of batch bb: one wave per block adds the block's chunk partials (in
  // chunk order), sums the piece columns, scales and stores.
  int done_b = 0;
  auto end_batch = [&]() {
    __syncthreads();
    const int nbl = blocks_in(done_b);
    for (int j = wave; j < nbl; j += kWaves) {
      v4f a = {0.f, 0.f, 0.f, 0.f};
      for (int cc = 0; cc < kw; ++cc) a += *reinterpret_cast<const v4f*>(slots + (j * kw + cc) * 1024 + 16 * lane);
      const long blk = bw0 + static_cast<long>(done_b) * nbb + j;
      const v4f sc = ops::block_scales(scale, blk, rows, g);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = ops::row16_sum(n < static_cast<unsigned>(ops::kSplits) ? a[i] : 0.f) * sc[i];
      const long r0 = blk * 16 + 4 * g;
      if (n == 0) {
        if (r0 + 3 < rows) {
          *(g_f32x4*)(y + r0) = f32x4{a[0], a[1], a[2], a[3]};
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (r0 + i < rows) ((g_float*)y)[r0 + i] = a[i];
        }
      }
    }
    __syncthreads();
    ++done_b;
  };

  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto compute_group = [&](const u32x4 (&r)[kG]) {
#pragma unroll
    for (int jj = 0; jj < kG; ++jj) {
      if (cs.b < nbatch) {
        v8i a0, a1;
        ops::ternary_unpack(r[jj], a0, a1);
        const int ct = cs.t;
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
        if (ct + 1 == t1) {  // end of this wave's chunk of the block: its partial to the block's slot
          *reinterpret_cast<v4f*>(slots + (cs.j * kw + c) * 1024 + 16 * lane) = acc0 + acc1;
          acc0 = v4f{0.f, 0.f, 0.f, 0.f};
          acc1 = v4f{0.f, 0.f, 0.f, 0.f};
        }
        const int b_before = cs.b;
        ++cs.t;
        norm(cs);
        for (int bb = b_before; bb < cs.b; ++bb) end_batch();
      }
    }
  };

  while (cs.b < nbatch) {
    load_group(rb);
    compute_group(ra);
    load_group(ra);
    compute_group(rb);
  }
  while (done_b < nbatch) end_batch();  // batches in which this wave had no chunk
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
  const size_t region = (ops::ternary_region_bytes(cols) + 1023) / 1024 * 1024;
  const int T = static_cast<int>((cols + 255) / 256);
  int kw = 8;
  while (kw > T) kw >>= 1;
  int slots = static_cast<int>((kLdsBudget - region) / 1024);
  slots = slots < kMaxSlots ? slots : kMaxSlots;
  int nbb = slots / kw;
  const size_t lds = region + static_cast<size_t>(nbb) * kw * 1024;
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
    void* args[] = {&wp, const_cast<float**>(&s), &r32, &c32, &xb, &yb, &kw, &nbb};
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
