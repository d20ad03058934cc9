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
// Work: each workgroup (8 waves) takes a contiguous range of 16-row blocks,
// in batches that its LDS slots hold.  When the workgroup has at least two
// blocks per wave, each wave streams whole blocks; with fewer, every block's
// K range is cut into KW chunks (a power of two <= 8) so that all waves
// stream even when the matrix has few rows.  At the end of its chunk a wave
// sums the piece columns and writes the chunk's 16 row sums to an LDS slot;
// at the end of a batch one wave per block adds the block's KW sums in chunk
// order (results do not depend on timing), scales and stores.  Two slot
// buffers alternate between batches, so a batch is reduced after the load
// group that crossed its end.  A tile is 16 rows x 64 bytes; one wave load
// instruction moves one tile (lane 16 q + i: row i, bytes 64 t + 16 q ..
// + 15), from the tiled arrangement (one contiguous KiB) or straight from
// the row-major blob (16 pieces of 64 bytes).  Loads go through a raw buffer
// resource over the workgroup's range: lanes past the matrix and loads past
// a wave's work read zeros without touching memory, so every load is issued
// unconditionally and the compiler waits only for the group being
// multiplied.  Each wave keeps two groups of kG tile loads in flight across
// chunk and batch boundaries; x is loaded first, then the first group, and
// the conversion waits for x alone.
#include "chain_input.h"
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


typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) float g_float;

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Raw buffer resource over [base, base + bytes): a lane whose offset lies
// past the end reads zeros and moves no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
constexpr unsigned kOff = 0x80000000u;  // an offset past every resource: the load returns zero
constexpr int kNt = 2;                  // streaming (non-temporal) cache policy

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNt));
}

enum Fmt { kT2Rows, kT2Tiled, kB3Tiled };

// Tile loads per register group (two groups in flight per wave).  Base-3
// tiles take more registers to decode; with shorter groups the kernel fits
// in 80 registers and three workgroups share a CU.
__host__ __device__ constexpr int group_tiles(int fmt) { return fmt == kB3Tiled ? 4 : 8; }
// Resident workgroups per CU the LDS sizing aims at for large matrices.
__host__ __device__ constexpr int target_residency(int fmt) { return fmt == kB3Tiled ? 3 : 2; }

__device__ __forceinline__ int fmt_windows(int fmt, int cols) {
  return fmt == kB3Tiled ? static_cast<int>(ops::b3_windows(cols)) : (cols + 255) >> 8;
}

// One conversion round of x: thread (beta, h, G) of round t0 converts
// summation group G of half h of 32-value block beta.  T2: it holds the
// half's 16 values x[32 beta + 16 h + i]; base-3 (block = 30-value group
// beta): its own 8 values x[30 beta + 16 h + 8 G + i] for 16 h + 8 G + i <
// 30.  Zeros past cols.
struct XRound {
  float v[16];
};
template <int kFmt>
__device__ __forceinline__ XRound load_x_round(__amdgpu_buffer_rsrc_t xr, int cols, int t0) {
  const int tid = t0 + static_cast<int>(threadIdx.x);
  const int beta = tid >> 2, h = (tid >> 1) & 1, G = tid & 1;
  XRound q;
  if (kFmt == kB3Tiled) {
    const int j0 = 16 * h + 8 * G, k0 = ops::kB3GroupWeights * beta + j0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = j0 + i < ops::kB3GroupWeights && k0 + i < cols;
      q.v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, in ? 4u * static_cast<unsigned>(k0 + i) : kOff, 0, 0));
    }
#pragma unroll
    for (int i = 8; i < 16; ++i) q.v[i] = 0.f;
  } else {
    const int k0 = 32 * beta + 16 * h;  // cols % 16 == 0: a half is all in or all out
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = buffer_load16(xr, k0 < cols ? 4u * static_cast<unsigned>(k0 + 4 * i) : kOff);
#pragma unroll
      for (int e = 0; e < 4; ++e) q.v[4 * i + e] = __uint_as_float(v[e]);
    }
  }
  return q;
}

// The same round of T2 quarters from a float vector in LDS.
__device__ __forceinline__ XRound stage_x_round(const float* stage, int cols, int t0) {
  const int tid = t0 + static_cast<int>(threadIdx.x);
  const int beta = tid >> 2, h = (tid >> 1) & 1;
  const int k0 = 32 * beta + 16 * h;  // cols % 16 == 0: a half is all in or all out
  XRound q;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 v = k0 < cols ? *reinterpret_cast<const f32x4*>(stage + k0 + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) q.v[4 * i + e] = v[e];
  }
  return q;
}

// Converts one round into the LDS operand region (blocks past cols up to the
// last window are written as zero).  Every thread takes part: the quarters
// of a block exchange their maxima with lane shuffles.
template <int kFmt>
__device__ __forceinline__ void convert_x_round(XRound& q, int cols, int t0, unsigned char* ops_lds) {
  const int T = fmt_windows(kFmt, cols);
  const int nquarter = T * 32;
  const int tid = t0 + static_cast<int>(threadIdx.x);
  const int beta = tid >> 2, h = (tid >> 1) & 1, G = tid & 1;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(q.v[i]));
  if (kFmt == kB3Tiled) amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));  // T2 quarters hold their whole half
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  if (tid < nquarter) {
    const size_t mf = static_cast<size_t>(2 * T);
    if (kFmt == kB3Tiled) {
      float r[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) r[i] = q.v[i];
      ops::write_b3_quarter(ops_lds, ops::operand_bsc_off(mf), ops::operand_asc_off(mf), beta, h, G, r,
                            ops::block_exponent(amax));
    } else {
      ops::write_ternary_quarter(ops_lds, ops::operand_bsc_off(mf), ops::operand_asc_off(mf), beta, h, G, q.v,
                                 ops::block_exponent(amax));
    }
  }
}

constexpr size_t kLdsBudget = 160 * 1024;
constexpr int kSlotBytes = 64;         // 16 float row sums of one (block, chunk)
constexpr size_t kSlotBudget = 64 * 1024;
constexpr size_t kSlotMin = 16 * 1024;

// Position of a wave in its sequence of tiles: batch b, block j of the
// batch, tile t of the wave's chunk [t0, t1).  b == nbatch: done.
struct Seq {
  int b, j, t;
};

// The 16 row scales of block blk through scalar loads (they count on the
// scalar memory counter, so waiting for them never waits for weight loads);
// lane i < 16 gets row 16 blk + i.
__device__ __forceinline__ float lane_row_scale(const float* scale, long blk, long rows, unsigned lane) {
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* s = (cfloat*)scale;
  const long base = blk * 16;
  float r[16];
  if (base + 16 <= rows) {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = s[base + i];
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) r[i] = s[base + i < rows ? base + i : rows - 1];
  }
  float out = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    out = lane == static_cast<unsigned>(i) ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(r[i]))) : out;
  return out;
}

// LDS: the operand region (rounded to 1 KiB), the base-3 nibble table
// (1 KiB, base-3 only), then the two slot buffers.
__host__ __device__ constexpr size_t fmt_region(int fmt, int64_t cols) {
  return (ops::operand_region_bytes(fmt == kB3Tiled ? ops::b3_mfmas(cols) : ops::ternary_mfmas(cols)) + 1023) / 1024 *
             1024 +
         (fmt == kB3Tiled ? 1024 : 0);
}

// kForm: the chained levels schedule's variant, which forms its input
// itself (every workgroup forms the whole vector from its sources into LDS,
// writes its own slice of it to x, and of the residual sum to resid_out),
// instead of a formation kernel before it.
template <int kFmt, bool kForm = false>
__global__ __launch_bounds__(kThreads) void t2_mfma_gemv_kernel(const unsigned char* __restrict__ w,
                                                                 const float* __restrict__ scale, int rows, int cols,
                                                                 const float* __restrict__ x, float* __restrict__ y,
                                                                 int kw, int nbb, chain::DevInput fin,
                                                                 chain::EmbedSrc femb) {
  extern __shared__ __align__(16) unsigned char smem[];
  const unsigned lane = threadIdx.x & 63u, n = lane & 15u, g = lane >> 4;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  constexpr bool kTiled = kFmt != kT2Rows;
  const int T = fmt_windows(kFmt, cols);
  constexpr int kTileBytes = kFmt == kB3Tiled ? ops::kB3TileBytes : 1024;
  constexpr int kLaneBytes = kTileBytes / 64;
  const int row_bytes = cols >> 2;  // T2 row-major only
  const int region = static_cast<int>(fmt_region(kFmt, cols));
  unsigned char* slots = smem + region;
  const unsigned* lut = reinterpret_cast<const unsigned*>(smem + region - 1024);  // base-3 only
  const int slot_buf = nbb * kw * kSlotBytes;  // one of two batch buffers
  const int bsc_off = static_cast<int>(ops::operand_bsc_off(2 * T)), asc_off = static_cast<int>(ops::operand_asc_off(2 * T));
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
  auto block_of = [&](const Seq& q) { return static_cast<long>(q.b) * nbb + q.j; };  // relative to bw0

  // This workgroup's weights as one buffer resource; offsets are relative to
  // its first block.  Rows past the matrix lie past the resource.
  const __amdgpu_buffer_rsrc_t wr =
      kTiled ? buffer_over(w + static_cast<size_t>(bw0) * T * kTileBytes, static_cast<unsigned>(nblk) * T * kTileBytes)
             : buffer_over(w + static_cast<size_t>(bw0) * 16 * row_bytes,
                           static_cast<unsigned>(min(static_cast<long>(rows), bw1 * 16) - bw0 * 16) * row_bytes);
  auto offset = [&](long blk, int t) -> unsigned {
    if (kTiled) return static_cast<unsigned>((blk * T + t) * kTileBytes + kLaneBytes * lane);
    const int off = 64 * t + 16 * static_cast<int>(g);
    return off < row_bytes ? static_cast<unsigned>((blk * 16 + n) * row_bytes + off) : kOff;
  };
  Seq ld{0, s0, t0}, cs{0, s0, t0};
  norm(ld);
  norm(cs);
  // kG loads per group, all issued (a load past the wave's sequence reads
  // nothing), so the compiler counts them and waits only for the group it
  // multiplies
  constexpr int kG = group_tiles(kFmt);
  auto load_group = [&](u32x4 (&r)[kG]) {
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const unsigned off = ld.b < nbatch ? offset(block_of(ld), ld.t) : kOff;
      if (kFmt == kB3Tiled) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b96(wr, off, 0, kNt);
        r[j] = u32x4{static_cast<unsigned>(v[0]), static_cast<unsigned>(v[1]), static_cast<unsigned>(v[2]), 0u};
      } else {
        r[j] = buffer_load16(wr, off);
      }
      ++ld.t;  // past the end norm() leaves b == nbatch
      norm(ld);
    }
  };
  const __amdgpu_buffer_rsrc_t xr = buffer_over(x, static_cast<unsigned>(cols) * 4u);
  // row scales of the first block this wave reduces (block `wave` of the
  // first batch), loaded before anything else so that the reduction does not
  // wait a memory latency for them
  const float sc_first = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      buffer_over(scale, static_cast<unsigned>(rows) * 4u),
      lane < 16u && wave < nblk ? static_cast<unsigned>(((bw0 + wave) * 16 + lane) * 4) : kOff, 0, 0));
  u32x4 ra[kG], rb[kG];
  if constexpr (kForm) {
    // the first weight loads go out before the sources are read; the formed
    // vector lies in LDS past the slot buffers
    float* stage = reinterpret_cast<float*>(slots + 2 * slot_buf);
    load_group(ra);
    chain::form_input<kThreads>(fin, cols, stage, stage + cols, femb, 0, cols);
    const int lo = static_cast<int>(static_cast<long>(blockIdx.x) * cols / gridDim.x);
    const int hi = static_cast<int>((static_cast<long>(blockIdx.x) + 1) * cols / gridDim.x);
    chain::store_formed(fin, cols, stage, const_cast<float*>(x), femb, lo, hi, static_cast<int>(threadIdx.x), kThreads);
    for (int r0 = 0; r0 < T * 32; r0 += kThreads) {
      XRound q = stage_x_round(stage, cols, r0);
      convert_x_round<kFmt>(q, cols, r0, smem);
    }
    __syncthreads();
  } else {
    XRound q = load_x_round<kFmt>(xr, cols, 0);  // x first: its wait leaves the weight loads in flight
    load_group(ra);
    if (kFmt == kB3Tiled && threadIdx.x < 256u)
      const_cast<unsigned*>(lut)[threadIdx.x] = ops::b3_nibbles(threadIdx.x);
    convert_x_round<kFmt>(q, cols, 0, smem);
    for (int r0 = kThreads; r0 < T * 32; r0 += kThreads) {
      XRound qn = load_x_round<kFmt>(xr, cols, r0);
      convert_x_round<kFmt>(qn, cols, r0, smem);
    }
    __syncthreads();
  }

  // End of batch b: all partials of the batch are in slot buffer b & 1; wave
  // j (step kWaves) adds block j's kw chunk sums in chunk order, scales and
  // stores its 16 rows.  The second barrier frees the buffer for batch b + 2.
  int done_b = 0;
  auto reduce_batch = [&]() {
    __syncthreads();
    const float* sl = reinterpret_cast<const float*>(slots + (done_b & 1) * slot_buf);
    const int nbl = blocks_in(done_b);
    for (int j = wave; j < nbl; j += kWaves) {
      const long blk = bw0 + static_cast<long>(done_b) * nbb + j;
      float v = 0.f;
      for (int cc = 0; cc < kw; ++cc) v += sl[(j * kw + cc) * 16 + (lane & 15u)];
      v *= done_b == 0 && j == wave ? sc_first : lane_row_scale(scale, blk, rows, lane);
      const long r = blk * 16 + lane;
      if (lane < 16u && r < rows) ((g_float*)y)[r] = v;
    }
    __syncthreads();
    ++done_b;
  };

  v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  auto compute_group = [&](const u32x4 (&r)[kG]) {
#pragma unroll
    for (int jj = 0; jj < kG; ++jj) {
      if (cs.b < nbatch) {
        const int ct = cs.t;
        v8i a0, a1;
        if (kFmt == kB3Tiled)
          ops::b3_unpack(lut, r[jj][0], r[jj][1], r[jj][2], a0, a1);
        else
          ops::ternary_unpack(r[jj], a0, a1);
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
        if (ct + 1 == t1) {  // end of this wave's chunk of the block: the piece columns summed, to its slot
          v4f a = acc0 + acc1;
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = ops::row16_sum(n < static_cast<unsigned>(ops::kSplits) ? a[i] : 0.f);
          if (n == 0)
            *reinterpret_cast<v4f*>(slots + (cs.b & 1) * slot_buf + (cs.j * kw + c) * kSlotBytes + 16 * g) = a;
          acc0 = v4f{0.f, 0.f, 0.f, 0.f};
          acc1 = v4f{0.f, 0.f, 0.f, 0.f};
        }
        ++cs.t;
        norm(cs);
      }
    }
  };

  // A group crosses at most one batch boundary (the host sizes batches so
  // that every wave has at least kG tiles in each full batch), so the
  // reduction of a batch can wait until the group ends: the next batch
  // writes the other slot buffer.
  while (cs.b < nbatch) {
    load_group(rb);
    compute_group(ra);
    while (done_b < cs.b) reduce_batch();
    load_group(ra);
    compute_group(rb);
    while (done_b < cs.b) reduce_batch();
  }
  while (done_b < nbatch) reduce_batch();  // batches in which this wave had no chunk
}

struct Instance {
  const void* fn;
  int fmt;
  // resident workgroups per CU for the last two LDS footprints queried
  size_t lds[2];
  int max_active[2];
  int occupancy(size_t bytes) {
    for (int i = 0; i < 2; ++i)
      if (lds[i] == bytes && max_active[i] > 0) return max_active[i];
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, bytes) != hipSuccess || n < 1) n = 1;
    lds[1] = lds[0];
    max_active[1] = max_active[0];
    lds[0] = bytes;
    max_active[0] = n;
    return n;
  }
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

// form: the input to form in the kernel (kForm instances), else null.
int launch(Instance& in, const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
           float* y, void* stream, const chain::DevInput* form = nullptr, const chain::EmbedSrc* emb = nullptr) {
  // a formed input: cols floats and the norm's per-wave sums past the slots
  const size_t stage = form ? (static_cast<size_t>(cols) * 4 + (kWaves + 1) * 4 + 15) / 16 * 16 : 0;
  const size_t budget = kLdsBudget - stage;
  const size_t region = fmt_region(in.fmt, cols);
  const int T = static_cast<int>(in.fmt == kB3Tiled ? ops::b3_windows(cols) : (cols + 255) / 256);
  // slots: all the LDS the operand region leaves (capped); or, for a matrix
  // with at least two blocks per wave at k workgroups per CU, room for k
  // resident workgroups (more waves to hide the load and LDS latencies)
  const long nb = (rows + 15) / 16;
  if (form && region + kSlotMin > budget)
    return fail(PWG_ERR_UNSUPPORTED, "ternary GEMV: %lld formed columns leave too little LDS",
                static_cast<long long>(cols));
  size_t slot_room = budget - region < kSlotBudget ? budget - region : kSlotBudget;
  for (int k = target_residency(in.fmt); k >= 2; --k) {
    if (budget / k >= region + kSlotMin && nb >= static_cast<long>(k) * device_cus() * 2 * kWaves) {
      slot_room = budget / k - region < slot_room ? budget / k - region : slot_room;
      break;
    }
  }
  const size_t lds = region + slot_room + stage;
  const long cap = static_cast<long>(device_cus()) * in.occupancy(lds);
  const unsigned grid = static_cast<unsigned>(nb < cap ? nb : cap);
  const long wg_blocks = (nb + grid - 1) / grid;
  // a workgroup's weights are addressed with 32-bit offsets
  if (wg_blocks * T * 1024 >= (1L << 31))
    return fail(PWG_ERR_UNSUPPORTED, "ternary GEMV: %lld rows exceed the per-workgroup addressing", static_cast<long long>(rows));
  // K chunks per block: a wave streams whole blocks when the workgroup has
  // at least two blocks per wave; with fewer, the K range is cut so that
  // every wave has tiles
  int kw = 1;
  while (kw < kWaves && 2 * kw <= T && wg_blocks * kw < 2 * kWaves) kw *= 2;
  // two slot buffers of nbb blocks x kw chunks; every wave needs at least kG
  // tiles in a full batch: nbb / P blocks of at least T / kw tiles each
  int nbb = static_cast<int>(slot_room / (2 * static_cast<size_t>(kw) * kSlotBytes));
  const int P = kWaves / kw;
  const int kG = group_tiles(in.fmt);
  const int need = P * ((kG + T / kw - 1) / (T / kw));
  if (nbb < need) return fail(PWG_ERR_UNSUPPORTED, "ternary GEMV: %lld columns leave too little LDS", static_cast<long long>(cols));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int r32 = static_cast<int>(rows), c32 = static_cast<int>(cols);
  const unsigned char* wp = static_cast<const unsigned char*>(w);
  for (int b = 0; b < batch; ++b) {
    const float* xb = x + static_cast<size_t>(b) * cols;
    float* yb = y + static_cast<size_t>(b) * rows;
    chain::DevInput fin = form ? *form : chain::DevInput{};
    chain::EmbedSrc femb = emb ? *emb : chain::EmbedSrc{};
    void* args[] = {&wp, const_cast<float**>(&s), &r32, &c32, &xb, &yb, &kw, &nbb, &fin, &femb};
    const hipError_t e = hipLaunchKernel(in.fn, dim3(grid), dim3(kThreads), args, lds, st);
    if (e != hipSuccess) return fail(PWG_ERR_HIP, "ternary GEMV launch: %s", hipGetErrorString(e));
  }
  return PWG_OK;
}

}  // namespace

// Row-major T2 blob; batch > 1 runs one pass per vector.
int launch_ternary_gemv(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
                        float* y, void* stream) {
  static Instance rowmajor{reinterpret_cast<const void*>(&t2_mfma_gemv_kernel<kT2Rows>), kT2Rows, {0, 0}, {0, 0}};
  return launch(rowmajor, w, s, rows, cols, x, batch, y, stream);
}

// Row-major T2 blob, batch 1, with the input formed in the kernel from its
// sources (the chained levels schedule); x receives the formed vector.
int launch_ternary_gemv_formed(const void* w, const float* s, int64_t rows, int64_t cols, const pwg_input& in,
                               const pwg_step_desc* d, float* x, float* y, void* stream) {
  static Instance formed{reinterpret_cast<const void*>(&t2_mfma_gemv_kernel<kT2Rows, true>), kT2Rows, {0, 0}, {0, 0}};
  const chain::DevInput fin = chain::from_abi(in);
  const chain::EmbedSrc emb{d->emb_table, d->emb_scale, d->token_in, static_cast<long>(d->vocab)};
  return launch(formed, w, s, rows, cols, x, 1, y, stream, &fin, &emb);
}

// Tiled T2 (cols % 256 == 0), batch 1.
int launch_ternary_gemv_tiled1(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, float* y,
                               void* stream) {
  static Instance tiled{reinterpret_cast<const void*>(&t2_mfma_gemv_kernel<kT2Tiled>), kT2Tiled, {0, 0}, {0, 0}};
  return launch(tiled, w, s, rows, cols, x, 1, y, stream);
}

// Base-3 weights in their device arrangement; batch > 1 runs one pass per
// vector.
int launch_ternary_gemv_b3(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
                           float* y, void* stream) {
  static Instance b3{reinterpret_cast<const void*>(&t2_mfma_gemv_kernel<kB3Tiled>), kB3Tiled, {0, 0}, {0, 0}};
  return launch(b3, w, s, rows, cols, x, batch, y, stream);
}

}  // namespace pwg
