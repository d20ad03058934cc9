// Small-batch int8 output projection + argmax on the CDNA4 matrix cores.
//
// Page "The Neutrino Engine", section "The 0.6B model does not get to
// decide": the large model scores a draft of several tokens in one batched
// pass, so the output table is read once for all of them.  Here
// Logits[b, v] = t_v * sum_k Q_vk H[b, k] for B = 4, 8 or 16 vectors and the
// greedy argmax of each (lowest row on ties), with Q read once from HBM in
// its stored row-major int8 layout.
//
// Operands.  Each vector's h is rounded per 256-value section to fixed point,
// X = rint(h * 2^(22 - e)) with max|h| < 2^e in the section (|X| <= 2^22),
// and X is written as three balanced base-256 digits (int8).  Four vectors
// share the 16 columns of one v_mfma_i32_16x16x64_i8 B operand: column
// 4 j + d holds digit d of vector j of the group, column 4 j + 3 is zero.
// The four instructions of a section sum exactly in int32 (|sum| < 2^24); one
// ldexp per section and column moves the sum into a float32 accumulator.
// A conversion kernel writes the digits into the workspace once per call.
//
// Work.  A workgroup takes a contiguous range of 16-row blocks and walks it in
// sweeps: in each sweep 7 compute waves hold two row blocks each and run over
// the whole K range in lock step through K-slices of 1,024 values, which a
// staging wave copies into two LDS buffers ahead of use (a 16-vector B
// operand for all of K would not fit in LDS).  Each compute wave keeps the
// tile loads of the next one or two sections in flight (8-16 KiB), across
// slice and sweep boundaries.  Lane L = 16 q + i of a tile load reads row i, bytes
// 16 q .. 16 q + 15 of the 64-value K-step: the A operand as stored.
#include "device_common.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

using namespace dev;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) unsigned g_u32;
typedef __attribute__((address_space(1))) float g_float;
typedef const __attribute__((address_space(4))) float c_float;

constexpr int kW = 8;                 // waves: wave 0 stages operand slices, waves 1..7 compute
constexpr int kCW = kW - 1;
constexpr int kThreadsB = kW * 64;
constexpr int kSliceSteps = 16;       // K-steps (64 values each) per staged slice
constexpr int kStepBytes = 1024;      // one group's B operand of one K-step: 64 lanes x 16 bytes
constexpr unsigned long long kSpinLimit = 50000000ull;  // 0.5 s of the 100 MHz real-time counter
static_assert(kSliceSteps % 8 == 0, "a slice holds whole pairs of sections");

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// LDS flag store that does not wait for this wave's outstanding copies into
// LDS first (the compiler would; the flags are never a copy's destination).
__device__ __forceinline__ void lds_publish(int* p, int v) {
  const unsigned addr = static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) int*)p));
  asm volatile("s_waitcnt lgkmcnt(0)\n\tds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ int lds_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// One wave converts section `blockIdx.x` of vector `blockIdx.y`; lane t owns
// values 4 t .. 4 t + 3.  Digits go to the B-operand layout of K-step
// m = 4 sec + t / 16 (lane group g = (t % 16) / 4, byte 4 (t % 4) of its 16).
__global__ __launch_bounds__(64) void i8b_convert_kernel(const float* __restrict__ h, int cols, int ngroups,
                                                         unsigned char* __restrict__ ops, int* __restrict__ exps) {
  const int sec = blockIdx.x, b = blockIdx.y, nb = 4 * ngroups;
  const unsigned lane = threadIdx.x;
  const float4 v = reinterpret_cast<const float4*>(h + static_cast<size_t>(b) * cols + 256 * sec)[lane];
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  const int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 0;  // amax < 2^e
  const float xv[4] = {v.x, v.y, v.z, v.w};
  unsigned dw[3] = {0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int X = static_cast<int>(rintf(ldexpf(xv[i], 22 - e)));  // |X| <= 2^22
    const int d0 = ((X + 128) & 255) - 128;
    const int X1 = (X - d0) >> 8;
    const int d1 = ((X1 + 128) & 255) - 128;
    const int d2 = (X1 - d1) >> 8;
    dw[0] |= (static_cast<unsigned>(d0) & 255u) << (8 * i);
    dw[1] |= (static_cast<unsigned>(d1) & 255u) << (8 * i);
    dw[2] |= (static_cast<unsigned>(d2) & 255u) << (8 * i);
  }
  const int m = 4 * sec + static_cast<int>(lane >> 4), g = static_cast<int>((lane & 15u) >> 2);
  const int j0 = 4 * static_cast<int>(lane & 3u);
  const int G = b >> 2, n0 = 4 * (b & 3);
  unsigned char* base = ops + (static_cast<size_t>(m) * ngroups + G) * kStepBytes + (16 * g + n0) * 16 + j0;
#pragma unroll
  for (int d = 0; d < 4; ++d) *(g_u32*)(base + d * 16) = d < 3 ? dw[d] : 0u;
  if (lane == 0) exps[sec * nb + b] = e - 22;
}

// Ternary levels: the same digits, stored in the K order in which the tile
// unpack below hands the weights to the instruction.  A 1 KiB ternary tile
// holds 256 values of each of its 16 rows (one section); lane (g, i) holds
// weights 64 g .. 64 g + 63, as four T2 words.  The unpack gives MFMA j
// (j = 0..3) word j; its byte k = 4 s + b is weight 16 j + m(s, b) of the
// lane's 64, m(s, b) = 8 (s / 2) + 2 b + s % 2 (the T2 bit order).  Lane t of
// the wave converts B bytes 4 s .. 4 s + 3 of lane group g = t / 16 for
// MFMA j = (t / 4) % 4, s = t % 4.
__global__ __launch_bounds__(64) void t2b_convert_kernel(const float* __restrict__ x, int cols, int ngroups,
                                                         unsigned char* __restrict__ ops, int* __restrict__ exps) {
  const int sec = blockIdx.x, b = blockIdx.y, nb = 4 * ngroups;
  const int t = static_cast<int>(threadIdx.x);
  const int g = t >> 4, j = (t >> 2) & 3, sq = t & 3;
  const float* xs = x + static_cast<size_t>(b) * cols + 256 * sec + 64 * g + 16 * j + 8 * (sq >> 1) + (sq & 1);
  const float xv[4] = {xs[0], xs[2], xs[4], xs[6]};
  float amax = fmaxf(fmaxf(fabsf(xv[0]), fabsf(xv[1])), fmaxf(fabsf(xv[2]), fabsf(xv[3])));
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  const int e = amax > 0.f ? __builtin_amdgcn_frexp_expf(amax) : 0;  // amax < 2^e
  unsigned dw[3] = {0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int X = static_cast<int>(rintf(ldexpf(xv[i], 22 - e)));  // |X| <= 2^22
    const int d0 = ((X + 128) & 255) - 128;
    const int X1 = (X - d0) >> 8;
    const int d1 = ((X1 + 128) & 255) - 128;
    const int d2 = (X1 - d1) >> 8;
    dw[0] |= (static_cast<unsigned>(d0) & 255u) << (8 * i);
    dw[1] |= (static_cast<unsigned>(d1) & 255u) << (8 * i);
    dw[2] |= (static_cast<unsigned>(d2) & 255u) << (8 * i);
  }
  const int m = 4 * sec + j, G = b >> 2, n0 = 4 * (b & 3);
  unsigned char* base = ops + (static_cast<size_t>(m) * ngroups + G) * kStepBytes + (16 * g + n0) * 16 + 4 * sq;
#pragma unroll
  for (int d = 0; d < 4; ++d) *(g_u32*)(base + d * 16) = d < 3 ? dw[d] : 0u;
  if (t == 0) exps[sec * nb + b] = e - 22;
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

// kTernary: T2 tiles (tiled arrangement), outputs y[b][row]; otherwise an
// int8 table (row-major or tiled), logits (optional) and argmax keys.
template <int NG, bool kTiled, bool kTernary>
__global__ __launch_bounds__(kThreadsB, 1) void i8b_kernel(const unsigned char* __restrict__ table,
                                                            const float* __restrict__ scale, int rows, int cols,
                                                            const unsigned char* __restrict__ ops,
                                                            const int* __restrict__ exps, float* __restrict__ logits,
                                                            unsigned long long* __restrict__ partials, int nparts,
                                                            const unsigned char* __restrict__ park,
                                                            unsigned* __restrict__ status) {
  // one tile load covers 1 K-step (int8) or 4 (ternary: a 256-value section)
  constexpr int kStepsPerLoad = kTernary ? 4 : 1;
  // row blocks per compute wave and sweep (ternary: 1, so that the unpacked
  // operands of 16 vectors stay in registers)
  constexpr int kR = kTernary ? 1 : 2;
  constexpr int kB = 4 * NG;
  constexpr int kSliceOps = kSliceSteps * NG * kStepBytes;                 // digits of one slice
  constexpr int kSliceBytes = kSliceOps + (kSliceSteps / 4) * kB * 4;      // + its sections' exponents
  extern __shared__ __align__(16) unsigned char smem[];
  int* ready = reinterpret_cast<int*>(smem + 2 * kSliceBytes);  // highest slice staged
  int* done = ready + 1;                                         // [kW]: highest slice a compute wave is done with
  unsigned long long* wkeys = reinterpret_cast<unsigned long long*>(smem + 2 * kSliceBytes + 64);  // [kW][kB]

  const unsigned lane = threadIdx.x & 63u;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const int nblocks = (rows + 15) / 16;
  const int rb0 = static_cast<int>(static_cast<long>(blockIdx.x) * nblocks / gridDim.x);
  const int rb1 = static_cast<int>(static_cast<long>(blockIdx.x + 1) * nblocks / gridDim.x);
  const int nsteps = cols / 64, nslices = nsteps / kSliceSteps;
  const int per_sweep = kCW * kR;
  const int nsweeps = (rb1 - rb0 + per_sweep - 1) / per_sweep;
  if (threadIdx.x == 0) *ready = -1;
  if (threadIdx.x < kW) done[threadIdx.x] = -1;
  __syncthreads();

  bool late = false;
  if (wave == 0) {
    // Staging wave: slice t (sweep t / nslices, K-slice t % nslices) goes
    // into buffer t & 1 once every compute wave is done with slice t - 2.
    const int total = nsweeps * nslices;
    for (int t = 0; t < total; ++t) {
      if (t >= 2) {
        const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
        while (true) {
          const int d = (lane >= 1 && lane < kW) ? lds_acquire(&done[lane]) : t;
          if (__all(d >= t - 2)) break;
          if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
            late = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      const int j = t % nslices;
      unsigned char* dst = smem + (t & 1) * kSliceBytes;
      const unsigned char* src = ops + static_cast<size_t>(j) * kSliceOps;
      for (int o = 0; o < kSliceOps; o += 1024)
        __builtin_amdgcn_global_load_lds(src + o + 16 * lane, (__attribute__((address_space(3))) void*)(dst + o), 16, 0, 0);
      const int ebytes = (kSliceSteps / 4) * kB * 4;  // a multiple of 16
      if (16 * static_cast<int>(lane) < ebytes)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(exps) + static_cast<size_t>(j) * ebytes + 16 * lane,
                                         (__attribute__((address_space(3))) void*)(dst + kSliceOps), 16, 0, 0);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
      lds_publish(ready, t);
    }
  } else {
    const int k = wave - 1;
    const unsigned n = lane & 15u, g = lane >> 4;
    const int vec_in_group = static_cast<int>(n >> 2), digit = static_cast<int>(n & 3u);
    float best[NG];
    unsigned bidx[NG];
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      best[G] = -__builtin_inff();
      bidx[G] = 0xFFFFFFFFu;
    }
    // Row block of slot r in sweep sw, or -1 past the workgroup's range.
    auto block_of = [&](int sw, int r) {
      const int rb = rb0 + sw * per_sweep + k * kR + r;
      return rb < rb1 ? rb : -1;
    };
    // This lane's 16 bytes of the first tile load of row block rb (rb < 0:
    // the park area, results unused).  Row-major int8: rows past the end
    // read the last row; tiled: the block's tiles are consecutive 1 KiB
    // (rows padded with zeros).
    const int nloads = nsteps / kStepsPerLoad;  // tile loads per row block
    constexpr int kStride = kTiled ? 1024 : 64;
    auto row_ptr = [&](int rb) -> const unsigned char* {
      if (rb < 0) return park + 16 * lane;
      if (kTiled) return table + static_cast<size_t>(rb) * nloads * 1024 + 16 * lane;
      int row = rb * 16 + static_cast<int>(lane & 15u);
      row = row < rows ? row : rows - 1;
      return table + static_cast<size_t>(row) * cols + 16 * (lane >> 4);
    };
    // Two register groups of 4 tile loads per row block: one group's loads
    // are in flight while the other is consumed.
    constexpr int kLoads = 4;
    u32x4 xa[kLoads][kR], xb[kLoads][kR];
    const unsigned char* lp[kR];  // each slot's first tile load of the sweep
    int lstride[kR];              // bytes between tile loads, or 0 for a parked slot
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int blk = nsweeps > 0 ? block_of(0, r) : -1;
      lp[r] = row_ptr(blk);
      lstride[r] = blk < 0 ? 0 : kStride;
    }
    auto issue = [&](u32x4(&x)[kLoads][kR], int load0) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u)
#pragma unroll
        for (int r = 0; r < kR; ++r)
          x[u][r] = __builtin_nontemporal_load((g_u32x4*)(lp[r] + lstride[r] * (load0 + u)));
    };
    // End of a 256-value section of the slice in `buf`: the exact sums
    // scaled by this column's exponent (digit weight 2^(8 d); column 4 j + 3
    // is zero).
    auto section_end = [&](const unsigned char* buf, int sec_in_slice, v4i(&iacc)[kR][NG], v4f(&facc)[kR][NG]) {
      const int* ex = reinterpret_cast<const int*>(buf + kSliceOps) + sec_in_slice * kB;
#pragma unroll
      for (int G = 0; G < NG; ++G) {
        const int ev = ex[4 * G + vec_in_group];
        const int e = digit < 3 ? ev + 8 * digit : -1000;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          facc[r][G].x += ldexpf(static_cast<float>(iacc[r][G].x), e);
          facc[r][G].y += ldexpf(static_cast<float>(iacc[r][G].y), e);
          facc[r][G].z += ldexpf(static_cast<float>(iacc[r][G].z), e);
          facc[r][G].w += ldexpf(static_cast<float>(iacc[r][G].w), e);
          iacc[r][G] = v4i{0, 0, 0, 0};
        }
      }
    };
    // One K-step (slice-relative s_in) of every row block and group.
    auto kstep = [&](const unsigned char* buf, int s_in, const v4i(&A)[kR], v4i(&iacc)[kR][NG]) {
#pragma unroll
      for (int G = 0; G < NG; ++G) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(buf + (s_in * NG + G) * kStepBytes + lane * 16);
        const v4i B = {static_cast<int>(bv.x), static_cast<int>(bv.y), static_cast<int>(bv.z), static_cast<int>(bv.w)};
#pragma unroll
        for (int r = 0; r < kR; ++r) iacc[r][G] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[r], B, iacc[r][G], 0, 0, 0);
      }
    };
    // One group: tile loads load0 .. load0 + 3 of every row block.
    auto group = [&](const u32x4(&x)[kLoads][kR], const unsigned char* buf, int load0, v4f(&facc)[kR][NG]) {
      v4i iacc[kR][NG];
#pragma unroll
      for (int r = 0; r < kR; ++r)
#pragma unroll
        for (int G = 0; G < NG; ++G) iacc[r][G] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < kLoads; ++u) {
        const int st0 = ((load0 + u) * kStepsPerLoad) % kSliceSteps;  // first K-step of the load in the slice
        if (kTernary) {
          // a ternary tile is one section: 4 K-steps from the lane's 4 words
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            v4i A[kR];
#pragma unroll
            for (int r = 0; r < kR; ++r) {
              const unsigned w = j == 0 ? x[u][r].x : j == 1 ? x[u][r].y : j == 2 ? x[u][r].z : x[u][r].w;
              int a[4];
              t2_unpack_i8(w, a);
              A[r] = v4i{a[0], a[1], a[2], a[3]};
            }
            kstep(buf, st0 + j, A, iacc);
            // one K-step's operands live at a time (no hoisting of the next
            // K-step's LDS reads or unpack above these instructions)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
          }
          section_end(buf, st0 / 4, iacc, facc);
        } else {
          v4i A[kR];
#pragma unroll
          for (int r = 0; r < kR; ++r)
            A[r] = v4i{static_cast<int>(x[u][r].x), static_cast<int>(x[u][r].y), static_cast<int>(x[u][r].z),
                       static_cast<int>(x[u][r].w)};
          kstep(buf, st0, A, iacc);
          if (u == kLoads - 1) section_end(buf, st0 / 4, iacc, facc);  // 4 int8 K-steps: one section
        }
      }
    };
    // Before the group starting at tile load `load`: enter its slice if it
    // starts one; returns the slice's buffer.
    auto slice_of = [&](int sw, int load) -> const unsigned char* {
      const int st = load * kStepsPerLoad;
      const int t = sw * nslices + st / kSliceSteps;
      if (st % kSliceSteps == 0) {
        lds_publish(&done[wave], t - 1);
        const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
        while (uni(lds_acquire(ready)) < t) {
          if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
            late = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      return smem + (t & 1) * kSliceBytes;
    };
    issue(xa, 0);

    for (int sw = 0; sw < nsweeps; ++sw) {
      v4f facc[kR][NG];
#pragma unroll
      for (int r = 0; r < kR; ++r)
#pragma unroll
        for (int G = 0; G < NG; ++G) facc[r][G] = v4f{0.f, 0.f, 0.f, 0.f};
      for (int l0 = 0; l0 < nloads; l0 += 2 * kLoads) {
        issue(xb, l0 + kLoads);
        __builtin_amdgcn_sched_barrier(0);
        group(xa, slice_of(sw, l0), l0, facc);
        __builtin_amdgcn_sched_barrier(0);
        // the next group: loads l0 + 8 .. of this sweep, or the first ones of
        // the next sweep (parked slots read the park area)
        int next = l0 + 2 * kLoads;
        if (next >= nloads) {
          next = 0;
#pragma unroll
          for (int r = 0; r < kR; ++r) {
            const int blk = sw + 1 < nsweeps ? block_of(sw + 1, r) : -1;
            lp[r] = row_ptr(blk);
            lstride[r] = blk < 0 ? 0 : kStride;
          }
        }
        issue(xa, next);
        __builtin_amdgcn_sched_barrier(0);
        group(xb, slice_of(sw, l0 + kLoads), l0 + kLoads, facc);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Sweep done: per row block, the four columns of each vector summed
      // (quad DPP), times the row scale; lanes 4 j of the quad hold vector
      // 4 G + j's logits of rows 4 g .. 4 g + 3.
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int rb = block_of(sw, r);
        if (rb < 0) continue;
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
                if (logits) ((g_float*)logits)[static_cast<size_t>(b) * rows + row] = a[i];  // ternary: y
                if (!kTernary && a[i] > best[G]) {  // a lane's rows ascend: ties keep the lower row
                  best[G] = a[i];
                  bidx[G] = static_cast<unsigned>(row);
                }
              }
            }
          }
        }
      }
    }
    lds_publish(&done[wave], 0x7FFFFFFF);
    // per vector: the max key over the four lane groups, then per wave in LDS
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      unsigned long long key = (digit == 0 && bidx[G] != 0xFFFFFFFFu) ? argmax_key(best[G], bidx[G]) : 0ull;
      unsigned long long o = __shfl_xor(key, 16, kWave);
      key = o > key ? o : key;
      o = __shfl_xor(key, 32, kWave);
      key = o > key ? o : key;
      if (lane < 16 && digit == 0) wkeys[wave * kB + 4 * G + vec_in_group] = key;
    }
  }
  if (late && lane == 0) __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (!kTernary && threadIdx.x < static_cast<unsigned>(kB)) {
    unsigned long long m = 0ull;
    for (int w = 1; w < kW; ++w) m = wkeys[w * kB + threadIdx.x] > m ? wkeys[w * kB + threadIdx.x] : m;
    partials[static_cast<size_t>(threadIdx.x) * nparts + blockIdx.x] = m;
  }
}

template <int NG>
constexpr size_t i8b_lds() {
  return 2 * (kSliceSteps * NG * kStepBytes + (kSliceSteps / 4) * 4 * NG * 4) + 64 + kW * 4 * NG * 8;
}

// Operand area (from its first 256-byte boundary): B-operand digits for
// `cap` values per vector, a 1 KiB park area (what an idle load slot reads),
// the section exponents, a status word.
struct OpsLayout {
  unsigned char* ops;
  unsigned char* park;
  int* exps;
  unsigned* status;
};
OpsLayout ops_layout(void* area, int64_t cap, int32_t batch) {
  OpsLayout L;
  L.ops = reinterpret_cast<unsigned char*>((reinterpret_cast<uintptr_t>(area) + 255) & ~uintptr_t{255});
  L.park = L.ops + static_cast<size_t>(cap / 64) * (batch / 4) * kStepBytes;
  L.exps = reinterpret_cast<int*>(L.park + kStepBytes);
  L.status = reinterpret_cast<unsigned*>(L.exps + (cap / 256) * batch);
  return L;
}

long batch_grid(int64_t rows, size_t cap) {
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  long grid = cus;
  const long nblocks = (rows + 15) / 16;
  if (grid > nblocks) grid = nblocks;
  if (grid > static_cast<long>(cap)) grid = static_cast<long>(cap);
  return grid;
}

}  // namespace

size_t batch_operand_bytes(int64_t cap, int32_t batch) {
  if (batch < 4) return 0;
  return 256 + static_cast<size_t>(cap / 64) * (batch / 4) * kStepBytes + kStepBytes + static_cast<size_t>(cap / 256) * batch * 4 + 64;
}

size_t i8b_operand_bytes(int32_t batch) { return batch_operand_bytes(kMaxInt8Cols, batch); }

bool i8b_supported(int64_t cols, int32_t batch) {
  return (batch == 4 || batch == 8 || batch == 16) && cols % (64 * kSliceSteps) == 0 && cols <= kMaxInt8Cols;
}

int launch_i8b(const int8_t* table, bool tiled, const float* s, int64_t rows, int64_t cols, const float* h,
               int32_t batch, unsigned long long* partials, size_t nparts, unsigned char* ops_area, float* logits,
               int32_t* token, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int ng = batch / 4;
  const OpsLayout L = ops_layout(ops_area, kMaxInt8Cols, batch);
  const int c32 = static_cast<int>(cols), r32 = static_cast<int>(rows);
  hipLaunchKernelGGL(i8b_convert_kernel, dim3(c32 / 256, batch), dim3(64), 0, st, h, c32, ng, L.ops, L.exps);
  const long grid = batch_grid(rows, nparts);
  const int np = static_cast<int>(nparts);
  const unsigned char* tp = reinterpret_cast<const unsigned char*>(table);
#define PWG_I8B(NG, T)                                                                                               \
  hipLaunchKernelGGL((i8b_kernel<NG, T, false>), dim3(grid), dim3(kThreadsB), i8b_lds<NG>(), st, tp, s, r32, c32, L.ops, \
                     L.exps, logits, partials, np, L.park, L.status)
  if (tiled) {
    if (ng == 1) PWG_I8B(1, true);
    else if (ng == 2) PWG_I8B(2, true);
    else PWG_I8B(4, true);
  } else {
    if (ng == 1) PWG_I8B(1, false);
    else if (ng == 2) PWG_I8B(2, false);
    else PWG_I8B(4, false);
  }
#undef PWG_I8B
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "int8_gemv_argmax (matrix-core batch) launch: %s", hipGetErrorString(e));
  return launch_argmax_reduce_batch(partials, static_cast<int>(grid), nparts, batch, token, stream);
}

int launch_t2b(const void* w_tiled, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch, float* y,
               void* ops_area, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int ng = batch / 4;
  const OpsLayout L = ops_layout(ops_area, cols, batch);
  const int c32 = static_cast<int>(cols), r32 = static_cast<int>(rows);
  hipLaunchKernelGGL(t2b_convert_kernel, dim3(c32 / 256, batch), dim3(64), 0, st, x, c32, ng, L.ops, L.exps);
  const long grid = batch_grid(rows, 1u << 20);
  const unsigned char* tp = static_cast<const unsigned char*>(w_tiled);
  unsigned long long* no_parts = nullptr;
#define PWG_T2B(NG)                                                                                                   \
  hipLaunchKernelGGL((i8b_kernel<NG, true, true>), dim3(grid), dim3(kThreadsB), i8b_lds<NG>(), st, tp, s, r32, c32, L.ops, \
                     L.exps, y, no_parts, 0, L.park, L.status)
  if (ng == 1) PWG_T2B(1);
  else if (ng == 2) PWG_T2B(2);
  else PWG_T2B(4);
#undef PWG_T2B
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "ternary_gemv_tiled launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

}  // namespace pwg
