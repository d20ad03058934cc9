// Small-batch ternary GEMV and int8 output projection + argmax on the CDNA4
// matrix cores, one call per matrix.
//
// Page "The Neutrino Engine", section "The 0.6B model does not get to
// decide": the large model scores a draft of several tokens in one batched
// pass, so each table is read once for all of them.  Here
// Y[b, r] = s_r * sum_k W_rk X[b, k] for B = 4, 8 or 16 vectors, and for int8
// tables also the greedy argmax of each vector (lowest row on ties).  The
// operand digits and the arithmetic are those of batch_core.h; a conversion
// kernel writes each call's digits into the workspace.
//
// Work.  A workgroup takes a contiguous range of 16-row blocks and walks it in
// sweeps: in each sweep 7 compute waves hold one (ternary) or two (int8) row
// blocks each and run over the whole K range in lock step through K-slices of
// 1,024 values, which a staging wave copies into two LDS buffers ahead of use
// (a 16-vector B operand for all of K would not fit in LDS).  Each compute
// wave keeps the tile loads of the next one or two register groups in flight,
// across slice and sweep boundaries.  Lane L = 16 q + i of an int8 tile load
// reads row i, bytes 16 q .. 16 q + 15 of the 64-value K-step: the A operand
// as stored (row-major tables gather the same bytes from 16 rows).
#include "batch_core.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

using namespace bcore;

constexpr int kThreadsB = bcore::kThreads;

__global__ __launch_bounds__(64) void i8b_convert_kernel(const float* __restrict__ h, int cols, int ngroups,
                                                         unsigned char* __restrict__ ops, int* __restrict__ exps) {
  convert_int8_section(h + static_cast<size_t>(blockIdx.y) * cols, blockIdx.x, blockIdx.y, ngroups, ops, exps,
                       threadIdx.x);
}

__global__ __launch_bounds__(64) void t2b_convert_kernel(const float* __restrict__ x, int cols, int ngroups,
                                                         unsigned char* __restrict__ ops, int* __restrict__ exps) {
  convert_ternary_block(x + static_cast<size_t>(blockIdx.y) * cols, blockIdx.x, blockIdx.y, ngroups, ops, exps,
                        threadIdx.x);
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
  using Core = Compute<NG, kTernary>;
  constexpr int kStepsPerLoad = Core::kStepsPerLoad;
  constexpr int kR = Core::kR;
  constexpr int kB = 4 * NG;
  constexpr int kSliceOps = SliceShape<NG>::kOps;
  constexpr int kSliceBytes = SliceShape<NG>::kBytes;
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
      const int ebytes = SliceShape<NG>::kExpBytes;  // a multiple of 16
      if (16 * static_cast<int>(lane) < ebytes)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const unsigned char*>(exps) + static_cast<size_t>(j) * ebytes + 16 * lane,
                                         (__attribute__((address_space(3))) void*)(dst + kSliceOps), 16, 0, 0);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
      lds_publish(ready, t);
    }
  } else {
    const int k = wave - 1;
    const Core core(lane);
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
    // Two register groups of kLoads tile loads per row block: one group's
    // loads are in flight while the other is consumed.
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
        core.group(xa, slice_of(sw, l0), l0, facc);
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
        core.group(xb, slice_of(sw, l0 + kLoads), l0 + kLoads, facc);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int rb = block_of(sw, r);
        if (rb >= 0) core.finish(facc, r, rb, scale, rows, logits, best, bidx);  // ternary: logits is y
      }
    }
    lds_publish(&done[wave], 0x7FFFFFFF);
    core.wave_keys(best, bidx, wkeys + wave * kB);
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
  return 2 * SliceShape<NG>::kBytes + 64 + kW * 4 * NG * 8;
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
  hipLaunchKernelGGL(t2b_convert_kernel, dim3(c32 / 1024, batch), dim3(64), 0, st, x, c32, ng, L.ops, L.exps);
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
