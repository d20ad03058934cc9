// Persistent level-ordered decode step: one kernel per step.
//
// Page "The Neutrino Engine", section "A 104 microsecond floor inside a 694
// microsecond step" and Fig. 1: most of a measured step was spent in about
// 120 kernel boundaries and their dependency chains, and one fused kernel
// with software barriers replaced the launches with similar waits.  Here the
// whole step (embedding row, every level in decoder order, output projection
// and argmax) runs as one kernel with one workgroup per CU.  Two things differ
// from a plain fused kernel:
//  * weights do not depend on activations, so before waiting for level L-1
//    each wave already has the first two tiles of its level-L rows in flight
//    (up to 16 MiB across the chip), and HBM keeps streaming through the wait;
//  * the level barrier is hierarchical over the 8 XCDs: workgroups of one XCD
//    count arrivals with an atomic in that XCD's L2, the last one publishes
//    the XCD's arrival to memory in 8 replicated flag lines, and waiters poll
//    the replica of their own XCD (no single hot address).  The kernel asks
//    for more than half of a CU's LDS, so every CU holds exactly one of its
//    workgroups and an XCD holds as many as it has CUs, whichever XCD the
//    dispatcher starts from.
// A level's outputs are stored device-coherent (they bypass the L2) before a
// workgroup arrives, so the next level may read them from any XCD.
// Every wait is bounded: after ~0.5 s a workgroup records a timeout in the
// status word and leaves, so a broken schedule ends with an error, not a hang.
#include <hip/hip_runtime.h>

#include <vector>

#include "device_common.h"
#include "pwg_internal.h"
#include "t2_rows.h"

namespace pwg {
namespace {

using namespace dev;

constexpr int kWpb = 8;              // waves per workgroup (one workgroup per CU)
constexpr int kThreads = kWpb * 64;
constexpr int kMaxC = 3;             // ternary levels: cols <= 64 * 64 * 3 = 12288
constexpr int kMaxI8C = 4;           // output projection: hidden <= 4096
constexpr int kReplicas = 8;
constexpr unsigned long long kSpinLimit = 50000000ull;  // 0.5 s at the 100 MHz real-time counter

enum : unsigned { kBarrierL2 = 0, kBarrierFlat = 1 };
enum : unsigned { kStatusOk = 0, kStatusTimeout = 1 };

// Dynamic LDS requested by the step kernel: more than half of the 160 KiB of
// a CU, so no CU can hold two of its workgroups.
constexpr size_t kStepLdsBytes = 96 * 1024;

struct DevLevel {
  const u32x4* w;
  const float* scale;
  const float* x;
  float* y;
  int rows;
  int cols;
  int nchunks;  // cols / 64
  int c;        // chunks per lane
};

// Device-side plan, written by pwg_step_plan into the workspace.
struct alignas(256) Plan {
  unsigned status;
  unsigned gen;            // completed steps (barrier epochs derive from it)
  unsigned n_levels;
  unsigned n_barriers;     // barriers per step: n_levels + 1 (ordered) or 1
  unsigned mode;           // kBarrierL2 or kBarrierFlat
  unsigned grid;
  unsigned per_xcd[8];
  unsigned xcd_mask;
  unsigned ordered;        // 1: level barriers; 0: levels only ordered within each workgroup
  int vocab, hidden, i8c;
  const u32x4* out_table;
  const float* out_scale;
  const float* h;
  const u32x4* emb_table;
  const float* emb_scale;
  const int* token_in;
  int* token_out;
  u32x4* emb_row_out;
  float* emb_scale_out;
  float4* emb_deq_out;
  float* logits_out;
  // offsets (bytes from the plan) of the barrier words, partial keys and level table
  unsigned long long counters_off, flags_off, partials_off, levels_off, calib_off;
};

constexpr size_t kCountersBytes = 8 * 128;                  // one 64-bit counter per 128-byte line
constexpr size_t kFlagsBytes = kReplicas * 256 + 4096;      // 8 XCD flags per replica line (+ flat mode)
constexpr size_t kMaxGrid = 1024;

__device__ __forceinline__ unsigned ld_sc(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_sc64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// true when flag value f has reached epoch e (wrap-safe)
__device__ __forceinline__ bool reached(unsigned f, unsigned e) { return static_cast<int>(f - e) >= 0; }

__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7u; }

struct Barrier {
  Plan* plan;
  unsigned long long* counters;
  unsigned* flags;
  unsigned xcd;
  unsigned base;  // gen * n_barriers

  // Arrive at barrier j: the workgroup's stores are complete before it counts.
  __device__ void arrive(unsigned j) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned epoch = base + j + 1;
      if (plan->mode == kBarrierL2) {
        // workgroup scope: the atomic executes in this XCD's L2, shared by its CUs
        const unsigned long long old =
            __hip_atomic_fetch_add(&counters[xcd * 16], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const unsigned long long target = static_cast<unsigned long long>(epoch) * plan->per_xcd[xcd];
        if (old + 1 == target) {
          for (int r = 0; r < kReplicas; ++r) st_sc(&flags[r * 64 + xcd], epoch);
        }
      } else {
        st_sc(&flags[kReplicas * 64 + blockIdx.x], epoch);
      }
    }
  }

  // Wait until every workgroup has arrived at barrier j.  Returns true when
  // the wait timed out; the answer is the same for every thread of the block.
  __device__ bool wait(unsigned j) {
    __shared__ int timed_out;
    if (threadIdx.x < 64) {
      const unsigned epoch = base + j + 1;
      const unsigned lane = threadIdx.x;
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      bool late = false;
      while (true) {
        bool ok = true;
        if (plan->mode == kBarrierL2) {
          if (lane < 8 && ((plan->xcd_mask >> lane) & 1u)) ok = reached(ld_sc(&flags[xcd * 64 + lane]), epoch);
        } else {
          for (unsigned b = lane; b < plan->grid; b += 64) ok = ok && reached(ld_sc(&flags[kReplicas * 64 + b]), epoch);
        }
        if (__all(ok)) break;
        // the real-time counter is a scalar read, so `late` is uniform
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
          late = true;
          break;
        }
      }
      if (lane == 0) {
        timed_out = late ? 1 : 0;
        if (late) st_sc(&plan->status, kStatusTimeout);
      }
    }
    __syncthreads();
    return timed_out != 0;
  }
};

// ----------------------------------------------------------------- ternary
// One ternary level for one wave: read the level input and prime NB tiles of
// the wave's rows, wait for the previous level, convert the input to limb
// planes, then stream the rows (t2_rows.h).  Returns false when the wait timed
// out (the same answer in every thread of the block).
// Wave 0 polls the barrier, so it issues no loads before the wait: a wave's
// loads complete in order, and its polls would otherwise queue behind them.
// The activation is loaded by waves 1..7; wave 0 loads its first tiles
// after the wait.
template <int C, int U, int NB, int G, class Wait>
__device__ bool t2_level(const DevLevel& L, long r0, long r1, unsigned lane, unsigned wave, unsigned* lds,
                         Wait&& wait_prev) {
  T2XRegs<G> xr;
  t2_x_load<G>(L.x, L.cols, xr, 64);
  T2Tile<C, U> tiles[NB];
  if (wave != 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (r0 + b * U < r1) t2_tile_load<C, U>(L.w, L.scale, L.nchunks, r0 + b * U, r1, lane, tiles[b]);
  }
  if (wait_prev()) return false;
  if (wave == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
      if (r0 + b * U < r1) t2_tile_load<C, U>(L.w, L.scale, L.nchunks, r0 + b * U, r1, lane, tiles[b]);
  }
  int* lds_e = reinterpret_cast<int*>(lds + L.nchunks * kT2ChunkDwords);
  t2_x_convert<G>(xr, L.cols, lds, lds_e, 64);
  T2Lane<C> st;
  t2_lane_init<C>(st, lds, lds_e, L.nchunks, lane);
  for (long r = r0; r < r1; r += NB * U) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const long rb = r + b * U;
      if (rb < r1) {
        const float v = t2_tile_compute<C, U>(st, tiles[b], rb, r1);
        const long row = rb + row_of<U>(static_cast<int>(lane >> 4));
        if ((lane & (64u / U - 1u)) == 0u && row < r1) st_sc(L.y + row, v);
        if (rb + NB * U < r1) t2_tile_load<C, U>(L.w, L.scale, L.nchunks, rb + NB * U, r1, lane, tiles[b]);
      }
    }
  }
  __syncthreads();  // every wave has its limbs in registers before the LDS is reused
  return true;
}

// ----------------------------------------------------------------- int8 vocab
template <int U>
struct I8Tile {
  u32x4 q[U][kMaxI8C];
  float s;  // scale of the tile row this lane reports
};

template <int U>
__device__ __forceinline__ void i8_tile_load(const Plan& P, long r, long r1, unsigned lane, I8Tile<U>& t) {
  const int nchunks = P.hidden >> 4;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (r + u < r1) {
      const u32x4* row = P.out_table + (r + u) * static_cast<long>(nchunks);
#pragma unroll
      for (int c = 0; c < kMaxI8C; ++c) {
        unsigned chunk = lane + 64u * c;
        chunk = chunk < static_cast<unsigned>(nchunks) ? chunk : static_cast<unsigned>(nchunks - 1);
        t.q[u][c] = __builtin_nontemporal_load(row + chunk);
      }
    }
  }
  const long rs = r + row_of<U>(static_cast<int>(lane >> 4));
  t.s = rs < r1 ? P.out_scale[rs] : 0.f;
}

// Logits of tile rows [r, r + U); each reporting lane (one per tile row)
// folds its row into its running (max, lowest index).
template <int U>
__device__ __forceinline__ void i8_tile_compute(const Plan& P, long r, long r1, unsigned lane, const I8Tile<U>& t,
                                                const unsigned (&H)[kMaxI8C][12], const int (&Ec)[kMaxI8C],
                                                float& best, unsigned& best_idx) {
  float p[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    p[u] = 0.f;
    if (r + u < r1) {
#pragma unroll
      for (int c = 0; c < kMaxI8C; ++c) {
        int a0 = 0, a1 = 0, a2 = 0;
        const unsigned qd[4] = {t.q[u][c].x, t.q[u][c].y, t.q[u][c].z, t.q[u][c].w};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          a0 = dot4(qd[g], H[c][3 * g + 0], a0);
          a1 = dot4(qd[g], H[c][3 * g + 1], a1);
          a2 = dot4(qd[g], H[c][3 * g + 2], a2);
        }
        // each limb sum is exact in float32 (|a| <= 16*127*128 < 2^24); the shifts are exact
        const float pc = fmaf(static_cast<float>(a2), 65536.0f, fmaf(static_cast<float>(a1), 256.0f, static_cast<float>(a0)));
        p[u] += ldexpf(pc, Ec[c]);
      }
    }
  }
  const float logit = t.s * tile_reduce<U>(p);
  const long row = r + row_of<U>(static_cast<int>(lane >> 4));
  if ((lane & (64u / U - 1u)) == 0u && row < r1) {
    if (P.logits_out) P.logits_out[row] = logit;
    // rows of one lane ascend, so ties keep the lower index
    if (logit > best) {
      best = logit;
      best_idx = static_cast<unsigned>(row);
    }
  }
}

template <bool kOrdered>
__global__ __launch_bounds__(kThreads, 1) void step_kernel(Plan* plan) {
  extern __shared__ __align__(16) unsigned lds[];
  const Plan& P = *plan;
  char* base_ptr = reinterpret_cast<char*>(plan);
  Barrier bar;
  bar.plan = plan;
  bar.counters = reinterpret_cast<unsigned long long*>(base_ptr + P.counters_off);
  bar.flags = reinterpret_cast<unsigned*>(base_ptr + P.flags_off);
  bar.xcd = xcc_id();
  const unsigned gen = ld_sc(&plan->gen);
  bar.base = gen * P.n_barriers;
  const DevLevel* levels = reinterpret_cast<const DevLevel*>(base_ptr + P.levels_off);
  unsigned long long* partials = reinterpret_cast<unsigned long long*>(base_ptr + P.partials_off);

  const unsigned lane = threadIdx.x & 63u;
  const unsigned wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long gw = static_cast<long>(blockIdx.x) * kWpb + wave, nw = static_cast<long>(gridDim.x) * kWpb;

  // embedding row of the previous token (workgroup 0)
  if (blockIdx.x == 0) {
    const int id = *P.token_in;
    const bool ok = id >= 0 && id < P.vocab;
    const int nchunks = P.hidden >> 4;
    const float s = ok ? P.emb_scale[id] : __builtin_nanf("");
    if (threadIdx.x == 0) *P.emb_scale_out = s;
    for (int c = threadIdx.x; c < nchunks; c += kThreads) {
      const u32x4 v = ok ? P.emb_table[static_cast<size_t>(id) * nchunks + c] : u32x4{0u, 0u, 0u, 0u};
      P.emb_row_out[c] = v;
      if (P.emb_deq_out) {
        const unsigned wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          P.emb_deq_out[4 * c + q] =
              ok ? make_float4(static_cast<float>(static_cast<int8_t>(wd[q] & 0xFF)) * s,
                               static_cast<float>(static_cast<int8_t>((wd[q] >> 8) & 0xFF)) * s,
                               static_cast<float>(static_cast<int8_t>((wd[q] >> 16) & 0xFF)) * s,
                               static_cast<float>(static_cast<int8_t>(wd[q] >> 24)) * s)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }

  for (unsigned li = 0; li < P.n_levels; ++li) {
    const DevLevel L = levels[li];
    const long r0 = gw * L.rows / nw, r1 = (gw + 1) * L.rows / nw;
    auto wait_prev = [&]() -> bool { return (kOrdered && li > 0) ? bar.wait(li - 1) : false; };
    bool ok;
    // G covers cols/16 groups with the 448 loading threads of waves 1..7
    if (L.c == 1) ok = t2_level<1, 4, 3, 1>(L, r0, r1, lane, wave, lds, wait_prev);
    else if (L.c == 2) ok = t2_level<2, 2, 2, 2>(L, r0, r1, lane, wave, lds, wait_prev);
    else ok = t2_level<3, 1, 1, 2>(L, r0, r1, lane, wave, lds, wait_prev);
    if (!ok) return;
    if (kOrdered) bar.arrive(li);
  }

  // output projection + per-workgroup argmax
  {
    constexpr int U = 2, NB = 2, G = 3;  // G * 448 threads * 4 elements covers hidden <= 4096
    const long r0 = gw * P.vocab / nw, r1 = (gw + 1) * P.vocab / nw;
    I8XRegs<G> hr;
    i8_x_load<G>(P.h, P.hidden, hr, 64);
    I8Tile<U> tiles[NB];
    if (wave != 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (r0 + b * U < r1) i8_tile_load<U>(P, r0 + b * U, r1, lane, tiles[b]);
    }
    if (kOrdered && P.n_levels > 0 && bar.wait(P.n_levels - 1)) return;
    if (wave == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (r0 + b * U < r1) i8_tile_load<U>(P, r0 + b * U, r1, lane, tiles[b]);
    }
    const int nchunks = P.hidden >> 4;
    int* lds_e = reinterpret_cast<int*>(lds + nchunks * kI8ChunkDwords);
    i8_x_convert<G>(hr, P.hidden, lds, lds_e, 64);
    unsigned H[kMaxI8C][12];
    int Ec[kMaxI8C];
#pragma unroll
    for (int c = 0; c < kMaxI8C; ++c) {
      const unsigned chunk = lane + 64u * c;
      const bool ok = chunk < static_cast<unsigned>(nchunks);
      Ec[c] = ok ? -lds_e[chunk] : 0;
      const u32x4* src = reinterpret_cast<const u32x4*>(lds + (ok ? chunk : 0u) * kI8ChunkDwords);
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const u32x4 v = ok ? src[q] : u32x4{0u, 0u, 0u, 0u};
        H[c][4 * q] = v.x; H[c][4 * q + 1] = v.y; H[c][4 * q + 2] = v.z; H[c][4 * q + 3] = v.w;
      }
    }
    float best = -__builtin_inff();
    unsigned best_idx = 0xFFFFFFFFu;
    for (long r = r0; r < r1; r += NB * U) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const long rb = r + b * U;
        if (rb < r1) {
          i8_tile_compute<U>(P, rb, r1, lane, tiles[b], H, Ec, best, best_idx);
          if (rb + NB * U < r1) i8_tile_load<U>(P, rb + NB * U, r1, lane, tiles[b]);
        }
      }
    }
    // wave (max, lowest index) over its reporting lanes, then the workgroup's
    unsigned long long k = best_idx == 0xFFFFFFFFu ? 0ull : argmax_key(best, best_idx);
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(k, off, kWave);
      k = o > k ? o : k;
    }
    __shared__ unsigned long long wkeys[kWpb];
    if (lane == 0) wkeys[wave] = k;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long m = 0ull;
      for (int i = 0; i < kWpb; ++i) m = wkeys[i] > m ? wkeys[i] : m;
      st_sc64(&partials[blockIdx.x], m);
    }
  }
  const unsigned final_barrier = kOrdered ? P.n_levels : 0u;
  bar.arrive(final_barrier);
  if (blockIdx.x == 0) {
    if (bar.wait(final_barrier)) return;
    if (threadIdx.x < 64) {
      unsigned long long k = 0ull;
      for (unsigned b = threadIdx.x; b < gridDim.x; b += 64) {
        const unsigned long long o = ld_sc64(&partials[b]);
        k = o > k ? o : k;
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(k, off, kWave);
        k = o > k ? o : k;
      }
      if (threadIdx.x == 0) {
        *P.token_out = static_cast<int>(argmax_key_index(k));
        st_sc(&plan->gen, gen + 1);
      }
    }
  }
}

__global__ void xcc_calibrate(unsigned* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

// ----------------------------------------------------------------- host side
struct Layout {
  size_t plan = 0, counters = 0, flags = 0, partials = 0, levels = 0, calib = 0, total = 0;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

Layout layout_for(int n_levels) {
  Layout L;
  L.plan = 0;
  L.counters = align_up(sizeof(Plan), 256);
  L.flags = L.counters + kCountersBytes;
  L.partials = align_up(L.flags + kFlagsBytes, 256);
  L.levels = align_up(L.partials + kMaxGrid * 8, 256);
  L.calib = align_up(L.levels + static_cast<size_t>(n_levels) * sizeof(DevLevel), 256);
  L.total = align_up(L.calib + kMaxGrid * 4, 256);
  return L;
}

struct GridInfo {
  int grid = 0;
  size_t lds = 0;
};

size_t step_lds_bytes(const pwg_step_desc* d) {
  size_t lds = i8_lds_bytes(d->hidden);
  for (int i = 0; i < d->n_levels; ++i) {
    const size_t b = t2_lds_bytes(d->levels[i].cols);
    lds = b > lds ? b : lds;
  }
  return lds > kStepLdsBytes ? lds : kStepLdsBytes;
}

int grid_for(const pwg_step_desc* d, GridInfo* gi) {
  int dev = 0, cus = 0, occ = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  gi->lds = step_lds_bytes(d);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(&step_kernel<true>), kThreads, gi->lds);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "persistent step: device query failed: %s", hipGetErrorString(e));
  if (occ < 1) return fail(PWG_ERR_UNSUPPORTED, "persistent step: kernel does not fit on a CU");
  gi->grid = cus < static_cast<int>(kMaxGrid) ? cus : static_cast<int>(kMaxGrid);  // one workgroup per CU
  return PWG_OK;
}

}  // namespace

size_t step_persistent_workspace(const pwg_step_desc* d) {
  if (!d || (d->schedule != PWG_SCHEDULE_PERSISTENT && d->schedule != PWG_SCHEDULE_STREAM) || d->n_levels < 0) return 0;
  return layout_for(d->n_levels).total + 256;  // + 256 for aligning the plan
}

static Plan* plan_ptr(const pwg_step_desc* d, size_t ws_offset) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(d->workspace) + ws_offset;
  return reinterpret_cast<Plan*>(align_up(p, 256));
}

int step_persistent_plan(const pwg_step_desc* d, size_t ws_offset, void* stream) {
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    if (L.cols > 64 * 64 * kMaxC)
      return fail(PWG_ERR_UNSUPPORTED, "pwg_step_plan: persistent schedule supports cols <= %d (level %d has %lld)",
                  64 * 64 * kMaxC, i, (long long)L.cols);
    if (L.rows >= (int64_t{1} << 31)) return fail(PWG_ERR_ARG, "pwg_step_plan: level %d has too many rows", i);
  }
  if (d->hidden > 16 * 64 * kMaxI8C)
    return fail(PWG_ERR_UNSUPPORTED, "pwg_step_plan: persistent schedule supports hidden <= %d", 16 * 64 * kMaxI8C);
  GridInfo gi;
  const int rc = grid_for(d, &gi);
  if (rc != PWG_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Layout lay = layout_for(d->n_levels);
  Plan* dplan = plan_ptr(d, ws_offset);
  char* dbase = reinterpret_cast<char*>(dplan);

  // XCD census: one workgroup per CU (same LDS request as the step kernel),
  // so the count on each XCD is that XCD's number of CUs.
  hipError_t e = hipMemsetAsync(dbase, 0, lay.total, st);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(xcc_calibrate, dim3(gi.grid), dim3(kThreads), gi.lds, st, reinterpret_cast<unsigned*>(dbase + lay.calib));
    e = hipGetLastError();
  }
  std::vector<unsigned> xcc(gi.grid);
  if (e == hipSuccess) e = hipMemcpyAsync(xcc.data(), dbase + lay.calib, gi.grid * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_plan: %s", hipGetErrorString(e));
  unsigned census[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int b = 0; b < gi.grid; ++b) census[xcc[b] & 7u] += 1;
  // The L2 barrier is valid when every XCD has the same number of CUs (then
  // any placement of one workgroup per CU gives the same per-XCD counts).
  bool uniform = true;
  for (int x = 1; x < 8; ++x) uniform = uniform && census[x] == census[0];

  Plan h{};
  h.status = kStatusOk;
  h.gen = 0;
  h.n_levels = static_cast<unsigned>(d->n_levels);
  h.ordered = d->schedule == PWG_SCHEDULE_STREAM ? 0u : 1u;
  h.n_barriers = h.ordered ? h.n_levels + 1 : 1u;  // unordered: only the final (argmax) barrier
  h.mode = uniform && census[0] > 0 ? kBarrierL2 : kBarrierFlat;
  h.grid = static_cast<unsigned>(gi.grid);
  h.xcd_mask = 0;
  for (int x = 0; x < 8; ++x) {
    h.per_xcd[x] = census[x];
    if (census[x]) h.xcd_mask |= 1u << x;
  }
  h.vocab = static_cast<int>(d->vocab);
  h.hidden = static_cast<int>(d->hidden);
  h.i8c = kMaxI8C;
  h.out_table = reinterpret_cast<const u32x4*>(d->out_table);
  h.out_scale = d->out_scale;
  h.h = d->h;
  h.emb_table = reinterpret_cast<const u32x4*>(d->emb_table);
  h.emb_scale = d->emb_scale;
  h.token_in = d->token_in;
  h.token_out = d->token_out;
  h.emb_row_out = reinterpret_cast<u32x4*>(d->emb_row_out);
  h.emb_scale_out = d->emb_scale_out;
  h.emb_deq_out = reinterpret_cast<float4*>(d->emb_deq_out);
  h.logits_out = d->logits_out;
  h.counters_off = lay.counters;
  h.flags_off = lay.flags;
  h.partials_off = lay.partials;
  h.levels_off = lay.levels;
  h.calib_off = lay.calib;
  std::vector<DevLevel> lv(d->n_levels);
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    lv[i].w = static_cast<const u32x4*>(L.w_packed);
    lv[i].scale = L.row_scale;
    lv[i].x = L.x;
    lv[i].y = L.y;
    lv[i].rows = static_cast<int>(L.rows);
    lv[i].cols = static_cast<int>(L.cols);
    lv[i].nchunks = static_cast<int>(L.cols / 64);
    lv[i].c = static_cast<int>((L.cols / 64 + 63) / 64);
  }
  e = hipMemcpyAsync(dplan, &h, sizeof(Plan), hipMemcpyHostToDevice, st);
  if (e == hipSuccess && d->n_levels > 0)
    e = hipMemcpyAsync(dbase + lay.levels, lv.data(), lv.size() * sizeof(DevLevel), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_plan: %s", hipGetErrorString(e));
  return PWG_OK;
}

int step_persistent_launch(const pwg_step_desc* d, size_t ws_offset, void* stream) {
  GridInfo gi;
  const int rc = grid_for(d, &gi);
  if (rc != PWG_OK) return rc;
  Plan* dplan = plan_ptr(d, ws_offset);
  if (d->schedule == PWG_SCHEDULE_STREAM)
    hipLaunchKernelGGL(step_kernel<false>, dim3(gi.grid), dim3(kThreads), gi.lds, reinterpret_cast<hipStream_t>(stream), dplan);
  else
    hipLaunchKernelGGL(step_kernel<true>, dim3(gi.grid), dim3(kThreads), gi.lds, reinterpret_cast<hipStream_t>(stream), dplan);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "persistent step launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

int step_persistent_status(const pwg_step_desc* d, size_t ws_offset, void* stream) {
  Plan* dplan = plan_ptr(d, ws_offset);
  unsigned s = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&s, &dplan->status, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_status: %s", hipGetErrorString(e));
  if (s == kStatusTimeout) return fail(PWG_ERR_HIP, "persistent step: a level barrier timed out");
  return PWG_OK;
}

}  // namespace pwg
