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

#include <cmath>
#include <vector>

#include "chain_input.h"
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
// state words: [0] status, [1] completed steps (barrier epochs derive from it)
enum : unsigned { kStateStatus = 0, kStateGen = 1 };



struct DevLevel {
  const u32x4* w;
  const float* scale;
  const float* x;
  float* y;
  int rows;
  int cols;
  int nchunks;  // cols / 64
  int c;        // chunks per lane
  chain::DevInput in;  // how x is formed (op 0: x as given)
};

// Device-side plan, written by pwg_step_plan into the workspace.  It is
// constant while a step runs (the kernel takes it as a read-only argument,
// so its fields are read with scalar loads); the words the kernel writes
// live in the state, counter, flag and partial-key areas that follow it.
struct alignas(256) Plan {
  unsigned n_levels;
  unsigned n_barriers;     // barriers per step: n_levels + 1
  unsigned mode;           // kBarrierL2 or kBarrierFlat
  unsigned grid;
  unsigned per_xcd[8];
  unsigned xcd_mask;
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
  chain::DevInput h_in;  // how h is formed (op 0: h as given)
  // offsets (bytes from the plan) of the state words, barrier words, partial keys and level table
  unsigned long long state_off, counters_off, flags_off, partials_off, levels_off, calib_off;
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
  const Plan* plan;
  unsigned* state;
  unsigned long long* counters;
  unsigned* flags;
  unsigned xcd;
  unsigned base;  // gen * n_barriers

  // Arrive at barrier j: the workgroup's stores are complete before it counts.
  __device__ __forceinline__ void arrive(unsigned j) {
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

  // Arrival by the control wave alone, after it stored the workgroup's
  // outputs of the level: the agent-scope release writes back this XCD's L2
  // and waits for the wave's stores, so the outputs are visible device-wide
  // before the count.  The compute waves are not held up: their outstanding
  // loads are weight prefetches, which need no ordering.
  __device__ __forceinline__ void arrive_release(unsigned j) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (threadIdx.x == 0) {
      const unsigned epoch = base + j + 1;
      if (plan->mode == kBarrierL2) {
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
  __device__ __forceinline__ bool wait(unsigned j) {
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
          for (unsigned b0 = 0; b0 < plan->grid; b0 += 64)  // wave-uniform trip count
            if (b0 + lane < plan->grid) ok = ok && reached(ld_sc(&flags[kReplicas * 64 + b0 + lane]), epoch);
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
        if (late) st_sc(&state[kStateStatus], kStatusTimeout);
      }
    }
    __syncthreads();
    return timed_out != 0;
  }
};

// ----------------------------------------------------------------- streaming
// LDS budget of the step kernel (bytes).
constexpr int kComputeWaves = kWpb - 1;                 // waves 1..7; wave 0 is the control wave
constexpr int kRing = 8;                                // 1 KiB ring slots per compute wave
constexpr int kSlotBytes = 1024;                        // 64 lanes x 16 bytes
constexpr int kMaxT2Cols = 64 * 64 * kMaxC;             // 12288
constexpr int kMaxWgRows = 640;                         // rows of one level per workgroup
constexpr size_t kRingBytes = static_cast<size_t>(kComputeWaves) * kRing * kSlotBytes;
constexpr size_t kStageBytes = kMaxT2Cols * 4;
constexpr size_t kPlaneBytes = static_cast<size_t>(kMaxT2Cols / 64) * (kT2ChunkDwords + 1) * 4;
constexpr size_t kScaleBytes = 2 * kMaxWgRows * 4;
constexpr size_t kOutBytes = kMaxWgRows * 4;              // a level's outputs of the workgroup
constexpr size_t kRedBytes = 64;                          // input formation: per-wave partial sums
// LDS: ring | raw input | planes | 2 x scales | outputs | partial sums.
constexpr size_t kStepSmem = kRingBytes + kStageBytes + kPlaneBytes + kScaleBytes + kOutBytes + kRedBytes;

#define PWG_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// One asynchronous 16-byte-per-lane copy from global memory into LDS: lane i
// lands at lds + 16 * i.  No VGPR is written; completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, PWG_LDS(lds), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, PWG_LDS(lds), 4, 0, 0);
}

// Waits until at most n of this wave's vector-memory operations are
// outstanding (n >= 15 waits for 15: waiting longer is always safe).  Loads
// retire in order, so when every load issued after a given one may still be
// pending, that one has completed.  The count is an immediate of the
// instruction, hence the branches; n is wave-uniform.
__device__ __forceinline__ void wait_vm_le(unsigned n) {
#define PWG_VM(k) __builtin_amdgcn_s_waitcnt(((k) & 15) | (((k) >> 4) << 14) | (7 << 4) | (15 << 8))
  switch (n < 15 ? n : 15) {
    case 15: PWG_VM(15); break;
    case 14: PWG_VM(14); break;
    case 13: PWG_VM(13); break;
    case 12: PWG_VM(12); break;
    case 11: PWG_VM(11); break;
    case 10: PWG_VM(10); break;
    case 9: PWG_VM(9); break;
    case 8: PWG_VM(8); break;
    case 7: PWG_VM(7); break;
    case 6: PWG_VM(6); break;
    case 5: PWG_VM(5); break;
    case 4: PWG_VM(4); break;
    case 3: PWG_VM(3); break;
    case 2: PWG_VM(2); break;
    case 1: PWG_VM(1); break;
    default: PWG_VM(0); break;
  }
#undef PWG_VM
}

// Rows of a level owned by workgroup `b` of `nb`: [R0, R1).  Compute wave k
// takes a contiguous share of them, share q = (k + li) mod kComputeWaves
// (rows first, first + 1, ...): each wave streams a contiguous block, and
// the waves whose share is one row longer change from item to item.
__device__ __forceinline__ void wg_rows(long rows, unsigned b, unsigned nb, long& R0, long& R1) {
  R0 = static_cast<long>(b) * rows / nb;
  R1 = static_cast<long>(b + 1) * rows / nb;
}
__device__ __forceinline__ void wave_rows(long R0, long R1, unsigned k, unsigned li, long& first, int& count) {
  const unsigned q = (k + li) % kComputeWaves;
  first = R0 + static_cast<long>(q) * (R1 - R0) / kComputeWaves;
  count = static_cast<int>(R0 + static_cast<long>(q + 1) * (R1 - R0) / kComputeWaves - first);
}
// Row stride between a wave's consecutive rows.
constexpr int kRowStride = 1;

// Wave-uniform copies (the values are the same in every lane; this keeps
// them in scalar registers, so the level table is read with scalar loads
// that do not wait behind the wave's outstanding weight copies).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ unsigned uni(unsigned v) { return static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(v))); }
template <typename T>
__device__ __forceinline__ T* uni(T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = uni(static_cast<unsigned>(v)), hi = uni(static_cast<unsigned>(v >> 32));
  return reinterpret_cast<T*>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// Workgroup row range [R0, R1) of level `item` (item n_levels: the
// vocabulary), split evenly over the workgroups.
__device__ __forceinline__ void item_rows(unsigned item, int vocab, const DevLevel* levels, unsigned n_levels,
                                          unsigned nwg, long& R0, long& R1) {
  wg_rows(item < n_levels ? uni(levels[item].rows) : vocab, blockIdx.x, nwg, R0, R1);
}

// The producer half of a compute wave: walks the wave's rows of every level
// and copies each row's slots into its ring of RS slots.  All state is
// wave-uniform.
template <int RS>
struct Producer {
  const DevLevel* levels;
  unsigned n_items;   // levels, then the vocabulary
  unsigned n_levels;
  int vocab, hidden;
  const u32x4* out_table;
  unsigned nwg;       // workgroups of the launch
  unsigned k;         // compute-wave index 0..6
  unsigned lane;
  unsigned issued;    // slots issued (one DMA each)
  unsigned item;      // item being produced (n_items = done)
  int rows_left;      // rows of the item still to issue, the current one included
  int chunk, chunks_per_row, nchunks;
  const u32x4* rowp;  // start of the current row
  unsigned char* ring;
  long first;         // the item's first row of this wave
  int count;          // the item's rows of this wave
  int fast_rows;      // upcoming rows issue_row_fast may issue (see plan_fast)

  // Moves to the first item, from `item` on, in which this wave has rows.
  __device__ __forceinline__ void enter_item() {
    item = uni(item);
    while (item < n_items) {
      long R0, R1;
      item_rows(item, vocab, levels, n_levels, nwg, R0, R1);
      const u32x4* base;
      if (item < n_levels) {
        nchunks = uni(levels[item].nchunks);
        chunks_per_row = uni(levels[item].c);
        base = uni(levels[item].w);
      } else {
        nchunks = hidden >> 4;
        chunks_per_row = (nchunks + 63) / 64;
        base = out_table;
      }
      wave_rows(R0, R1, k, item, first, count);
      rows_left = uni(count);
      rowp = uni(base + first * nchunks);
      chunk = 0;
      if (rows_left > 0) {
        plan_fast();
        return;
      }
      item = uni(item + 1);
    }
    fast_rows = 0;
  }

  // Rows from the next one on that are plain: whole rows of 64-chunk
  // multiples, not the item's last row.  Those take the straight-line
  // issue_row_fast.
  __device__ __forceinline__ void plan_fast() {
    int n = rows_left - 1;
    if (chunk != 0 || (nchunks & 63) != 0) n = 0;
    fast_rows = uni(n);
  }

  __device__ __forceinline__ bool active() const { return item < n_items; }

  // Whether the next slot may be issued: the ring has room.
  __device__ __forceinline__ bool can_issue(unsigned consumed) const {
    return active() && uni(issued) - uni(consumed) < static_cast<unsigned>(RS);
  }

  // Issues the next slot (the caller checks can_issue()).
  __device__ __forceinline__ void issue() {
    unsigned c = lane + 64u * static_cast<unsigned>(chunk);
    c = c < static_cast<unsigned>(nchunks) ? c : static_cast<unsigned>(nchunks - 1);
    dma16(rowp + c, ring + (issued % RS) * kSlotBytes);
    issued = uni(issued + 1);
    chunk = uni(chunk + 1);
    if (chunk == chunks_per_row) {
      chunk = 0;
      rowp = uni(rowp + kRowStride * nchunks);
      rows_left = uni(rows_left - 1);
      if (rows_left == 0) {
        item = uni(item + 1);
        enter_item();
      } else {
        plan_fast();
      }
    } else {
      fast_rows = 0;
    }
  }

  // Issues one plain row of C chunks (fast_rows > 0, chunks_per_row == C,
  // and the ring has C free slots): no bookkeeping branches.
  template <int C>
  __device__ __forceinline__ void issue_row_fast() {
#pragma unroll
    for (int c = 0; c < C; ++c) dma16(rowp + lane + 64u * c, ring + ((issued + c) % RS) * kSlotBytes);
    issued = uni(issued + C);
    rowp = uni(rowp + kRowStride * nchunks);
    rows_left = uni(rows_left - 1);
    fast_rows = uni(fast_rows - 1);
  }

  // Refills the ring after the consumer freed slots.
  __device__ __forceinline__ void fill(unsigned consumed) {
    while (can_issue(consumed)) issue();
  }
};

// The consumer half: takes the next row's C slots out of the ring and
// refills the ring before the caller computes on them.
template <int C, int RS>
__device__ __forceinline__ void take_row(Producer<RS>& pr, unsigned& consumed, const unsigned char* ring, unsigned lane,
                                         u32x4 (&w)[C]) {
  // The row's last slot has index consumed + C - 1; everything issued after
  // it may still be in flight.  Slots are refilled one row late (below), so
  // in the steady state RS - C slots are ahead and RS - 2C may stay in flight.
  const unsigned ahead = uni(pr.issued) - uni(consumed);
  if (ahead == static_cast<unsigned>(RS - C)) {
    __builtin_amdgcn_s_waitcnt(((RS - 2 * C) & 15) | (((RS - 2 * C) >> 4) << 14) | (7 << 4) | (15 << 8));
  } else {
    wait_vm_le(ahead - C);
  }
#pragma unroll
  for (int c = 0; c < C; ++c)
    w[c] = *reinterpret_cast<const u32x4*>(ring + ((consumed + c) % RS) * kSlotBytes + lane * 16);
  // Refill the slots of the rows before this one: their LDS reads have
  // returned (their values were used), while this row's reads may still be
  // in flight, so its slots wait until the next row.  In the steady state
  // that is one plain row of the same shape: the straight-line issue.
  if (pr.fast_rows > 0 && pr.chunks_per_row == C && ahead == static_cast<unsigned>(RS) - C) {
    pr.template issue_row_fast<C>();
  } else {
    pr.fill(consumed);
  }
  consumed = uni(consumed + C);
}

// Row scale for the tile row this lane stores (tile row row_of<4>(lane >> 4),
// row index i + that), from the workgroup's LDS copy of the level's scales
// starting at row R0.
__device__ __forceinline__ float tile_scale(const float* scales, long first, int i, int count, long R0, unsigned lane) {
  const int t = row_of<4>(static_cast<int>(lane >> 4));
  const int iu = i + t < count ? i + t : i;
  return scales[first + static_cast<long>(kRowStride) * iu - R0];
}

// Consumes the wave's rows of one ternary level (C chunks of 64 words per
// lane and row), four rows per tile reduction; results go to the
// workgroup's LDS output buffer (stored to y by the control wave).
template <int C, int RS>
__device__ __forceinline__ void t2_consume_level(const DevLevel& L, long first, int count, long R0, const float* scales,
                                                 unsigned lane, Producer<RS>& pr, unsigned& consumed,
                                                 const unsigned char* ring, const unsigned* planes,
                                                 const int* plane_e, float* out_buf) {
  T2Lane<C> st;
  t2_lane_init<C>(st, planes, plane_e, L.nchunks, lane);
  for (int i = 0; i < count; i += 4) {
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      p[u] = 0.f;
      if (i + u < count) {
        u32x4 w[C];
        take_row<C, RS>(pr, consumed, ring, lane, w);
#pragma unroll
        for (int c = 0; c < C; ++c) {
          t2_chunk_dot(w[c], st.X[c], st.acc[c]);
          const unsigned comb = combine_limbs6(st.acc[c]);
          const int v = static_cast<int>(comb - st.prev[c]);
          st.prev[c] = comb;
          p[u] += ldexpf(static_cast<float>(v), st.Ec[c]);
        }
      }
    }
    const int iu = i + row_of<4>(static_cast<int>(lane >> 4));
    const long row = first + static_cast<long>(kRowStride) * iu;
    const float sc = tile_scale(scales, first, i, count, R0, lane);
    const float total = tile_reduce<4>(p);
    if ((lane & 15u) == 0u && iu < count) out_buf[row - R0] = sc * total;
  }
}

// Consumes the wave's vocabulary rows: logits, and the wave's (max, lowest
// row) of them.
template <int RS>
__device__ __forceinline__ void i8_consume_level(const Plan& P, long first, int count, long R0, const float* scales, unsigned lane,
                                 Producer<RS>& pr, unsigned& consumed, const unsigned char* ring,
                                 const unsigned* planes, const int* plane_e, float& best, unsigned& best_idx) {
  const int nchunks = P.hidden >> 4;
  unsigned H[kMaxI8C][12];
  int Ec[kMaxI8C];
#pragma unroll
  for (int c = 0; c < kMaxI8C; ++c) {
    const unsigned chunk = lane + 64u * c;
    const bool ok = chunk < static_cast<unsigned>(nchunks);
    Ec[c] = ok ? -plane_e[chunk] : 0;
    const u32x4* src = reinterpret_cast<const u32x4*>(planes + (ok ? chunk : 0u) * kI8ChunkDwords);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const u32x4 v = ok ? src[q] : u32x4{0u, 0u, 0u, 0u};
      H[c][4 * q] = v.x; H[c][4 * q + 1] = v.y; H[c][4 * q + 2] = v.z; H[c][4 * q + 3] = v.w;
    }
  }
  const int cpr = (nchunks + 63) / 64;  // slots per row (4 for hidden = 4096)
  for (int i = 0; i < count; i += 4) {
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      p[u] = 0.f;
      if (i + u < count) {
        u32x4 q[kMaxI8C];
        const unsigned ahead = uni(pr.issued) - uni(consumed);
        if (ahead == static_cast<unsigned>(RS - kMaxI8C) && cpr == kMaxI8C) {  // steady state (see take_row)
          __builtin_amdgcn_s_waitcnt(((RS - 2 * kMaxI8C) & 15) | (((RS - 2 * kMaxI8C) >> 4) << 14) | (7 << 4) | (15 << 8));
        } else {
          wait_vm_le(ahead - cpr);
        }
#pragma unroll
        for (int c = 0; c < kMaxI8C; ++c)
          q[c] = c < cpr ? *reinterpret_cast<const u32x4*>(ring + ((consumed + c) % RS) * kSlotBytes + lane * 16)
                         : u32x4{0u, 0u, 0u, 0u};
        if (pr.fast_rows > 0 && pr.chunks_per_row == kMaxI8C && ahead == static_cast<unsigned>(RS - kMaxI8C)) {
          pr.template issue_row_fast<kMaxI8C>();  // slots of the rows before this one (see take_row)
        } else {
          pr.fill(consumed);
        }
        consumed = uni(consumed + cpr);
#pragma unroll
        for (int c = 0; c < kMaxI8C; ++c) {
          int a0 = 0, a1 = 0, a2 = 0;
          const unsigned qd[4] = {q[c].x, q[c].y, q[c].z, q[c].w};
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
    const int iu = i + row_of<4>(static_cast<int>(lane >> 4));
    const long row = first + static_cast<long>(kRowStride) * iu;
    const float sc = tile_scale(scales, first, i, count, R0, lane);
    const float total = tile_reduce<4>(p);
    if ((lane & 15u) == 0u && iu < count) {
      const float logit = sc * total;
      if (P.logits_out) P.logits_out[row] = logit;
      if (logit > best) {  // rows of one lane ascend: ties keep the lower index
        best = logit;
        best_idx = static_cast<unsigned>(row);
      }
    }
  }
}

// Control wave: copies level `li`'s input vector into LDS (li == n_levels:
// the hidden state).
__device__ __forceinline__ void stage_x(const Plan& P, const DevLevel* levels, unsigned li, unsigned lane,
                                        float* stage) {
  const float* x = li < P.n_levels ? levels[li].x : P.h;
  const int cols = li < P.n_levels ? levels[li].cols : static_cast<int>(P.hidden);
  // Lanes past the end are masked off: a masked lane neither reads nor writes.
  for (int o = 0; o < cols; o += 256)
    if (o + 4 * static_cast<int>(lane) < cols) dma16(x + o + 4 * lane, stage + o);
}

// Control wave: copies the workgroup's row scales of level `li` into LDS
// (li == n_levels: the vocabulary scales).  Scales are constant inputs.
__device__ __forceinline__ void stage_scales(const Plan& P, const DevLevel* levels, unsigned li, unsigned lane,
                                             float* scales) {
  const float* s = li < P.n_levels ? levels[li].scale : P.out_scale;
  const long rows = li < P.n_levels ? levels[li].rows : P.vocab;
  long R0, R1;
  wg_rows(rows, blockIdx.x, P.grid, R0, R1);
  for (long o = R0; o < R1; o += 64)
    if (o + lane < R1) dma4(s + o + lane, scales + (o - R0));
}

// Embedding row of the previous token (workgroup 0, control wave).
__device__ __forceinline__ void embed_row(const Plan& P, unsigned lane) {
  const int id = *P.token_in;
  const bool ok = id >= 0 && id < P.vocab;
  const int nchunks = P.hidden >> 4;
  const float s = ok ? P.emb_scale[id] : __builtin_nanf("");
  if (lane == 0) *P.emb_scale_out = s;
  // wave-uniform trip count: a loop whose exit differed between lanes would
  // make everything the caller merges after this branch divergent
  for (int c0 = 0; c0 < nchunks; c0 += 64) {
    const int c = c0 + static_cast<int>(lane);
    if (c < nchunks) {
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
}

// A compute wave's rows of level li (workgroup rows [R0, R1)); planes: the
// level's input limbs in LDS; scales: the workgroup's LDS copy of its row
// scales.
template <int RS>
__device__ __forceinline__ void consume_item(const Plan& P, const DevLevel* levels, unsigned li, long R0, long R1,
                                             unsigned k, const float* scales, unsigned lane, Producer<RS>& pr,
                                             unsigned& consumed, const unsigned char* ring, const unsigned* planes,
                                             float* out_buf, float& best, unsigned& best_idx) {
  long first;
  int count;
  wave_rows(R0, R1, k, li, first, count);
  if (li == P.n_levels) {
    const int* plane_e = reinterpret_cast<const int*>(planes + (P.hidden >> 4) * kI8ChunkDwords);
    i8_consume_level<RS>(P, first, count, R0, scales, lane, pr, consumed, ring, planes, plane_e, best, best_idx);
    return;
  }
  const DevLevel& L = levels[li];
  const int* plane_e = reinterpret_cast<const int*>(planes + L.nchunks * kT2ChunkDwords);
  if (L.c == 1) t2_consume_level<1, RS>(L, first, count, R0, scales, lane, pr, consumed, ring, planes, plane_e, out_buf);
  else if (L.c == 2) t2_consume_level<2, RS>(L, first, count, R0, scales, lane, pr, consumed, ring, planes, plane_e, out_buf);
  else t2_consume_level<3, RS>(L, first, count, R0, scales, lane, pr, consumed, ring, planes, plane_e, out_buf);
}

__global__ __launch_bounds__(kThreads, 1) void step_kernel(const Plan* __restrict__ plan,
                                                            const DevLevel* __restrict__ levels, unsigned* state,
                                                            unsigned long long* counters, unsigned* flags,
                                                            unsigned long long* partials) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring_all = smem;
  // ordered: raw input, one plane buffer, scales, outputs
  float* stage = reinterpret_cast<float*>(smem + kRingBytes);
  unsigned* planes1 = reinterpret_cast<unsigned*>(smem + kRingBytes + kStageBytes);
  float* scale_buf = reinterpret_cast<float*>(smem + kRingBytes + kStageBytes + kPlaneBytes);
  float* out_buf = reinterpret_cast<float*>(smem + kRingBytes + kStageBytes + kPlaneBytes + kScaleBytes);
  float* red = out_buf + kMaxWgRows;

  const Plan& P = *plan;
  Barrier bar;
  bar.plan = plan;
  bar.state = state;
  bar.counters = counters;
  bar.flags = flags;
  bar.xcd = xcc_id();
  const unsigned gen = ld_sc(&state[kStateGen]);
  bar.base = gen * P.n_barriers;

  const unsigned lane = threadIdx.x & 63u;
  const unsigned wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned k = wave - 1;  // compute-wave index (unused by wave 0)
  constexpr int RS = kRing;
  unsigned char* ring = ring_all + static_cast<size_t>(wave == 0 ? 0 : k) * RS * kSlotBytes;

  Producer<RS> pr;
  pr.levels = levels;
  pr.n_items = P.n_levels + 1;
  pr.n_levels = P.n_levels;
  pr.vocab = P.vocab;
  pr.hidden = P.hidden;
  pr.out_table = P.out_table;
  pr.nwg = P.grid;
  pr.k = k;
  pr.lane = lane;
  pr.issued = 0;
  pr.item = 0;
  pr.ring = ring;
  pr.first = 0;
  pr.count = 0;
  unsigned consumed = 0;

  // how each level's input is formed (op 0: staged as given); a formed
  // input reads earlier outputs, so it is formed after the level barrier
  auto input_of = [&](unsigned li) -> const chain::DevInput& { return li < P.n_levels ? levels[li].in : P.h_in; };
  const chain::EmbedSrc emb{reinterpret_cast<const int8_t*>(P.emb_table), P.emb_scale, P.token_in,
                            static_cast<long>(P.vocab)};
  if (wave == 0) {
    if (input_of(0).op == PWG_INPUT_GIVEN) stage_x(P, levels, 0, lane, stage);
    stage_scales(P, levels, 0, lane, scale_buf);
    if (blockIdx.x == 0) embed_row(P, lane);
  } else {
    pr.enter_item();
    pr.fill(consumed);
  }

  float best = -__builtin_inff();
  unsigned best_idx = 0xFFFFFFFFu;
  {
    for (unsigned li = 0; li <= P.n_levels; ++li) {
      float* scales = scale_buf + (li & 1u) * kMaxWgRows;
      const bool vocab = li == P.n_levels;
      long R0, R1;
      wg_rows(vocab ? P.vocab : levels[li].rows, blockIdx.x, P.grid, R0, R1);
      // Level li starts once level li-1 is complete everywhere, and only
      // then is its input read (it may be an output of level li-1).  The
      // agent-scope acquire drops stale lines of the input from this XCD's L2.
      if (li > 0) {
        if (bar.wait(li - 1)) return;
        if (wave == 0) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          if (input_of(li).op == PWG_INPUT_GIVEN) stage_x(P, levels, li, lane, stage);
        }
      }
      if (wave == 0) __builtin_amdgcn_s_waitcnt(0);  // this level's input and scales have landed
      __syncthreads();
      const int cols = vocab ? P.hidden : levels[li].cols;
      // A formed input: every wave reads the sources after the barrier
      // (the control wave's acquire above has invalidated this CU's and
      // this XCD's stale lines before the workgroup barrier), and the
      // workgroup forms the vector in the staging buffer.
      const chain::DevInput& fin = input_of(li);
      if (fin.op != PWG_INPUT_GIVEN) chain::form_input<kThreads>(fin, cols, stage, red, emb, 0, cols);
      int* plane_e = reinterpret_cast<int*>(planes1 + (vocab ? (cols >> 4) * kI8ChunkDwords : (cols >> 6) * kT2ChunkDwords));
      if (vocab) i8_prepare_x(stage, cols, planes1, plane_e);
      else t2_convert_staged(stage, cols, planes1, plane_e);
      // compute waves copy their limbs into registers inside the consume
      // functions; the planes are rewritten only after the block barrier below
      if (wave == 0) {
        if (li < P.n_levels) stage_scales(P, levels, li + 1, lane, scale_buf + ((li + 1) & 1u) * kMaxWgRows);
        // every workgroup writes its slice of the formed input (and of the
        // residual sum); the release at this level's arrival publishes them
        if (fin.op != PWG_INPUT_GIVEN)
          chain::store_formed(fin, cols, stage, const_cast<float*>(li < P.n_levels ? levels[li].x : P.h), emb,
                              static_cast<int>(blockIdx.x * static_cast<unsigned>(cols) / P.grid),
                              static_cast<int>((blockIdx.x + 1) * static_cast<unsigned>(cols) / P.grid),
                              static_cast<int>(lane), 64);
      } else {
        consume_item<RS>(P, levels, li, R0, R1, k, scales, lane, pr, consumed, ring, planes1, out_buf, best, best_idx);
      }
      __syncthreads();  // planes, this level's scales and outputs are complete
      if (!vocab && wave == 0) {
        float* y = levels[li].y;
        for (long o0 = 0; o0 < R1 - R0; o0 += 64)  // wave-uniform trip count
          if (o0 + lane < R1 - R0) y[R0 + o0 + lane] = out_buf[o0 + lane];
        bar.arrive_release(li);
      }
    }
  }

  // workgroup (max, lowest index) of the vocabulary rows
  {
    unsigned long long key = best_idx == 0xFFFFFFFFu ? 0ull : argmax_key(best, best_idx);
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(key, off, kWave);
      key = o > key ? o : key;
    }
    __shared__ unsigned long long wkeys[kWpb];
    if (lane == 0) wkeys[wave] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
      unsigned long long m = 0ull;
      for (int i = 0; i < kWpb; ++i) m = wkeys[i] > m ? wkeys[i] : m;
      st_sc64(&partials[blockIdx.x], m);
    }
  }
  const unsigned final_barrier = P.n_levels;
  bar.arrive(final_barrier);
  if (blockIdx.x == 0) {
    if (bar.wait(final_barrier)) return;
    if (threadIdx.x < 64) {
      unsigned long long m = 0ull;
      for (unsigned b = threadIdx.x; b < P.grid; b += 64) {
        const unsigned long long o = ld_sc64(&partials[b]);
        m = o > m ? o : m;
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(m, off, kWave);
        m = o > m ? o : m;
      }
      if (threadIdx.x == 0) {
        *P.token_out = static_cast<int>(argmax_key_index(m));
        st_sc(&state[kStateGen], gen + 1);
      }
    }
  }
}

__global__ void xcc_calibrate(unsigned* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

// ----------------------------------------------------------------- host side
struct Layout {
  size_t plan = 0, state = 0, counters = 0, flags = 0, partials = 0, levels = 0, calib = 0, total = 0;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout of a step (offsets from the 256-byte aligned plan).
Layout layout_for(const pwg_step_desc* d) {
  const int n_levels = d->n_levels;
  Layout L;
  L.plan = 0;
  L.state = align_up(sizeof(Plan), 256);
  L.counters = L.state + 256;
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

size_t step_lds_bytes(const pwg_step_desc*) { return kStepSmem; }

int grid_for(const pwg_step_desc* d, GridInfo* gi) {
  int dev = 0, cus = 0, occ = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  gi->lds = step_lds_bytes(d);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(&step_kernel), kThreads, gi->lds);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "persistent step: device query failed: %s", hipGetErrorString(e));
  if (occ < 1) return fail(PWG_ERR_UNSUPPORTED, "persistent step: kernel does not fit on a CU");
  gi->grid = cus < static_cast<int>(kMaxGrid) ? cus : static_cast<int>(kMaxGrid);  // one workgroup per CU
  return PWG_OK;
}

}  // namespace

size_t step_persistent_workspace(const pwg_step_desc* d) {
  if (!d || d->schedule != PWG_SCHEDULE_PERSISTENT || d->n_levels < 0) return 0;
  return layout_for(d).total + 256;  // + 256 for aligning the plan
}

static Plan* plan_ptr(const pwg_step_desc* d, size_t ws_offset) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(d->workspace) + ws_offset;
  return reinterpret_cast<Plan*>(align_up(p, 256));
}

int step_persistent_plan(const pwg_step_desc* d, size_t ws_offset, void* stream) {
  GridInfo gi0;
  const int rc0 = grid_for(d, &gi0);
  if (rc0 != PWG_OK) return rc0;
  // a workgroup keeps its row scales and outputs of a level in LDS
  auto too_many = [&](int64_t rows) { return (rows + gi0.grid - 1) / gi0.grid > kMaxWgRows; };
  if (too_many(d->vocab))
    return fail(PWG_ERR_UNSUPPORTED, "pwg_step_plan: persistent schedules support up to %d vocabulary rows per CU",
                kMaxWgRows);
  for (int i = 0; i < d->n_levels; ++i) {
    if (too_many(d->levels[i].rows))
      return fail(PWG_ERR_UNSUPPORTED, "pwg_step_plan: level %d has more than %d rows per CU", i, kMaxWgRows);
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
  const Layout lay = layout_for(d);
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
  h.n_levels = static_cast<unsigned>(d->n_levels);
  h.n_barriers = h.n_levels + 1;
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
  h.h_in = chain::from_abi(d->h_in);
  h.state_off = lay.state;
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
    lv[i].in = chain::from_abi(L.in);
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
  char* dbase = reinterpret_cast<char*>(dplan);
  const Layout lay = layout_for(d);
  const DevLevel* lv = reinterpret_cast<const DevLevel*>(dbase + lay.levels);
  unsigned* state = reinterpret_cast<unsigned*>(dbase + lay.state);
  auto* counters = reinterpret_cast<unsigned long long*>(dbase + lay.counters);
  auto* flags = reinterpret_cast<unsigned*>(dbase + lay.flags);
  auto* partials = reinterpret_cast<unsigned long long*>(dbase + lay.partials);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(step_kernel, dim3(gi.grid), dim3(kThreads), gi.lds, st, dplan, lv, state, counters, flags, partials);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "persistent step launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

int step_persistent_status(const pwg_step_desc* d, size_t ws_offset, void* stream) {
  Plan* dplan = plan_ptr(d, ws_offset);
  unsigned s = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const unsigned* state = reinterpret_cast<const unsigned*>(reinterpret_cast<char*>(dplan) + layout_for(d).state);
  hipError_t e = hipMemcpyAsync(&s, &state[kStateStatus], 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_status: %s", hipGetErrorString(e));
  if (s == kStatusTimeout) return fail(PWG_ERR_HIP, "persistent step: a level barrier timed out");
  return PWG_OK;
}

}  // namespace pwg
