// Stream schedule of the decode step on the CDNA4 matrix cores.
//
// Page "The Neutrino Engine": section "A 104 microsecond floor inside a 694
// microsecond step" (batch-1 decode applies every projection to the current
// activations once per token, the output projection scores the whole
// vocabulary, the token is the greedy argmax), section "The file is not the
// traffic" (ternary projections with row scales, int8 vocabulary tables) and
// section "The same weights take four execution paths" (the loader arranges
// the stored values for the device at load time: here, 16-row x 64-byte
// tiles, one 1 KiB tile per wave load instruction).
//
// Ternary levels run on v_mfma_scale_f32_16x16x128_f8f6f4 with A in FP4
// (e2m1) and B in FP8 (e4m3).  Operand A is 16 weight rows x 128 weights:
// masking a T2 word with 0xCCCCCCCC, and again after a 2-bit left shift,
// leaves nibbles 0b0100 / 0b1100 / 0 for w = +1 / -1 / 0, which are the FP4
// values +2, -2 and 0, so a 16-byte tile slice becomes the A operands of two
// instructions with three VALU operations per word.  Operand B is 128 x 16:
// column j < 6 holds e4m3 piece j of the activations (operands.h: six pieces
// of four significant bits, each with its own exponent per value, that sum to
// x exactly); the E8M0 block scales (one per 32 K-values and column) carry
// the block exponent and the piece's weight.  Every product is exact; the
// instruction sums in float32.  The instruction's destination must not share
// registers with its A or B operands (with an FP8 operand that gives wrong
// sums on gfx950), so every operand stays live past its instruction.
//
// The int8 output projection runs on v_mfma_i32_16x16x64_i8: A is the tile
// as stored, B's columns are six balanced base-256 digits of h rounded to
// 47-bit fixed point per 256-element section; four instructions accumulate
// exactly in int32 before one conversion to float per section and column.
//
// Work: 16-row blocks of every level and of the vocabulary.  Each workgroup
// (one per CU) first takes a contiguous range of the ternary levels of equal
// cost, then claims blocks of a shared pool (the vocabulary, then a few
// small-block ternary levels) from a global counter.  Inside a workgroup, 6
// compute waves claim blocks one at a time and stream their tiles through two
// register groups (one group's loads in flight while the other is consumed,
// across block, level and segment boundaries).  Wave 0 claims pool blocks
// ahead into an LDS ring and records which pool segments its claims fall
// in; wave 1 copies the converted activation operands of each static
// segment and of each claimed pool segment into a ring of LDS regions ahead
// of the compute waves.  The last workgroup to finish reduces the argmax.
#include <algorithm>
#include <cmath>
#include <vector>

#include "device_common.h"
#include "operands.h"
#include "pwg_internal.h"
#include "step_stream.h"

namespace pwg {
namespace {

using namespace dev;
using namespace stream;
using ops::block_scales;
using ops::row16_sum;
using ops::ternary_unpack;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = kStreamWaves;     // wave 0 claims pool blocks, wave 1 stages operands, the others compute
constexpr int kControl = 2;
constexpr int kCompute = kWaves - kControl;
constexpr int kThreads = kWaves * 64;
constexpr unsigned long long kSpinLimit = 50000000ull;  // 0.5 s of the 100 MHz real-time counter
enum : unsigned { kStatusOk = 0, kStatusTimeout = 1 };

#define PWG_LDS(p) ((__attribute__((address_space(3))) void*)(p))
typedef const __attribute__((address_space(4))) float cfloat;
// Global-address-space views: generic (flat) accesses would also count on
// the LDS counter, and every LDS wait would then wait for the weight loads.
typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) float g_float;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) f32x4 g_f32x4;
typedef const __attribute__((address_space(1))) f32x4 cg_f32x4;

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ unsigned uni(unsigned v) {
  return static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
}
template <typename T>
__device__ __forceinline__ T* uni(T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = uni(static_cast<unsigned>(v)), hi = uni(static_cast<unsigned>(v >> 32));
  return reinterpret_cast<T*>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// LDS flag store that does not make the compiler wait for outstanding
// global-to-LDS copies first (the flags are never a copy's destination).
__device__ __forceinline__ void lds_publish(int* p, int v) {
  const unsigned addr = static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) int*)p));
  asm volatile("s_waitcnt lgkmcnt(0)\n\tds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ int lds_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The producer half of a compute wave: issues the 1 KiB tile loads of the
// wave's current block, then of the next block the consumer half has
// already claimed; parks on a scratch area once nothing is left.  A block's
// tiles are read starting at tile `rot` (a multiple of the group size) and
// wrapping around, rot depending on the block index only: the ~1,800 blocks
// in flight across the chip then do not all read the same offset of their
// block at the same time.  Loop-free, so the tile loop stays simple enough
// for the compiler to keep the tile registers in one assignment.  State is
// wave-uniform.
struct Producer {
  const unsigned char* base;   // this lane's 16 bytes of tile 0 of the current block
  int T, rot, pos;             // tiles per block, first tile, tiles issued (T = 0: parked)
  const unsigned char* nbase;  // the next block (nT = 0: none)
  int nT, nrot;

  // Moves to the claimed next block once the current one is fully issued.
  __device__ __forceinline__ void step_block() {
    if (pos >= T) {
      base = nbase;
      T = nT;
      rot = nrot;
      pos = 0;
      nT = 0;
    }
  }
  template <int GR>
  __device__ __forceinline__ void issue(u32x4 (&x)[GR]) {
    step_block();
    int off = rot + pos;
    off = off >= T ? off - T : off;
#pragma unroll
    for (int j = 0; j < GR; ++j) x[j] = __builtin_nontemporal_load((const g_u32x4*)(base + 1024 * (off + j)));
    pos = uni(pos + (T > 0 ? GR : 0));
  }
};

// First tile of block `blk` of a level with T tiles per block (groups of G).
template <int G>
__device__ __forceinline__ int block_rot(int blk, int T) {
  if (G == 0) return 0;
  return ((blk * 5) % (T / G)) * G;
}

// Two FP4 x FP8 MFMAs over K-values 256 t .. 256 t + 255 of a ternary block.
// buf: the level's operand region in LDS; kOdd: t is odd (the scale bytes of
// MFMAs 2t, 2t + 1 are then bytes 2 and 3 of the dwords read at t - 1).
template <bool kOdd>
__device__ __forceinline__ void ternary_mfma(const v8i& a0, const v8i& a1, int t, const unsigned char* buf,
                                             int bsc_off, int asc_off, unsigned boff, unsigned lane, unsigned g,
                                             unsigned& sb, unsigned& sa, v4f& acc0, v4f& acc1) {
  const u32x4* p0 = reinterpret_cast<const u32x4*>(buf + (2 * t) * kTernaryMfmaBytes + boff);
  const u32x4* p1 = reinterpret_cast<const u32x4*>(buf + (2 * t + 1) * kTernaryMfmaBytes + boff);
  const u32x4 b0 = p0[0], b0h = p0[1], b1 = p1[0], b1h = p1[1];
  if (!kOdd) {  // scales of MFMAs 2t .. 2t + 3 (one byte each)
    sb = *reinterpret_cast<const unsigned*>(buf + bsc_off + (t >> 1) * 256 + lane * 4);
    sa = *reinterpret_cast<const unsigned*>(buf + asc_off + (t >> 1) * 16 + g * 4);
  }
  const v8i B0 = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z), static_cast<int>(b0.w),
                  static_cast<int>(b0h.x), static_cast<int>(b0h.y), static_cast<int>(b0h.z), static_cast<int>(b0h.w)};
  const v8i B1 = {static_cast<int>(b1.x), static_cast<int>(b1.y), static_cast<int>(b1.z), static_cast<int>(b1.w),
                  static_cast<int>(b1h.x), static_cast<int>(b1h.y), static_cast<int>(b1h.z), static_cast<int>(b1h.w)};
  if (kOdd) {
    acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, B0, acc0, 4, 0, 2, static_cast<int>(sa), 2, static_cast<int>(sb));
    acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, B1, acc1, 4, 0, 3, static_cast<int>(sa), 3, static_cast<int>(sb));
  } else {
    acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, B0, acc0, 4, 0, 0, static_cast<int>(sa), 0, static_cast<int>(sb));
    acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, B1, acc1, 4, 0, 1, static_cast<int>(sa), 1, static_cast<int>(sb));
  }
  // operands live past the instructions: no destination shares their registers
  asm volatile("" ::"v"(a0), "v"(a1), "v"(B0), "v"(B1));
}

// One int8 MFMA over K-values 64 t .. 64 t + 63 of a vocabulary block.
__device__ __forceinline__ void int8_mfma(const u32x4 v, int t, const unsigned char* buf, unsigned boff, v4i& iacc) {
  const u32x4 b = *reinterpret_cast<const u32x4*>(buf + t * kInt8MfmaBytes + boff);
  const v4i A = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
  const v4i B = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w)};
  iacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, iacc, 0, 0, 0);
}
// End of an exponent section (4 tiles): the exact int32 sums, scaled into
// the float accumulator.
__device__ __forceinline__ void int8_section(int t, const unsigned char* buf, int exp_off, int cexp, v4i& iacc,
                                             v4f& facc) {
  const int e = *reinterpret_cast<const int*>(buf + exp_off + (t / kSectionMfmas) * 4) + cexp;
  // |iacc| <= 4 * 64 * 127 * 128 < 2^23: the conversion is exact
  facc.x += ldexpf(static_cast<float>(iacc.x), e);
  facc.y += ldexpf(static_cast<float>(iacc.y), e);
  facc.z += ldexpf(static_cast<float>(iacc.z), e);
  facc.w += ldexpf(static_cast<float>(iacc.w), e);
  iacc = v4i{0, 0, 0, 0};
}

// Embedding row of the previous token (workgroup 0, control wave).
__device__ __forceinline__ void embed_row(const Plan& P, unsigned lane) {
  const int id = *P.token_in;
  const bool ok = id >= 0 && id < P.vocab;
  const int nchunks = P.hidden >> 4;
  const float s = ok ? P.emb_scale[id] : __builtin_nanf("");
  if (lane == 0) *P.emb_scale_out = s;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {  // wave-uniform trip count
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

// Segment s of a workgroup: its static segments first, then the pool's.
__device__ __forceinline__ Seg seg_at(const Seg* segs, int nseg, const Plan& P, int s) {
  Seg r;
  if (s < nseg) {
    r.level = uni(segs[s].level);
    r.b0 = uni(segs[s].b0);
    r.b1 = uni(segs[s].b1);
  } else {
    r.level = uni(P.pool_segs[s - nseg].level);
    r.b0 = uni(P.pool_segs[s - nseg].b0);
    r.b1 = uni(P.pool_segs[s - nseg].b1);
  }
  r.pad = 0;
  return r;
}

template <int G>
__global__ __launch_bounds__(kThreads, 1) void stream_step_kernel(const Plan* __restrict__ plan,
                                                                   const Level* __restrict__ levels,
                                                                   const Seg* __restrict__ all_segs) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Plan& P = *plan;
  const unsigned lane = threadIdx.x & 63u;
  const unsigned wave = uni(threadIdx.x >> 6);
  const int nseg = uni(P.seg_count[blockIdx.x]);   // static segments
  const int nall = nseg + uni(P.pool_nseg);         // with the pool's
  const Seg* segs = all_segs + static_cast<size_t>(blockIdx.x) * P.seg_stride;
  const int buf_bytes = P.buf_bytes;
  unsigned char* flags = smem + 2 * buf_bytes;
  int* ready = reinterpret_cast<int*>(flags);        // highest segment whose operands are in LDS
  int* wcnt = ready + 1;                              // claims of static blocks
  int* phead = ready + 2;                             // pool claims popped from the ring
  int* done = ready + 4;                              // [kWaves]: highest segment a wave is done with
  int* pool_mask = ready + 4 + kWaves;                // bit q: this workgroup claimed a block of pool segment q
  int* pool_past = pool_mask + 1;                     // no later claim of this workgroup falls below pool segment pool_past
  unsigned long long* wkeys = reinterpret_cast<unsigned long long*>(flags + 128);  // [kWaves]
  int* seg_first = reinterpret_cast<int*>(flags + kSegFirstOff);               // [kMaxWgSegs + 1]
  unsigned long long* ring = reinterpret_cast<unsigned long long*>(flags + kRingOff);  // [kRing]
  int* seg_pos = reinterpret_cast<int*>(flags + kSegOffOff);                   // [kMaxSegs][2]
  if (threadIdx.x == 0) {
    *ready = -1;
    *wcnt = 0;
    *phead = 0;
    *pool_mask = 0;
    *pool_past = 0;
  }
  if (threadIdx.x < kWaves) done[threadIdx.x] = -1;
  if (threadIdx.x < kRing) ring[threadIdx.x] = ~0ull;  // tag 0xFFFFFFFF: empty
  if (threadIdx.x == 64) {  // prefix sums of the static segments' block counts (padded with the total)
    int acc = 0;
    for (int i = 0; i <= kMaxWgSegs; ++i) {
      seg_first[i] = acc;
      if (i < nseg) acc += segs[i].b1 - segs[i].b0;
    }
  }
  __syncthreads();
  const int total_blocks = uni(seg_first[kMaxWgSegs]);

  float best = -__builtin_inff();
  unsigned best_idx = 0xFFFFFFFFu;
  if (wave == 0) {
    // Claim wave: keeps up to kPoolAhead pool claims queued in the claim
    // ring beyond the compute waves' pops (one global atomic per batch of
    // claims); after the pool runs out, one end marker per compute wave.
    bool late = false;
    int tail = 0, ends = 0, batch = kClaimBatch, mask = 0;
    bool exhausted = false;
    const int pool_total = uni(P.pool_total);
    unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (ends < kCompute) {
      if (tail - uni(lds_acquire(phead)) < kPoolAhead) {
        // claims come in batches of `batch` consecutive pool blocks (one
        // atomic each; under a full memory load an atomic takes microseconds),
        // smaller batches once the pool is nearly used up
        if (!exhausted) {
          int p = 0;
          if (lane == 0)
            p = static_cast<int>(__hip_atomic_fetch_add(P.pool_next, static_cast<unsigned>(batch), __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT));
          p = uni(p);
          int past = 0;
          for (int q = 0; q < batch; ++q) {
            const int pq = p + q < pool_total ? p + q : -1;
            if (pq < 0) {
              exhausted = true;
              break;
            }
            // the pool segment of the block: its operands will be needed
            int sq = 0;  // pool_first[j] = pool_total for j >= pool_nseg
#pragma unroll
            for (int step = kMaxPoolSegs / 2; step >= 1; step >>= 1)
              if (P.pool_first[sq + step] <= pq) sq += step;
            mask |= 1 << uni(sq);
            past = uni(sq);
            if (lane == 0)
              __hip_atomic_store(&ring[tail & (kRing - 1)],
                                 (static_cast<unsigned long long>(static_cast<unsigned>(tail)) << 32) | static_cast<unsigned>(pq),
                                 __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            tail = uni(tail + 1);
          }
          // claims only move forward through the pool: segments below the
          // last claimed one will not be claimed again (none at all once the
          // pool is used up)
          if (lane == 0) {
            __hip_atomic_store(pool_mask, mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_store(pool_past, exhausted ? kMaxPoolSegs : past, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          if (pool_total - (p + batch) < kLateClaims * P.grid) batch = kLateBatch;
        } else {
          if (lane == 0)
            __hip_atomic_store(&ring[tail & (kRing - 1)],
                               (static_cast<unsigned long long>(static_cast<unsigned>(tail)) << 32) | 0xFFFFFFFFull,
                               __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
          tail = uni(tail + 1);
          ends = uni(ends + 1);
        }
        t0 = __builtin_amdgcn_s_memrealtime();
      } else {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
          late = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (late && lane == 0) __hip_atomic_store(P.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (wave == 1) {
    // Staging wave: copies segment s's operand region into the LDS region
    // ring as soon as it has room.  The ring is 2 buf_bytes long, buf_bytes
    // >= the largest region; a region goes right after the previous one,
    // never straddles the middle, and may not overlap a region a compute
    // wave may still read (segments after the lowest one every compute wave
    // is done with).  So small regions are staged several segments ahead,
    // and a region always fits once only the previous segment is in use.
    bool late = false;
    int s = 0, head = 0;
    unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (s < nall) {
      if (s >= nseg) {
        // a pool segment: stage it once this workgroup has claimed one of
        // its blocks; skip it (no region) once the claims have moved past it
        const int q = s - nseg;
        const int past = uni(__hip_atomic_load(pool_past, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
        const int mask = uni(__hip_atomic_load(pool_mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (!((mask >> q) & 1)) {
          if (past > q) {
            if (lane == 0) {
              seg_pos[2 * s] = 0;
              seg_pos[2 * s + 1] = 0;  // an empty region overlaps nothing
            }
            lds_publish(ready, s);
            s = uni(s + 1);
            t0 = __builtin_amdgcn_s_memrealtime();
          } else if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
            late = true;
            break;
          } else {
            __builtin_amdgcn_s_sleep(1);
          }
          continue;
        }
      }
      const Level& L = levels[seg_at(segs, nseg, P, s).level];
      const int bytes = uni(L.b_bytes);
      int d = (lane >= kControl && lane < kWaves) ? lds_acquire(&done[lane]) : 0x7FFFFFFF;
      for (int off = 32; off >= 1; off >>= 1) d = min(d, __shfl_xor(d, off, kWave));
      const int live0 = uni(d) + 1 > 0 ? uni(d) + 1 : 0;  // regions of segments live0 .. s - 1 may be in use
      int c = head;
      if (c < buf_bytes && c + bytes > buf_bytes) c = buf_bytes;
      if (c + bytes > 2 * buf_bytes) c = 0;
      int pos = -1;
      for (int k = 0; k < 3 && pos < 0; ++k) {
        const int cand = k == 0 ? c : (k == 1 ? 0 : buf_bytes);
        bool free = true;
        for (int j = live0; j < s; ++j)
          if (cand < uni(seg_pos[2 * j + 1]) && uni(seg_pos[2 * j]) < cand + bytes) free = false;
        if (free) pos = cand;
      }
      if (pos >= 0) {
        const unsigned char* src = uni(L.b);
        unsigned char* dst = smem + pos;
        if (lane == 0) {
          seg_pos[2 * s] = pos;
          seg_pos[2 * s + 1] = pos + bytes;
        }
        head = pos + bytes;
        for (int o = 0; o < bytes; o += 1024)
          if (o + 16 * static_cast<int>(lane) < bytes)
            __builtin_amdgcn_global_load_lds(src + o + 16 * lane, PWG_LDS(dst + o), 16, 0, 0);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed in LDS
        lds_publish(ready, s);
        if (s == 0 && blockIdx.x == 0) embed_row(P, lane);
        s = uni(s + 1);
        t0 = __builtin_amdgcn_s_memrealtime();
      } else {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
          late = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (nall == 0 && blockIdx.x == 0) embed_row(P, lane);
    if (late && lane == 0) __hip_atomic_store(P.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    const unsigned n = lane & 15u, g = lane >> 4;
    bool late = false;
    // Claims the next block: a static block from the workgroup counter (the
    // segment from a fixed-depth search of the prefix sums), else a pool
    // block from the ring.  Returns the segment (-1: nothing left).
    bool static_done = false;
    auto claim = [&](int& blk) -> int {
      if (!static_done) {
        int f = 0;
        if (lane == 0) f = __hip_atomic_fetch_add(wcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        f = uni(f);
        if (f < total_blocks) {
          int sidx = 0;
#pragma unroll
          for (int step = kMaxWgSegs / 2; step >= 1; step >>= 1)
            if (seg_first[sidx + step] <= f) sidx += step;  // seg_first[i] = total for i >= nseg
          sidx = uni(sidx);
          blk = uni(segs[sidx].b0) + f - uni(seg_first[sidx]);
          return sidx;
        }
        static_done = true;
      }
      int i = 0;
      if (lane == 0) i = __hip_atomic_fetch_add(phead, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      i = uni(i);
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      unsigned long long v;
      while (true) {
        v = __hip_atomic_load(&ring[i & (kRing - 1)], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (uni(static_cast<int>(v >> 32)) == i) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
          late = true;
          return -1;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      const int p = uni(static_cast<int>(static_cast<unsigned>(v)));
      if (p < 0) return -1;
      int q = 0;  // pool_first[j] = pool_total for j >= pool_nseg
#pragma unroll
      for (int step = kMaxPoolSegs / 2; step >= 1; step >>= 1)
        if (P.pool_first[q + step] <= p) q += step;
      q = uni(q);
      blk = uni(P.pool_segs[q].b0) + p - uni(P.pool_first[q]);
      return nseg + q;
    };
    auto block_at = [&](int sidx, int blk, const unsigned char*& base, int& tiles, int& rot) {
      const Level& L = levels[seg_at(segs, nseg, P, sidx).level];
      tiles = uni(L.tiles);
      base = uni(L.w) + static_cast<size_t>(blk) * static_cast<size_t>(tiles) * 1024u + lane * 16u;
      rot = block_rot<G>(blk, tiles);
    };

    Producer pr;
    pr.base = P.park + lane * 16u;
    pr.T = pr.rot = pr.pos = 0;
    pr.nbase = P.park + lane * 16u;
    pr.nT = pr.nrot = 0;
    int cs, cblk = 0;  // the consumer's current block
    cs = claim(cblk);
    if (cs >= 0) block_at(cs, cblk, pr.base, pr.T, pr.rot);
    // Two groups of G tile registers: one group's loads are in flight while
    // the other group is consumed (G == 0: one tile at a time, no prefetch).
    constexpr int GR = G > 0 ? G : 1;
    u32x4 ra[GR], rb[GR];
    if (G > 0) pr.template issue<GR>(ra);

    const unsigned tboff = ops::ternary_b_entry(n, g);                 // ternary B entry of this lane
    const unsigned iboff = ops::int8_b_entry(n, g);                    // int8 B entry of this lane
    const int icexp = n < static_cast<unsigned>(ops::kInt8Digits) ? static_cast<int>(8u * n) : -1000;  // digit weight (other columns vanish)
    int cur = -1;  // segment whose operands this wave is using
    const unsigned char* buf = smem;
    int T = 0, rows = 0, kind = 0, bsc_off = 0, asc_off = 0;
    const float* scale = nullptr;
    float* y = nullptr;
    while (cs >= 0) {
      // Without prefetch the loads have not crossed into this block yet:
      // make it current before the next claim replaces the claimed block.
      if (G == 0) pr.step_block();
      // The next block is claimed late, so that a wave holds as little
      // unstarted work as possible when the pool runs out: just before the
      // iteration whose loads cross into it (at the start for blocks of one
      // iteration and without prefetch).
      int nblk = 0, ns = -1;
      auto claim_next = [&]() {
        ns = claim(nblk);
        if (ns >= 0) {
          block_at(ns, nblk, pr.nbase, pr.nT, pr.nrot);
        } else {
          pr.nbase = P.park + lane * 16u;
          pr.nT = pr.nrot = 0;
        }
      };
      if (cs != cur) {
        lds_publish(&done[wave], cs - 1);  // done with every segment before cs
        const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
        while (uni(lds_acquire(ready)) < cs) {
          if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
            late = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        cur = cs;
        buf = smem + uni(seg_pos[2 * cs]);
        const Level& L = levels[seg_at(segs, nseg, P, cs).level];
        T = uni(L.tiles);
        rows = uni(L.rows);
        scale = uni(L.scale);
        y = uni(L.y);
        kind = uni(L.kind);
        bsc_off = uni(L.bsc_off);
        asc_off = uni(L.asc_off);
      }
      const int blk = cblk;
      const int rot = block_rot<G>(blk, T);
      auto wrap = [&](int t) { return t >= T ? t - T : t; };
      // One block: T tiles from tile rot on, 2 G per iteration; both kinds
      // share the loop so that the tile registers keep one assignment.
      v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};  // ternary: two chains; int8: acc0 = sum
      v4i iacc = {0, 0, 0, 0};
      unsigned sb = 0, sa = 0;
      auto group = [&](const u32x4(&x)[GR], int t0) {
        if (kind == kKindTernary) {
#pragma unroll
          for (int j = 0; j < GR; ++j) {
            v8i a0, a1;
            ternary_unpack(x[j], a0, a1);
            const int t = t0 + j;
            const bool odd = G > 0 ? (j & 1) != 0 : (t & 1) != 0;
            if (odd) ternary_mfma<true>(a0, a1, t, buf, bsc_off, asc_off, tboff, lane, g, sb, sa, acc0, acc1);
            else ternary_mfma<false>(a0, a1, t, buf, bsc_off, asc_off, tboff, lane, g, sb, sa, acc0, acc1);
          }
        } else {
#pragma unroll
          for (int j = 0; j < GR; ++j) {
            const int t = t0 + j;
            int8_mfma(x[j], t, buf, iboff, iacc);
            // exponent sections of 4 tiles (T and G are multiples of 4 unless G == 0)
            const bool end = G > 0 ? (j % kSectionMfmas) == kSectionMfmas - 1 : (t % kSectionMfmas) == kSectionMfmas - 1;
            if (end) int8_section(t, buf, bsc_off, icexp, iacc, acc0);
          }
        }
      };
      if (G > 0) {
        auto iterations = [&](int from, int to) {
          for (int it = from; it < to; it += 2 * GR) {
            pr.template issue<GR>(rb);
            __builtin_amdgcn_sched_barrier(0);
            group(ra, wrap(rot + it));
            __builtin_amdgcn_sched_barrier(0);
            pr.template issue<GR>(ra);
            __builtin_amdgcn_sched_barrier(0);
            group(rb, wrap(rot + it + GR));
            __builtin_amdgcn_sched_barrier(0);
          }
        };
        const int tc = T - 2 * GR;  // the last iteration's loads cross into the next block
        iterations(0, tc);
        claim_next();
        iterations(tc, T);
      } else {
        claim_next();
        for (int it = 0; it < T; ++it) {
          pr.template issue<GR>(ra);
          group(ra, it);
        }
      }
      const v4f sc = block_scales(scale, blk, rows, g);
      v4f a = kind == kKindTernary ? acc0 + acc1 : acc0;  // rows 4g + i, digit column n
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = row16_sum(kind != kKindTernary || n < static_cast<unsigned>(ops::kSplits) ? a[i] : 0.f) * sc[i];
      const int r0 = blk * 16 + static_cast<int>(4 * g);
      if (n == 0) {
        if (y) {
          if (r0 + 3 < rows) {
            *(g_f32x4*)(y + r0) = f32x4{a[0], a[1], a[2], a[3]};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (r0 + i < rows) ((g_float*)y)[r0 + i] = a[i];
          }
        }
        if (kind != kKindTernary) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (r0 + i < rows && a[i] > best) {  // a lane's rows of one block ascend; ties keep the lower index
              best = a[i];
              best_idx = static_cast<unsigned>(r0 + i);
            }
        }
      }
      cs = ns;
      cblk = nblk;
    }
    lds_publish(&done[wave], nall);  // this wave reads no operand buffer any more
    if (late && lane == 0) __hip_atomic_store(P.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // Workgroup (max, lowest index) of its vocabulary rows, then the last
  // workgroup to arrive reduces every workgroup's key into the token.
  unsigned long long key = best_idx == 0xFFFFFFFFu ? 0ull : argmax_key(best, best_idx);
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(key, off, kWave);
    key = o > key ? o : key;
  }
  if (lane == 0) wkeys[wave] = key;
  __syncthreads();
  if (wave == 0) {
    unsigned last = 0;
    if (lane == 0) {
      unsigned long long m = 0ull;
      for (int i = 0; i < kWaves; ++i) m = wkeys[i] > m ? wkeys[i] : m;
      __hip_atomic_store(&P.partials[blockIdx.x], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned prev = __hip_atomic_fetch_add(P.arrivals, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      last = prev == static_cast<unsigned>(P.grid) - 1u ? 1u : 0u;
    }
    if (uni(last)) {
      unsigned long long m = 0ull;
      for (int b = static_cast<int>(lane); b < P.grid; b += 64) {
        const unsigned long long o = __hip_atomic_load(&P.partials[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        m = o > m ? o : m;
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(m, off, kWave);
        m = o > m ? o : m;
      }
      if (lane == 0) {
        *P.token_out = static_cast<int>(argmax_key_index(m));
        // every workgroup has arrived, so nobody claims any more: reset for the next step
        __hip_atomic_store(P.pool_next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(P.arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// --------------------------------------------------------------- conversion
// Ternary level input: thread (beta, h, G) of level L converts summation
// group G of half h of the 32-element block beta (operands.h); the four
// quarters of a block are adjacent lanes and share the block exponent.
__device__ void convert_ternary(const Level& L, int tid, unsigned lane) {
  const int beta = tid >> 2, h = (tid >> 1) & 1, G = tid & 1;
  const bool ok = beta < L.cols / 32;
  float xs[16];
  float amax = 0.f;
  const cg_f32x4* src = (const cg_f32x4*)(L.x + 32 * (ok ? beta : 0) + 16 * h);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = ok ? src[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    xs[4 * q] = v.x; xs[4 * q + 1] = v.y; xs[4 * q + 2] = v.z; xs[4 * q + 3] = v.w;
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));  // the other half of the block
  (void)lane;
  if (ok) ops::write_ternary_quarter(L.b_out, L.bsc_off, L.asc_off, beta, h, G, xs, ops::block_exponent(amax));
}

// Vocabulary input h: wave `sec` converts section sec (256 elements); lane
// t owns elements 4t .. 4t + 3 of it.
__device__ void convert_int8(const Level& L, const float* h, int sec, unsigned lane) {
  const f32x4 v = ((const cg_f32x4*)(h + 256 * sec))[lane];
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
  const int e = ops::block_exponent(amax);
  const float hv[4] = {v.x, v.y, v.z, v.w};
  unsigned dw[ops::kInt8Digits];
  ops::int8_digits4(hv, e, dw);
  const int m = 4 * sec + static_cast<int>(lane >> 4), g = static_cast<int>((lane & 15u) >> 2), j0 = 4 * static_cast<int>(lane & 3u);
  unsigned char* b = L.b_out;
#pragma unroll
  for (int d = 0; d < ops::kInt8Digits; ++d)
    *reinterpret_cast<unsigned*>(b + m * kInt8MfmaBytes + ops::int8_b_entry(d, g) + j0) = dw[d];
  if (lane == 0) *reinterpret_cast<int*>(b + L.bsc_off + 4 * sec) = e - ops::kInt8FixedBits;
}

// One-dimensional grid: the workgroups of level i are conv0(i) ..
// conv0(i + 1) - 1 (ternary: 64 blocks of 32 inputs per workgroup, four
// threads per block; the vocabulary: four 256-value sections of h, one per
// wave); the plan's table names each workgroup's level.
__global__ __launch_bounds__(256) void stream_convert_kernel(const Plan* __restrict__ plan,
                                                             const Level* __restrict__ levels) {
  const Plan& P = *plan;
  const int wg = static_cast<int>(blockIdx.x);
  const int lo = ((const __attribute__((address_space(4))) int*)P.conv_level)[wg];  // a scalar load
  const Level& L = levels[lo];
  const int local = wg - L.conv0;
  if (lo < P.n_levels) {
    convert_ternary(L, local * 256 + static_cast<int>(threadIdx.x), threadIdx.x & 63u);
  } else {
    const int sec = local * 4 + static_cast<int>(threadIdx.x >> 6);
    if (sec < P.hidden / 256) convert_int8(L, P.h, sec, threadIdx.x & 63u);
  }
}

}  // namespace

// ----------------------------------------------------------------- host side
namespace {

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
constexpr int kMaxGrid = 1024;

struct SLayout {
  size_t plan, partials, arrivals, levels, segs, seg_count, conv_level, park, regions, total;
};

// Conversion workgroups of level i (the vocabulary: i == n_levels): 4
// threads per 32-input ternary block, one wave per 256-value section of h.
int conv_blocks(const pwg_step_desc* d, int i) {
  if (i < d->n_levels) return static_cast<int>((d->levels[i].cols / 32 * 4 + 255) / 256);
  return static_cast<int>((d->hidden / 256 + 3) / 4);
}

size_t region_bytes(const pwg_step_desc* d, int i) {
  return i < d->n_levels ? ternary_region_bytes(d->levels[i].cols) : int8_region_bytes(d->hidden);
}

SLayout layout_for(const pwg_step_desc* d) {
  SLayout L{};
  L.plan = 0;
  L.partials = align_up(sizeof(Plan), 256);
  L.arrivals = L.partials + kMaxGrid * 8;
  L.levels = align_up(L.arrivals + 256, 256);
  L.segs = align_up(L.levels + static_cast<size_t>(d->n_levels + 1) * sizeof(Level), 256);
  L.seg_count = align_up(L.segs + static_cast<size_t>(kMaxGrid) * (d->n_levels + 1) * sizeof(Seg), 256);
  int conv = 0;
  for (int i = 0; i <= d->n_levels; ++i) conv += conv_blocks(d, i);
  L.conv_level = align_up(L.seg_count + kMaxGrid * 4, 256);
  L.park = align_up(L.conv_level + static_cast<size_t>(conv) * 4, 256);
  L.regions = L.park + kParkBytes;
  size_t end = L.regions;
  for (int i = 0; i <= d->n_levels; ++i) end += align_up(region_bytes(d, i), 256);
  L.total = end;
  return L;
}

// LDS of the step kernel: two operand buffers, then flags, the segments'
// first-block table and the pool claim ring.
size_t lds_bytes(const pwg_step_desc* d) {
  size_t need = 0;
  for (int i = 0; i <= d->n_levels; ++i) need = std::max(need, region_bytes(d, i));
  return 2 * align_up(need, 16) + kLdsTailBytes;
}

Plan* plan_ptr(const pwg_step_desc* d, size_t ws_offset) {
  const uintptr_t p = reinterpret_cast<uintptr_t>(d->workspace) + ws_offset;
  return reinterpret_cast<Plan*>(align_up(p, 256));
}

int grid_size(int* grid) {
  static int cus_of[64] = {};  // CUs per device, queried once
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && dev >= 0 && dev < 64 && cus_of[dev] > 0) {
    cus = cus_of[dev];
  } else {
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(PWG_ERR_HIP, "stream step: device query failed: %s", hipGetErrorString(e));
    if (dev >= 0 && dev < 64) cus_of[dev] = cus;
  }
  *grid = cus < kMaxGrid ? cus : kMaxGrid;
  return PWG_OK;
}


// The ternary levels that end the shared pool: the last levels (in
// decoder order) with the fewest tiles per block, until they hold
// kPoolTailShare of the weight bytes.  Small blocks make the last claims
// even out; the vocabulary's blocks are four times larger.
std::vector<int> pool_tail_levels(const pwg_step_desc* d) {
  std::vector<int> out;
  if (d->n_levels == 0) return out;
  int64_t min_cols = d->levels[0].cols, total = d->vocab * d->hidden;
  for (int i = 0; i < d->n_levels; ++i) {
    min_cols = std::min<int64_t>(min_cols, d->levels[i].cols);
    total += d->levels[i].rows * d->levels[i].cols / 4;
  }
  int64_t acc = 0;
  for (int i = d->n_levels - 1; i >= 0 && static_cast<int>(out.size()) < kMaxPoolSegs - 1; --i) {
    if (d->levels[i].cols != min_cols) continue;
    out.insert(out.begin(), i);
    acc += d->levels[i].rows * d->levels[i].cols / 4;
    if (static_cast<double>(acc) >= kPoolTailShare * static_cast<double>(total)) break;
  }
  return out;
}

// Splits the concatenation of the ternary levels' 16-row blocks (all but
// the pool's tail levels) into `grid` contiguous ranges of equal size; each
// workgroup's ranges are its static segments, one per level it touches.
void partition(const pwg_step_desc* d, int grid, const std::vector<int>& tail, std::vector<std::vector<Seg>>& out) {
  std::vector<int> lvl;
  for (int i = 0; i < d->n_levels; ++i)
    if (std::find(tail.begin(), tail.end(), i) == tail.end()) lvl.push_back(i);
  const int n = static_cast<int>(lvl.size());
  out.assign(grid, {});
  if (n == 0) return;
  std::vector<long long> blocks(n);
  std::vector<double> cost(n), start(n + 1);
  for (int i = 0; i < n; ++i) {
    blocks[i] = (d->levels[lvl[i]].rows + 15) / 16;
    cost[i] = static_cast<double>(d->levels[lvl[i]].cols / 256);
  }
  start[0] = 0.0;
  for (int i = 0; i < n; ++i) start[i + 1] = start[i] + static_cast<double>(blocks[i]) * cost[i];
  const double total = start[n];
  auto pos = [&](double x, int& lv, long long& b) {
    lv = 0;
    while (lv < n - 1 && x >= start[lv + 1]) ++lv;
    b = static_cast<long long>(std::llround((x - start[lv]) / cost[lv]));
    b = b < 0 ? 0 : (b > blocks[lv] ? blocks[lv] : b);
  };
  int lv0 = 0;
  long long b0 = 0;
  for (int w = 0; w < grid; ++w) {
    int lv1;
    long long b1;
    if (w + 1 == grid) {
      lv1 = n - 1;
      b1 = blocks[n - 1];
    } else {
      pos(total * (w + 1) / grid, lv1, b1);
    }
    for (int lv = lv0; lv <= lv1; ++lv) {
      const long long a = lv == lv0 ? b0 : 0;
      const long long e = lv == lv1 ? b1 : blocks[lv];
      if (e > a) out[w].push_back(Seg{lvl[lv], static_cast<int>(a), static_cast<int>(e), 0});
    }
    lv0 = lv1;
    b0 = b1;
  }
}

// Prefetch group: G tiles per register group (two groups per compute wave),
// 2G dividing every level's tiles per block, so that the register of a tile
// is known at compile time; 0 (no prefetch) for other shapes.
int prefetch_depth(const pwg_step_desc* d) {
  long long gcd = d->hidden / 64;
  for (int i = 0; i < d->n_levels; ++i) {
    long long a = gcd, b = d->levels[i].cols / 256;
    while (b) {
      const long long t = a % b;
      a = b;
      b = t;
    }
    gcd = a;
  }
  return gcd % 16 == 0 ? 8 : 0;
}

}  // namespace

int step_stream_check(const pwg_step_desc* d) {
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    if (L.cols % 256 != 0 || L.cols > kMaxStreamCols)
      return fail(PWG_ERR_UNSUPPORTED, "stream schedule: level %d needs cols %% 256 == 0 and cols <= %d (has %lld)", i,
                  kMaxStreamCols, static_cast<long long>(L.cols));
    if (L.rows >= (int64_t{1} << 30)) return fail(PWG_ERR_ARG, "stream schedule: level %d has too many rows", i);
  }
  if (d->hidden % 256 != 0 || d->hidden > kMaxStreamCols)
    return fail(PWG_ERR_UNSUPPORTED, "stream schedule: hidden must be a multiple of 256 and at most %d", kMaxStreamCols);
  if (d->vocab >= (int64_t{1} << 30)) return fail(PWG_ERR_ARG, "stream schedule: vocabulary too large");
  if (lds_bytes(d) > kMaxLds)
    return fail(PWG_ERR_UNSUPPORTED, "stream schedule: operands and claim counters need %zu bytes of LDS", lds_bytes(d));
  return PWG_OK;
}

size_t step_stream_workspace(const pwg_step_desc* d) { return layout_for(d).total + 256; }

int step_stream_plan(const pwg_step_desc* d, size_t ws_offset, void* stream) {
  TRY(step_stream_check(d));
  int grid = 0;
  TRY(grid_size(&grid));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const SLayout lay = layout_for(d);
  Plan* dplan = plan_ptr(d, ws_offset);
  char* dbase = reinterpret_cast<char*>(dplan);
  size_t need = 0;
  for (int i = 0; i <= d->n_levels; ++i) need = std::max(need, region_bytes(d, i));

  Plan h{};
  h.n_levels = d->n_levels;
  h.grid = grid;
  h.buf_bytes = static_cast<int>(align_up(need, 16));
  h.vocab = static_cast<int>(d->vocab);
  h.hidden = static_cast<int>(d->hidden);
  h.depth = prefetch_depth(d);
  h.h = d->h;
  h.emb_table = reinterpret_cast<const u32x4*>(d->emb_table);
  h.emb_scale = d->emb_scale;
  h.token_in = d->token_in;
  h.token_out = d->token_out;
  h.emb_row_out = reinterpret_cast<u32x4*>(d->emb_row_out);
  h.emb_scale_out = d->emb_scale_out;
  h.emb_deq_out = reinterpret_cast<float4*>(d->emb_deq_out);
  h.park = reinterpret_cast<const unsigned char*>(dbase + lay.park);
  h.partials = reinterpret_cast<unsigned long long*>(dbase + lay.partials);
  h.arrivals = reinterpret_cast<unsigned*>(dbase + lay.arrivals);
  h.status = reinterpret_cast<unsigned*>(dbase + lay.arrivals + 64);
  h.seg_count = reinterpret_cast<const int*>(dbase + lay.seg_count);
  h.conv_level = reinterpret_cast<const int*>(dbase + lay.conv_level);

  std::vector<Level> lv(d->n_levels + 1);
  size_t off = lay.regions;
  for (int i = 0; i <= d->n_levels; ++i) {
    Level& L = lv[i];
    L.b = reinterpret_cast<const unsigned char*>(dbase + off);
    L.b_out = reinterpret_cast<unsigned char*>(dbase + off);
    L.b_bytes = static_cast<int>(region_bytes(d, i));
    if (i < d->n_levels) {
      const pwg_level& S = d->levels[i];
      L.w = static_cast<const unsigned char*>(S.w_packed);
      L.scale = S.row_scale;
      L.x = S.x;
      L.y = S.y;
      L.rows = static_cast<int>(S.rows);
      L.cols = static_cast<int>(S.cols);
      L.tiles = static_cast<int>(S.cols / 256);
      L.kind = kKindTernary;
      L.bsc_off = static_cast<int>(ternary_bsc_off(S.cols));
      L.asc_off = static_cast<int>(ternary_asc_off(S.cols));
    } else {
      L.w = reinterpret_cast<const unsigned char*>(d->out_table);
      L.scale = d->out_scale;
      L.x = d->h;
      L.y = d->logits_out;
      L.rows = static_cast<int>(d->vocab);
      L.cols = static_cast<int>(d->hidden);
      L.tiles = static_cast<int>(d->hidden / 64);
      L.kind = kKindInt8;
      L.bsc_off = static_cast<int>(int8_exp_off(d->hidden));
      L.asc_off = 0;
    }
    off += align_up(region_bytes(d, i), 256);
  }
  int conv = 0;
  std::vector<int> conv_level;
  for (int i = 0; i <= d->n_levels; ++i) {
    lv[i].conv0 = conv;
    conv += conv_blocks(d, i);
    conv_level.insert(conv_level.end(), conv_blocks(d, i), i);
  }

  const std::vector<int> tail = pool_tail_levels(d);
  h.pool_nseg = 0;
  h.pool_first[0] = 0;
  auto add_pool = [&](int level, int blocks) {
    h.pool_segs[h.pool_nseg] = Seg{level, 0, blocks, 0};
    h.pool_first[h.pool_nseg + 1] = h.pool_first[h.pool_nseg] + blocks;
    h.pool_nseg += 1;
  };
  add_pool(d->n_levels, static_cast<int>((d->vocab + 15) / 16));
  for (int t : tail) add_pool(t, static_cast<int>((d->levels[t].rows + 15) / 16));
  h.pool_total = h.pool_first[h.pool_nseg];
  for (int i = h.pool_nseg + 1; i <= kMaxPoolSegs; ++i) h.pool_first[i] = h.pool_total;
  h.pool_next = reinterpret_cast<unsigned*>(dbase + lay.arrivals + 128);
  std::vector<std::vector<Seg>> parts;
  partition(d, grid, tail, parts);
  int stride = 1;
  for (const auto& v : parts) stride = std::max(stride, static_cast<int>(v.size()));
  std::vector<Seg> seg_flat(static_cast<size_t>(grid) * stride, Seg{0, 0, 0, 0});
  std::vector<int> seg_count(grid);
  for (int b = 0; b < grid; ++b) {
    seg_count[b] = static_cast<int>(parts[b].size());
    for (size_t j = 0; j < parts[b].size(); ++j) seg_flat[static_cast<size_t>(b) * stride + j] = parts[b][j];
  }
  h.seg_stride = stride;
  if (stride > kMaxWgSegs)
    return fail(PWG_ERR_UNSUPPORTED, "stream schedule: a workgroup would touch %d levels (at most %d)", stride,
                kMaxWgSegs);

  hipError_t e = hipMemsetAsync(dbase, 0, lay.regions, st);  // partials, arrival counter, status, park
  if (e == hipSuccess) e = hipMemcpyAsync(dplan, &h, sizeof(Plan), hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dbase + lay.levels, lv.data(), lv.size() * sizeof(Level), hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dbase + lay.segs, seg_flat.data(), seg_flat.size() * sizeof(Seg), hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dbase + lay.seg_count, seg_count.data(), seg_count.size() * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dbase + lay.conv_level, conv_level.data(), conv_level.size() * 4, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_plan: %s", hipGetErrorString(e));
  return PWG_OK;
}

int step_stream_launch(const pwg_step_desc* d, size_t ws_offset, void* stream) {
  int grid = 0;  // (the description was checked by the caller)
  TRY(grid_size(&grid));
  Plan* dplan = plan_ptr(d, ws_offset);
  char* dbase = reinterpret_cast<char*>(dplan);
  const SLayout lay = layout_for(d);
  const Level* lv = reinterpret_cast<const Level*>(dbase + lay.levels);
  const Seg* segs = reinterpret_cast<const Seg*>(dbase + lay.segs);
  int conv = 0;
  for (int i = 0; i <= d->n_levels; ++i) conv += conv_blocks(d, i);
  const size_t lds = lds_bytes(d);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(stream_convert_kernel, dim3(conv), dim3(256), 0, st, dplan, lv);
  if (prefetch_depth(d) == 8)
    hipLaunchKernelGGL(stream_step_kernel<8>, dim3(grid), dim3(kThreads), lds, st, dplan, lv, segs);
  else
    hipLaunchKernelGGL(stream_step_kernel<0>, dim3(grid), dim3(kThreads), lds, st, dplan, lv, segs);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "stream step launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

int step_stream_status(const pwg_step_desc* d, size_t ws_offset, void* stream) {
  Plan* dplan = plan_ptr(d, ws_offset);
  const SLayout lay = layout_for(d);
  unsigned s = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&s, reinterpret_cast<char*>(dplan) + lay.arrivals + 64, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_status: %s", hipGetErrorString(e));
  if (s == kStatusTimeout) return fail(PWG_ERR_HIP, "stream step: a workgroup's operand wait timed out");
  return PWG_OK;
}

}  // namespace pwg
