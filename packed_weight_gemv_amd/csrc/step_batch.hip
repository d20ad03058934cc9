// Batched decode step on the CDNA4 matrix cores: one pass over every weight
// for B = 4, 8 or 16 vectors.
//
// Page "The Neutrino Engine": section "The 0.6B model does not get to
// decide" (the large model scores several drafted tokens in one batched
// forward pass) and section "A 104 microsecond floor inside a 694
// microsecond step" (every projection applied once per pass, the output
// projection over the whole vocabulary, greedy tokens).  Each level's
// Y[b, r] = s_r * sum_k W_rk X[b, k], the output projection's logits and each
// vector's greedy token, with every weight byte read once per pass.
//
// Two kernels.  The conversion kernel writes the operand digits of every
// level's inputs and of h (batch_core.h) into the workspace and gathers the
// B embedding rows.  The pass kernel (one workgroup per CU) claims work items
// from one global counter: an item is up to 14 row blocks of the vocabulary
// or 7 of one ternary level (two or one per compute wave), which the seven
// compute waves run over K in lock step with the arithmetic of the per-call
// kernels, while a staging wave claims the next item and copies operand
// slices into two or three LDS buffers.  Items come in a fixed order,
// largest first (ternary levels wider than h, the vocabulary, the other
// ternary levels widest K first, halves of the last ones), so that the
// workgroups finish close together.  The last
// workgroup to arrive reduces the per-workgroup argmax keys into each
// vector's token and resets the counters for the next pass.
#include <algorithm>
#include <vector>

#include "batch_core.h"
#include "pwg_internal.h"

namespace pwg {
namespace bstep {

enum : int { kKindTernary = 0, kKindInt8 = 1 };

// One ternary level or (last entry) the vocabulary.
struct BLevel {
  const unsigned char* w;   // tiled weights (16-row x 64-byte tiles)
  const float* scale;       // row scales
  const float* x;           // input [batch][cols] (vocabulary: h)
  float* y;                 // output [batch][rows] (vocabulary: logits or null)
  unsigned char* ops;       // operand digits (workspace)
  int* exps;                // section exponents [cols / 256][batch] (workspace)
  int rows, cols, kind, pad;
};

// Row blocks [rb0, rb1) of one level.
struct BItem {
  int level, rb0, rb1, pad;
};

struct BPlan {
  int n_levels, batch, n_items, n_static;  // items [0, n_static) go round-robin (a multiple of grid)
  int vocab, hidden, grid, pad;
  const BLevel* levels;           // [n_levels + 1], the vocabulary last
  const BItem* items;             // [n_items], in claim order
  const int2* conv_wg;            // [conversion workgroups]: (level or -1 for the embedding rows, first unit)
  unsigned* item_next;            // global claim counter
  unsigned* arrivals;
  unsigned* status;
  unsigned long long* partials;   // [batch][grid] argmax keys
  const unsigned char* park;      // 1 KiB that idle load slots read
  const dev::u32x4* emb_table;
  const float* emb_scale;
  const int32_t* token_in;        // [batch]
  int32_t* token_out;             // [batch]
  dev::u32x4* emb_row_out;        // [batch][hidden / 16]
  float* emb_scale_out;           // [batch]
  float4* emb_deq_out;            // [batch][hidden / 4] or null
};

}  // namespace bstep

namespace {

using namespace bcore;
using namespace bstep;

constexpr int kRing = 8;        // claimed items a workgroup holds (ring in LDS)
constexpr int kTernarySets = 4; // row-block sets per ternary item and compute wave
constexpr int kMaxGrid = 1024;
enum : unsigned { kStatusOk = 0, kStatusTimeout = 1 };

// Embedding row of vector b's previous token (one wave).
__device__ void embed_row(const BPlan& P, int b, unsigned lane) {
  const int id = P.token_in[b];
  const bool ok = id >= 0 && id < P.vocab;
  const int nchunks = P.hidden >> 4;
  const float s = ok ? P.emb_scale[id] : __builtin_nanf("");
  if (lane == 0) P.emb_scale_out[b] = s;
  for (int c0 = 0; c0 < nchunks; c0 += 64) {  // wave-uniform trip count
    const int c = c0 + static_cast<int>(lane);
    if (c < nchunks) {
      const u32x4 v = ok ? P.emb_table[static_cast<size_t>(id) * nchunks + c] : u32x4{0u, 0u, 0u, 0u};
      P.emb_row_out[static_cast<size_t>(b) * nchunks + c] = v;
      if (P.emb_deq_out) {
        const unsigned wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          P.emb_deq_out[static_cast<size_t>(b) * (nchunks * 4) + 4 * c + q] =
              ok ? make_float4(static_cast<float>(static_cast<int8_t>(wd[q] & 0xFF)) * s,
                               static_cast<float>(static_cast<int8_t>((wd[q] >> 8) & 0xFF)) * s,
                               static_cast<float>(static_cast<int8_t>((wd[q] >> 16) & 0xFF)) * s,
                               static_cast<float>(static_cast<int8_t>(wd[q] >> 24)) * s)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
}

// Units: per level, (block, vector) pairs, blocks of 1,024 values (ternary)
// or 256 (the vocabulary's h); unit u of a level is block u / batch of
// vector u % batch.  Each wave of the grid converts one unit: workgroup w
// converts units c.y .. c.y + 3 of level c.x (c = conv_wg[w]; units past the
// level's last are skipped), or, for c.x < 0, the embedding rows of vectors
// c.y .. c.y + 3.
__global__ __launch_bounds__(256) void bstep_convert_kernel(const BPlan* __restrict__ plan) {
  const BPlan& P = *plan;
  const unsigned lane = threadIdx.x & 63u;
  typedef const __attribute__((address_space(4))) int cint;
  const cint* cw = (const cint*)P.conv_wg + 2 * blockIdx.x;  // scalar loads
  const int level = cw[0], u = uni(cw[1] + static_cast<int>(threadIdx.x >> 6));
  if (level >= 0) {
    const BLevel& L = P.levels[level];
    const int cols = uni(L.cols), kind = uni(L.kind), batch = P.batch;
    unsigned char* ops = uni(L.ops);
    int* exps = uni(L.exps);
    const int blk = u / batch, b = u % batch;
    if (blk >= cols / (kind == kKindTernary ? 1024 : 256)) return;
    const float* xb = uni(L.x) + static_cast<size_t>(b) * cols;
    if (kind == kKindTernary) convert_ternary_block(xb, blk, b, batch / 4, ops, exps, lane);
    else convert_int8_section(xb, blk, b, batch / 4, ops, exps, lane);
  } else if (u < P.batch) {
    embed_row(P, u, lane);
  }
}

// Operand slice buffers in LDS: three for 4 and 8 vectors (the staging wave
// runs two slices ahead), two for 16 (three 64 KiB slices would not fit).
template <int NG>
constexpr int slice_bufs() {
  return NG <= 2 ? 3 : 2;
}

template <int NG>
constexpr size_t bstep_lds() {
  return slice_bufs<NG>() * SliceShape<NG>::kBytes + 64 + 16 * kRing + kW * 4 * NG * 8;
}

// Compute-wave state shared by the two phases (int8 items, then ternary).
struct WaveState {
  int item;   // local sequence number of the current item
  int t0;     // first slice number of the current item
  int4 cur;   // the current item (level < 0: none left)
  bool late;
};

template <int NG>
struct Pass {
  static constexpr int kB = 4 * NG;
  static constexpr int kSliceBytes = SliceShape<NG>::kBytes;
  static constexpr int kBufs = slice_bufs<NG>();
  const BPlan& P;
  unsigned char* smem;
  int* ready;        // highest slice staged
  int* nknown;       // items claimed so far (ring entries written)
  int* done;         // [kW]: highest slice a compute wave is done with
  int4* ring;        // [kRing] claimed items
  unsigned lane;
  int wave;

  __device__ __forceinline__ Pass(const BPlan& p, unsigned char* s, unsigned l, int w)
      : P(p), smem(s), lane(l), wave(w) {
    ready = reinterpret_cast<int*>(smem + kBufs * kSliceBytes);
    nknown = ready + 1;
    done = ready + 2;
    ring = reinterpret_cast<int4*>(smem + kBufs * kSliceBytes + 64);
  }

  // Item i of this workgroup once the staging wave has claimed it.
  __device__ __forceinline__ int4 wait_item(int i, bool& late) const {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    while (uni(lds_acquire(nknown)) <= i) {
      if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
        late = true;
        return make_int4(-1, 0, 0, 0);
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const int4 v = ring[i % kRing];
    return make_int4(uni(v.x), uni(v.y), uni(v.z), 0);
  }

  __device__ __forceinline__ int kind_of(int level) const { return uni(P.levels[level].kind); }

  // The staging wave: claims items into the ring and copies each item's
  // operand slices (t counts slices over the items) into buffer t & 1 once
  // every compute wave is done with slice t - kBufs.  The item after the current
  // one is claimed before the current one's second-to-last slice, so that
  // the compute waves can issue its first tile loads in time.
  __device__ void stage(bool& late) {
    int claimed = 0;
    // Claim k of this workgroup: item blockIdx.x + k grid while those are
    // round-robin items (no atomic: under the full memory load an atomic
    // takes microseconds, and its wait drains the slice copies in flight),
    // then the next item of the global counter.
    auto claim = [&]() -> int4 {
      unsigned j = 0;
      if (claimed < P.n_static / P.grid) {
        j = blockIdx.x + static_cast<unsigned>(claimed) * static_cast<unsigned>(P.grid);
      } else {
        if (lane == 0)
          j = static_cast<unsigned>(P.n_static) + __hip_atomic_fetch_add(P.item_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        j = static_cast<unsigned>(uni(static_cast<int>(j)));
      }
      int4 it = make_int4(-1, 0, 0, 0);
      if (j < static_cast<unsigned>(P.n_items)) {
        const BItem& I = P.items[j];
        it = make_int4(uni(I.level), uni(I.rb0), uni(I.rb1), 0);
      }
      if (lane == 0) ring[claimed % kRing] = it;
      ++claimed;
      lds_publish(nknown, claimed);  // waits for the ring write first
      return it;
    };
    constexpr int kOps = SliceShape<NG>::kOps, kEb = SliceShape<NG>::kExpBytes;  // kEb: a multiple of 16
    int4 cur = claim();
    int t = 0;
    while (cur.x >= 0) {
      const BLevel& L = P.levels[cur.x];
      const int nsl = uni(L.cols) / (64 * kSliceSteps);
      const unsigned char* ops = L.ops;
      const unsigned char* exps = reinterpret_cast<const unsigned char*>(L.exps);
      int4 nxt = make_int4(-1, 0, 0, 0);
      for (int j = 0; j < nsl; ++j, ++t) {
        if (j == (nsl > 1 ? nsl - 2 : 0)) nxt = claim();
        if (t >= kBufs) {
          const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
          while (true) {
            const int d = (lane >= 1 && lane < kW) ? lds_acquire(&done[lane]) : t;
            if (__all(d >= t - kBufs)) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
              late = true;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        }
        unsigned char* dst = smem + (t % kBufs) * kSliceBytes;
        const unsigned char* src = ops + static_cast<size_t>(j) * kOps;
        for (int o = 0; o < kOps; o += 1024)
          __builtin_amdgcn_global_load_lds(src + o + 16 * lane, (__attribute__((address_space(3))) void*)(dst + o), 16, 0, 0);
        if (16 * static_cast<int>(lane) < kEb)
          __builtin_amdgcn_global_load_lds(exps + static_cast<size_t>(j) * kEb + 16 * lane,
                                           (__attribute__((address_space(3))) void*)(dst + kOps), 16, 0, 0);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
        lds_publish(ready, t);
      }
      cur = nxt;
    }
  }

  // Compute wave k (0..6): the items of one kind, starting at S.cur, until
  // an item of the other kind or the end.  An item's row blocks form up to
  // kL sets of kCW x kR (set l of wave k: blocks rb0 + (l kCW + k) kR + r);
  // the wave runs every set of the item through each staged slice before
  // the next slice, so a slice serves up to kL x kCW x kR row blocks.  Tile
  // loads go in register groups of kLoads per set, two groups in flight
  // (one group's loads are issued before the previous group is consumed),
  // across set, slice and item boundaries.
  template <bool kTernary>
  __device__ void phase(int k, WaveState& S, float (&best)[NG], unsigned (&bidx)[NG]) {
    using Core = Compute<NG, kTernary>;
    constexpr int kR = Core::kR;
    constexpr int kSPL = Core::kStepsPerLoad;
    constexpr int kL = kTernary ? kTernarySets : 1;
    constexpr int kGps = kSliceSteps / kSPL / kLoads;  // register groups per slice and set: int8 4, ternary 1
    constexpr int kMaxGroups = kL * kGps;              // register groups per slice: 4
    static_assert(kMaxGroups % 2 == 0 && kGps >= 1, "groups alternate between two register sets");
    constexpr int kMine = kTernary ? kKindTernary : kKindInt8;
    const Core core(lane);
    u32x4 xa[kLoads][kR], xb[kLoads][kR];
    const unsigned char* lp[kL][kR];  // each slot's first tile load of the item
    int lstride[kL][kR];              // bytes between tile loads, or 0 for a parked slot
    int ngroups = 0;                  // register groups per slice of the current item (even)
    // Points the slots at this wave's row blocks of item `it` (park when it
    // is the end or of the other kind); returns its groups per slice.
    auto set_item = [&](int4 it) -> int {
      const bool mine = it.x >= 0 && kind_of(it.x) == kMine;
      const unsigned char* w = nullptr;
      int nloads = 0;
      if (mine) {
        const BLevel& L = P.levels[it.x];
        w = L.w;
        nloads = uni(L.cols) / (64 * kSPL);
      }
#pragma unroll
      for (int l = 0; l < kL; ++l)
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int rb = it.y + (l * kCW + k) * kR + r;
          const bool valid = mine && rb < it.z;
          lp[l][r] = valid ? w + static_cast<size_t>(rb) * nloads * 1024 + 16 * lane : P.park + 16 * lane;
          lstride[l][r] = valid ? 1024 : 0;
        }
      int sets = (it.z - it.y + kCW * kR - 1) / (kCW * kR);
      sets = sets > kL ? kL : sets;
      return mine ? ((sets * kGps + 1) & ~1) : 2;
    };
    auto issue = [&](u32x4(&x)[kLoads][kR], const unsigned char* const (&p)[kR], const int (&st)[kR], int load0) {
#pragma unroll
      for (int u = 0; u < kLoads; ++u)
#pragma unroll
        for (int r = 0; r < kR; ++r)
          x[u][r] = __builtin_nontemporal_load((g_u32x4*)(p[r] + st[r] * (load0 + u)));
    };
    // Slice t: waits until it is staged (after publishing that this wave is
    // done with slice t - 1); returns its buffer.
    auto enter_slice = [&](int t) -> const unsigned char* {
      lds_publish(&done[wave], t - 1);
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      while (uni(lds_acquire(ready)) < t) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
          S.late = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      return smem + (t % kBufs) * kSliceBytes;
    };

    ngroups = set_item(S.cur);
    issue(xa, lp[0], lstride[0], 0);
    while (S.cur.x >= 0 && kind_of(S.cur.x) == kMine) {
      const BLevel& L = P.levels[S.cur.x];
      const int nsl = uni(L.cols) / (64 * kSliceSteps);
      int4 nxt = make_int4(-1, 0, 0, 0);
      int ng_next = 2;
      v4f facc[kL][kR][NG];
#pragma unroll
      for (int l = 0; l < kL; ++l)
#pragma unroll
        for (int r = 0; r < kR; ++r)
#pragma unroll
          for (int G = 0; G < NG; ++G) facc[l][r][G] = v4f{0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < nsl; ++s) {
        const unsigned char* buf = enter_slice(S.t0 + s);
#pragma unroll
        for (int gi = 0; gi < kMaxGroups; ++gi) {
          if (gi < ngroups) {
            const int l = gi / kGps, q = gi % kGps;
            const int gn = gi + 1 < kMaxGroups ? gi + 1 : kMaxGroups - 1;  // next group in this slice
            const int ln = gn / kGps, qn = gn % kGps;
            auto& xc = (gi % 2 == 0) ? xa : xb;
            auto& xn = (gi % 2 == 0) ? xb : xa;
            if (gi + 1 < ngroups) {
              issue(xn, lp[ln], lstride[ln], (s * kGps + qn) * kLoads);
            } else if (s + 1 < nsl) {
              issue(xn, lp[0], lstride[0], (s + 1) * kGps * kLoads);
            } else {
              nxt = wait_item(S.item + 1, S.late);
              ng_next = set_item(nxt);
              issue(xn, lp[0], lstride[0], 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            core.group(xc, buf, (s * kGps + q) * kLoads, facc[l]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // set_item(nxt) has moved the slots on: results by the item's own blocks
      const int rows = uni(L.rows);
#pragma unroll
      for (int l = 0; l < kL; ++l)
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int rb = S.cur.y + (l * kCW + k) * kR + r;
          if (rb < S.cur.z) core.finish(facc[l], r, rb, L.scale, rows, L.y, best, bidx);
        }
      S.t0 += nsl;
      S.item += 1;
      S.cur = nxt;
      ngroups = ng_next;
    }
  }
};

template <int NG>
__global__ __launch_bounds__(kThreads, 1) void bstep_kernel(const BPlan* __restrict__ plan) {
  constexpr int kB = 4 * NG;
  extern __shared__ __align__(16) unsigned char smem[];
  const BPlan& P = *plan;
  const unsigned lane = threadIdx.x & 63u;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  Pass<NG> pass(P, smem, lane, wave);
  unsigned long long* wkeys =
      reinterpret_cast<unsigned long long*>(smem + slice_bufs<NG>() * SliceShape<NG>::kBytes + 64 + 16 * kRing);  // [kW][kB]
  if (threadIdx.x == 0) {
    *pass.ready = -1;
    *pass.nknown = 0;
  }
  if (threadIdx.x < kW) pass.done[threadIdx.x] = -1;
  if (threadIdx.x < kW * kB) wkeys[threadIdx.x] = 0ull;
  __syncthreads();

  bool late = false;
  if (wave == 0) {
    pass.stage(late);
  } else {
    float best[NG];
    unsigned bidx[NG];
#pragma unroll
    for (int G = 0; G < NG; ++G) {
      best[G] = -__builtin_inff();
      bidx[G] = 0xFFFFFFFFu;
    }
    WaveState S{0, 0, make_int4(-1, 0, 0, 0), false};
    S.cur = pass.wait_item(0, S.late);
    while (S.cur.x >= 0) {  // runs of items of one kind
      if (pass.kind_of(S.cur.x) == kKindInt8) pass.template phase<false>(wave - 1, S, best, bidx);
      else pass.template phase<true>(wave - 1, S, best, bidx);
    }
    late = S.late;
    lds_publish(&pass.done[wave], 0x7FFFFFFF);
    Compute<NG, false>(lane).wave_keys(best, bidx, wkeys + wave * kB);
  }
  if (late && lane == 0) __hip_atomic_store(P.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();

  // Per vector, the workgroup's (max, lowest index) key; the last workgroup
  // to arrive reduces every workgroup's keys into the tokens.
  if (wave == 0) {
    unsigned last = 0;
    if (lane == 0) {
      for (int b = 0; b < kB; ++b) {
        unsigned long long m = 0ull;
        for (int w = 1; w < kW; ++w) m = wkeys[w * kB + b] > m ? wkeys[w * kB + b] : m;
        __hip_atomic_store(&P.partials[static_cast<size_t>(b) * P.grid + blockIdx.x], m, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      const unsigned prev = __hip_atomic_fetch_add(P.arrivals, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      last = prev == static_cast<unsigned>(P.grid) - 1u ? 1u : 0u;
    }
    if (uni(static_cast<int>(last))) {
      // every vector's keys are loaded before any is reduced, so that the
      // loads' latencies overlap
      unsigned long long m[kB];
#pragma unroll
      for (int b = 0; b < kB; ++b) m[b] = 0ull;
      for (int i = static_cast<int>(lane); i < P.grid; i += 64) {
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          const unsigned long long o =
              __hip_atomic_load(&P.partials[static_cast<size_t>(b) * P.grid + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          m[b] = o > m[b] ? o : m[b];
        }
      }
#pragma unroll
      for (int b = 0; b < kB; ++b) {
        for (int off = 32; off >= 1; off >>= 1) {
          const unsigned long long o = __shfl_xor(m[b], off, kWave);
          m[b] = o > m[b] ? o : m[b];
        }
        if (lane == 0) P.token_out[b] = static_cast<int>(argmax_key_index(m[b]));
      }
      if (lane == 0) {
        // every workgroup has arrived, so nobody claims any more: reset for the next pass
        __hip_atomic_store(P.item_next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(P.arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ----------------------------------------------------------------- host side
size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Row blocks per item: kR per compute wave (int8), kR per set and compute
// wave (ternary).
constexpr int kVocabItemBlocks = kCW * Compute<1, false>::kR;
constexpr int kTernaryItemBlocks = kCW * Compute<1, true>::kR * kTernarySets;

struct BLayout {
  size_t plan, counters, partials, park, levels, items, conv, regions, total;
  int n_items;
};

// Conversion workgroups (four units each): per level ceil(units / 4), then
// the embedding rows.
std::vector<int2> conv_table(const pwg_step_desc* d) {
  std::vector<int2> out;
  for (int i = 0; i <= d->n_levels; ++i) {
    const int64_t cols = i < d->n_levels ? d->levels[i].cols : d->hidden;
    const int units = static_cast<int>(cols / (i < d->n_levels ? 1024 : 256)) * d->batch;
    for (int u = 0; u < units; u += 4) out.push_back(make_int2(i, u));
  }
  for (int u = 0; u < d->batch; u += 4) out.push_back(make_int2(-1, u));
  return out;
}

size_t conv_count(const pwg_step_desc* d) {
  size_t n = static_cast<size_t>(d->batch + 3) / 4;
  for (int i = 0; i <= d->n_levels; ++i) {
    const int64_t cols = i < d->n_levels ? d->levels[i].cols : d->hidden;
    n += static_cast<size_t>((cols / (i < d->n_levels ? 1024 : 256)) * d->batch + 3) / 4;
  }
  return n;
}

// Claim order, largest items first: the items of ternary levels wider than
// h (a ternary byte costs the matrix cores more than an int8 byte), the
// vocabulary's, then the other ternary levels' widest K first; the last
// `grid` ternary-item halves are separate items, so that the final claims
// are small.
std::vector<BItem> make_items(const pwg_step_desc* d, int grid) {
  std::vector<BItem> out;
  auto add = [&](int level, int64_t rows, int per) {
    const int nb = static_cast<int>((rows + 15) / 16);
    for (int b = 0; b < nb; b += per) out.push_back(BItem{level, b, std::min(nb, b + per), 0});
  };
  std::vector<int> order(d->n_levels);
  for (int i = 0; i < d->n_levels; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return d->levels[a].cols > d->levels[b].cols; });
  for (int i : order)
    if (d->levels[i].cols > d->hidden) add(i, d->levels[i].rows, kTernaryItemBlocks);
  add(d->n_levels, d->vocab, kVocabItemBlocks);
  const size_t first_ternary = out.size();
  for (int i : order)
    if (d->levels[i].cols <= d->hidden) add(i, d->levels[i].rows, kTernaryItemBlocks);
  const size_t n_split = std::min(out.size() - first_ternary, static_cast<size_t>(grid / 2));
  std::vector<BItem> tail(out.end() - n_split, out.end());
  out.resize(out.size() - n_split);
  for (const BItem& it : tail) {
    const int mid = std::min(it.rb1, it.rb0 + kTernaryItemBlocks / 2);
    out.push_back(BItem{it.level, it.rb0, mid, 0});
    if (mid < it.rb1) out.push_back(BItem{it.level, mid, it.rb1, 0});
  }
  return out;
}

size_t count_items(const pwg_step_desc* d) {
  size_t n = static_cast<size_t>((d->vocab + 15) / 16 + kVocabItemBlocks - 1) / kVocabItemBlocks;
  for (int i = 0; i < d->n_levels; ++i)
    n += static_cast<size_t>((d->levels[i].rows + 15) / 16 + kTernaryItemBlocks - 1) / kTernaryItemBlocks;
  return 2 * n;  // an upper bound: items split in two at the end
}

BLayout layout_for(const pwg_step_desc* d) {
  BLayout L{};
  L.n_items = static_cast<int>(count_items(d));
  L.plan = 0;
  L.counters = align_up(sizeof(BPlan), 256);
  L.partials = L.counters + 256;
  L.park = L.partials + static_cast<size_t>(d->batch) * kMaxGrid * 8;
  L.levels = align_up(L.park + kStepBytes, 256);
  L.items = align_up(L.levels + static_cast<size_t>(d->n_levels + 1) * sizeof(BLevel), 256);
  L.conv = align_up(L.items + static_cast<size_t>(L.n_items) * sizeof(BItem), 256);
  L.regions = align_up(L.conv + conv_count(d) * sizeof(int2), 256);
  size_t end = L.regions;
  for (int i = 0; i < d->n_levels; ++i) end += operand_bytes(d->levels[i].cols, d->batch);
  end += operand_bytes(d->hidden, d->batch);
  L.total = end;
  return L;
}

BPlan* plan_ptr(const pwg_step_desc* d) {
  return reinterpret_cast<BPlan*>(align_up(reinterpret_cast<uintptr_t>(d->workspace), 256));
}

int grid_size(int* grid) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "batched step: device query failed: %s", hipGetErrorString(e));
  *grid = cus < kMaxGrid ? cus : kMaxGrid;
  return PWG_OK;
}

}  // namespace

int step_batch_check(const pwg_step_desc* d) {
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    if (L.cols % 2048 != 0)
      return fail(PWG_ERR_UNSUPPORTED, "batched step: level %d needs cols %% 2048 == 0 (has %lld)", i,
                  static_cast<long long>(L.cols));
    if (L.rows >= (int64_t{1} << 30)) return fail(PWG_ERR_ARG, "batched step: level %d has too many rows", i);
  }
  if (d->hidden % 1024 != 0)
    return fail(PWG_ERR_UNSUPPORTED, "batched step: hidden must be a multiple of 1024 (has %lld)",
                static_cast<long long>(d->hidden));
  if (d->vocab >= (int64_t{1} << 30)) return fail(PWG_ERR_ARG, "batched step: vocabulary too large");
  if (count_items(d) >= (size_t{1} << 30)) return fail(PWG_ERR_ARG, "batched step: too many work items");
  return PWG_OK;
}

size_t step_batch_workspace(const pwg_step_desc* d) { return layout_for(d).total + 256; }

int step_batch_plan(const pwg_step_desc* d, void* stream) {
  TRY(step_batch_check(d));
  int grid = 0;
  TRY(grid_size(&grid));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const BLayout lay = layout_for(d);
  BPlan* dplan = plan_ptr(d);
  char* dbase = reinterpret_cast<char*>(dplan);

  BPlan h{};
  h.n_levels = d->n_levels;
  h.batch = d->batch;
  h.n_items = 0;  // set below
  h.vocab = static_cast<int>(d->vocab);
  h.hidden = static_cast<int>(d->hidden);
  h.grid = grid;
  h.levels = reinterpret_cast<const BLevel*>(dbase + lay.levels);
  h.items = reinterpret_cast<const BItem*>(dbase + lay.items);
  h.conv_wg = reinterpret_cast<const int2*>(dbase + lay.conv);
  h.item_next = reinterpret_cast<unsigned*>(dbase + lay.counters);
  h.arrivals = reinterpret_cast<unsigned*>(dbase + lay.counters + 64);
  h.status = reinterpret_cast<unsigned*>(dbase + lay.counters + 128);
  h.partials = reinterpret_cast<unsigned long long*>(dbase + lay.partials);
  h.park = reinterpret_cast<const unsigned char*>(dbase + lay.park);
  h.emb_table = reinterpret_cast<const u32x4*>(d->emb_table);
  h.emb_scale = d->emb_scale;
  h.token_in = d->token_in;
  h.token_out = d->token_out;
  h.emb_row_out = reinterpret_cast<u32x4*>(d->emb_row_out);
  h.emb_scale_out = d->emb_scale_out;
  h.emb_deq_out = reinterpret_cast<float4*>(d->emb_deq_out);

  std::vector<BLevel> lv(d->n_levels + 1);
  size_t off = lay.regions;
  for (int i = 0; i <= d->n_levels; ++i) {
    BLevel& L = lv[i];
    const bool vocab = i == d->n_levels;
    const int64_t cols = vocab ? d->hidden : d->levels[i].cols;
    L.w = vocab ? reinterpret_cast<const unsigned char*>(d->out_table)
                : static_cast<const unsigned char*>(d->levels[i].w_packed);
    L.scale = vocab ? d->out_scale : d->levels[i].row_scale;
    L.x = vocab ? d->h : d->levels[i].x;
    L.y = vocab ? d->logits_out : d->levels[i].y;
    L.ops = reinterpret_cast<unsigned char*>(dbase + off);
    L.exps = reinterpret_cast<int*>(dbase + off + operand_digit_bytes(cols, d->batch));
    L.rows = static_cast<int>(vocab ? d->vocab : d->levels[i].rows);
    L.cols = static_cast<int>(cols);
    L.kind = vocab ? kKindInt8 : kKindTernary;
    L.pad = 0;
    off += operand_bytes(cols, d->batch);
  }
  const std::vector<BItem> items = make_items(d, grid);
  const std::vector<int2> conv = conv_table(d);

  h.n_items = static_cast<int>(items.size());
  // three quarters of the items (whole rounds) round-robin, the rest claimed
  h.n_static = static_cast<int>((3 * items.size() / 4) / grid) * grid;
  hipError_t e = hipMemsetAsync(dbase + lay.counters, 0, lay.levels - lay.counters, st);  // counters, partials, park
  if (e == hipSuccess) e = hipMemcpyAsync(dplan, &h, sizeof(BPlan), hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dbase + lay.levels, lv.data(), lv.size() * sizeof(BLevel), hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dbase + lay.items, items.data(), items.size() * sizeof(BItem), hipMemcpyHostToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dbase + lay.conv, conv.data(), conv.size() * sizeof(int2), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_plan: %s", hipGetErrorString(e));
  return PWG_OK;
}

int step_batch_launch(const pwg_step_desc* d, void* stream) {
  TRY(step_batch_check(d));
  int grid = 0;
  TRY(grid_size(&grid));
  const BPlan* dplan = plan_ptr(d);
  const int conv_blocks = static_cast<int>(conv_count(d));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(bstep_convert_kernel, dim3(conv_blocks), dim3(256), 0, st, dplan);
  if (d->batch == 4)
    hipLaunchKernelGGL(bstep_kernel<1>, dim3(grid), dim3(kThreads), bstep_lds<1>(), st, dplan);
  else if (d->batch == 8)
    hipLaunchKernelGGL(bstep_kernel<2>, dim3(grid), dim3(kThreads), bstep_lds<2>(), st, dplan);
  else
    hipLaunchKernelGGL(bstep_kernel<4>, dim3(grid), dim3(kThreads), bstep_lds<4>(), st, dplan);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "batched step launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

int step_batch_status(const pwg_step_desc* d, void* stream) {
  const BLayout lay = layout_for(d);
  const char* status = reinterpret_cast<const char*>(plan_ptr(d)) + lay.counters + 128;
  unsigned s = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&s, status, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_status: %s", hipGetErrorString(e));
  if (s == kStatusTimeout) return fail(PWG_ERR_HIP, "batched step: a workgroup's wait timed out");
  return PWG_OK;
}

}  // namespace pwg
