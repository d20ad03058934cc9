// Ordered decode step on the CDNA4 matrix cores: one persistent kernel runs
// the embedding row, every level in decoder order and the output projection
// with greedy argmax, for chained levels (each input formed from earlier
// outputs) as well as given ones.
//
// Page "The Neutrino Engine", section "A 104 microsecond floor inside a 694
// microsecond step" and Fig. 1: each projection waits for the activations of
// the one before it; most of a measured step went to kernel boundaries and
// dependency waits, and a fused kernel with software barriers replaced the
// launches with similar waits.  What this kernel does about the waits:
//  * weights do not depend on activations, so while level L is computed the
//    compute waves already have their level-L+1 tiles in flight (one
//    register buffer per level parity), and HBM streams through the barrier;
//  * every workgroup forms the whole input of a level itself, straight from
//    its sources (previous outputs, the residual stream, the embedding row
//    in the table), so one barrier per level orders everything;
//  * outputs leave through device-coherent stores (past the XCD's L2) from
//    a control wave that has no loads in flight, and the barrier is
//    hierarchical over the 8 XCDs: an atomic in each XCD's L2 counts that
//    XCD's arrivals, the last one publishes the XCD's arrival to 8
//    replicated flag lines, and waiters poll their XCD's replica.
// Arithmetic: the stream step's (operands.h): FP4 weights x six e4m3 pieces
// of x on v_mfma_scale_f32_16x16x128_f8f6f4, the int8 table x six digits of
// h on v_mfma_i32_16x16x64_i8; weights in the 16-row x 64-byte tiled
// arrangement.
//
// Work: one workgroup of 8 waves per CU (the kernel asks for more than half
// of a CU's LDS, so all workgroups are resident at once).  Workgroup w takes
// 16-row blocks [w nb / G, (w + 1) nb / G) of every level; its 7 compute
// waves split the workgroup's tiles (block-major) into contiguous ranges,
// sum piece columns at each block end into 64-byte LDS slots, and the
// control wave adds each block's slots in wave order (results do not depend
// on timing), scales, stores and arrives.  The vocabulary is split the same
// way in whole blocks per compute wave and streamed through both register
// buffers; the last workgroup to finish reduces the argmax keys.  Every wait
// is bounded (~0.5 s): a broken schedule ends with a status, never a hang.
#include <algorithm>
#include <cstddef>
#include <cstring>
#include <vector>

#include "chain_input.h"
#include "device_common.h"
#include "operands.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

using namespace dev;
using ops::v4f;
using ops::v8i;
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kCompute = kWaves - 1;   // waves 1..7; wave 0 controls
constexpr int kMaxT = 16;              // tiles per compute wave in one register buffer
constexpr int kPrefetchFirst = 8;      // tiles of the next level loaded before a level's conversion
constexpr int kMaxCols = 12288;
constexpr int kMaxBlk = 16;            // 16-row blocks of one level per workgroup
constexpr int kReplicas = 8;
constexpr unsigned long long kSpinLimit = 50000000ull;  // 0.5 s of the 100 MHz real-time counter
enum : unsigned { kBarrierL2 = 0, kBarrierFlat = 1 };
enum : unsigned { kStatusOk = 0, kStatusTimeout = 1 };
enum : unsigned { kStateStatus = 0, kStateGen = 1 };
// Level trace events (100 MHz real-time counter), per level and workgroup:
// control wave before its barrier wait, after it, with the level's sources
// in LDS; every wave past the sources' barrier, past the converted operands,
// past the products; control wave after its arrival.
enum : int {
  kEvWait = 0, kEvPassed = 1, kEvSources = 2, kEvStart = 3, kEvConverted = 4, kEvProducts = 5, kEvArrived = 6,
  kTraceEvents = 8
};

// LDS: the formed input (float), the operand region, the partial slots,
// the norm reduction and the waves' argmax keys.
constexpr size_t kStageBytes = kMaxCols * 4;
constexpr size_t kRegionBytes = 80256;  // ternary operands of 12,288 columns (int8 of 12,288: 73,920)
static_assert(kRegionBytes >= ops::ternary_region_bytes(kMaxCols) && kRegionBytes >= ops::int8_region_bytes(kMaxCols),
              "operand region");
constexpr size_t kSlotsBytes = static_cast<size_t>(kMaxBlk) * kCompute * 64;
constexpr int kMaxSlice = 256;           // formed values one workgroup writes back
constexpr int kMaxNormCols = 9984;       // RMSNORM: source and gain staged in the operand region
constexpr size_t kLevelBytes = 160;      // one level descriptor (OLevel)
// red[16], wkeys[8], hsave[kMaxSlice], two level descriptors
constexpr size_t kMiscBytes = 128 + 4 * kMaxSlice + 2 * kLevelBytes;
constexpr size_t kLds = kStageBytes + kRegionBytes + kSlotsBytes + kMiscBytes;
static_assert(kLds > 80 * 1024 && kLds <= 160 * 1024, "one resident workgroup per CU");
// formation staging in the operand region: two float rows, or an int8 row
// (rounded to KiB) and a float row
static_assert(kRegionBytes >= 4 * kMaxCols && kRegionBytes >= (kMaxCols + 1023) / 1024 * 1024 + 4 * kMaxCols &&
                  kRegionBytes >= 8 * kMaxNormCols,
              "formation staging");

// A level input formed by the previous level (its producer) from its own
// outputs: the input op kInputPrenorm takes src = gamma h, written by the
// producer, and the producer's per-workgroup sums of h^2 (`part`); the
// consumer only applies the norm's scale.
constexpr int kInputPrenorm = 100;
// What a level's control wave forms from the level's outputs for the next
// consumer (the next level, or h): nothing, RMSNORM's gamma h and h (with
// the sums of h^2), or SwiGLU's input (rows assigned as gate/up block pairs).
enum : int { kEpiNone = 0, kEpiNorm = 1, kEpiSwiglu = 2 };

struct OLevel {
  const unsigned char* w;  // tiled T2
  const float* scale;
  const float* x;          // given input, or where the formed input is written
  float* y;
  int rows, cols, T, nb;   // T = cols / 256 tiles per block, nb = 16-row blocks
  chain::DevInput in;
  int epi;                 // kEpi*
  int seg;                 // 1: block j of the first half paired with block j of the second
  int pad0, pad1;
  const float* part;       // in.op == kInputPrenorm: the producer's sums of h^2, one per workgroup
  float* e_out;            // kEpiNorm: gamma h; kEpiSwiglu: the consumer's input
  const float* e_resid;    // kEpiNorm: the residual stream added to y
  const float* e_gamma;
  float* e_resid_out;      // kEpiNorm: h (or null)
  float* e_part;           // kEpiNorm: this launch's per-workgroup sums of h^2
};

static_assert(sizeof(OLevel) == kLevelBytes && kLevelBytes % 4 == 0, "level descriptor size");

struct alignas(256) OPlan {
  unsigned n_levels, n_barriers, grid, mode;
  unsigned long long grid_magic;  // ceil(2^40 / grid): x / grid = x grid_magic >> 40 for x < 2^26
  unsigned per_xcd[8];
  unsigned xcd_mask;
  int vocab, hidden;
  const unsigned char* out_table;  // tiled int8
  const float* out_scale;
  const float* h;
  const int8_t* emb_table;
  const float* emb_scale;
  const int* token_in;
  int* token_out;
  int8_t* emb_row_out;
  float* emb_scale_out;
  float* emb_deq_out;
  float* logits_out;
  chain::DevInput h_in;
  const float* h_part;     // h_in.op == kInputPrenorm: the producer's sums of h^2
  unsigned long long* trace;  // null, or [n_levels + 1][grid][kTraceEvents] real-time stamps
};

constexpr size_t kMaxGrid = 1024;
constexpr size_t kStateBytes = 256;
constexpr size_t kCountersBytes = 8 * 128;               // one 64-bit counter per 128-byte line
constexpr size_t kFlagsBytes = kReplicas * 256 + 4096;   // 8 XCD flags per replica line (+ flat mode)

struct OLayout {
  size_t plan, state, counters, flags, partials, arrivals, levels, calib, uvec, sums, total;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

OLayout olayout(int n_levels) {
  OLayout L{};
  L.plan = 0;
  L.state = align_up(sizeof(OPlan), 256);
  L.counters = L.state + kStateBytes;
  L.flags = L.counters + kCountersBytes;
  L.partials = L.flags + kFlagsBytes;
  L.arrivals = L.partials + kMaxGrid * 8;
  L.levels = L.arrivals + 256;
  L.calib = align_up(L.levels + static_cast<size_t>(n_levels) * sizeof(OLevel), 256);
  L.uvec = align_up(L.calib + kMaxGrid * 4, 256);        // two vectors of gamma h (consumer parity)
  L.sums = L.uvec + 2 * kMaxCols * 4;                     // two arrays of per-workgroup sums of h^2
  L.total = align_up(L.sums + 2 * kMaxGrid * 4, 256);
  return L;
}

// ------------------------------------------------------------------ device
__device__ __forceinline__ unsigned ld_sc(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool reached(unsigned f, unsigned e) { return static_cast<int>(f - e) >= 0; }
__device__ __forceinline__ unsigned xcc_id() { return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7u; }
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uni_ptr(T* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(v)));
  const unsigned hi = static_cast<unsigned>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)));
  return reinterpret_cast<T*>((static_cast<unsigned long long>(hi) << 32) | lo);
}

struct Barrier {
  const OPlan* plan;
  unsigned* state;
  unsigned long long* counters;
  unsigned* flags;
  unsigned xcd;
  unsigned base;  // gen * n_barriers

  // Arrival of the workgroup at barrier j, by its control wave once its
  // device-coherent stores of the level have completed.  Everything another
  // workgroup reads from this launch is stored and loaded at device scope,
  // so no L2 write-back (or invalidation) is needed: those are cache-wide
  // operations, and every workgroup of an XCD would run them each level.
  __device__ __forceinline__ void arrive(unsigned j) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores have completed
    if ((threadIdx.x & 63u) == 0) {
      const unsigned epoch = base + j + 1;
      if (plan->mode == kBarrierL2) {
        // workgroup scope: the atomic executes in this XCD's L2, shared by its CUs
        const unsigned long long old =
            __hip_atomic_fetch_add(&counters[xcd * 16], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const unsigned long long target = static_cast<unsigned long long>(epoch) * plan->per_xcd[xcd];
        if (old + 1 == target)
          for (int r = 0; r < kReplicas; ++r) st_sc(&flags[r * 64 + xcd], epoch);
      } else {
        st_sc(&flags[kReplicas * 64 + blockIdx.x], epoch);
      }
    }
  }

  // Wait (control wave) until every workgroup has arrived at barrier j;
  // true when the wait timed out (uniform).
  __device__ __forceinline__ bool wait(unsigned j) {
    const unsigned epoch = base + j + 1;
    const unsigned lane = threadIdx.x & 63u;
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    bool late = false;
    while (true) {
      bool ok = true;
      if (plan->mode == kBarrierL2) {
        if (lane < 8 && ((plan->xcd_mask >> lane) & 1u)) ok = reached(ld_sc(&flags[xcd * 64 + lane]), epoch);
      } else {
        for (unsigned b0 = 0; b0 < plan->grid; b0 += 64)
          if (b0 + lane < plan->grid) ok = ok && reached(ld_sc(&flags[kReplicas * 64 + b0 + lane]), epoch);
      }
      if (__all(ok)) break;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinLimit) {
        late = true;
        break;
      }
    }
    if (late && lane == 0) st_sc(&state[kStateStatus], kStatusTimeout);
    return late;
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
constexpr unsigned kOff = 0x80000000u;  // past every resource: the load returns zero and moves nothing

// Tiles [s, e) (e - s <= kMaxT) of a block-major sequence of 1 KiB tiles (T
// per block, first block b0): consecutive tiles of the sequence are
// consecutive KiB of the arrangement, so this lane's 16 bytes of tile s + j
// are at KiB b0 T + s + j, byte 16 lane.  The resource ends after tile e - 1:
// the slots past it read zeros and move nothing.  Every slot's load is
// issued, so the compiler can count them.
__device__ __forceinline__ void load_tiles(u32x4 (&r)[kMaxT], const unsigned char* w, int T, int b0, int s, int e) {
  const long first = static_cast<long>(b0) * T + s;
  const __amdgpu_buffer_rsrc_t rs = buffer_over(w + first * 1024, e > s ? static_cast<unsigned>(e - s) * 1024u : 0u);
  const unsigned off = 16u * (threadIdx.x & 63u);
#pragma unroll
  for (int j = 0; j < kMaxT; ++j)
    r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024u * j, 0, 2));
}

// A workgroup's tiles of a level: tile idx of the workgroup's block-major
// sequence is tile a0 + idx of the matrix below `split`, b0 + idx - split
// from there (rows assigned as two segments; split = the first segment's
// tiles).  Tile t is KiB t of the arrangement.
struct TileMap {
  int a0, b0, split;
};
__device__ __forceinline__ unsigned tile_byte(const TileMap& m, int idx) {
  return static_cast<unsigned>(idx < m.split ? m.a0 + idx : m.b0 + (idx - m.split)) * 1024u;
}

// Tiles [s, e) (e - s <= kMaxT) of the sequence, for a prefetch whose
// registers are not read until every load of the wave has completed: only
// the tiles that exist are loaded (a load past the end still costs the wave
// an address-unit slot).  `bytes`: the matrix's size.
// Slots [J0, J1) only: a large prefetch is issued in two parts.
template <int J0, int J1>
__device__ __forceinline__ void prefetch_tiles(u32x4 (&r)[kMaxT], const unsigned char* w, unsigned bytes,
                                               const TileMap& m, int s, int e) {
  const __amdgpu_buffer_rsrc_t rs = buffer_over(w, bytes);
  const unsigned lo = 16u * (threadIdx.x & 63u);
  const int n = e - s;
#pragma unroll
  for (int j = J0; j < J1; ++j)
    if (j < n) r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, tile_byte(m, s + j) + lo, 0, 2));
}

// The same with every slot's load issued (slots past e read zeros), for
// tiles used right after: the compiler counts the loads.
__device__ __forceinline__ void load_tiles_map(u32x4 (&r)[kMaxT], const unsigned char* w, unsigned bytes,
                                               const TileMap& m, int s, int e) {
  const __amdgpu_buffer_rsrc_t rs = buffer_over(w, bytes);
  const unsigned lo = 16u * (threadIdx.x & 63u);
#pragma unroll
  for (int j = 0; j < kMaxT; ++j) {
    const unsigned off = s + j < e ? tile_byte(m, s + j) + lo : kOff;
    r[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
  }
}

// Ternary tiles [s, e) (at most kMaxT, the ones in r) of a compute wave's
// range that ends at e_all: two MFMAs per tile against the operand region;
// at a block's last tile, or the range's end, the piece columns are summed
// and the block's 16 row sums go to slot (block, wave).
__device__ __forceinline__ void ternary_tiles(const u32x4 (&r)[kMaxT], int T, int s, int e, int e_all,
                                              const unsigned char* region, int bsc_off, int asc_off, float* slots,
                                              int k, v4f& acc0, v4f& acc1) {
  const unsigned lane = threadIdx.x & 63u, n = lane & 15u, g = lane >> 4;
  const unsigned tboff = ops::ternary_b_entry(n, g);
  int blk = s / T, t = s - blk * T;
#pragma unroll
  for (int j = 0; j < kMaxT; ++j) {
    if (s + j < e) {
      v8i a0, a1;
      ops::ternary_unpack(r[j], a0, a1);
      const unsigned char* bp = region + static_cast<size_t>(2 * t) * ops::kTernaryMfmaBytes + tboff;
      const u32x4 b0l = *reinterpret_cast<const u32x4*>(bp), b0h = *reinterpret_cast<const u32x4*>(bp + 16);
      const u32x4 b1l = *reinterpret_cast<const u32x4*>(bp + ops::kTernaryMfmaBytes);
      const u32x4 b1h = *reinterpret_cast<const u32x4*>(bp + ops::kTernaryMfmaBytes + 16);
      const int sb = *reinterpret_cast<const int*>(region + bsc_off + (t >> 1) * 256 + 4 * lane);
      const int sa = *reinterpret_cast<const int*>(region + asc_off + (t >> 1) * 16 + 4 * g);
      const v8i B0 = {static_cast<int>(b0l.x), static_cast<int>(b0l.y), static_cast<int>(b0l.z), static_cast<int>(b0l.w),
                      static_cast<int>(b0h.x), static_cast<int>(b0h.y), static_cast<int>(b0h.z), static_cast<int>(b0h.w)};
      const v8i B1 = {static_cast<int>(b1l.x), static_cast<int>(b1l.y), static_cast<int>(b1l.z), static_cast<int>(b1l.w),
                      static_cast<int>(b1h.x), static_cast<int>(b1h.y), static_cast<int>(b1h.z), static_cast<int>(b1h.w)};
      if (t & 1) {  // instructions 2 t, 2 t + 1: scale bytes 2 and 3 of their quad's dwords
        acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, B0, acc0, 4, 0, 2, sa, 2, sb);
        acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, B1, acc1, 4, 0, 3, sa, 3, sb);
      } else {
        acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, B0, acc0, 4, 0, 0, sa, 0, sb);
        acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, B1, acc1, 4, 0, 1, sa, 1, sb);
      }
      // operands live past the instructions: no destination shares their registers
      asm volatile("" ::"v"(a0), "v"(a1), "v"(B0), "v"(B1));
      if (t == T - 1 || s + j == e_all - 1) {
        v4f a = acc0 + acc1;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = ops::row16_sum(n < static_cast<unsigned>(ops::kSplits) ? a[i] : 0.f);
        if (n == 0) *reinterpret_cast<v4f*>(slots + (blk * kCompute + k) * 16 + 4 * g) = a;
        acc0 = v4f{0.f, 0.f, 0.f, 0.f};
        acc1 = v4f{0.f, 0.f, 0.f, 0.f};
      }
      const int wrap = t + 1 == T;
      t = wrap ? 0 : t + 1;
      blk += wrap;
    }
  }
}

// One round of the vocabulary: tiles t0 .. t0 + kMaxT - 1 of one block (t0
// a multiple of kMaxT, so the exponent sections of 4 tiles fall at fixed
// places): one MFMA per tile, exact int32 sums per section moved into float
// with the section's power of two.
__device__ __forceinline__ void int8_round(const u32x4 (&r)[kMaxT], int t0, const unsigned char* region, int exp_off,
                                           v4i& iacc, v4f& facc) {
  const unsigned lane = threadIdx.x & 63u, n = lane & 15u, g = lane >> 4;
  const unsigned iboff = ops::int8_b_entry(n, g);
  const int cexp = n < static_cast<unsigned>(ops::kInt8Digits) ? static_cast<int>(8u * n) : -1000;
#pragma unroll
  for (int j = 0; j < kMaxT; ++j) {
    const int t = t0 + j;
    const u32x4 b = *reinterpret_cast<const u32x4*>(region + t * ops::kInt8MfmaBytes + iboff);
    const v4i A = {static_cast<int>(r[j].x), static_cast<int>(r[j].y), static_cast<int>(r[j].z), static_cast<int>(r[j].w)};
    const v4i B = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w)};
    iacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, iacc, 0, 0, 0);
    if ((j % ops::kSectionMfmas) == ops::kSectionMfmas - 1) {
      const int ex = *reinterpret_cast<const int*>(region + exp_off + (t / ops::kSectionMfmas) * 4) + cexp;
      // |iacc| <= 4 * 64 * 127 * 128 < 2^23: the conversion is exact
      facc.x += ldexpf(static_cast<float>(iacc.x), ex);
      facc.y += ldexpf(static_cast<float>(iacc.y), ex);
      facc.z += ldexpf(static_cast<float>(iacc.z), ex);
      facc.w += ldexpf(static_cast<float>(iacc.w), ex);
      iacc = v4i{0, 0, 0, 0};
    }
  }
}

// End of vocabulary block blk: the digit columns summed and scaled, the
// logits stored (through a resource that is empty when none are wanted, so
// the store is not a branch) and the lane's running (max, lowest row)
// updated.
__device__ __forceinline__ void int8_block_end(long blk, const OPlan& P, __amdgpu_buffer_rsrc_t lr, v4f& facc,
                                               float& best, unsigned& best_idx) {
  const unsigned lane = threadIdx.x & 63u, n = lane & 15u, g = lane >> 4;
  const v4f sc = ops::block_scales(P.out_scale, blk, P.vocab, g);
  const long r0 = blk * 16 + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = ops::row16_sum(n < static_cast<unsigned>(ops::kInt8Digits) ? facc[i] : 0.f) * sc[i];
    const bool mine = n == 0 && r0 + i < P.vocab;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), lr, mine ? static_cast<unsigned>(4 * (r0 + i)) : kOff, 0, 0);
    if (mine && a > best) {  // a lane's rows ascend; ties keep the lower index
      best = a;
      best_idx = static_cast<unsigned>(r0 + i);
    }
  }
  facc = v4f{0.f, 0.f, 0.f, 0.f};
}

// Any vocabulary width (T a multiple of 4): the wave's n tiles from block
// b0 on, one load per tile as it is used.  For widths that are not a
// multiple of 64 kMaxT values (never the 8B shape): no prefetch, few
// registers.
__device__ __noinline__ unsigned long long int8_tiles_any(const OPlan& P, int T, int nbv, long b0, int n,
                                                          const unsigned char* region, int exp_off,
                                                          __amdgpu_buffer_rsrc_t lr) {
  float best = -__builtin_inff();
  unsigned best_idx = 0xFFFFFFFFu;
  const unsigned lane = threadIdx.x & 63u, nl = lane & 15u, g = lane >> 4;
  const unsigned iboff = ops::int8_b_entry(nl, g);
  const int cexp = nl < static_cast<unsigned>(ops::kInt8Digits) ? static_cast<int>(8u * nl) : -1000;
  const __amdgpu_buffer_rsrc_t rs = buffer_over(P.out_table, static_cast<unsigned>(nbv) * static_cast<unsigned>(T) * 1024u);
  v4i iacc = {0, 0, 0, 0};
  v4f facc = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < n; ++i) {
    const int blk = i / T, t = i - blk * T;
    const u32x4 v = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<unsigned>(((b0 + blk) * T + t) * 1024) + 16u * lane, 0, 2));
    const u32x4 b = *reinterpret_cast<const u32x4*>(region + t * ops::kInt8MfmaBytes + iboff);
    const v4i A = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
    const v4i B = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w)};
    iacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, iacc, 0, 0, 0);
    if ((t % ops::kSectionMfmas) == ops::kSectionMfmas - 1) {
      const int ex = *reinterpret_cast<const int*>(region + exp_off + (t / ops::kSectionMfmas) * 4) + cexp;
      facc.x += ldexpf(static_cast<float>(iacc.x), ex);
      facc.y += ldexpf(static_cast<float>(iacc.y), ex);
      facc.z += ldexpf(static_cast<float>(iacc.z), ex);
      facc.w += ldexpf(static_cast<float>(iacc.w), ex);
      iacc = v4i{0, 0, 0, 0};
    }
    if (t == T - 1) int8_block_end(b0 + blk, P, lr, facc, best, best_idx);
  }
  return best_idx == 0xFFFFFFFFu ? 0ull : argmax_key(best, best_idx);  // this lane's (max, lowest row)
}

// A level descriptor held in LDS, read as wave-uniform (scalar) values.
__device__ __forceinline__ OLevel uni_level(const OLevel* p) {
  constexpr int kDw = static_cast<int>(kLevelBytes / 4);
  int w[kDw];
  __builtin_memcpy(w, p, kLevelBytes);
#pragma unroll
  for (int i = 0; i < kDw; ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
  OLevel o;
  __builtin_memcpy(&o, w, kLevelBytes);
  return o;
}

// ------------------------------------------------------------ formation
// A level's input is formed in three steps: the control wave copies its
// sources into LDS with device-coherent loads (no registers, one memory round
// trip; the sources that do not depend on the previous level are copied
// before its barrier), every thread then forms the values element by element
// (the norm's sum of squares, SwiGLU), and every thread converts the result
// into the matrix-core operand region.  The arithmetic is chain_input.h's:
// same element order, same reductions.
constexpr int kSc1 = 16;  // cache-policy bits of a device-coherent (SC1) load
typedef __attribute__((address_space(3))) void* lds_ptr;

// LDS-destination load: lane l's 16 bytes at byte `off` of rs go to lds + 16 l.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, unsigned off, unsigned char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)lds, 16, off, 0, 0, kSc1);
}

// One wave copies bytes [0, bytes) of p to LDS at dst, 1 KiB per instruction
// (lanes past the end read zeros).
__device__ __forceinline__ void lds_copy(const void* p, unsigned bytes, unsigned char* dst) {
  const __amdgpu_buffer_rsrc_t rs = buffer_over(p, bytes);
  const unsigned lane = threadIdx.x & 63u;
  for (unsigned o = 0; o < bytes; o += 1024u) lds_load16(rs, o + 16u * lane, dst + o);
}

__device__ __forceinline__ bool is_norm(int op) { return op == PWG_INPUT_RMSNORM || op == PWG_INPUT_EMBED_RMSNORM; }
__device__ __forceinline__ int embed_gamma_off(int n) { return (n + 1023) / 1024 * 1024; }

// LDS use while forming (raw = the operand region, free until conversion):
//   GIVEN          x -> stage
//   RMSNORM        resid -> stage, src -> raw[0, n), gamma -> raw[n, 2n)
//                  (n <= kMaxNormCols)
//   EMBED_RMSNORM  int8 row -> raw bytes [0, n), gamma -> raw bytes from
//                  embed_gamma_off(n) (past the row copy's last KiB)
//   ATTN1          gathered value rows -> stage
//   SWIGLU         gate -> raw[0, n), up -> stage
//   kInputPrenorm  gamma h -> stage, the producer's sums of h^2 -> sums
//                  (the slot area, free until the products)
// Control wave, any time after the previous level's operands were used: the
// sources that are constant in the launch.
__device__ __forceinline__ void issue_static_sources(const chain::DevInput& in, int n, unsigned char* raw,
                                                     const chain::EmbedSrc& e, float* red) {
  const unsigned nb = static_cast<unsigned>(n) * 4u;
  if (in.op == PWG_INPUT_RMSNORM) lds_copy(in.gamma, nb, raw + nb);
  if (in.op == PWG_INPUT_EMBED_RMSNORM) {
    const int id = *e.token_in;
    const bool valid = id >= 0 && id < e.vocab;
    if (valid) lds_copy(e.table + static_cast<long>(id) * n, static_cast<unsigned>(n), raw);
    lds_copy(in.gamma, nb, raw + embed_gamma_off(n));
    if ((threadIdx.x & 63u) == 0) {
      red[12] = valid ? e.scale[id] : 0.f;
      red[13] = valid ? 1.f : 0.f;
    }
  }
}

// Control wave, after the previous level's barrier: the sources written
// earlier in this launch.
__device__ __forceinline__ void issue_dynamic_sources(const chain::DevInput& in, int n, const float* x, float* stage,
                                                      unsigned char* raw, const float* part, int grid, float* sums) {
  const unsigned nb = static_cast<unsigned>(n) * 4u;
  unsigned char* st = reinterpret_cast<unsigned char*>(stage);
  if (in.op == PWG_INPUT_GIVEN) {
    lds_copy(x, nb, st);
  } else if (in.op == kInputPrenorm) {
    lds_copy(in.src, nb, st);
    lds_copy(part, static_cast<unsigned>(grid) * 4u, reinterpret_cast<unsigned char*>(sums));
  } else if (in.op == PWG_INPUT_RMSNORM) {
    lds_copy(in.resid, nb, st);
    if (in.src) lds_copy(in.src, nb, raw);
  } else if (in.op == PWG_INPUT_SWIGLU) {
    lds_copy(in.src, nb, raw);
    lds_copy(in.src + n, nb, st);
  } else if (in.op == PWG_INPUT_ATTN1) {
    // element i is value element i % head_dim of key/value head i / span;
    // a lane's 4 elements lie in one head (head_dim is a multiple of 4)
    const int span = in.head_dim * in.group;
    const unsigned src_bytes = static_cast<unsigned>(((n - 1) / span + 1) * in.head_dim) * 4u;
    const __amdgpu_buffer_rsrc_t rs = buffer_over(in.src, src_bytes);
    // i / head_dim and its quotient by group through multiply-high by
    // ceil(2^32 / d): exact, since i d < n^2 < 2^32 (the host bounds n)
    const unsigned hd = static_cast<unsigned>(in.head_dim), grp = static_cast<unsigned>(in.group);
    const unsigned m_hd = 0xFFFFFFFFu / hd + 1u, m_grp = grp > 1 ? 0xFFFFFFFFu / grp + 1u : 0u;
    const unsigned lane = threadIdx.x & 63u;
    for (int i0 = 0; i0 < n; i0 += 256) {
      const unsigned i = static_cast<unsigned>(i0) + 4u * lane;
      const unsigned q = __umulhi(i, m_hd), kv = grp > 1 ? __umulhi(q, m_grp) : q;
      lds_load16(rs, (kv * hd + (i - q * hd)) * 4u, st + 4 * i0);
    }
  }
}

// Element-wise formation by every thread: element i = base + kThreads u +
// tid, kU per thread per round, every LDS read of a round issued before the
// first use, indices clamped so that the reads need no branch.
constexpr int kU = 8;

__device__ __forceinline__ void form_swiglu(int n, float* stage, const float* gate) {
  const int tid = static_cast<int>(threadIdx.x);
  for (int base = 0; base < n; base += kU * kThreads) {
    float g[kU], up[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(base + u * kThreads + tid, n - 1);
      g[u] = gate[i];
      up[u] = stage[i];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // silu(g) = g * sigmoid(g), sigmoid from e^-|g| (no overflow)
      const float gv = g[u], ez = expf(-fabsf(gv));
      const float sig = gv >= 0.f ? 1.0f / (1.0f + ez) : ez / (1.0f + ez);
      const float v = gv * sig * up[u];
      const int i = base + u * kThreads + tid;
      if (i < n) stage[i] = v;
    }
  }
}

// RMSNORM (kEmbed: of the embedding row q * s, else of resid + src): gamma *
// h to stage, h of elements [s0, s1) to hsave, and the thread's sum of
// squares (elements past n add 0), in chain_input.h's order.
template <bool kEmbed, bool kSrc>
__device__ __forceinline__ float form_norm(int n, float* stage, const float* src, const int8_t* q, float s,
                                           const float* gamma, float* hsave, int s0, int s1) {
  const int tid = static_cast<int>(threadIdx.x);
  float acc = 0.f;
  for (int base = 0; base < n; base += kU * kThreads) {
    float h[kU], gm[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(base + u * kThreads + tid, n - 1);
      if (kEmbed) h[u] = static_cast<float>(q[i]) * s;
      else h[u] = kSrc ? stage[i] + src[i] : stage[i];
      gm[u] = gamma[i];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * kThreads + tid;
      const float hv = i < n ? h[u] : 0.f;
      if (i < n) stage[i] = gm[u] * hv;
      if (static_cast<unsigned>(i - s0) < static_cast<unsigned>(s1 - s0)) hsave[i - s0] = hv;
      acc = fmaf(hv, hv, acc);
    }
  }
  return acc;
}

// Every thread: the formed input (before the norm's scale) in stage, the
// waves' sums of squares in red[0, 8) (norm ops) and the residual-stream
// values of elements [s0, s1) in hsave.  EMBED_RMSNORM: red[12] holds the
// row's scale and red[13] whether the token id was valid.  True when it
// wrote LDS.
__device__ __forceinline__ bool form_elementwise(const chain::DevInput& in, int n, float* stage,
                                                 const unsigned char* raw, float* red, float* hsave, int s0, int s1) {
  const float* rawf = reinterpret_cast<const float*>(raw);
  if (in.op == PWG_INPUT_SWIGLU) {
    form_swiglu(n, stage, rawf);
    return true;
  }
  if (!is_norm(in.op)) return false;
  float acc;
  if (in.op == PWG_INPUT_EMBED_RMSNORM) {
    // an invalid id gathers a zero row (scale 0)
    const float s = red[13] != 0.f ? red[12] : 0.f;
    acc = form_norm<true, false>(n, stage, nullptr, reinterpret_cast<const int8_t*>(raw), s,
                                 reinterpret_cast<const float*>(raw + embed_gamma_off(n)), hsave, s0, s1);
  } else if (in.src) {
    acc = form_norm<false, true>(n, stage, rawf, nullptr, 0.f, rawf + n, hsave, s0, s1);
  } else {
    acc = form_norm<false, false>(n, stage, nullptr, nullptr, 0.f, rawf + n, hsave, s0, s1);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if ((threadIdx.x & 63u) == 0) red[threadIdx.x >> 6] = acc;
  return true;
}

// The norm's scale 1 / sqrt(mean + eps) from the waves' sums (fixed order),
// or 1 for the other ops.
__device__ __forceinline__ float norm_scale(const chain::DevInput& in, int n, const float* red, const float* sums,
                                            int grid) {
  if (in.op == kInputPrenorm) {
    // the producer's sums: lane l adds sums l, l + 64, ... in order, then a
    // fixed tree over the lanes; every wave of every workgroup gets the same
    float v = 0.f;
    for (int w = static_cast<int>(threadIdx.x & 63u); w < grid; w += 64) v += sums[w];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return 1.0f / sqrtf(v / static_cast<float>(n) + in.eps);
  }
  if (!is_norm(in.op)) return 1.f;
  float sum = 0.f;
  for (int w = 0; w < kWaves; ++w) sum += red[w];
  return 1.0f / sqrtf(sum / static_cast<float>(n) + in.eps);
}

// Control wave: the formed input's elements [s0, s1) to x and, for the norm
// ops, the residual-stream values to resid_out (device scope).
__device__ __forceinline__ void store_slice(const chain::DevInput& in, const float* stage, const float* hsave,
                                            float inv, float* x, int s0, int s1) {
  if (in.op == PWG_INPUT_GIVEN) return;
  const bool norm = is_norm(in.op) && in.resid_out;
  for (int i = s0 + static_cast<int>(threadIdx.x & 63u); i < s1; i += 64) {
    __hip_atomic_store(&x[i], stage[i] * inv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (norm) __hip_atomic_store(&in.resid_out[i], hsave[i - s0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Converts stage * sc (cols values) into the ternary operand region: four
// threads per 32-value block, one summation group each.
__device__ __forceinline__ void convert_ternary(const float* stage, int cols, unsigned char* region, float sc) {
  const int T = cols >> 8;
  const size_t mf = static_cast<size_t>(2 * T);
  const size_t bsc = ops::operand_bsc_off(mf), asc = ops::operand_asc_off(mf);
  for (int t0 = 0; t0 < T * 32; t0 += kThreads) {  // uniform trip count (shuffles below)
    const int tid = t0 + static_cast<int>(threadIdx.x);
    const int beta = tid >> 2, h = (tid >> 1) & 1, G = tid & 1;
    const bool in = tid < T * 32;
    float xs[16];
    float amax = 0.f;
    const float4* src = reinterpret_cast<const float4*>(stage + 32 * (in ? beta : 0) + 16 * h);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = src[q];
      xs[4 * q + 0] = in ? v.x * sc : 0.f;
      xs[4 * q + 1] = in ? v.y * sc : 0.f;
      xs[4 * q + 2] = in ? v.z * sc : 0.f;
      xs[4 * q + 3] = in ? v.w * sc : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xs[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));  // the other half of the block
    if (in) ops::write_ternary_quarter(region, bsc, asc, beta, h, G, xs, ops::block_exponent(amax));
  }
}

// Converts stage * sc (hidden values) into the int8 operand region: one wave
// per 256-value section, lane t owning values 4t .. 4t + 3.
__device__ __forceinline__ void convert_int8(const float* stage, int hidden, unsigned char* region, float sc) {
  const unsigned lane = threadIdx.x & 63u;
  const int exp_off = static_cast<int>(ops::int8_exp_off(hidden));
  for (int sec = static_cast<int>(threadIdx.x >> 6); sec < hidden / 256; sec += kWaves) {
    const float4 v4 = *reinterpret_cast<const float4*>(stage + 256 * sec + 4 * lane);
    const float hv[4] = {v4.x * sc, v4.y * sc, v4.z * sc, v4.w * sc};
    float amax = fmaxf(fmaxf(fabsf(hv[0]), fabsf(hv[1])), fmaxf(fabsf(hv[2]), fabsf(hv[3])));
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    const int e = ops::block_exponent(amax);
    unsigned dw[ops::kInt8Digits];
    ops::int8_digits4(hv, e, dw);
    const int m = 4 * sec + static_cast<int>(lane >> 4), g = static_cast<int>((lane & 15u) >> 2),
              j0 = 4 * static_cast<int>(lane & 3u);
#pragma unroll
    for (int d = 0; d < ops::kInt8Digits; ++d)
      *reinterpret_cast<unsigned*>(region + m * ops::kInt8MfmaBytes + ops::int8_b_entry(d, g) + j0) = dw[d];
    if (lane == 0) *reinterpret_cast<int*>(region + exp_off + 4 * sec) = e - ops::kInt8FixedBits;
  }
}

// Embedding row of the step's token (control wave of workgroup 0).
__device__ __forceinline__ void embed_outputs(const OPlan& P) {
  const unsigned lane = threadIdx.x & 63u;
  const int id = *P.token_in;
  const bool ok = id >= 0 && id < P.vocab;
  const float s = ok ? P.emb_scale[id] : __builtin_nanf("");
  if (lane == 0) *P.emb_scale_out = s;
  for (int i = static_cast<int>(lane); i < P.hidden; i += 64) {
    const int8_t q = ok ? P.emb_table[static_cast<long>(id) * P.hidden + i] : static_cast<int8_t>(0);
    P.emb_row_out[i] = q;
    if (P.emb_deq_out) P.emb_deq_out[i] = ok ? static_cast<float>(q) * s : 0.f;
  }
}

// Tiles [s, e) of compute wave k of a workgroup with nblk blocks of T tiles.
__device__ __forceinline__ void wave_range(int nblk, int T, int k, int& s, int& e) {
  const int n = nblk * T;
  s = k * n / kCompute;
  e = (k + 1) * n / kCompute;
}

__global__ __launch_bounds__(kThreads, 1) void ordered_step_kernel(const OPlan* __restrict__ plan,
                                                                   const OLevel* __restrict__ levels, unsigned* state,
                                                                   unsigned long long* counters, unsigned* flags,
                                                                   unsigned long long* partials, unsigned* arrivals) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* stage = reinterpret_cast<float*>(smem);
  unsigned char* region = smem + kStageBytes;
  float* slots = reinterpret_cast<float*>(smem + kStageBytes + kRegionBytes);
  float* red = reinterpret_cast<float*>(smem + kStageBytes + kRegionBytes + kSlotsBytes);
  unsigned long long* wkeys = reinterpret_cast<unsigned long long*>(red + 16);
  float* hsave = red + 32;
  OLevel* ring = reinterpret_cast<OLevel*>(hsave + kMaxSlice);  // descriptors of levels li & 1

  const OPlan& P = *plan;
  const unsigned lane = threadIdx.x & 63u;
  const int wave = uni(static_cast<int>(threadIdx.x >> 6));
  const int k = wave - 1;  // compute-wave index (wave 0: -1)
  const unsigned G = P.grid, wg = blockIdx.x;
  const unsigned nl = P.n_levels;
  Barrier bar{plan, state, counters, flags, xcc_id(), 0};
  bar.base = ld_sc(&state[kStateGen]) * P.n_barriers;
  const chain::EmbedSrc emb{P.emb_table, P.emb_scale, P.token_in, static_cast<long>(P.vocab)};
  constexpr int kDw = static_cast<int>(kLevelBytes / 4);
  unsigned long long* const trace = P.trace;
  auto stamp = [&](unsigned li, int ev) {
    if (trace && threadIdx.x == 0)
      trace[(static_cast<size_t>(li) * G + wg) * kTraceEvents + ev] = __builtin_amdgcn_s_memrealtime();
  };

  // [b0, b1) of a range of n units owned by this workgroup
  auto wg_split = [&](int n, int& b0, int& b1) {
    const unsigned long long m = P.grid_magic;
    b0 = static_cast<int>((static_cast<unsigned long long>(wg * static_cast<unsigned>(n)) * m) >> 40);
    b1 = static_cast<int>((static_cast<unsigned long long>((wg + 1) * static_cast<unsigned>(n)) * m) >> 40);
  };
  // The workgroup's 16-row blocks of a level: local block lb is block
  // a0 + lb below na, c0 + lb - na from there (seg: block j of the first half
  // paired with block j of the second).
  struct WgRows {
    int a0, na, c0, nblk;
    __device__ int block(int lb) const { return lb < na ? a0 + lb : c0 + (lb - na); }
  };
  auto wg_rows = [&](const OLevel& L) -> WgRows {
    int b0, b1;
    if (L.seg) {
      const int half = L.nb / 2;
      wg_split(half, b0, b1);
      return WgRows{b0, b1 - b0, half + b0, 2 * (b1 - b0)};
    }
    wg_split(L.nb, b0, b1);
    return WgRows{b0, b1 - b0, 0, b1 - b0};
  };
  auto tile_map = [&](const WgRows& R, int T) { return TileMap{R.a0 * T, R.c0 * T, R.na * T}; };
  // elements of a formed input of n values this workgroup writes back
  auto wg_slice = [&](int n, int& s0, int& s1) { wg_split(n, s0, s1); };
  // tiles of level li (descriptor L; li == nl: the vocabulary's first kMaxT;
  // past it: none) for this compute wave; every load of the wave completes
  // before they are read
  // A prefetch of level li's tiles (li == nl: the output table's first
  // round) for this compute wave: where the tiles are, then the loads.
  struct Pref {
    const unsigned char* w;
    unsigned bytes;
    TileMap m;
    int s, e;
  };
  auto pref_plan = [&](unsigned li, const OLevel& L) -> Pref {
    int s = 0, e = 0;
    unsigned bytes = 0;
    const unsigned char* w = P.out_table;
    TileMap m{0, 0, 0};
    if (li < nl) {
      const WgRows R = wg_rows(L);
      w = L.w;
      bytes = static_cast<unsigned>(L.nb) * static_cast<unsigned>(L.T) * 1024u;
      m = tile_map(R, L.T);
      wave_range(R.nblk, L.T, k, s, e);
    } else if (li == nl) {
      const int T = P.hidden / 64, nbv = (P.vocab + 15) / 16;
      int b0, b1;
      wg_split(nbv, b0, b1);
      const int w0 = b0 + k * (b1 - b0) / kCompute, w1 = b0 + (k + 1) * (b1 - b0) / kCompute;
      bytes = static_cast<unsigned>(nbv) * static_cast<unsigned>(T) * 1024u;
      m = TileMap{w0 * T, 0, 1 << 30};
      e = (w1 - w0) * T;
    }
    return Pref{w, bytes, m, s, e};
  };
  auto pref_issue = [&](u32x4 (&r)[kMaxT], const Pref& p, int part) {
    const int e = p.e < p.s + kMaxT ? p.e : p.s + kMaxT;
    if (part == 0) prefetch_tiles<0, kPrefetchFirst>(r, p.w, p.bytes, p.m, p.s, e);
    if (part != 0) prefetch_tiles<kPrefetchFirst, kMaxT>(r, p.w, p.bytes, p.m, p.s, e);
  };
  // control wave: per row lane + 64 j of the workgroup's rows of a level, its
  // scale and, for a norm epilogue, the gain and the residual stream there
  // (`dynamic`: the residual stream only, after the previous level's barrier,
  // since the previous level may have written it)
  float rsc[4] = {0.f, 0.f, 0.f, 0.f}, rres[4] = {0.f, 0.f, 0.f, 0.f}, rgam[4] = {0.f, 0.f, 0.f, 0.f};
  auto load_rows = [&](const OLevel& L, bool dynamic) {
    const WgRows R = wg_rows(L);
    const unsigned nb = static_cast<unsigned>(L.rows) * 4u;
    const __amdgpu_buffer_rsrc_t rs = buffer_over(L.scale, nb);
    const __amdgpu_buffer_rsrc_t rr_res = buffer_over(L.e_resid, L.epi == kEpiNorm ? nb : 0u);
    const __amdgpu_buffer_rsrc_t rr_gam = buffer_over(L.e_gamma, L.epi == kEpiNorm ? nb : 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = static_cast<int>(lane) + 64 * j, row = R.block(rr >> 4) * 16 + (rr & 15);
      const unsigned off = rr < R.nblk * 16 && row < L.rows ? static_cast<unsigned>(row) * 4u : kOff;
      if (dynamic) {
        // written earlier in this launch: device scope
        rres[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr_res, off, 0, kSc1));
      } else {
        rsc[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
        rgam[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr_gam, off, 0, 0));
      }
    }
  };

  u32x4 ra[kMaxT], rb[kMaxT];
  if (wave == 0) {
    if (wg == 0) embed_outputs(P);
    if (nl > 0 && lane < kDw)  // level 0's descriptor
      reinterpret_cast<int*>(ring)[lane] = reinterpret_cast<const int*>(levels)[lane];
  } else {
    const Pref p0 = pref_plan(0, levels[0]);
    pref_issue(ra, p0, 0);
    pref_issue(ra, p0, 1);
  }

  // The sources of level li's input (li == nl: h) in LDS, after the previous
  // level's barrier, and level li + 1's descriptor in the ring; true
  // (uniform) when the wait timed out.
  auto gather = [&](unsigned li) -> bool {
    const bool vocab = li == nl;
    if (wave == 0) {
      const OLevel L = vocab ? OLevel{} : uni_level(&ring[li & 1]);
      const chain::DevInput in = vocab ? P.h_in : L.in;
      const int n = vocab ? P.hidden : L.cols;
      int next_dw = 0;
      if (li + 1 < nl && lane < kDw) next_dw = reinterpret_cast<const int*>(levels + li + 1)[lane];
      if (!vocab) load_rows(L, false);
      issue_static_sources(in, n, region, emb, red);
      stamp(li, kEvWait);
      bool late = false;
      if (li > 0) late = bar.wait(li - 1);
      stamp(li, kEvPassed);
      if (!late) {
        issue_dynamic_sources(in, n, vocab ? P.h : L.x, stage, region, vocab ? P.h_part : L.part,
                              static_cast<int>(G), slots);
        if (!vocab && L.epi == kEpiNorm) load_rows(L, true);
      }
      if (li + 1 < nl && lane < kDw) reinterpret_cast<int*>(&ring[(li + 1) & 1])[lane] = next_dw;
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the sources are in LDS
      stamp(li, kEvSources);
      if (lane == 0) red[15] = late ? 1.f : 0.f;
    }
    __syncthreads();
    stamp(li, kEvStart);
    return red[15] != 0.f;
  };

  // One level: its tiles are in `cur` (loaded during the previous level's
  // conversion and products); the next level's go into `nxt` as soon as this
  // level's sources are in LDS, so the weight stream overlaps the conversion
  // and the products and stays off the paths of the level's inputs and
  // outputs.
  auto level = [&](unsigned li, u32x4(&cur)[kMaxT], u32x4(&nxt)[kMaxT]) -> bool {
    if (gather(li)) return true;
    const OLevel L = uni_level(&ring[li & 1]);
    const int T = L.T, cols = L.cols, rows = L.rows;
    const WgRows R = wg_rows(L);
    int s0, s1;
    wg_slice(cols, s0, s1);
    // where the next level's tiles are (worked out while this level's last
    // loads land)
    const OLevel Ln = uni_level(&ring[(li + 1) & 1]);  // not read past the last level
    const Pref pn = pref_plan(li + 1, Ln);
    // every earlier load (this level's tiles) has completed; saying so on
    // every path lets the compiler count the prefetch below instead of
    // draining it before the products
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    // the first kPrefetchFirst tiles of the next level now; the rest after
    // this level's products, so that a large next level holds up neither the
    // conversion nor the products alone
    if (wave > 0) pref_issue(nxt, pn, 0);
    if (form_elementwise(L.in, cols, stage, region, red, hsave, s0, s1)) __syncthreads();
    const float inv = norm_scale(L.in, cols, red, slots, static_cast<int>(G));
    convert_ternary(stage, cols, region, inv);
    __syncthreads();  // the operand region is complete
    stamp(li, kEvConverted);
    if (wave > 0) {
      int s, e;
      wave_range(R.nblk, T, k, s, e);
      const size_t mf = static_cast<size_t>(2 * T);
      const int bsc = static_cast<int>(ops::operand_bsc_off(mf)), asc = static_cast<int>(ops::operand_asc_off(mf));
      v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      // rounds past the first (levels wider than 7 x kMaxT tiles per
      // workgroup) load on demand
      ternary_tiles(cur, T, s, e < s + kMaxT ? e : s + kMaxT, e, region, bsc, asc, slots, k, acc0, acc1);
      for (int r0 = s + kMaxT; r0 < e; r0 += kMaxT) {
        load_tiles_map(cur, L.w, static_cast<unsigned>(L.nb) * static_cast<unsigned>(T) * 1024u, tile_map(R, T), r0,
                       e < r0 + kMaxT ? e : r0 + kMaxT);
        ternary_tiles(cur, T, r0, e < r0 + kMaxT ? e : r0 + kMaxT, e, region, bsc, asc, slots, k, acc0, acc1);
      }
    } else {
      store_slice(L.in, stage, hsave, inv, const_cast<float*>(L.x), s0, s1);
    }
    __syncthreads();  // every slot of the level is written
    stamp(li, kEvProducts);
    // the rest of the next level's tiles, while the control wave publishes
    if (wave > 0) pref_issue(nxt, pn, 1);
    if (wave == 0) {
      // rows of the workgroup: block bl's sum over the compute waves that
      // touched it, in wave order; then what the rows form for the next
      // consumer
      const int nrow = R.nblk * 16;
      float hh = 0.f;  // kEpiNorm: this lane's sum of h^2
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = static_cast<int>(lane) + 64 * j;
        if (rr < nrow) {
          const int bl = rr >> 4, i = rr & 15;
          float v = 0.f;
          for (int kk = 0; kk < kCompute; ++kk) {
            int s, e;
            wave_range(R.nblk, T, kk, s, e);
            if (s < e && s < (bl + 1) * T && e > bl * T) v += slots[(bl * kCompute + kk) * 16 + i];
          }
          const int row = R.block(bl) * 16 + i;
          const float y = v * rsc[j];
          if (row < rows) {
            __hip_atomic_store(&L.y[row], y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (L.epi == kEpiNorm) {
              // chain_input.h's h = resid + src, then gamma h
              const float h = rres[j] + y;
              if (L.e_resid_out) __hip_atomic_store(&L.e_resid_out[row], h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              __hip_atomic_store(&L.e_out[row], rgam[j] * h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              hh = fmaf(h, h, hh);
            }
          }
          if (L.epi == kEpiSwiglu) hsave[rr] = y;
        }
      }
      if (L.epi == kEpiNorm) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) hh += __shfl_xor(hh, o, kWave);
        if (lane == 0) __hip_atomic_store(&L.e_part[wg], hh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else if (L.epi == kEpiSwiglu) {
        // gate row g of local block bl < na pairs with up row g + rows / 2 of
        // local block bl + na; SwiGLU as chain_input.h forms it
        const int ng = R.na * 16;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int rr = static_cast<int>(lane) + 64 * j;
          if (rr < ng) {
            const float gv = hsave[rr], up = hsave[rr + ng], ez = expf(-fabsf(gv));
            const float sig = gv >= 0.f ? 1.0f / (1.0f + ez) : ez / (1.0f + ez);
            __hip_atomic_store(&L.e_out[(R.a0 + (rr >> 4)) * 16 + (rr & 15)], gv * sig * up, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      bar.arrive(li);
      stamp(li, kEvArrived);
    }
    return false;
  };

  // levels in pairs, so that each buffer has one static role per call
  for (unsigned li = 0; li < nl; li += 2) {
    if (level(li, ra, rb)) return;
    if (li + 1 < nl && level(li + 1, rb, ra)) return;
  }
  const bool vocab_in_a = (nl & 1u) == 0;  // the vocabulary's first round: prefetched into ra for even nl

  // Output projection: h formed after the last level, then every compute
  // wave streams its whole vocabulary blocks through both register buffers.
  if (gather(nl)) return;
  {
    int s0, s1;
    wg_slice(P.hidden, s0, s1);
    if (form_elementwise(P.h_in, P.hidden, stage, region, red, hsave, s0, s1)) __syncthreads();
    const float inv = norm_scale(P.h_in, P.hidden, red, slots, static_cast<int>(G));
    convert_int8(stage, P.hidden, region, inv);
    __syncthreads();
    stamp(nl, kEvConverted);
    if (wave == 0) store_slice(P.h_in, stage, hsave, inv, const_cast<float*>(P.h), s0, s1);
  }
  float best = -__builtin_inff();
  unsigned best_idx = 0xFFFFFFFFu;
  unsigned long long key_any = 0ull;  // the any-width path's key
  if (wave > 0) {
    const int T = P.hidden / 64, nbv = (P.vocab + 15) / 16;
    int b0, b1;
    wg_split(nbv, b0, b1);
    const int w0 = b0 + k * (b1 - b0) / kCompute, w1 = b0 + (k + 1) * (b1 - b0) / kCompute;
    const int n = (w1 - w0) * T;
    const int exp_off = static_cast<int>(ops::int8_exp_off(P.hidden));
    v4i iacc = {0, 0, 0, 0};
    v4f facc = {0.f, 0.f, 0.f, 0.f};
    const __amdgpu_buffer_rsrc_t lr =
        buffer_over(P.logits_out, P.logits_out ? static_cast<unsigned>(P.vocab) * 4u : 0u);
    const int rpb = T / kMaxT;  // rounds per block (T is a multiple of kMaxT)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first round has arrived
    auto stream = [&](u32x4(&a)[kMaxT], u32x4(&b)[kMaxT]) {
      if (T % kMaxT != 0) {  // any width: tiles loaded one at a time (the prefetched round is not used)
        key_any = int8_tiles_any(P, T, nbv, w0, n, region, exp_off, lr);
        return;
      }
      // a holds round 0; rounds alternate between the buffers
      for (int r0 = 0; r0 < n; r0 += 2 * kMaxT) {
        load_tiles(b, P.out_table, T, w0, r0 + kMaxT, n < r0 + 2 * kMaxT ? n : r0 + 2 * kMaxT);
        int8_round(a, r0 % T, region, exp_off, iacc, facc);
        if ((r0 / kMaxT) % rpb == rpb - 1) int8_block_end(w0 + r0 / T, P, lr, facc, best, best_idx);
        if (r0 + kMaxT >= n) break;
        load_tiles(a, P.out_table, T, w0, r0 + 2 * kMaxT, n < r0 + 3 * kMaxT ? n : r0 + 3 * kMaxT);
        int8_round(b, (r0 + kMaxT) % T, region, exp_off, iacc, facc);
        if ((r0 / kMaxT + 1) % rpb == rpb - 1) int8_block_end(w0 + (r0 + kMaxT) / T, P, lr, facc, best, best_idx);
      }
    };
    if (vocab_in_a) stream(ra, rb);
    else stream(rb, ra);
  }

  // Workgroup (max, lowest index), then the last workgroup to arrive reduces
  // every workgroup's key into the token and starts the next step's epoch.
  unsigned long long key = best_idx == 0xFFFFFFFFu ? 0ull : argmax_key(best, best_idx);
  key = key_any > key ? key_any : key;
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(key, off, kWave);
    key = o > key ? o : key;
  }
  if (lane == 0) wkeys[wave] = key;
  __syncthreads();
  stamp(nl, kEvProducts);
  if (wave == 0) {
    unsigned last = 0;
    if (lane == 0) {
      unsigned long long m = 0ull;
      for (int i = 0; i < kWaves; ++i) m = wkeys[i] > m ? wkeys[i] : m;
      __hip_atomic_store(&partials[wg], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned prev = __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      last = prev == G - 1u ? 1u : 0u;
    }
    if (uni(static_cast<int>(last))) {
      unsigned long long m = 0ull;
      for (unsigned b = lane; b < G; b += 64) {
        const unsigned long long o = __hip_atomic_load(&partials[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        m = o > m ? o : m;
      }
      for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(m, off, kWave);
        m = o > m ? o : m;
      }
      if (lane == 0) {
        *P.token_out = static_cast<int>(argmax_key_index(m));
        __hip_atomic_store(arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        st_sc(&state[kStateGen], ld_sc(&state[kStateGen]) + 1u);
      }
    }
  }
}

__global__ void xcc_census_kernel(unsigned* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

int ordered_grid() {
  int dev = 0, cus = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&ordered_step_kernel), kThreads,
                                                   kLds) != hipSuccess || n != 1)
    return -1;
  return cus;
}

}  // namespace

// ------------------------------------------------------------------- host
size_t step_ordered_workspace(const pwg_step_desc* d) { return olayout(d->n_levels).total; }

namespace {
// The control wave copies a level's sources into LDS 16 bytes per lane.
int check_sources(const pwg_input& in, int64_t n, const float* x, const char* fn, const char* what) {
  const void* ptrs[4] = {in.op == PWG_INPUT_GIVEN ? static_cast<const void*>(x) : nullptr, in.src, in.resid, in.gamma};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(PWG_ERR_ALIGN, "%s: %s: sources must be 16-byte aligned", fn, what);
  if (in.op == PWG_INPUT_ATTN1 && in.head_dim % 4 != 0)
    return fail(PWG_ERR_UNSUPPORTED, "%s: %s: head_dim must be a multiple of 4 on the persistent schedule", fn, what);
  if (in.op == PWG_INPUT_RMSNORM && n > kMaxNormCols)
    return fail(PWG_ERR_UNSUPPORTED, "%s: %s: RMSNORM over more than %d values is not on the persistent schedule", fn,
                what, kMaxNormCols);
  return PWG_OK;
}
}  // namespace

int step_ordered_check(const pwg_step_desc* d, const char* fn) {
  if (d->weight_layout != PWG_LAYOUT_TILED)
    return fail(PWG_ERR_UNSUPPORTED, "%s: the persistent schedule reads tiled weights (PWG_LAYOUT_TILED)", fn);
  if (d->batch > 1) return fail(PWG_ERR_UNSUPPORTED, "%s: the persistent schedule runs one vector", fn);
  if (d->hidden < 256 || d->hidden % 256 != 0 || d->hidden > kMaxCols)
    return fail(PWG_ERR_UNSUPPORTED, "%s: hidden must be a multiple of 256 in [256, %d] on the persistent schedule", fn,
                kMaxCols);
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    if (L.cols % 256 != 0 || L.cols > kMaxCols)
      return fail(PWG_ERR_UNSUPPORTED, "%s: level %d: cols must be a multiple of 256 in [256, %d] on the persistent "
                  "schedule", fn, i, kMaxCols);
    TRY(check_sources(L.in, L.cols, L.x, fn, "level input"));
  }
  TRY(check_sources(d->h_in, d->hidden, d->h, fn, "h"));
  return PWG_OK;
}

namespace {
OLayout layout_of(const pwg_step_desc* d) { return olayout(d->n_levels); }
unsigned char* ws_base(const pwg_step_desc* d) { return static_cast<unsigned char*>(d->workspace); }
}  // namespace

int step_ordered_plan(const pwg_step_desc* d, void* stream) {
  const char* fn = "pwg_step_plan";
  TRY(step_ordered_check(d, fn));
  const int G = ordered_grid();
  if (G < 1 || G > static_cast<int>(kMaxGrid))
    return fail(PWG_ERR_UNSUPPORTED, "%s: the persistent kernel needs one resident workgroup on every CU", fn);
  if ((kMaxCols + G - 1) / G > kMaxSlice)
    return fail(PWG_ERR_UNSUPPORTED, "%s: %d CUs are too few for the persistent kernel", fn, G);
  const OLayout lay = layout_of(d);
  std::vector<OLevel> lv(static_cast<size_t>(d->n_levels));
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    OLevel& o = lv[i];
    o.w = static_cast<const unsigned char*>(L.w_packed);
    o.scale = L.row_scale;
    o.x = L.x;
    o.y = L.y;
    o.rows = static_cast<int>(L.rows);
    o.cols = static_cast<int>(L.cols);
    o.T = static_cast<int>(L.cols / 256);
    o.nb = static_cast<int>((L.rows + 15) / 16);
    o.in = chain::from_abi(L.in);
    if ((o.nb + G - 1) / G > kMaxBlk)
      return fail(PWG_ERR_UNSUPPORTED, "%s: level %d has more than %d rows per CU", fn, i, kMaxBlk * 16);
    if (static_cast<long>(o.nb) * o.T * 1024 >= (1L << 32))
      return fail(PWG_ERR_UNSUPPORTED, "%s: level %d is larger than 4 GiB", fn, i);
  }
  if ((d->vocab + 15) / 16 * (d->hidden / 64) * 1024 >= (int64_t{1} << 32))
    return fail(PWG_ERR_UNSUPPORTED, "%s: the output table is larger than 4 GiB", fn);
  if (d->vocab > (int64_t{1} << 20))  // 16-row blocks split over the grid by multiply-shift
    return fail(PWG_ERR_UNSUPPORTED, "%s: vocab above 2^20 on the persistent schedule", fn);
  OPlan h;
  std::memset(&h, 0, sizeof h);
  h.n_levels = static_cast<unsigned>(d->n_levels);
  h.n_barriers = static_cast<unsigned>(d->n_levels > 0 ? d->n_levels : 1);
  h.grid = static_cast<unsigned>(G);
  // x / G for x < 2^26: x ceil(2^40 / G) / 2^40 exceeds x / G by less than
  // 2^-14 < 1 / G, which cannot carry past the next integer
  h.grid_magic = ((1ull << 40) + static_cast<unsigned long long>(G) - 1) / static_cast<unsigned long long>(G);
  h.vocab = static_cast<int>(d->vocab);
  h.hidden = static_cast<int>(d->hidden);
  h.out_table = static_cast<const unsigned char*>(static_cast<const void*>(d->out_table));
  h.out_scale = d->out_scale;
  h.h = d->h;
  h.emb_table = d->emb_table;
  h.emb_scale = d->emb_scale;
  h.token_in = d->token_in;
  h.token_out = d->token_out;
  h.emb_row_out = d->emb_row_out;
  h.emb_scale_out = d->emb_scale_out;
  h.emb_deq_out = d->emb_deq_out;
  h.logits_out = d->logits_out;
  h.h_in = chain::from_abi(d->h_in);

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  unsigned char* base = ws_base(d);

  // Producer epilogues: where a consumer (the next level, or h) forms its
  // input from the previous level's output alone, that level's control wave
  // forms it as it writes the output (RMSNORM: h, gamma h and the sums of
  // h^2, the consumer applying the scale; SwiGLU: the input itself, with the
  // gate and up rows of one index in one workgroup).  Buffers alternate with
  // the consumer's parity: a consumer reads them before its barrier, the
  // next writer of the same buffer runs after it.
  float* uvec = reinterpret_cast<float*>(base + lay.uvec);
  float* sums = reinterpret_cast<float*>(base + lay.sums);
  auto link = [&](OLevel& p, chain::DevInput& in, int n, float* cons_x, const float** cons_part, int parity,
                  bool level_consumer) {
    if (in.op == PWG_INPUT_RMSNORM && in.src == p.y && n == p.rows && n <= kMaxNormCols) {
      p.epi = kEpiNorm;
      p.e_out = uvec + static_cast<size_t>(parity) * kMaxCols;
      p.e_resid = in.resid;
      p.e_gamma = in.gamma;
      p.e_resid_out = in.resid_out;
      p.e_part = sums + static_cast<size_t>(parity) * kMaxGrid;
      in.op = kInputPrenorm;
      in.src = p.e_out;
      in.resid = nullptr;
      in.gamma = nullptr;
      in.resid_out = nullptr;
      *cons_part = p.e_part;
    } else if (level_consumer && in.op == PWG_INPUT_SWIGLU && in.src == p.y && p.rows == 2 * n && n % 16 == 0 &&
               (p.nb / 2 + G - 1) / G * 2 <= kMaxBlk) {
      p.epi = kEpiSwiglu;
      p.seg = 1;
      p.e_out = cons_x;
      in.op = PWG_INPUT_GIVEN;
    }
  };
  for (int i = 0; i + 1 < d->n_levels; ++i)
    link(lv[i], lv[i + 1].in, lv[i + 1].cols, const_cast<float*>(lv[i + 1].x), &lv[i + 1].part, (i + 1) & 1, true);
  if (d->n_levels > 0)
    link(lv[d->n_levels - 1], h.h_in, h.hidden, const_cast<float*>(h.h), &h.h_part, d->n_levels & 1, false);
  // XCD census: one workgroup per CU (the step kernel's LDS request); the
  // barrier counts per XCD when every XCD holds the same number of them
  hipLaunchKernelGGL(xcc_census_kernel, dim3(G), dim3(kThreads), kLds, st, reinterpret_cast<unsigned*>(base + lay.calib));
  std::vector<unsigned> xcc(static_cast<size_t>(G));
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(xcc.data(), base + lay.calib, static_cast<size_t>(G) * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "%s: XCD census: %s", fn, hipGetErrorString(e));
  unsigned census[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int b = 0; b < G; ++b) census[xcc[b] & 7u] += 1;
  bool uniform = true;
  for (int x = 1; x < 8; ++x) uniform = uniform && (census[x] == census[0] || census[x] == 0);
  h.mode = uniform ? kBarrierL2 : kBarrierFlat;
  for (int x = 0; x < 8; ++x) {
    h.per_xcd[x] = census[x];
    if (census[x]) h.xcd_mask |= 1u << x;
  }
  e = hipMemcpyAsync(base + lay.plan, &h, sizeof h, hipMemcpyHostToDevice, st);
  if (e == hipSuccess && !lv.empty())
    e = hipMemcpyAsync(base + lay.levels, lv.data(), lv.size() * sizeof(OLevel), hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipMemsetAsync(base + lay.state, 0, lay.levels - lay.state, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return PWG_OK;
}

int step_ordered_launch(const pwg_step_desc* d, void* stream) {
  const OLayout lay = layout_of(d);
  static int grid = -1;
  if (grid < 0) grid = ordered_grid();
  if (grid < 1) return fail(PWG_ERR_UNSUPPORTED, "persistent step: no resident grid");
  unsigned char* base = ws_base(d);
  hipLaunchKernelGGL(ordered_step_kernel, dim3(grid), dim3(kThreads), kLds, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const OPlan*>(base + lay.plan), reinterpret_cast<const OLevel*>(base + lay.levels),
                     reinterpret_cast<unsigned*>(base + lay.state), reinterpret_cast<unsigned long long*>(base + lay.counters),
                     reinterpret_cast<unsigned*>(base + lay.flags), reinterpret_cast<unsigned long long*>(base + lay.partials),
                     reinterpret_cast<unsigned*>(base + lay.arrivals));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "persistent step launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

size_t step_ordered_trace_bytes(const pwg_step_desc* d) {
  const int G = ordered_grid();
  if (G < 1 || d->n_levels < 0) return 0;
  return static_cast<size_t>(d->n_levels + 1) * static_cast<size_t>(G) * kTraceEvents * 8;
}

int step_ordered_set_trace(const pwg_step_desc* d, void* trace, void* stream) {
  const OLayout lay = layout_of(d);
  unsigned long long* t = static_cast<unsigned long long*>(trace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(ws_base(d) + lay.plan + offsetof(OPlan, trace), &t, sizeof t, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_set_trace: %s", hipGetErrorString(e));
  return PWG_OK;
}

int step_ordered_status(const pwg_step_desc* d, void* stream) {
  const OLayout lay = layout_of(d);
  unsigned s = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&s, ws_base(d) + lay.state + 4 * kStateStatus, 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "pwg_step_status: %s", hipGetErrorString(e));
  if (s == kStatusTimeout) return fail(PWG_ERR_HIP, "persistent step: a level barrier timed out (re-plan the step)");
  return PWG_OK;
}

}  // namespace pwg
