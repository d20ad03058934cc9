// Data layout of the stream schedule (matrix-core step): the converted
// activation operands of each level in the workspace, and the plan tables.
#pragma once
#include <cstddef>
#include <cstdint>

#include "device_common.h"
#include "operands.h"

namespace pwg {
namespace stream {

using ops::kTernaryMfmaBytes;
using ops::kInt8MfmaBytes;
using ops::kSectionMfmas;
constexpr int kMaxStreamCols = 12288;             // two operand buffers of this width fit in LDS
constexpr size_t kMaxLds = 160 * 1024;
constexpr int kStreamWaves = 8;                   // waves per workgroup (two control waves)
constexpr size_t kFlagBytes = 256;                // ready word, claim counters, done words, per-wave argmax keys
static_assert(kStreamWaves <= 16, "flag words");
constexpr int kMaxWgSegs = 32;                    // static segments (levels touched) per workgroup
constexpr int kMaxPoolSegs = 16;                  // levels of the shared pool (the vocabulary first)
constexpr double kPoolTailShare = 0.04;           // small-block ternary levels that end the pool: this share of the bytes
constexpr int kRing = 64;                         // pool claims queued per workgroup (ring entries)
constexpr int kPoolAhead = 2;                     // claims a workgroup keeps ready beyond its pops
constexpr int kClaimBatch = 8;                    // pool blocks per global atomic ...
constexpr int kLateClaims = 8;                   // ... until fewer than this many per workgroup remain,
constexpr int kLateBatch = 1;                     // then this many
// LDS after the operand regions: flag words and argmax keys, the static
// segments' first-block table, the pool claim ring, the segments' region
// offsets.
constexpr int kMaxSegs = kMaxWgSegs + kMaxPoolSegs;  // segments of one workgroup
constexpr size_t kSegFirstOff = kFlagBytes;
constexpr size_t kRingOff = kSegFirstOff + (4 * (kMaxWgSegs + 1) + 15) / 16 * 16;
constexpr size_t kSegOffOff = kRingOff + 8 * kRing;   // [kMaxSegs][2]: LDS start and end of each segment's operands
constexpr size_t kLdsTailBytes = kSegOffOff + 8 * kMaxSegs;
constexpr size_t kParkBytes = 16 * 1024;          // tiles a wave re-reads after its last one
enum { kKindTernary = 0, kKindInt8 = 1 };

// Operand regions (operands.h): the ternary levels' FP8 pieces of x and the
// vocabulary's base-256 digits of h.
using ops::ternary_mfmas;
using ops::ternary_quads;
using ops::ternary_bsc_off;
using ops::ternary_asc_off;
using ops::ternary_region_bytes;
using ops::int8_exp_off;
using ops::int8_region_bytes;
static_assert(ternary_region_bytes(kMaxStreamCols) % 16 == 0, "regions are copied in 16-byte units");

// One ternary level or (last entry) the vocabulary.
struct Level {
  const unsigned char* w;   // tiled weights (16-row x 64-byte tiles)
  const float* scale;       // row scales
  const float* x;           // input (ternary: x; vocabulary: h)
  float* y;                 // output (ternary: y; vocabulary: logits or null)
  const unsigned char* b;   // converted operand region (workspace)
  unsigned char* b_out;     // same region, written by the conversion kernel
  int rows, cols;
  int tiles;                // tiles per 16-row block
  int kind;                 // kKindTernary or kKindInt8
  int bsc_off, asc_off;     // ternary: scale offsets; int8: bsc_off = exponent offset
  int b_bytes;              // region bytes (a multiple of 16)
  int conv0;                // first workgroup of the conversion kernel that converts this level's input
};

// Blocks [b0, b1) of level `level`: one contiguous part of a workgroup's range.
struct Seg {
  int level, b0, b1, pad;
};

// Work split: every workgroup first takes its static segments (contiguous
// ranges of the ternary levels), then claims blocks of the shared pool (the
// vocabulary, then one small-block ternary level) from one global counter,
// so that workgroups that stream faster take more of the pool.
struct Plan {
  int n_levels;             // ternary levels; levels[n_levels] is the vocabulary
  int grid;
  int seg_stride;
  int buf_bytes;            // LDS for operand regions (a ring of variable-size regions)
  int vocab, hidden;
  int depth;                // tiles in flight per compute wave
  int pool_nseg;            // pool segments (levels), in claim order
  int pool_total;           // pool blocks
  int pool_first[kMaxPoolSegs + 1];  // first pool index of each pool segment (then pool_total)
  Seg pool_segs[kMaxPoolSegs];
  unsigned* pool_next;      // global claim counter
  const int* seg_count;     // [grid]
  const int* conv_level;    // [conversion workgroups]: the level each one converts
  const float* h;
  const dev::u32x4* emb_table;
  const float* emb_scale;
  const int32_t* token_in;
  int32_t* token_out;
  dev::u32x4* emb_row_out;
  float* emb_scale_out;
  float4* emb_deq_out;
  const unsigned char* park; // kParkBytes of workspace
  unsigned long long* partials;
  unsigned* arrivals;
  unsigned* status;
};

}  // namespace stream
}  // namespace pwg
