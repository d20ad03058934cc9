// Internal declarations shared by the library's translation units.
#pragma once
#include <cstdint>
#include <cstddef>

#include "../../include/pwg.h"

namespace pwg {

// Records a formatted message for pwg_last_error() on this thread and
// returns `code`, so call sites can write `return fail(PWG_ERR_ARG, ...)`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

#define TRY(expr)                  \
  do {                             \
    const int _rc = (expr);        \
    if (_rc != PWG_OK) return _rc; \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_batch(int32_t b) { return b == 1 || b == 4 || b == 8 || b == 16; }
inline bool valid_cols(int64_t cols) { return cols >= 64 && cols % 64 == 0 && cols <= PWG_MAX_COLS; }
// The VALU int8 kernel keeps 80 dwords of activation limbs per 4,096 columns
// in VGPRs; beyond 8,192 columns they would spill.
constexpr int64_t kMaxInt8Cols = 8192;

// Launchers (asynchronous, arguments already validated).
int launch_ternary_gemv(const void* w, const float* s, int64_t rows, int64_t cols,
                        const float* x, int32_t batch, float* y, void* stream);
int launch_int8_gemv_argmax(const int8_t* table, const float* s, int64_t rows, int64_t cols,
                            const float* h, int32_t batch, void* ws, int32_t* token,
                            float* logits, void* stream);
size_t int8_partials(int64_t rows);
// Batch-1 ternary GEMV on the tiled arrangement (gemv_mfma.hip).
int launch_ternary_gemv_b3(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
                           float* y, void* stream);
int launch_ternary_gemv_formed(const void* w, const float* s, int64_t rows, int64_t cols, const pwg_input& in,
                               const pwg_step_desc* d, float* x, float* y, void* stream);
int launch_ternary_gemv_tiled1(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, float* y,
                               void* stream);
int launch_argmax_reduce_batch(const unsigned long long* partials, int n, size_t nparts, int32_t batch, int32_t* token,
                               void* stream);
// Matrix-core variant of the batched int8 projection (batch_mfma.hip): for
// batch 4, 8, 16 and cols a multiple of 1,024 up to kMaxInt8Cols.  Its
// operands live in the workspace after the partial keys.
bool i8b_supported(int64_t cols, int32_t batch);
size_t i8b_operand_bytes(int32_t batch);
// Operand area of a batched matrix-core call for up to `cap` values per vector.
size_t batch_operand_bytes(int64_t cap, int32_t batch);
// Batched ternary GEMV on tiled T2 weights (batch 4, 8, 16; cols % 2048 == 0).
int launch_t2b(const void* w_tiled, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch, float* y,
               void* ops_area, void* stream);
int launch_i8b(const int8_t* table, bool tiled, const float* s, int64_t rows, int64_t cols, const float* h,
               int32_t batch, unsigned long long* partials, size_t nparts, unsigned char* ops_area, float* logits,
               int32_t* token, void* stream);
size_t i8_lds_bytes(int64_t cols);
// Decode attention over a bfloat16 KV cache (attention.hip).
bool attention_supported(int n_heads, int n_kv, int head_dim);
size_t attention_workspace(int n_heads, int n_kv, int head_dim, long ctx);
int launch_attention(const uint16_t* k, const uint16_t* v, const float* q, int n_heads, int n_kv, int head_dim,
                     long ctx, float scale, float* out, void* workspace, void* stream);

// Verify-pass acceptance (verify.hip).
int launch_verify_accept(const int32_t* tokens_in, const int32_t* targets, int32_t n_drafts, int32_t* accepted,
                         int32_t* next_token, void* stream);

// Chained step, levels schedule (chain.hip): forms one level's input into x.
int launch_chain_input(const pwg_input& in, int64_t n, float* x, const pwg_step_desc* d, void* stream);

int launch_embed_gather(const int8_t* table, const float* s, int64_t rows, int64_t cols,
                        const int32_t* ids, int32_t n, int8_t* rows_out, float* scales_out,
                        float* deq_out, void* stream);


// Stream schedule on the matrix cores (step_stream.hip): tiled weights.
int step_stream_check(const pwg_step_desc* d);
size_t step_stream_workspace(const pwg_step_desc* d);
int step_stream_plan(const pwg_step_desc* d, size_t ws_offset, void* stream);
int step_stream_launch(const pwg_step_desc* d, size_t ws_offset, void* stream);
int step_stream_status(const pwg_step_desc* d, size_t ws_offset, void* stream);

// Batched pass (step_batch.hip): batch 4, 8 or 16, tiled weights.
// The ordered (persistent) step on the matrix cores: step_ordered.hip.
size_t step_ordered_workspace(const pwg_step_desc* d);
int step_ordered_check(const pwg_step_desc* d, const char* fn);
int step_ordered_plan(const pwg_step_desc* d, void* stream);
int step_ordered_launch(const pwg_step_desc* d, void* stream);
int step_ordered_status(const pwg_step_desc* d, void* stream);
size_t step_ordered_trace_bytes(const pwg_step_desc* d);
int step_ordered_set_trace(const pwg_step_desc* d, void* trace, void* stream);

int step_batch_check(const pwg_step_desc* d);
size_t step_batch_workspace(const pwg_step_desc* d);
int step_batch_plan(const pwg_step_desc* d, void* stream);
int step_batch_launch(const pwg_step_desc* d, void* stream);
int step_batch_status(const pwg_step_desc* d, void* stream);

// Host-only checks of a step description (validate.cpp).
// PWG_ERR_UNSUPPORTED when a level input or h overlaps a buffer the step
// writes (schedules that run levels in no fixed order).
int check_unordered_aliasing(const pwg_step_desc* d, const char* fn);
uint64_t step_fingerprint(const pwg_step_desc* d);
// The fingerprint of the description a workspace was last planned for.
void plan_record(const pwg_step_desc* d);
void plan_forget(const pwg_step_desc* d);
// PWG_ERR_ARG unless `d` is the description its workspace was planned for.
int plan_check(const pwg_step_desc* d, const char* fn);

// 16-row x 64-byte tile arrangement (tile.hip).
size_t tiled_bytes(int64_t rows, int64_t row_bytes);
int launch_tile_rows(const void* src, int64_t rows, int64_t row_bytes, void* dst, void* stream);
size_t b3_tiled_bytes(int64_t rows, int64_t cols);
int launch_tile_b3(const void* src, int64_t rows, int64_t cols, void* dst, void* stream);

}  // namespace pwg
