// C entry points: argument validation, then the launchers.  Nothing here
// allocates or synchronises except pwg_step_plan (documented as such).
#include <hip/hip_runtime.h>

#include <cmath>

#include "operands.h"
#include "pwg_internal.h"

using namespace pwg;

namespace {

int check_ptr(const void* p, const char* fn, const char* name) {
  if (p == nullptr) return fail(PWG_ERR_ARG, "%s: %s is null", fn, name);
  if (!aligned16(p)) return fail(PWG_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, name);
  return PWG_OK;
}

int check_shape(int64_t rows, int64_t cols, const char* fn) {
  if (rows < 1 || rows > (int64_t{1} << 30))
    return fail(PWG_ERR_ARG, "%s: rows must be in [1, 2^30] (got %lld)", fn, (long long)rows);
  if (!valid_cols(cols))
    return fail(PWG_ERR_ARG, "%s: cols must be a multiple of 64 in [64, %d] (got %lld)", fn, PWG_MAX_COLS,
                (long long)cols);
  return PWG_OK;
}

int validate_ternary(const void* w, const float* s, int64_t rows, int64_t cols, const float* x, int32_t batch,
                     const float* y, const char* fn) {
  TRY(check_shape(rows, cols, fn));
  if (!valid_batch(batch)) return fail(PWG_ERR_ARG, "%s: batch must be 1, 4, 8 or 16 (got %d)", fn, batch);
  TRY(check_ptr(w, fn, "w_packed"));
  TRY(check_ptr(s, fn, "row_scale"));
  TRY(check_ptr(x, fn, "x"));
  TRY(check_ptr(y, fn, "y"));
  return PWG_OK;
}

int validate_int8(const int8_t* t, const float* s, int64_t rows, int64_t cols, const char* fn) {
  TRY(check_shape(rows, cols, fn));
  if (cols > kMaxInt8Cols)
    return fail(PWG_ERR_UNSUPPORTED, "%s: int8 tables wider than %lld columns are not supported", fn,
                (long long)kMaxInt8Cols);
  if (rows >= (int64_t{1} << 31) - 1) return fail(PWG_ERR_ARG, "%s: too many rows", fn);
  TRY(check_ptr(t, fn, "table"));
  TRY(check_ptr(s, fn, "row_scale"));
  return PWG_OK;
}

// Partial (max, index) keys of every vector; for batch > 1 also the operand
// area of the matrix-core kernel (sized for the widest table).
size_t argmax_ws(int64_t rows, int32_t batch) {
  return int8_partials(rows) * sizeof(unsigned long long) * batch + i8b_operand_bytes(batch);
}

}  // namespace

extern "C" int pwg_ternary_gemv(const void* w_packed, const float* row_scale, int64_t rows, int64_t cols,
                                const float* x, int32_t batch, float* y, void* stream) {
  TRY(validate_ternary(w_packed, row_scale, rows, cols, x, batch, y, "pwg_ternary_gemv"));
  return launch_ternary_gemv(w_packed, row_scale, rows, cols, x, batch, y, stream);
}

extern "C" size_t pwg_argmax_workspace_bytes(int64_t rows, int32_t batch) {
  if (rows < 1 || !valid_batch(batch)) return 0;
  return argmax_ws(rows, batch);
}

extern "C" int pwg_int8_gemv_argmax(const int8_t* table, const float* row_scale, int64_t rows, int64_t cols,
                                    const float* h, int32_t batch, void* workspace, size_t workspace_bytes,
                                    int32_t* token_out, float* logits_out, void* stream) {
  const char* fn = "pwg_int8_gemv_argmax";
  TRY(validate_int8(table, row_scale, rows, cols, fn));
  if (!valid_batch(batch)) return fail(PWG_ERR_ARG, "%s: batch must be 1, 4, 8 or 16 (got %d)", fn, batch);
  TRY(check_ptr(h, fn, "h"));
  TRY(check_ptr(workspace, fn, "workspace"));
  TRY(check_ptr(token_out, fn, "token_out"));
  if (logits_out && !aligned16(logits_out)) return fail(PWG_ERR_ALIGN, "%s: logits_out is not 16-byte aligned", fn);
  if (workspace_bytes < argmax_ws(rows, batch))
    return fail(PWG_ERR_SIZE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, argmax_ws(rows, batch));
  return launch_int8_gemv_argmax(table, row_scale, rows, cols, h, batch, workspace, token_out, logits_out, stream);
}

extern "C" size_t pwg_batch_workspace_bytes(int64_t cols, int32_t batch) {
  if (batch == 1) return (cols >= 256 && cols % 256 == 0 && cols <= PWG_MAX_COLS) ? 16 : 0;  // no scratch used
  if (cols < 2048 || cols % 2048 != 0 || cols > PWG_MAX_COLS || !(batch == 4 || batch == 8 || batch == 16)) return 0;
  return batch_operand_bytes(cols, batch);
}

extern "C" int pwg_ternary_gemv_tiled(const void* w_tiled, const float* row_scale, int64_t rows, int64_t cols,
                                      const float* x, int32_t batch, float* y, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const char* fn = "pwg_ternary_gemv_tiled";
  TRY(check_shape(rows, cols, fn));
  if (rows >= (int64_t{1} << 30)) return fail(PWG_ERR_ARG, "%s: too many rows", fn);
  if (!(batch == 1 || batch == 4 || batch == 8 || batch == 16))
    return fail(PWG_ERR_ARG, "%s: batch must be 1, 4, 8 or 16 (got %d)", fn, batch);
  if (cols % (batch == 1 ? 256 : 2048) != 0)
    return fail(PWG_ERR_UNSUPPORTED, "%s: cols must be a multiple of %d at batch %d (got %lld)", fn,
                batch == 1 ? 256 : 2048, batch, static_cast<long long>(cols));
  TRY(check_ptr(w_tiled, fn, "w_tiled"));
  TRY(check_ptr(row_scale, fn, "row_scale"));
  TRY(check_ptr(x, fn, "x"));
  TRY(check_ptr(y, fn, "y"));
  TRY(check_ptr(workspace, fn, "workspace"));
  const size_t need = pwg_batch_workspace_bytes(cols, batch);
  if (workspace_bytes < need) return fail(PWG_ERR_SIZE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  if (batch == 1) return launch_ternary_gemv_tiled1(w_tiled, row_scale, rows, cols, x, y, stream);
  return launch_t2b(w_tiled, row_scale, rows, cols, x, batch, y, workspace, stream);
}

extern "C" int pwg_int8_gemv_argmax_tiled(const int8_t* table_tiled, const float* row_scale, int64_t rows,
                                          int64_t cols, const float* h, int32_t batch, void* workspace,
                                          size_t workspace_bytes, int32_t* token_out, float* logits_out,
                                          void* stream) {
  const char* fn = "pwg_int8_gemv_argmax_tiled";
  TRY(validate_int8(table_tiled, row_scale, rows, cols, fn));
  if (!(batch == 4 || batch == 8 || batch == 16)) return fail(PWG_ERR_ARG, "%s: batch must be 4, 8 or 16 (got %d)", fn, batch);
  if (!i8b_supported(cols, batch))
    return fail(PWG_ERR_UNSUPPORTED, "%s: cols must be a multiple of 1024 (got %lld)", fn, static_cast<long long>(cols));
  TRY(check_ptr(h, fn, "h"));
  TRY(check_ptr(workspace, fn, "workspace"));
  TRY(check_ptr(token_out, fn, "token_out"));
  if (logits_out && !aligned16(logits_out)) return fail(PWG_ERR_ALIGN, "%s: logits_out is not 16-byte aligned", fn);
  if (workspace_bytes < argmax_ws(rows, batch))
    return fail(PWG_ERR_SIZE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, argmax_ws(rows, batch));
  const size_t nparts = int8_partials(rows);
  return launch_i8b(table_tiled, true, row_scale, rows, cols, h, batch, static_cast<unsigned long long*>(workspace),
                    nparts, static_cast<unsigned char*>(workspace) + nparts * sizeof(unsigned long long) * batch,
                    logits_out, token_out, stream);
}

extern "C" int pwg_embed_gather(const int8_t* table, const float* row_scale, int64_t rows, int64_t cols,
                                const int32_t* ids, int32_t n, int8_t* rows_out, float* scales_out, float* deq_out,
                                void* stream) {
  const char* fn = "pwg_embed_gather";
  TRY(check_shape(rows, cols, fn));
  if (rows >= (int64_t{1} << 31) - 1) return fail(PWG_ERR_ARG, "%s: too many rows", fn);
  if (n < 0 || n > (1 << 24)) return fail(PWG_ERR_ARG, "%s: n must be in [0, 2^24] (got %d)", fn, n);
  if (n == 0) return PWG_OK;
  TRY(check_ptr(table, fn, "table"));
  TRY(check_ptr(row_scale, fn, "row_scale"));
  TRY(check_ptr(ids, fn, "ids"));
  TRY(check_ptr(rows_out, fn, "rows_out"));
  TRY(check_ptr(scales_out, fn, "scales_out"));
  if (deq_out && !aligned16(deq_out)) return fail(PWG_ERR_ALIGN, "%s: deq_out is not 16-byte aligned", fn);
  return launch_embed_gather(table, row_scale, rows, cols, ids, n, rows_out, scales_out, deq_out, stream);
}

// ---------------------------------------------------------------------------
// Tiled arrangement
// ---------------------------------------------------------------------------
extern "C" size_t pwg_tiled_size(int64_t rows, int64_t row_bytes) { return tiled_bytes(rows, row_bytes); }

extern "C" int pwg_tile_rows(const void* src, int64_t rows, int64_t row_bytes, void* dst, size_t dst_bytes,
                             void* stream) {
  const char* fn = "pwg_tile_rows";
  if (rows < 1 || rows > (int64_t{1} << 30) || row_bytes < 64 || row_bytes % 64 != 0 || row_bytes > (int64_t{1} << 20))
    return fail(PWG_ERR_ARG, "%s: rows must be in [1, 2^30] and row_bytes a multiple of 64 in [64, 2^20]", fn);
  TRY(check_ptr(src, fn, "src"));
  TRY(check_ptr(dst, fn, "dst"));
  const size_t need = tiled_bytes(rows, row_bytes);
  if (dst_bytes < need) return fail(PWG_ERR_SIZE, "%s: dst has %zu bytes, needs %zu", fn, dst_bytes, need);
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const size_t src_bytes = static_cast<size_t>(rows) * static_cast<size_t>(row_bytes);
  if (s0 < d0 + need && d0 < s0 + src_bytes) return fail(PWG_ERR_ARG, "%s: src and dst overlap", fn);
  return launch_tile_rows(src, rows, row_bytes, dst, stream);
}

// ---------------------------------------------------------------------------
// Base-3 weights
// ---------------------------------------------------------------------------
namespace {
int check_b3_shape(int64_t rows, int64_t cols, const char* fn) {
  if (rows < 1 || rows > (int64_t{1} << 30))
    return fail(PWG_ERR_ARG, "%s: rows must be in [1, 2^30] (got %lld)", fn, (long long)rows);
  if (cols < 1 || cols > PWG_MAX_COLS)
    return fail(PWG_ERR_ARG, "%s: cols must be in [1, %d] (got %lld)", fn, PWG_MAX_COLS, (long long)cols);
  return PWG_OK;
}
}  // namespace

extern "C" size_t pwg_b3_tiled_size(int64_t rows, int64_t cols) { return b3_tiled_bytes(rows, cols); }

extern "C" int pwg_tile_b3(const void* src, int64_t rows, int64_t cols, void* dst, size_t dst_bytes, void* stream) {
  const char* fn = "pwg_tile_b3";
  TRY(check_b3_shape(rows, cols, fn));
  if (src == nullptr) return fail(PWG_ERR_ARG, "%s: src is null", fn);
  TRY(check_ptr(dst, fn, "dst"));
  const size_t need = b3_tiled_bytes(rows, cols);
  if (dst_bytes < need) return fail(PWG_ERR_SIZE, "%s: dst has %zu bytes, needs %zu", fn, dst_bytes, need);
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const size_t src_bytes = static_cast<size_t>(rows) * static_cast<size_t>(ops::b3_row_bytes(cols));
  if (s0 < d0 + need && d0 < s0 + src_bytes) return fail(PWG_ERR_ARG, "%s: src and dst overlap", fn);
  return launch_tile_b3(src, rows, cols, dst, stream);
}

extern "C" int pwg_ternary_gemv_b3(const void* w_b3_tiled, const float* row_scale, int64_t rows, int64_t cols,
                                   const float* x, int32_t batch, float* y, void* stream) {
  const char* fn = "pwg_ternary_gemv_b3";
  TRY(check_b3_shape(rows, cols, fn));
  if (!valid_batch(batch)) return fail(PWG_ERR_ARG, "%s: batch must be 1, 4, 8 or 16 (got %d)", fn, batch);
  TRY(check_ptr(w_b3_tiled, fn, "w_b3_tiled"));
  TRY(check_ptr(row_scale, fn, "row_scale"));
  TRY(check_ptr(x, fn, "x"));
  TRY(check_ptr(y, fn, "y"));
  return launch_ternary_gemv_b3(w_b3_tiled, row_scale, rows, cols, x, batch, y, stream);
}

// ---------------------------------------------------------------------------
// Decode step
// ---------------------------------------------------------------------------
namespace {

bool batched(const pwg_step_desc* d) { return d->batch > 1; }

bool chained(const pwg_input& in) { return in.op != PWG_INPUT_GIVEN; }

constexpr int64_t kMaxFormedInput = 12288;

// A level input op (pwg.h, pwg_input): n is the level's cols (hidden for h).
int validate_input(const pwg_input& in, int64_t n, const float* x, const char* fn, const char* what) {
  if (in.op == PWG_INPUT_GIVEN) return PWG_OK;
  if (in.op < PWG_INPUT_GIVEN || in.op > PWG_INPUT_SWIGLU)
    return fail(PWG_ERR_ARG, "%s: %s: unknown input op %d", fn, what, in.op);
  if (n > kMaxFormedInput)
    return fail(PWG_ERR_UNSUPPORTED, "%s: %s: formed inputs hold at most %d values", fn, what, kMaxFormedInput);
  const void* bufs[5] = {x, in.resid_out, in.src, in.resid, in.gamma};
  for (int a = 0; a < 5; ++a)
    for (int b = a + 1; b < 5; ++b)
      if (bufs[a] && bufs[a] == bufs[b]) return fail(PWG_ERR_ARG, "%s: %s: input buffers overlap", fn, what);
  if (in.op == PWG_INPUT_RMSNORM || in.op == PWG_INPUT_EMBED_RMSNORM) {
    if (!(in.eps >= 0.f) || in.eps > 1e30f) return fail(PWG_ERR_ARG, "%s: %s: eps must be >= 0", fn, what);
    TRY(check_ptr(in.gamma, fn, "gamma"));
    if (in.op == PWG_INPUT_RMSNORM) TRY(check_ptr(in.resid, fn, "resid"));
  } else {
    TRY(check_ptr(in.src, fn, "src"));
    if (in.op == PWG_INPUT_ATTN1) {
      if (in.head_dim < 1 || in.group < 1 || n % (static_cast<int64_t>(in.head_dim) * in.group) != 0)
        return fail(PWG_ERR_ARG, "%s: %s: %lld values are not whole groups of %d heads of %d", fn, what,
                    static_cast<long long>(n), in.group, in.head_dim);
    }
  }
  return PWG_OK;
}

// A chained level's output may not overlap anything its input is formed
// from or written to: the level's workgroups form the input while others
// may already store their rows.
int check_output_apart(const pwg_input& in, int64_t n, const float* x, const float* y, int64_t rows, const char* fn) {
  if (in.op == PWG_INPUT_GIVEN) return PWG_OK;
  const int64_t src_n = in.op == PWG_INPUT_SWIGLU ? 2 * n : in.op == PWG_INPUT_ATTN1 ? n / (in.group > 0 ? in.group : 1) : n;
  const struct {
    const float* p;
    int64_t count;
    const char* what;
  } bufs[5] = {{x, n, "x"}, {in.resid_out, n, "resid_out"}, {in.src, src_n, "src"}, {in.resid, n, "resid"},
               {in.gamma, n, "gamma"}};
  const uintptr_t y0 = reinterpret_cast<uintptr_t>(y), y1 = y0 + static_cast<uintptr_t>(rows) * 4;
  for (const auto& b : bufs) {
    if (!b.p) continue;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(b.p), b1 = b0 + static_cast<uintptr_t>(b.count) * 4;
    if (b0 < y1 && y0 < b1) return fail(PWG_ERR_ARG, "%s: the level's y overlaps its input's %s", fn, b.what);
  }
  return PWG_OK;
}

int validate_step(const pwg_step_desc* d) {
  const char* fn = "pwg_decode_step_weights";
  if (!d) return fail(PWG_ERR_ARG, "%s: desc is null", fn);
  if (d->schedule != PWG_SCHEDULE_LEVELS && d->schedule != PWG_SCHEDULE_PERSISTENT &&
      d->schedule != PWG_SCHEDULE_STREAM)
    return fail(PWG_ERR_ARG, "%s: unknown schedule %d", fn, d->schedule);
  if (d->n_levels < 0 || d->n_levels > 4096) return fail(PWG_ERR_ARG, "%s: n_levels out of range", fn);
  if (d->weight_layout != PWG_LAYOUT_ROWS && d->weight_layout != PWG_LAYOUT_TILED)
    return fail(PWG_ERR_ARG, "%s: unknown weight layout %d", fn, d->weight_layout);
  const int want = d->schedule == PWG_SCHEDULE_LEVELS ? PWG_LAYOUT_ROWS : PWG_LAYOUT_TILED;
  if (d->weight_layout != want)
    return fail(PWG_ERR_UNSUPPORTED, "%s: schedule %d takes weight layout %d (got %d)", fn, d->schedule, want,
                d->weight_layout);
  if (d->batch != 0 && d->batch != 1) {
    if (!(d->batch == 4 || d->batch == 8 || d->batch == 16))
      return fail(PWG_ERR_ARG, "%s: batch must be 0, 1, 4, 8 or 16 (got %d)", fn, d->batch);
    if (d->schedule != PWG_SCHEDULE_STREAM)
      return fail(PWG_ERR_UNSUPPORTED, "%s: batch %d takes the stream schedule", fn, d->batch);
  }
  if (d->n_levels > 0 && !d->levels) return fail(PWG_ERR_ARG, "%s: levels is null", fn);
  bool any_chained = chained(d->h_in);
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    int rc = validate_ternary(L.w_packed, L.row_scale, L.rows, L.cols, L.x, 1, L.y, fn);
    if (rc == PWG_OK) rc = validate_input(L.in, L.cols, L.x, fn, "level input");
    if (rc == PWG_OK) rc = check_output_apart(L.in, L.cols, L.x, L.y, L.rows, fn);
    if (rc != PWG_OK) return fail(rc, "%s (level %d)", pwg_last_error(), i);
    any_chained = any_chained || chained(L.in);
  }
  TRY(validate_input(d->h_in, d->hidden, d->h, fn, "h"));
  if (any_chained && (d->schedule == PWG_SCHEDULE_STREAM || batched(d)))
    return fail(PWG_ERR_UNSUPPORTED, "%s: formed level inputs need an ordered schedule (levels or persistent) at batch 1",
                fn);
  if (d->schedule == PWG_SCHEDULE_STREAM) {
    TRY(check_shape(d->vocab, d->hidden, fn));
    TRY(check_ptr(d->out_table, fn, "out_table"));
    TRY(check_ptr(d->out_scale, fn, "out_scale"));
    TRY(batched(d) ? step_batch_check(d) : step_stream_check(d));
  } else if (d->schedule == PWG_SCHEDULE_PERSISTENT) {
    TRY(check_shape(d->vocab, d->hidden, fn));
    TRY(check_ptr(d->out_table, fn, "out_table"));
    TRY(check_ptr(d->out_scale, fn, "out_scale"));
    TRY(step_ordered_check(d, fn));
  } else {
    TRY(validate_int8(d->out_table, d->out_scale, d->vocab, d->hidden, fn));
  }
  TRY(check_ptr(d->h, fn, "h"));
  TRY(check_ptr(d->emb_table, fn, "emb_table"));
  TRY(check_ptr(d->emb_scale, fn, "emb_scale"));
  TRY(check_ptr(d->token_in, fn, "token_in"));
  TRY(check_ptr(d->token_out, fn, "token_out"));
  TRY(check_ptr(d->emb_row_out, fn, "emb_row_out"));
  TRY(check_ptr(d->emb_scale_out, fn, "emb_scale_out"));
  if (d->emb_deq_out && !aligned16(d->emb_deq_out)) return fail(PWG_ERR_ALIGN, "%s: emb_deq_out misaligned", fn);
  if (d->logits_out && !aligned16(d->logits_out)) return fail(PWG_ERR_ALIGN, "%s: logits_out misaligned", fn);
  TRY(check_ptr(d->workspace, fn, "workspace"));
  if (d->schedule == PWG_SCHEDULE_STREAM) TRY(check_unordered_aliasing(d, fn));
  return PWG_OK;
}

}  // namespace

extern "C" size_t pwg_step_workspace_bytes(const pwg_step_desc* d) {
  if (!d || d->vocab < 1) return 0;
  if (!(d->batch == 0 || d->batch == 1 || d->batch == 4 || d->batch == 8 || d->batch == 16)) return 0;
  if (batched(d)) {
    if (d->schedule != PWG_SCHEDULE_STREAM || d->n_levels < 0 || (d->n_levels > 0 && !d->levels)) return 0;
    return step_batch_workspace(d);
  }
  if (d->schedule == PWG_SCHEDULE_STREAM) return step_stream_workspace(d);
  if (d->schedule == PWG_SCHEDULE_PERSISTENT) return step_ordered_workspace(d);
  if (d->schedule != PWG_SCHEDULE_LEVELS) return 0;
  return argmax_ws(d->vocab, 1);
}

extern "C" int pwg_step_plan(const pwg_step_desc* d, void* stream) {
  TRY(validate_step(d));
  if (d->workspace_bytes < pwg_step_workspace_bytes(d))
    return fail(PWG_ERR_SIZE, "pwg_step_plan: workspace %zu < %zu bytes", d->workspace_bytes,
                pwg_step_workspace_bytes(d));
  if (d->schedule == PWG_SCHEDULE_LEVELS) return PWG_OK;
  plan_forget(d);
  if (d->schedule == PWG_SCHEDULE_PERSISTENT) TRY(step_ordered_plan(d, stream));
  else TRY(batched(d) ? step_batch_plan(d, stream) : step_stream_plan(d, 0, stream));
  plan_record(d);
  return PWG_OK;
}

extern "C" int pwg_step_status(const pwg_step_desc* d, void* stream) {
  TRY(validate_step(d));
  if (d->schedule == PWG_SCHEDULE_LEVELS) return PWG_OK;
  if (d->schedule == PWG_SCHEDULE_PERSISTENT) return step_ordered_status(d, stream);
  if (batched(d)) return step_batch_status(d, stream);
  return step_stream_status(d, 0, stream);
}

extern "C" size_t pwg_step_trace_bytes(const pwg_step_desc* d) {
  if (!d || d->schedule != PWG_SCHEDULE_PERSISTENT || d->n_levels < 0 || d->n_levels > 4096) return 0;
  return step_ordered_trace_bytes(d);
}

extern "C" int pwg_step_set_trace(const pwg_step_desc* d, void* trace, size_t trace_bytes, void* stream) {
  const char* fn = "pwg_step_set_trace";
  TRY(validate_step(d));
  if (d->schedule != PWG_SCHEDULE_PERSISTENT)
    return fail(PWG_ERR_UNSUPPORTED, "%s: only the persistent schedule records a level trace", fn);
  TRY(plan_check(d, fn));
  if (trace) {
    const size_t need = pwg_step_trace_bytes(d);
    if (trace_bytes < need) return fail(PWG_ERR_SIZE, "%s: trace buffer %zu < %zu bytes", fn, trace_bytes, need);
    if (!aligned16(trace)) return fail(PWG_ERR_ALIGN, "%s: trace buffer is not 16-byte aligned", fn);
  }
  return step_ordered_set_trace(d, trace, stream);
}

extern "C" int pwg_decode_step_weights(const pwg_step_desc* d, void* stream) {
  TRY(validate_step(d));
  if (d->workspace_bytes < pwg_step_workspace_bytes(d))
    return fail(PWG_ERR_SIZE, "pwg_decode_step_weights: workspace %zu < %zu bytes", d->workspace_bytes,
                pwg_step_workspace_bytes(d));
  if (d->schedule != PWG_SCHEDULE_LEVELS) {
    // the kernels take every pointer and shape from the device plan
    TRY(plan_check(d, "pwg_decode_step_weights"));
    if (d->schedule == PWG_SCHEDULE_PERSISTENT) return step_ordered_launch(d, stream);
    return batched(d) ? step_batch_launch(d, stream) : step_stream_launch(d, 0, stream);
  }
  // Levels schedule: embedding row, every level in decoder order, output
  // projection + argmax, all on one stream.
  TRY(launch_embed_gather(d->emb_table, d->emb_scale, d->vocab, d->hidden, d->token_in, 1, d->emb_row_out,
                          d->emb_scale_out, d->emb_deq_out, stream));
  for (int i = 0; i < d->n_levels; ++i) {
    const pwg_level& L = d->levels[i];
    if (chained(L.in))  // the GEMV forms its input itself
      TRY(launch_ternary_gemv_formed(L.w_packed, L.row_scale, L.rows, L.cols, L.in, d, const_cast<float*>(L.x), L.y,
                                     stream));
    else
      TRY(launch_ternary_gemv(L.w_packed, L.row_scale, L.rows, L.cols, L.x, 1, L.y, stream));
  }
  if (chained(d->h_in)) TRY(launch_chain_input(d->h_in, d->hidden, const_cast<float*>(d->h), d, stream));
  return launch_int8_gemv_argmax(d->out_table, d->out_scale, d->vocab, d->hidden, d->h, 1, d->workspace,
                                 d->token_out, d->logits_out, stream);
}

// ---------------------------------------------------------------------------
// Decode attention
// ---------------------------------------------------------------------------
extern "C" size_t pwg_attention_workspace_bytes(int32_t n_heads, int32_t n_kv, int32_t head_dim, int64_t ctx) {
  if (ctx < 1 || ctx > (int64_t{1} << 31) || !attention_supported(n_heads, n_kv, head_dim)) return 0;
  return attention_workspace(n_heads, n_kv, head_dim, static_cast<long>(ctx));
}

extern "C" int pwg_gqa_decode_attention(const uint16_t* k_cache, const uint16_t* v_cache, const float* q,
                                        int32_t n_heads, int32_t n_kv, int32_t head_dim, int64_t ctx, float scale,
                                        float* out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pwg_gqa_decode_attention";
  if (n_heads < 1 || n_kv < 1 || head_dim < 1 || n_heads % n_kv != 0)
    return fail(PWG_ERR_ARG, "%s: %d query heads are not a multiple of %d key/value heads", fn, n_heads, n_kv);
  if (ctx < 1 || ctx > (int64_t{1} << 31)) return fail(PWG_ERR_ARG, "%s: ctx must be in [1, 2^31]", fn);
  if (!std::isfinite(scale)) return fail(PWG_ERR_ARG, "%s: scale is not finite", fn);
  if (!attention_supported(n_heads, n_kv, head_dim))
    return fail(PWG_ERR_UNSUPPORTED, "%s: head_dim %d with %d query heads per key/value head", fn, head_dim,
                n_heads / n_kv);
  TRY(check_ptr(k_cache, fn, "k_cache"));
  TRY(check_ptr(v_cache, fn, "v_cache"));
  TRY(check_ptr(q, fn, "q"));
  TRY(check_ptr(out, fn, "out"));
  TRY(check_ptr(workspace, fn, "workspace"));
  const size_t need = attention_workspace(n_heads, n_kv, head_dim, static_cast<long>(ctx));
  if (workspace_bytes < need) return fail(PWG_ERR_SIZE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, need);
  return launch_attention(k_cache, v_cache, q, n_heads, n_kv, head_dim, static_cast<long>(ctx), scale, out,
                          workspace, stream);
}

// ---------------------------------------------------------------------------
// Verify-pass acceptance
// ---------------------------------------------------------------------------
extern "C" int pwg_verify_accept(const int32_t* tokens_in, const int32_t* targets, int32_t n_drafts,
                                 int32_t* accepted, int32_t* next_token, void* stream) {
  const char* fn = "pwg_verify_accept";
  if (n_drafts < 0 || n_drafts > 15) return fail(PWG_ERR_ARG, "%s: n_drafts must be in [0, 15] (got %d)", fn, n_drafts);
  TRY(check_ptr(tokens_in, fn, "tokens_in"));
  TRY(check_ptr(targets, fn, "targets"));
  TRY(check_ptr(accepted, fn, "accepted"));
  TRY(check_ptr(next_token, fn, "next_token"));
  return launch_verify_accept(tokens_in, targets, n_drafts, accepted, next_token, stream);
}
