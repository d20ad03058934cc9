/*
 * pwg.h - C ABI of the packed ternary weight-streaming decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes comes from the page "The Neutrino Engine"
 * (fermionresearch.com):
 *   - section "A 104 microsecond floor inside a 694 microsecond step": batch-1
 *     decode applies every layer's attention and feed-forward projections to
 *     the current activations, one multiply-accumulate per weight per token;
 *     the output projection scores the hidden state against the whole
 *     vocabulary; packed weights are read in place, with no float copy and no
 *     tensor read twice per token;
 *   - section "The file is not the traffic": projections are ternary with row
 *     scales; two int8 vocabulary tables of 151,936 x 4,096; the input side
 *     reads only the selected rows, the output side scores the whole table;
 *   - intro and section "The same weights take four execution paths": decode
 *     is greedy (argmax) and the loader re-arranges the same values for the
 *     device at load time.
 *
 * Conventions (every entry point):
 *   - Return value: PWG_OK (0) on success, a negative PWG_ERR_* code on
 *     failure; pwg_last_error() then returns a message for the calling thread.
 *     Arguments are validated before anything is enqueued; a failed call has
 *     enqueued no work.  No C++ exception crosses this boundary.
 *   - Ownership: the caller owns and allocates every buffer.  The GPU entry
 *     points allocate nothing, free nothing and never synchronise, so they may
 *     be recorded into a HIP graph with stream capture.
 *   - Device pointers are plain device addresses (e.g. a torch tensor's
 *     data_ptr()); host pointers are plain host addresses.  Every device
 *     pointer must be 16-byte aligned (PWG_ERR_ALIGN otherwise).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  GPU
 *     entry points are asynchronous on that stream.
 *   - Shapes: rows >= 1; cols a multiple of 64 and at most PWG_MAX_COLS.
 *     batch is 1, 4, 8 or 16.
 *   - Floating-point inputs must be finite.
 */
#ifndef PWG_H
#define PWG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif
#pragma GCC visibility push(default)

#define PWG_VERSION 7
#define PWG_MAX_COLS 16384

enum {
  PWG_OK = 0,
  PWG_ERR_ARG = -1,         /* null pointer, bad shape, bad batch, bad id on host */
  PWG_ERR_ALIGN = -2,       /* a device pointer is not 16-byte aligned */
  PWG_ERR_SIZE = -3,        /* an output buffer or workspace is too small */
  PWG_ERR_VALUE = -4,       /* a weight outside {-1, 0, +1}; message names (row, col) */
  PWG_ERR_HIP = -5,         /* a HIP runtime error; message has hipGetErrorString */
  PWG_ERR_UNSUPPORTED = -6  /* valid request this build does not implement */
};

/* Step schedules for pwg_decode_step_weights. */
enum {
  PWG_SCHEDULE_LEVELS = 0,      /* one kernel per dependency level, in decoder order */
  PWG_SCHEDULE_PERSISTENT = 1,  /* one resident matrix-core kernel that runs the
                                   levels in decoder order, separated by device-wide
                                   barriers; each workgroup's weight tiles of a level
                                   are loaded before that level's input is ready.
                                   Honours every dependency (chained inputs allowed).
                                   Needs PWG_LAYOUT_TILED weights, batch 1, hidden and
                                   every level's cols a multiple of 256 and at most
                                   12288; pwg_step_plan before the first call */
  PWG_SCHEDULE_STREAM = 2       /* one matrix-core kernel (after a small input
                                   conversion kernel) without level barriers: the
                                   16-row blocks of all levels and of the vocabulary
                                   are split over the CUs, so levels overlap.  Valid
                                   only when no level reads another level's output
                                   (as in a step over fixed inputs); it measures the
                                   weight stream alone, without dependency waits.
                                   Needs PWG_LAYOUT_TILED weights, every level's cols
                                   and hidden a multiple of 256 and at most 12288 */
};

/* Weight arrangements of a step description (pwg_step_desc.weight_layout). */
enum {
  PWG_LAYOUT_ROWS = 0,   /* T2 blobs and the int8 output table row-major
                            (schedule LEVELS) */
  PWG_LAYOUT_TILED = 1   /* the same bytes in 16-row x 64-byte tiles, see
                            pwg_tile_rows (schedules STREAM and PERSISTENT) */
};

/* ---------------------------------------------------------------------------
 * Packed ternary format "T2" (2 bits per weight).  The pages name their own
 * packed type but do not specify it; this is the library's format, arranged
 * at load time as the page's loader does.
 *   - logical W in {-1,0,+1}^(rows x cols), cols % 64 == 0;
 *   - row-major: row r is bytes [r*cols/4, (r+1)*cols/4);
 *   - each row is little-endian 32-bit words; word j holds weights
 *     k = 16*j + m (m = 0..15); weight m's code is at bit
 *     p(m) = 8*((m%8)/2) + 4*(m/8) + 2*(m%2): byte b holds weights 2b, 2b+1
 *     in its low nibble and 8+2b, 9+2b in its high nibble;
 *   - code = two's complement of w in 2 bits (0 -> 00, +1 -> 01, -1 -> 11);
 *   - no header; row scales are separate float32 arrays.
 * ------------------------------------------------------------------------- */

/* Bytes of a packed T2 blob: rows*cols/4.  Returns 0 for an invalid shape
 * (rows < 1, cols < 64, cols % 64 != 0).  Pure host function. */
size_t pwg_packed_size(int64_t rows, int64_t cols);

/* Pack a logical ternary matrix into T2 (page section "The same weights take
 * four execution paths": the same values arranged for the device at load
 * time).  Synchronous host code; may use several threads internally.
 *   w_host       host, int8 row-major rows x cols, values in {-1, 0, +1}
 *   out_host     host, at least pwg_packed_size(rows, cols) bytes
 *   out_bytes    host, receives the bytes written (may be NULL)
 * Errors: PWG_ERR_ARG (null / bad shape), PWG_ERR_SIZE (capacity too small),
 * PWG_ERR_VALUE (a value outside {-1,0,1}; out_host contents unspecified). */
int pwg_pack_weights(const int8_t* w_host, int64_t rows, int64_t cols,
                     void* out_host, size_t out_capacity, size_t* out_bytes);

/* Inverse of pwg_pack_weights (host).  PWG_ERR_VALUE on a 0b10 code. */
int pwg_unpack_weights(const void* packed_host, int64_t rows, int64_t cols,
                       int8_t* w_out_host);

/* Ternary GEMV (page section "A 104 microsecond floor ...": each projection
 * applied to the current activations; section "The file is not the
 * traffic": ternary weights with row scales):
 *     y[b, r] = row_scale[r] * sum_k W[r, k] * x[b, k]
 *   w_packed     device, T2 blob of rows x cols
 *   row_scale    device, float32[rows]
 *   x            device, float32[batch][cols] row-major
 *   y            device, float32[batch][rows] row-major (written, not accumulated)
 * Arithmetic: the matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4), the
 * weights as FP4 and x as six e4m3 pieces per value with a shared E8M0 scale
 * per 32 values; the pieces sum to x to within 2^-24 of each value (2^-30 of
 * its 32-value block's maximum at worst), every product is exact and the
 * sums are float32: the accuracy of a float32 GEMV, outliers included.
 * batch > 1 runs one pass over the weights per vector.
 * Errors: PWG_ERR_ARG, PWG_ERR_ALIGN, PWG_ERR_HIP. */
int pwg_ternary_gemv(const void* w_packed, const float* row_scale,
                     int64_t rows, int64_t cols,
                     const float* x, int32_t batch,
                     float* y, void* stream);

/* ---------------------------------------------------------------------------
 * Tiled arrangement (page section "The same weights take four execution
 * paths": the loader arranges the stored values for the device at load
 * time).  A row-major byte matrix of `rows` rows of `row_bytes` bytes (a T2
 * blob: row_bytes = cols / 4; an int8 table: row_bytes = cols) becomes
 * 16-row x 64-byte tiles of 1 KiB:
 *   - rows are padded with zero bytes to a multiple of 16;
 *   - tile (rb, tc) covers rows 16 rb .. 16 rb + 15 and bytes 64 tc .. 64 tc + 63
 *     and sits at byte offset (rb * (row_bytes / 64) + tc) * 1024;
 *   - inside a tile, byte (row 16 rb + i, column 64 tc + 16 q + b) is at
 *     offset 256 q + 16 i + b  (i < 16, q < 4, b < 16).
 * One wave load instruction (64 lanes x 16 bytes) then reads one tile and
 * lane 16 q + i holds row i's bytes 16 q .. 16 q + 15 of the window: the
 * operand layout of the 16 x 16 matrix-core instructions.
 * ------------------------------------------------------------------------- */

/* Bytes of the tiled arrangement: ceil(rows / 16) * 16 * row_bytes; 0 for an
 * invalid shape (rows < 1, row_bytes < 64 or not a multiple of 64). */
size_t pwg_tiled_size(int64_t rows, int64_t row_bytes);

/* Writes the tiled arrangement of a row-major device matrix (asynchronous on
 * `stream`, capturable, allocates nothing).
 *   src          device, rows x row_bytes bytes, row-major
 *   dst          device, at least pwg_tiled_size(rows, row_bytes) bytes; must
 *                not overlap src
 * Errors: PWG_ERR_ARG (null, bad shape), PWG_ERR_ALIGN, PWG_ERR_SIZE, PWG_ERR_HIP. */
int pwg_tile_rows(const void* src, int64_t rows, int64_t row_bytes,
                  void* dst, size_t dst_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Base-3 packed ternary format "B3" (five weights per byte, 0.2 bytes per
 * weight against T2's 0.25).  Page "The Neutrino Engine", section "A 104
 * microsecond floor inside a 694 microsecond step": weight bytes over memory
 * bandwidth bound a batch-1 step, and a smaller artifact lowers that bound on
 * every backend; section "The file is not the traffic": the page's own
 * 72,351,744-byte layer slab (3 bits per weight).  The pages do not specify
 * their format; this is the library's:
 *   - logical W in {-1,0,+1}^(rows x cols), 1 <= cols <= PWG_MAX_COLS;
 *   - row-major: row r is bytes [r*B, (r+1)*B), B = ceil(cols/5);
 *   - byte m of a row holds weights k = 5m + i (i = 0..4) as base-3 digits
 *     d_i = w_k + 1, least significant first:
 *         byte = d_0 + 3 d_1 + 9 d_2 + 27 d_3 + 81 d_4;
 *     weights past the row end are 0 (digit 1); bytes 243..255 never occur;
 *   - no header; row scales are separate float32 arrays.
 * One layer of the 8B shape is 38,617,088 bytes (0.534 of the slab).
 * ------------------------------------------------------------------------- */

/* Bytes of a B3 blob: rows * ceil(cols / 5); 0 for an invalid shape (rows <
 * 1, cols outside [1, PWG_MAX_COLS]).  Pure host function. */
size_t pwg_b3_packed_size(int64_t rows, int64_t cols);

/* Pack a logical ternary matrix into B3 on the host (multi-threaded):
 *   w_host       host, int8 rows x cols row-major, values in {-1, 0, 1}
 *   out_host     host, >= pwg_b3_packed_size(rows, cols) bytes
 *   out_bytes    may be NULL; receives the blob size
 * Errors: PWG_ERR_ARG (null / bad shape), PWG_ERR_SIZE (capacity too small),
 * PWG_ERR_VALUE (a value outside {-1,0,1}; out_host contents unspecified). */
int pwg_pack_weights_b3(const int8_t* w_host, int64_t rows, int64_t cols,
                        void* out_host, size_t out_capacity, size_t* out_bytes);

/* Inverse of pwg_pack_weights_b3 (host).  PWG_ERR_VALUE on a byte > 242. */
int pwg_unpack_weights_b3(const void* packed_host, int64_t rows, int64_t cols,
                          int8_t* w_out_host);

/* Bytes of the device arrangement of a B3 blob: ceil(rows/16) 16-row blocks
 * of W = ceil(ceil(ceil(cols/5)/6)/8) windows of 768 bytes (40,304,640 bytes
 * for one layer of the 8B shape); 0 for an invalid shape. */
size_t pwg_b3_tiled_size(int64_t rows, int64_t cols);

/* Load-time device arrangement of a B3 blob (page section "The same weights
 * take four execution paths": the loader arranges the same stored values for
 * the device).  Each row's bytes are cut into 30-weight groups of 6 bytes and
 * padded with the zero-weight byte 121 to whole windows of 8 groups; rows are
 * padded to a multiple of 16 with zero-weight rows.  Window tile (rb, t) is
 * the (rb * W + t)-th 768 bytes; its 12 bytes at offset 12 L (L = 16 g + i)
 * are group 8t+g and then group 8t+4+g of row 16 rb + i: one lane's A
 * operands of two matrix-core instructions.
 *   src          device, the B3 blob (no alignment needed)
 *   dst          device, >= pwg_b3_tiled_size(rows, cols) bytes, 16-byte
 *                aligned, not overlapping src
 * Asynchronous on `stream`.  Errors: PWG_ERR_ARG (null, bad shape, overlap),
 * PWG_ERR_ALIGN, PWG_ERR_SIZE, PWG_ERR_HIP. */
int pwg_tile_b3(const void* src, int64_t rows, int64_t cols,
                void* dst, size_t dst_bytes, void* stream);

/* Ternary GEMV on B3 weights in their device arrangement:
 *     y[b, r] = row_scale[r] * sum_k W[r, k] * x[b, k]
 *   w_b3_tiled   device, pwg_tile_b3 output for rows x cols
 *   row_scale    device, float32[rows]
 *   x            device, float32[batch][cols]
 *   y            device, float32[batch][rows] (written)
 * The same arithmetic and accuracy as pwg_ternary_gemv (six e4m3 pieces of x
 * per value, FP4 weights, float32 sums; one E8M0 exponent per 30-value group
 * of x).  Each byte becomes five FP4 weights through a 256-entry table in
 * LDS (bytes 243..255 read as zero weights).  batch > 1 runs one pass per
 * vector.  Errors: PWG_ERR_ARG (null, shape, batch), PWG_ERR_ALIGN
 * (pointers are 16-byte aligned), PWG_ERR_HIP. */
int pwg_ternary_gemv_b3(const void* w_b3_tiled, const float* row_scale, int64_t rows, int64_t cols,
                        const float* x, int32_t batch, float* y, void* stream);

/* ---------------------------------------------------------------------------
 * Small batch on the tiled arrangement (page section "The 0.6B model does not
 * get to decide": several drafted tokens are scored in one batched pass, so
 * each weight is read once for all of them).  Both calls take the weights as
 * pwg_tile_rows arranges them (the arrangement the stream step reads), run on
 * the int8 matrix cores (v_mfma_i32_16x16x64_i8) and form every row sum
 * exactly in int32 per 256-value section (int8 tables) or 1,024-value block
 * (ternary weights) over a fixed-point rounding of the activations (four
 * balanced base-256 digits of rint(x * 2^(30 - e)), e the exponent of the
 * section or block: at most 2^(e - 31) per value); float32 after that.
 * Asynchronous on `stream`, capturable, allocate nothing. */

/* Workspace bytes of pwg_ternary_gemv_tiled for (cols, batch): the converted
 * activations (4 bytes per value and vector) and a few KiB; 16 (unused) for
 * batch 1; 0 for an unsupported shape (batch 1: cols not a multiple of 256 in
 * [256, PWG_MAX_COLS]; batch 4, 8, 16: cols not a multiple of 2048 in [2048,
 * PWG_MAX_COLS]; other batches). */
size_t pwg_batch_workspace_bytes(int64_t cols, int32_t batch);

/* Batched ternary GEMV on tiled T2 weights:
 *     y[b, r] = row_scale[r] * sum_k W[r, k] * x[b, k]
 *   w_tiled      device, pwg_tiled_size(rows, cols / 4) bytes (pwg_tile_rows
 *                of the T2 blob)
 *   row_scale    device, float32[rows]
 *   x            device, float32[batch][cols]
 *   y            device, float32[batch][rows] (written)
 *   workspace    device, >= pwg_batch_workspace_bytes(cols, batch); scratch
 * batch 1 (cols a multiple of 256): the matrix-core kernel of
 * pwg_ternary_gemv on the tiled weights (FP8 pieces of x, float32-accurate;
 * the workspace is not used).  batch 4, 8 or 16 (cols a multiple of 2048):
 * the digits above, the 2-bit codes expanded to int8 in registers.
 * Errors: PWG_ERR_ARG (null, shape, batch), PWG_ERR_ALIGN (pointers are
 * 16-byte aligned), PWG_ERR_SIZE, PWG_ERR_UNSUPPORTED (cols), PWG_ERR_HIP. */
int pwg_ternary_gemv_tiled(const void* w_tiled, const float* row_scale, int64_t rows, int64_t cols,
                           const float* x, int32_t batch, float* y, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Batched int8 projection + per-vector greedy argmax on a tiled table
 * (pwg_tile_rows of the rows x cols int8 table): the same results as
 * pwg_int8_gemv_argmax (bit for bit: the same digits and sums), with the
 * table streamed as contiguous 1 KiB tiles.  batch 4, 8 or 16; cols a
 * multiple of 1024, at most 8192; workspace >= pwg_argmax_workspace_bytes(rows,
 * batch).  Errors as pwg_int8_gemv_argmax, plus PWG_ERR_UNSUPPORTED (cols). */
int pwg_int8_gemv_argmax_tiled(const int8_t* table_tiled, const float* row_scale, int64_t rows,
                               int64_t cols, const float* h, int32_t batch, void* workspace,
                               size_t workspace_bytes, int32_t* token_out, float* logits_out,
                               void* stream);

/* Workspace bytes needed by pwg_int8_gemv_argmax for (rows, batch): the
 * partial (max, index) keys of every vector and, for batch 4, 8 and 16, the
 * matrix-core kernel's operand area (the digits of h for a table of up to
 * 8,192 columns, 4 bytes per value and vector: 512 KiB at batch 16). */
size_t pwg_argmax_workspace_bytes(int64_t rows, int32_t batch);

/* int8 output projection fused with greedy argmax (page sections "A 104
 * microsecond floor ..." - the output projection scores the full vocabulary -
 * and "The file is not the traffic" - int8 tables of 151,936 x 4,096):
 *     logit[b, v] = row_scale[v] * sum_k table[v, k] * h[b, k]
 *     token_out[b] = argmax_v logit[b, v], lowest v on ties
 *   table        device, int8 rows x cols row-major (read in place)
 *   row_scale    device, float32[rows]
 *   h            device, float32[batch][cols]
 *   workspace    device, >= pwg_argmax_workspace_bytes(rows, batch); scratch
 *                (contents on entry are ignored)
 *   token_out    device, int32[batch]
 *   logits_out   device float32[batch][rows] or NULL (written only if given)
 * batch 1: a fused GEMV + per-block (max, index), then one block that
 * reduces the pairs; h is rounded to five int8 limbs per value (39-bit fixed
 * point per 16-value chunk: at most 2^(e - 39) per value, e the exponent of
 * the chunk maximum) and each limb's sum is exact in int32 (v_dot4_i32_i8).
 * batch 4, 8, 16 with cols a multiple of 1,024: h is converted into
 * matrix-core operands in the workspace, one kernel computes every vector's
 * logits on v_mfma_i32_16x16x64_i8 (exact int32 sums per 256-value section
 * over four digits, as pwg_ternary_gemv_tiled) with the table read once, and
 * one block per vector reduces its keys; other widths run the batch-1 kernel
 * per vector.  Deterministic bit for bit on every path.
 * Errors: PWG_ERR_ARG, PWG_ERR_ALIGN, PWG_ERR_SIZE, PWG_ERR_HIP. */
int pwg_int8_gemv_argmax(const int8_t* table, const float* row_scale,
                         int64_t rows, int64_t cols,
                         const float* h, int32_t batch,
                         void* workspace, size_t workspace_bytes,
                         int32_t* token_out, float* logits_out,
                         void* stream);

/* pwg_int8_gemv_argmax for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and results, bit for bit, with no
 * workspace argument.  Its scratch (the per-workgroup (max, index) keys and,
 * for batch 4, 8, 16, the matrix-core operands of h) is a fixed device array
 * of this library, 1 MiB per GPU, held by each GPU the library runs on until
 * the process ends; the call allocates and frees nothing.  Requests needing
 * more than 1 MiB (pwg_argmax_workspace_bytes(rows, batch) > 1 MiB, e.g.
 * batch 16 over more than about 4,000 rows) fail with PWG_ERR_SIZE.  Every
 * call on one GPU shares that GPU's array and leaves its contents behind
 * (nothing in it needs to start at zero): calls that overlap on one GPU
 * (other streams, other threads) race.  The first call on a device looks up
 * the array's address (hipGetSymbolAddress), so make it outside stream
 * capture.  Arguments and errors as pwg_int8_gemv_argmax, plus PWG_ERR_SIZE
 * for the limit. */
int pwg_int8_gemv_argmax_noalloc(const int8_t* table, const float* row_scale,
                                 int64_t rows, int64_t cols,
                                 const float* h, int32_t batch,
                                 int32_t* token_out, float* logits_out,
                                 void* stream);

/* Embedding-row gather (page section "The file is not the traffic": only the
 * selected input rows are read):
 *     rows_out[i, :] = table[ids[i], :]; scales_out[i] = row_scale[ids[i]];
 *     deq_out[i, k] = float32(table[ids[i], k] * row_scale[ids[i]])
 *   table        device, int8 rows x cols;  row_scale device float32[rows]
 *   ids          device, int32[n]
 *   rows_out     device, int8[n][cols];  scales_out device float32[n]
 *   deq_out      device float32[n][cols] or NULL
 * An id outside [0, rows) is not dereferenced: its output row is zero and
 * its scale NaN.  n == 0 is a no-op.
 * Errors: PWG_ERR_ARG, PWG_ERR_ALIGN, PWG_ERR_HIP. */
int pwg_embed_gather(const int8_t* table, const float* row_scale,
                     int64_t rows, int64_t cols,
                     const int32_t* ids, int32_t n,
                     int8_t* rows_out, float* scales_out, float* deq_out,
                     void* stream);

/* How a level's input vector is formed when the level starts (chained step).
 * Page "The Neutrino Engine", section "A 104 microsecond floor inside a 694
 * microsecond step": a decoder layer applies its projections to the current
 * activations, so each projection depends on the ones before it.  The pages
 * do not give the operations between projections; these are the pre-norm
 * decoder layer's (RMSNorm with a gain, grouped-query attention taken at the
 * first position of a sequence, SwiGLU, residual adds).
 *
 * With any op other than PWG_INPUT_GIVEN the library WRITES the formed
 * vector to the level's x (float32[cols]), then the level multiplies it;
 * `src`, `resid` and `gamma` are device float32 vectors read during the
 * step, `resid_out` (nullable) receives the residual sum.  In the formulas
 * n = the level's cols:
 *   PWG_INPUT_RMSNORM:        h = resid + src (src NULL: h = resid);
 *                             x = gamma * h / sqrt(mean(h^2) + eps);
 *   PWG_INPUT_EMBED_RMSNORM:  h = the step's dequantised embedding row of
 *                             *token_in (emb_table[id][k] * emb_scale[id]),
 *                             then as RMSNORM; resid and src unused;
 *   PWG_INPUT_ATTN1:          x[i] = src[(i / (head_dim*group))*head_dim + i % head_dim]
 *                             (each of n/head_dim query heads reads the value
 *                             vector of key/value head (i/head_dim)/group:
 *                             attention over one cached position, whose
 *                             softmax weight is 1);
 *   PWG_INPUT_SWIGLU:         x[i] = silu(src[i]) * src[n + i], silu(g) = g / (1 + e^-g)
 *                             (src: the stacked gate|up output, gate first).
 * Buffers may not overlap: x, resid_out, src, resid and gamma are distinct
 * (PWG_ERR_ARG where pointers are equal), and the level's y overlaps none
 * of them over their extents (src: 2n values for SWIGLU, n/group for
 * ATTN1, n otherwise; PWG_ERR_ARG).  Only the ordered schedules
 * (LEVELS, PERSISTENT) at batch 1 take such levels (PWG_ERR_UNSUPPORTED
 * otherwise).  Arithmetic is float32: the mean of squares is a float32 sum,
 * the root and the quotient IEEE float32. */
enum {
  PWG_INPUT_GIVEN = 0,
  PWG_INPUT_RMSNORM = 1,
  PWG_INPUT_EMBED_RMSNORM = 2,
  PWG_INPUT_ATTN1 = 3,
  PWG_INPUT_SWIGLU = 4
};

typedef struct pwg_input {
  int32_t op;            /* PWG_INPUT_* (0: x is used as given) */
  int32_t head_dim;      /* ATTN1: values per head (n % (head_dim*group) == 0) */
  int32_t group;         /* ATTN1: query heads per key/value head */
  float eps;             /* RMSNORM, EMBED_RMSNORM: added to the mean of squares (>= 0) */
  const float* src;      /* RMSNORM (nullable), ATTN1, SWIGLU (2n values) */
  const float* resid;    /* RMSNORM: the residual stream, float32[n] */
  const float* gamma;    /* RMSNORM, EMBED_RMSNORM: the gain, float32[n] */
  float* resid_out;      /* RMSNORM, EMBED_RMSNORM: receives h (nullable) */
} pwg_input;

/* One ternary GEMV level of a decode step (matrices that share an input are
 * stacked by rows: q|k|v and gate|up). */
typedef struct pwg_level {
  const void* w_packed;    /* device, T2 rows x cols (arranged as weight_layout says) */
  const float* row_scale;  /* device, float32[rows] */
  const float* x;          /* device, float32[cols] */
  float* y;                /* device, float32[rows] */
  int64_t rows;
  int64_t cols;
  pwg_input in;            /* how x is formed (zero-filled: x as given) */
} pwg_level;

/* Whole batch-1 decode step over the weights (page section "A 104
 * microsecond floor ...", Fig. 1: one step = embedding row, every layer's
 * projections in decoder order, the output projection and the greedy token):
 *   embedding gather of *token_in -> levels[0 .. n_levels-1] in order ->
 *   int8 output projection of h + argmax -> *token_out.
 * All pointers except `levels` are device pointers; `levels` is a host
 * array: the levels schedule reads it during each call, the stream and
 * persistent schedules and the batched pass read it in pwg_step_plan (their
 * device plan then holds the pointers and shapes).  token_in and token_out may alias (the token then
 * feeds the next step on the device).
 *
 * Batched pass (batch = 4, 8 or 16; page section "The 0.6B model does not get
 * to decide": several drafted tokens scored in one batched forward pass).
 * Schedule STREAM with tiled weights only; every level's cols a multiple of
 * 2048 and hidden a multiple of 1024 (PWG_ERR_UNSUPPORTED otherwise).  Every
 * buffer then holds `batch` rows: x float32[batch][cols], y
 * float32[batch][rows], h float32[batch][hidden], token_in and token_out
 * int32[batch], emb_row_out int8[batch][hidden], emb_scale_out
 * float32[batch], emb_deq_out and logits_out float32[batch][hidden] and
 * [batch][vocab].  The levels take their given inputs (they do not feed one
 * another), each weight byte is read once per pass, and the levels' outputs
 * and tokens are those of pwg_ternary_gemv_tiled and
 * pwg_int8_gemv_argmax_tiled on the same inputs, bit for bit.  token_in and
 * token_out may alias. */
typedef struct pwg_step_desc {
  int32_t n_levels;
  int32_t schedule;              /* PWG_SCHEDULE_* */
  int32_t weight_layout;         /* PWG_LAYOUT_*: of every w_packed and of out_table */
  int32_t batch;                 /* vectors per step: 0 or 1 (batch-1 step), or 4, 8, 16 */
  const pwg_level* levels;       /* host array [n_levels] */
  const int8_t* out_table;       /* int8 vocab x hidden (arranged as weight_layout says) */
  const float* out_scale;        /* float32[vocab] */
  const float* h;                /* float32[hidden] */
  int64_t vocab;
  int64_t hidden;
  const int8_t* emb_table;       /* int8 vocab x hidden, row-major (rows are gathered) */
  const float* emb_scale;        /* float32[vocab] */
  const int32_t* token_in;       /* int32[1] */
  int32_t* token_out;            /* int32[1] */
  int8_t* emb_row_out;           /* int8[hidden] */
  float* emb_scale_out;          /* float32[1] */
  float* emb_deq_out;            /* float32[hidden] or NULL */
  float* logits_out;             /* float32[vocab] or NULL */
  void* workspace;               /* >= pwg_step_workspace_bytes(desc) */
  size_t workspace_bytes;
  pwg_input h_in;                /* how h is formed (zero-filled: h as given); with
                                    another op the library writes h (hidden values) */
} pwg_step_desc;

/* Workspace bytes for a step description (depends on shapes and schedule). */
size_t pwg_step_workspace_bytes(const pwg_step_desc* desc);

/* Prepare the workspace of a step: validates the description and, for the
 * stream and persistent schedules and the batched pass, writes the
 * device-side level table and work split and resets the claim counters,
 * barrier counters and status words.  Synchronous (it waits
 * for its own copies); call it once per set of buffers, outside stream
 * capture, before pwg_decode_step_weights.
 * Errors: PWG_ERR_ARG, PWG_ERR_ALIGN, PWG_ERR_SIZE, PWG_ERR_HIP,
 * PWG_ERR_UNSUPPORTED (a shape or layout the schedule does not take). */
int pwg_step_plan(const pwg_step_desc* desc, void* stream);

/* Enqueue one step on `stream` (capturable; no allocation, no sync).
 * Levels schedule: one kernel per level (and one per formed input), the
 * output projection and the argmax reduction, in decoder order.
 * Stream schedule: a conversion kernel (every level's input and h into
 * matrix-core operands in the workspace), then one kernel with one workgroup
 * per CU; its only waits are inside a workgroup and are bounded (about
 * 0.5 s), after which the kernel records a timeout and ends instead of
 * hanging; pwg_step_status reports it.
 * Persistent schedule: one kernel with one workgroup per CU (all resident at
 * once); the levels run in order, separated by device-wide barriers whose
 * waits are bounded the same way (a timed-out wait ends the kernel and
 * pwg_step_status reports it).  Level outputs, formed inputs and h are
 * written and read at device scope inside the launch.
 * Batched pass: a conversion kernel (operands and embedding rows), then one
 * kernel with one workgroup per CU that claims its work from a counter in the
 * workspace; its waits are inside a workgroup and bounded the same way.
 * The step's workspace is rewritten by every call: calls that overlap on one
 * workspace race. */
int pwg_decode_step_weights(const pwg_step_desc* desc, void* stream);

/* Synchronously reads the step's status word (stream and persistent
 * schedules and batched pass; always PWG_OK for the levels schedule): PWG_ERR_HIP with a
 * message if a bounded wait timed out.  Not for the hot path. */
int pwg_step_status(const pwg_step_desc* desc, void* stream);

/* Level trace of the persistent schedule (page "The Neutrino Engine",
 * section "A 104 microsecond floor inside a 694 microsecond step" and Fig. 1:
 * where a step's time goes between its dependent levels).
 * pwg_step_trace_bytes: bytes of a trace buffer for the description (0 for
 * the other schedules, or where no device is present).
 * pwg_step_set_trace, after pwg_step_plan (synchronous): later calls of
 * pwg_decode_step_weights on this workspace record, for every level and the
 * output projection (index n_levels) and every workgroup, eight uint64
 * stamps of the GPU's 100 MHz real-time counter, laid out
 * [level][workgroup][event]:
 *   0 the control wave starts waiting for the previous level's barrier,
 *   1 the barrier has passed, 2 the level's sources are in LDS, 3 every wave
 *   is past them, 4 the operands are converted, 5 the products are done,
 *   6 the control wave has arrived (its stores complete), 7 unused.
 * Events a level does not reach keep their previous contents.
 * trace: device, 16-byte aligned, >= pwg_step_trace_bytes(desc) bytes; NULL
 * turns tracing off, and so does pwg_step_plan.  Each event adds a store by
 * one thread: tracing lengthens the step it measures.
 * Errors: PWG_ERR_UNSUPPORTED (another schedule), PWG_ERR_ARG (no plan for
 * this description), PWG_ERR_SIZE, PWG_ERR_ALIGN, PWG_ERR_HIP. */
size_t pwg_step_trace_bytes(const pwg_step_desc* desc);
int pwg_step_set_trace(const pwg_step_desc* desc, void* trace, size_t trace_bytes, void* stream);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* pwg_last_error(void);

/* ---------------------------------------------------------------------------
 * Grouped-query decode attention over a bfloat16 key/value cache (one layer,
 * one new token).  Page "The Neutrino Engine", KV-cache section: 8 key/value
 * heads of 128 values per layer, 2 bytes per value for keys and for values;
 * every cached position is read once per token.
 *   out[j*head_dim + d] = sum_t p_jt * V[t][j/group][d],
 *   p_jt = softmax over t of scale * sum_d q[j*head_dim + d] * K[t][j/group][d],
 * for query heads j < n_heads, group = n_heads / n_kv.
 *   k_cache, v_cache: device bfloat16 bit patterns (the upper half of a
 *       float32), position-major [ctx][n_kv][head_dim];
 *   q: device float32[n_heads*head_dim]; out: device float32[n_heads*head_dim];
 *   workspace: device, >= pwg_attention_workspace_bytes(...) bytes (partial
 *       results per range of positions); calls on one workspace must not
 *       overlap.  Two kernels on `stream`.
 * Every pointer is 16-byte aligned (PWG_ERR_ALIGN), none null (PWG_ERR_ARG).
 * Accumulation is float32 (online softmax in base 2, partial results per
 * range of positions merged at the end).  Supported: head_dim 64 or 128 and
 * group 1, 2 or 4 (PWG_ERR_UNSUPPORTED otherwise); ctx >= 1 (PWG_ERR_ARG);
 * scale finite. */
size_t pwg_attention_workspace_bytes(int32_t n_heads, int32_t n_kv, int32_t head_dim, int64_t ctx);
int pwg_gqa_decode_attention(const uint16_t* k_cache, const uint16_t* v_cache, const float* q,
                             int32_t n_heads, int32_t n_kv, int32_t head_dim, int64_t ctx, float scale,
                             float* out, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Acceptance of drafted tokens after a batched verify pass (page "The
 * Neutrino Engine", section "The 0.6B model does not get to decide": the
 * large model scores the drafts in one batched pass and keeps them only while
 * its greedy choice agrees).  Device int32 arrays of at least n_drafts + 1
 * entries: tokens_in[0] = the last accepted token, tokens_in[1..n_drafts] =
 * the drafts (the batched pass's token_in); targets[i] = the large model's
 * greedy token after position i (the batched pass's token_out).  Writes *accepted = k, the largest k <=
 * n_drafts with targets[i] == tokens_in[i+1] for all i < k, and *next_token =
 * targets[k]; the step emits drafts 1..k, then *next_token.  Positions past
 * n_drafts (padding up to the pass's batch) are ignored.  0 <= n_drafts <= 15
 * (PWG_ERR_ARG); pointers 16-byte aligned.  One small kernel on `stream`. */
int pwg_verify_accept(const int32_t* tokens_in, const int32_t* targets, int32_t n_drafts, int32_t* accepted,
                      int32_t* next_token, void* stream);

/* ---------------------------------------------------------------------------
 * Packed-blob header (page "The Neutrino Engine", sections "The same weights
 * take four execution paths" and "What ships": every path reads the same
 * stored values, and a converted pack must match the engine before it is
 * used).  A 64-byte little-endian header that a loader writes in front of a
 * packed payload and checks before use: format version, layout, shape, the
 * payload size and a checksum of the LOGICAL values, FNV-1a 64 (Fowler, Noll,
 * Vo: h = 14695981039346656037, then h = (h ^ byte) * 1099511628211 mod 2^64)
 * over W as int8, row-major.  The 2-bit and base-3 packings of one matrix,
 * stored or arranged for the device, carry the same checksum.  Host
 * functions; the library's kernels take payloads without headers.
 * ------------------------------------------------------------------------- */
#define PWG_BLOB_MAGIC 0x42475750u /* "PWGB" */
#define PWG_BLOB_VERSION 1

enum {
  PWG_BLOB_T2 = 1,        /* T2, row-major (pwg_pack_weights); cols % 64 == 0 */
  PWG_BLOB_T2_TILED = 2,  /* T2 in 16-row x 64-byte tiles (pwg_tile_rows); cols % 256 == 0 */
  PWG_BLOB_B3 = 3,        /* base-3, stored (pwg_pack_weights_b3) */
  PWG_BLOB_B3_TILED = 4   /* base-3, device arrangement (pwg_tile_b3) */
};

typedef struct pwg_blob_header {
  uint32_t magic;          /* PWG_BLOB_MAGIC */
  uint16_t version;        /* PWG_BLOB_VERSION */
  uint16_t layout;         /* PWG_BLOB_* */
  int64_t rows;            /* >= 1 */
  int64_t cols;            /* >= 1, <= PWG_MAX_COLS */
  uint64_t payload_bytes;  /* size of the payload that follows */
  uint64_t logical_fnv1a;  /* FNV-1a 64 of W (int8, row-major, rows * cols bytes) */
  uint64_t header_fnv1a;   /* FNV-1a 64 of the 40 bytes above */
  uint64_t reserved[2];    /* zero */
} pwg_blob_header;

/* Payload bytes of `layout` for rows x cols; 0 for an invalid combination. */
size_t pwg_blob_payload_bytes(int32_t layout, int64_t rows, int64_t cols);

/* Fills *out for the logical matrix w_host (host int8 rows x cols, values in
 * {-1, 0, 1}) in `layout`.  Errors: PWG_ERR_ARG (null, layout / shape),
 * PWG_ERR_VALUE (a value outside {-1, 0, 1}). */
int pwg_blob_header_init(int32_t layout, const int8_t* w_host, int64_t rows, int64_t cols, pwg_blob_header* out);

/* Checks a header without reading the payload: magic, version, header
 * checksum, reserved words, layout and shape, and that its payload size is
 * the layout's and equals payload_bytes.  Errors: PWG_ERR_ARG (null),
 * PWG_ERR_VALUE (a malformed header), PWG_ERR_SIZE (payload size). */
int pwg_blob_header_check(const pwg_blob_header* h, size_t payload_bytes);

/* pwg_blob_header_check, then decodes every weight of the host payload in
 * its layout and compares the logical checksum.  Errors as the check, plus
 * PWG_ERR_ARG (null payload) and PWG_ERR_VALUE (an invalid code, or a
 * payload whose logical values differ from the header's). */
int pwg_blob_verify(const pwg_blob_header* h, const void* payload_host, size_t payload_bytes);

/* PWG_VERSION of the built library. */
int pwg_version(void);

#pragma GCC visibility pop
#ifdef __cplusplus
}
#endif
#endif /* PWG_H */
