// Forming a level's input vector from earlier outputs (chained decode step).
//
// Page "The Neutrino Engine", section "A 104 microsecond floor inside a 694
// microsecond step": each projection of a decoder layer reads the activations
// the previous one produced.  The operations between projections (RMSNorm
// with a gain, one-position grouped-query attention, SwiGLU, residual adds)
// are the pre-norm decoder layer's; pwg.h defines each op.
//
// form_input() is called by every thread of a workgroup of T threads and
// leaves the formed float32 vector in LDS; store_formed() writes it, and the
// residual sum, to memory.  The ordered step schedules call both: the levels
// schedule from a one-workgroup kernel before the level's GEMV, the
// persistent schedule in every workgroup after the level barrier.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/pwg.h"

namespace pwg {
namespace chain {

struct DevInput {
  int op;
  int head_dim;
  int group;
  float eps;
  const float* src;
  const float* resid;
  const float* gamma;
  float* resid_out;
};

inline DevInput from_abi(const pwg_input& in) {
  return DevInput{in.op, in.head_dim, in.group, in.eps, in.src, in.resid, in.gamma, in.resid_out};
}

// Where the embedding row of the step's token comes from (EMBED_RMSNORM).
struct EmbedSrc {
  const int8_t* table;  // vocab x n, row-major
  const float* scale;
  const int* token_in;
  long vocab;
};

// Residual-stream value h[i] of a norm op (the dequantised embedding entry,
// or resid + src); `row`/`s` describe the embedding row (s = 0: invalid id).
__device__ __forceinline__ float norm_value(const DevInput& in, int i, const int8_t* row, float s) {
  if (in.op == PWG_INPUT_EMBED_RMSNORM) return row ? static_cast<float>(row[i]) * s : 0.f;
  return in.src ? in.resid[i] + in.src[i] : in.resid[i];
}

__device__ __forceinline__ void embed_row(const EmbedSrc& e, int n, const int8_t*& row, float& s) {
  const int id = *e.token_in;
  if (id >= 0 && id < e.vocab) {
    row = e.table + static_cast<long>(id) * n;
    s = e.scale[id];
  } else {
    row = nullptr;  // an invalid id gathers a zero row (as the gather does)
    s = 0.f;
  }
}

// Every thread of the workgroup (T threads) calls this; `v` is LDS
// float[n], `red` LDS float[T / 64 + 1].  On return (after a workgroup
// barrier) v holds the formed input.
template <int T>
__device__ __forceinline__ void form_input(const DevInput& in, int n, float* v, float* red, const EmbedSrc& e) {
  const int tid = threadIdx.x;
  if (in.op == PWG_INPUT_ATTN1) {
    const int span = in.head_dim * in.group;
    for (int i = tid; i < n; i += T) v[i] = in.src[(i / span) * in.head_dim + i % in.head_dim];
    __syncthreads();
    return;
  }
  if (in.op == PWG_INPUT_SWIGLU) {
    for (int i = tid; i < n; i += T) {
      const float g = in.src[i];
      v[i] = g / (1.0f + expf(-g)) * in.src[n + i];
    }
    __syncthreads();
    return;
  }
  // RMSNORM / EMBED_RMSNORM
  const int8_t* row = nullptr;
  float s = 0.f;
  if (in.op == PWG_INPUT_EMBED_RMSNORM) embed_row(e, n, row, s);
  float acc = 0.f;
  for (int i = tid; i < n; i += T) {
    const float h = norm_value(in, i, row, s);
    v[i] = h;
    acc = fmaf(h, h, acc);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
    for (int w = 0; w < T / 64; ++w) sum += red[w];  // fixed order: deterministic
    red[T / 64] = 1.0f / sqrtf(sum / static_cast<float>(n) + in.eps);
  }
  __syncthreads();
  const float inv = red[T / 64];
  for (int i = tid; i < n; i += T) v[i] = in.gamma[i] * v[i] * inv;
  __syncthreads();
}

// Writes the formed input v (LDS) to x and, for the norm ops, h to
// resid_out.  Called by `nt` threads with index t (a whole workgroup, or one
// wave); h is recomputed from its sources, which form_input only read.
__device__ __forceinline__ void store_formed(const DevInput& in, int n, const float* v, float* x, const EmbedSrc& e,
                                             int t, int nt) {
  for (int i = t; i < n; i += nt) x[i] = v[i];
  if ((in.op == PWG_INPUT_RMSNORM || in.op == PWG_INPUT_EMBED_RMSNORM) && in.resid_out) {
    const int8_t* row = nullptr;
    float s = 0.f;
    if (in.op == PWG_INPUT_EMBED_RMSNORM) embed_row(e, n, row, s);
    for (int i = t; i < n; i += nt) in.resid_out[i] = norm_value(in, i, row, s);
  }
}

}  // namespace chain
}  // namespace pwg
