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
// residual sum, to memory.  The levels schedule calls both: every workgroup
// of a level's GEMV kernel forms the level's whole input, and a small kernel
// (chain.hip) forms the output projection's.  The persistent schedule forms
// its inputs with its own routines on the descriptors declared here.
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

// A load of a value another workgroup of the same launch may have written:
// kCoherent reads it at device scope (past this XCD's L2, which may hold a
// stale line), so the kernel needs no cache invalidation.
template <bool kCoherent>
__device__ __forceinline__ float ld(const float* p) {
  if (kCoherent) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

// Residual-stream value h[i] of a norm op (the dequantised embedding entry,
// or resid + src); `row`/`s` describe the embedding row (s = 0: invalid id).
template <bool kCoherent = false>
__device__ __forceinline__ float norm_value(const DevInput& in, int i, const int8_t* row, float s) {
  if (in.op == PWG_INPUT_EMBED_RMSNORM) return row ? static_cast<float>(row[i]) * s : 0.f;
  return in.src ? ld<kCoherent>(in.resid + i) + ld<kCoherent>(in.src + i) : ld<kCoherent>(in.resid + i);
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
// barrier) v holds the formed input: all of it for the norm ops (whose sum
// of squares needs every element), elements [lo, hi) for the others.  Loads are issued in batches of kU per
// thread before any of them is used, so a batch costs one memory round trip
// (the sources were just written by other CUs and come from HBM).
constexpr int kU = 8;

template <int T, bool kCoherent = false>
__device__ __forceinline__ void form_input(const DevInput& in, int n, float* v, float* red, const EmbedSrc& e,
                                           int lo, int hi) {
  const int tid = threadIdx.x;
  if (in.op == PWG_INPUT_ATTN1) {
    const int span = in.head_dim * in.group;
    for (int base = lo; base < hi; base += kU * T) {
      float a[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * T + tid;
        a[u] = i < hi ? ld<kCoherent>(in.src + (i / span) * in.head_dim + i % in.head_dim) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * T + tid;
        if (i < hi) v[i] = a[u];
      }
    }
    __syncthreads();
    return;
  }
  if (in.op == PWG_INPUT_SWIGLU) {
    for (int base = lo; base < hi; base += kU * T) {
      float g[kU], up[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * T + tid;
        g[u] = i < hi ? ld<kCoherent>(in.src + i) : 0.f;
        up[u] = i < hi ? ld<kCoherent>(in.src + n + i) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * T + tid;
        if (i < hi) {
          // silu(g) = g * sigmoid(g), with sigmoid from e^-|g| in (0, 1]: no
          // overflow for very negative g (g / (1 + e^-g) would give 0 there)
          const float gv = g[u], ez = expf(-fabsf(gv));
          const float sig = gv >= 0.f ? 1.0f / (1.0f + ez) : ez / (1.0f + ez);
          v[i] = gv * sig * up[u];
        }
      }
    }
    __syncthreads();
    return;
  }
  // RMSNORM / EMBED_RMSNORM: v holds gamma * h until the sum of squares of
  // h is known, then the product is scaled by 1 / sqrt(mean + eps).
  const int8_t* row = nullptr;
  float s = 0.f;
  if (in.op == PWG_INPUT_EMBED_RMSNORM) embed_row(e, n, row, s);
  float acc = 0.f;
  for (int base = 0; base < n; base += kU * T) {
    float h[kU], gm[kU];
    if (in.op == PWG_INPUT_EMBED_RMSNORM) {
      int q[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * T + tid;
        q[u] = (i < n && row) ? static_cast<int>(row[i]) : 0;
        gm[u] = i < n ? in.gamma[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) h[u] = static_cast<float>(q[u]) * s;
    } else if (in.src) {
      float r[kU], a[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * T + tid;
        r[u] = i < n ? ld<kCoherent>(in.resid + i) : 0.f;
        a[u] = i < n ? ld<kCoherent>(in.src + i) : 0.f;
        gm[u] = i < n ? in.gamma[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) h[u] = r[u] + a[u];
    } else {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int i = base + u * T + tid;
        h[u] = i < n ? ld<kCoherent>(in.resid + i) : 0.f;
        gm[u] = i < n ? in.gamma[i] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * T + tid;
      if (i < n) v[i] = gm[u] * h[u];
      acc = fmaf(h[u], h[u], acc);  // lanes past the end add 0
    }
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
  for (int i = tid; i < n; i += T) v[i] *= inv;
  __syncthreads();
}

// Writes elements [lo, hi) of the formed input v (LDS) to x and, for the
// norm ops, of h to resid_out.  Called by `nt` threads with index t; h is
// recomputed from its sources (form_input only read them), with each
// thread's loads of a batch issued before its stores.
// kCoherent: agent-scope stores that reach memory past this XCD's L2, for a
// kernel whose other workgroups read the residual sum later in the same launch.
template <bool kCoherent = false>
__device__ __forceinline__ void store_formed(const DevInput& in, int n, const float* v, float* x, const EmbedSrc& e,
                                             int lo, int hi, int t, int nt) {
  const bool norm = (in.op == PWG_INPUT_RMSNORM || in.op == PWG_INPUT_EMBED_RMSNORM) && in.resid_out;
  const int8_t* row = nullptr;
  float s = 0.f;
  if (norm && in.op == PWG_INPUT_EMBED_RMSNORM) embed_row(e, n, row, s);
  for (int base = lo; base < hi; base += kU * nt) {
    float h[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * nt + t;
      h[u] = (norm && i < hi) ? norm_value<kCoherent>(in, i, row, s) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = base + u * nt + t;
      if (i < hi) {
        if (kCoherent) {
          __hip_atomic_store(&x[i], v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (norm) __hip_atomic_store(&in.resid_out[i], h[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          x[i] = v[i];
          if (norm) in.resid_out[i] = h[u];
        }
      }
    }
  }
}

}  // namespace chain
}  // namespace pwg
