// Grouped-query decode attention over a bfloat16 key/value cache.
//
// Page "The Neutrino Engine", KV-cache section: per layer the cache holds 8
// key/value heads of 128 values, 2 bytes each for keys and values, and every
// cached position is read once per generated token, so at long contexts the
// cache, not the weights, is the larger stream.  One call is one layer:
// out_j = sum_t softmax_t(scale * q_j . k_t) v_t for every query head j,
// query head j reading key/value head j / group.
//
// The kernel is an HBM stream over K and V: workgroup (split, kv) takes a
// contiguous range of positions of one key/value head; inside it 16-byte
// lane loads cover 8 values of one position's key (or value) row, HD/8 lanes
// a row, so one wave load reads 64/(HD/8) positions.  Each lane group keeps
// a running maximum, normaliser and weighted value sum per query head of the
// group (online softmax in base 2, the query pre-scaled by scale * log2 e),
// taking U positions per step so the K and V loads of U positions are in
// flight together.  The lane groups are merged through LDS, each workgroup
// writes one partial (maximum, normaliser, sum) per query head to the
// workspace, and a second kernel (one workgroup per query head) merges the
// splits into the output.
#include <cmath>

#include "device_common.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnU = 4;  // positions per lane group per step
constexpr int kMergeBatch = 32;  // split partials loaded together by the merging workgroup
constexpr int kMaxSplits = 512;  // splits per key/value head (workgroups in all <= ~512)

struct AttnArgs {
  const dev::u32x4* k;
  const dev::u32x4* v;
  const float* q;
  float* out;
  float* part;            // [n_heads][splits][HD] weighted sums
  float2* part_ml;        // [n_heads][splits] (maximum, normaliser)
  int n_kv, splits, per;  // positions per split
  long ctx;
  float qscale;           // scale * log2(e)
};

// Sum over the L lanes of a row group (L = 8 or 16, aligned), every lane
// receiving the sum: DPP lane exchanges inside 16-lane rows (xor 1 and xor
// 2 within quads, then mirrors of 8 and of 16 lanes), full-rate VALU
// operands instead of LDS-crossbar shuffles.
template <int L>
__device__ __forceinline__ float row_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row half mirror
  if constexpr (L == 16)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// 2^x for x <= 0 by the hardware instruction alone: a result below 2^-126
// (flushed to zero) weighs less than 2^-126 against the running maximum's 1.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float lo_bf16(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int HD, int G>
__global__ __launch_bounds__(kAttnThreads) void attn_decode_kernel(AttnArgs a) {
  constexpr int L = HD / 8;                   // lanes per row
  static_assert(L == 8 || L == 16, "row sums cover 8 or 16 lanes");
  constexpr int P = 64 / L;                   // rows per wave load
  constexpr int NGR = (kAttnThreads / 64) * P;  // lane groups per workgroup
  __shared__ float sm_ml[NGR][G][2];
  __shared__ float sm_acc[NGR][G][HD];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % L, r = wave * P + lane / L;
  const int split = blockIdx.x, kvh = blockIdx.y;
  const long t0 = static_cast<long>(split) * a.per;
  const long t1 = t0 + a.per < a.ctx ? t0 + a.per : a.ctx;
  const long npos = t1 - t0;

  float q[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) q[g][i] = a.q[(kvh * G + g) * HD + 8 * sub + i] * a.qscale;

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
  }

  const long row_stride = static_cast<long>(a.n_kv) * L;  // uint4 per position
  const long trips = (npos + NGR * kAttnU - 1) / (NGR * kAttnU);  // uniform over the workgroup
  for (long it = 0; it < trips; ++it) {
    dev::u32x4 kw[kAttnU], vw[kAttnU];
    bool valid[kAttnU];
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      const long t = t0 + (it * kAttnU + u) * NGR + r;
      valid[u] = t < t1;
      // positions past the range read row 0 (in bounds) and are discarded
      const long idx = (valid[u] ? t * row_stride : 0) + static_cast<long>(kvh) * L + sub;
      const dev::u32x4 zero = {0u, 0u, 0u, 0u};
      const dev::u32x4 kl = __builtin_nontemporal_load(a.k + idx);
      const dev::u32x4 vl = __builtin_nontemporal_load(a.v + idx);
      kw[u] = valid[u] ? kl : zero;
      vw[u] = valid[u] ? vl : zero;
    }
    float s[G][kAttnU];
#pragma unroll
    for (int u = 0; u < kAttnU; ++u) {
      const unsigned w[4] = {kw[u].x, kw[u].y, kw[u].z, kw[u].w};
      float kf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kf[2 * i] = lo_bf16(w[i]);
        kf[2 * i + 1] = hi_bf16(w[i]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) d = fmaf(q[g][i], kf[i], d);
        d = row_sum<L>(d);
        s[g][u] = valid[u] ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < kAttnU; ++u) mx = fmaxf(mx, s[g][u]);
      const float corr = mx == -INFINITY ? 1.f : fast_exp2(m[g] - mx);
      l[g] *= corr;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] *= corr;
#pragma unroll
      for (int u = 0; u < kAttnU; ++u) {
        const float p = valid[u] ? fast_exp2(s[g][u] - mx) : 0.f;
        l[g] += p;
        const unsigned w[4] = {vw[u].x, vw[u].y, vw[u].z, vw[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[g][2 * i] = fmaf(p, lo_bf16(w[i]), acc[g][2 * i]);
          acc[g][2 * i + 1] = fmaf(p, hi_bf16(w[i]), acc[g][2 * i + 1]);
        }
      }
      m[g] = mx;
    }
  }

  // merge the lane groups of the workgroup
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (sub == 0) {
      sm_ml[r][g][0] = m[g];
      sm_ml[r][g][1] = l[g];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sm_acc[r][g][8 * sub + i] = acc[g][i];
  }
  __syncthreads();
  for (int o = threadIdx.x; o < G * HD; o += kAttnThreads) {
    const int g = o / HD, d = o % HD;
    float M = -INFINITY;
    for (int j = 0; j < NGR; ++j) M = fmaxf(M, sm_ml[j][g][0]);
    float A = 0.f, Z = 0.f;
    for (int j = 0; j < NGR; ++j) {
      const float mj = sm_ml[j][g][0];
      const float w = mj == -INFINITY ? 0.f : exp2f(mj - M);
      A = fmaf(sm_acc[j][g][d], w, A);
      Z = fmaf(sm_ml[j][g][1], w, Z);
    }
    const int head = kvh * G + g;
    a.part[(static_cast<long>(head) * a.splits + split) * HD + d] = A;
    if (d == 0) a.part_ml[static_cast<long>(head) * a.splits + split] = make_float2(M, Z);
  }

}

// Merge of the split partials: workgroup `head`, one thread per value index.
// The partials are complete (stream order after the split kernel).  Each
// round of up to kMergeBatch splits issues every load it needs at once (the
// threads' value sums, and the splits' (maximum, normaliser) pairs shared
// through LDS), so that a round waits for one round trip; a running maximum
// rescales across rounds.
template <int HD>
__global__ __launch_bounds__(HD) void attn_merge_kernel(AttnArgs a) {
  __shared__ float2 sm[kMergeBatch];
  const int head = blockIdx.x, d = threadIdx.x;
  const float2* ml = a.part_ml + static_cast<long>(head) * a.splits;
  const float* pa = a.part + static_cast<long>(head) * a.splits * HD + d;
  float M = -INFINITY, A = 0.f, Z = 0.f;
  for (int j0 = 0; j0 < a.splits; j0 += kMergeBatch) {
    const int nb = a.splits - j0 < kMergeBatch ? a.splits - j0 : kMergeBatch;
    float pv[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) pv[u] = u < nb ? pa[static_cast<long>(j0 + u) * HD] : 0.f;
    for (int u = d; u < kMergeBatch; u += HD) sm[u] = u < nb ? ml[j0 + u] : make_float2(-INFINITY, 0.f);
    __syncthreads();
    float mb = M;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) mb = fmaxf(mb, sm[u].x);
    const float c = M == -INFINITY ? 0.f : exp2f(M - mb);
    A *= c;
    Z *= c;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float2 mz = sm[u];
      const float w = mz.x == -INFINITY ? 0.f : exp2f(mz.x - mb);
      A = fmaf(pv[u], w, A);
      Z = fmaf(mz.y, w, Z);
    }
    M = mb;
    __syncthreads();  // sm is rewritten by the next round
  }
  a.out[head * HD + d] = A / Z;
}

struct Shape {
  int splits, per;
};

Shape split_for(int n_kv, long ctx) {
  // ~128 positions per split at short contexts (two steps of 16 lane
  // groups x 4 positions for heads of 128), at most ~512 workgroups in all
  // at long ones
  long splits = (ctx + 127) / 128;
  const long cap = kMaxSplits / n_kv > 0 ? kMaxSplits / n_kv : 1;
  if (splits > cap) splits = cap;
  if (splits < 1) splits = 1;
  const long per = (ctx + splits - 1) / splits;
  return Shape{static_cast<int>((ctx + per - 1) / per), static_cast<int>(per)};
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

template <int HD, int G>
const void* kernel_for() {
  return reinterpret_cast<const void*>(&attn_decode_kernel<HD, G>);
}

const void* pick(int hd, int g) {
  // group sizes up to 4 (the per-workgroup merge buffer is G * 16 KiB)
  if (hd == 128) {
    if (g == 1) return kernel_for<128, 1>();
    if (g == 2) return kernel_for<128, 2>();
    if (g == 4) return kernel_for<128, 4>();
  } else if (hd == 64) {
    if (g == 1) return kernel_for<64, 1>();
    if (g == 2) return kernel_for<64, 2>();
    if (g == 4) return kernel_for<64, 4>();
  }
  return nullptr;
}

}  // namespace

bool attention_supported(int n_heads, int n_kv, int head_dim) {
  return n_kv >= 1 && n_heads >= n_kv && n_heads % n_kv == 0 && pick(head_dim, n_heads / n_kv) != nullptr;
}

size_t attention_workspace(int n_heads, int n_kv, int head_dim, long ctx) {
  const Shape s = split_for(n_kv, ctx);
  return align256(static_cast<size_t>(n_heads) * s.splits * 8) + static_cast<size_t>(n_heads) * s.splits * head_dim * 4;
}

int launch_attention(const uint16_t* k, const uint16_t* v, const float* q, int n_heads, int n_kv, int head_dim,
                     long ctx, float scale, float* out, void* workspace, void* stream) {
  const Shape s = split_for(n_kv, ctx);
  char* ws = static_cast<char*>(workspace);
  AttnArgs a;
  a.k = reinterpret_cast<const dev::u32x4*>(k);
  a.v = reinterpret_cast<const dev::u32x4*>(v);
  a.q = q;
  a.out = out;
  a.part_ml = reinterpret_cast<float2*>(ws);
  a.part = reinterpret_cast<float*>(ws + align256(static_cast<size_t>(n_heads) * s.splits * 8));
  a.n_kv = n_kv;
  a.splits = s.splits;
  a.per = s.per;
  a.ctx = ctx;
  a.qscale = scale * 1.4426950408889634f;
  void* args[] = {&a};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipLaunchKernel(pick(head_dim, n_heads / n_kv), dim3(s.splits, n_kv), dim3(kAttnThreads), args, 0, st);
  if (e == hipSuccess) {
    const void* merge = head_dim == 128 ? reinterpret_cast<const void*>(&attn_merge_kernel<128>)
                                        : reinterpret_cast<const void*>(&attn_merge_kernel<64>);
    e = hipLaunchKernel(merge, dim3(n_heads), dim3(head_dim), args, 0, st);
  }
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

}  // namespace pwg
