// int8 output projection fused with greedy argmax, and the embedding gather.
//
// Page "The Neutrino Engine", section "A 104 microsecond floor inside a 694
// microsecond step": the output projection maps the final hidden state onto
// the whole vocabulary and runs at the DRAM limit; section "The file is not
// the traffic": two untied int8 tables of 151,936 x 4,096, the output table
// scored in full, the input table read only at the selected rows.  Decode is
// greedy (intro), so the step's result is the argmax of the logits.
//
// Stage 1 (one kernel): every wave streams a contiguous range of table rows
// (64 lanes x 16 B = 1 KiB per load instruction, four per 4,096-byte row),
// forms each logit with v_dot4_i32_i8 against five int8 limbs of the hidden
// state rounded to 39-bit fixed point per 16-element chunk (exact integer
// sums per limb and chunk, then float32), keeps a running (max, lowest index),
// and each workgroup writes one 64-bit key.  Stage 2 (one workgroup) reduces
// the keys.  Both stages use a fixed reduction order, so the token is
// reproducible bit for bit.
#include "device_common.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

using namespace dev;

template <int C, int U, int WPB>
__global__ __launch_bounds__(WPB * 64) void int8_gemv_argmax_kernel(const u32x4* __restrict__ table,
                                                                    const float* __restrict__ scale, int rows,
                                                                    int cols, const float* __restrict__ h,
                                                                    float* __restrict__ logits,
                                                                    unsigned long long* __restrict__ partials) {
  extern __shared__ __align__(16) unsigned lds[];
  const int nchunks = cols >> 4;  // 16 int8 per 128-bit chunk
  int* lds_e = reinterpret_cast<int*>(lds + nchunks * kI8ChunkDwords);
  i8_prepare_x(h, cols, lds, lds_e);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned H[C][kI8ChunkDwords];
  int Ec[C];  // -E_c
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int chunk = lane + 64 * c;
    Ec[c] = chunk < nchunks ? -lds_e[chunk] : 0;
    if (chunk < nchunks) {
      const u32x4* src = reinterpret_cast<const u32x4*>(lds + chunk * kI8ChunkDwords);
#pragma unroll
      for (int q = 0; q < kI8Limbs; ++q) {
        const u32x4 v = src[q];
        H[c][4 * q + 0] = v.x; H[c][4 * q + 1] = v.y; H[c][4 * q + 2] = v.z; H[c][4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kI8ChunkDwords; ++q) H[c][q] = 0u;
    }
  }

  const long gw = static_cast<long>(blockIdx.x) * WPB + wave, nw = static_cast<long>(gridDim.x) * WPB;
  const long r0 = gw * rows / nw, r1 = (gw + 1) * rows / nw;

  float best = -__builtin_inff();
  unsigned best_idx = 0xFFFFFFFFu;

  auto load = [&](long r, u32x4 (&Q)[U][C], float (&sv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = r + u < r1;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int chunk = lane + 64 * c;
        Q[u][c] = (valid && chunk < nchunks) ? __builtin_nontemporal_load(table + (r + u) * nchunks + chunk)
                                             : u32x4{0u, 0u, 0u, 0u};
      }
      sv[u] = valid ? scale[r + u] : 0.f;
    }
  };
  auto compute = [&](long r, const u32x4 (&Q)[U][C], const float (&sv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        int a[kI8Limbs];
        const unsigned qd[4] = {Q[u][c].x, Q[u][c].y, Q[u][c].z, Q[u][c].w};
#pragma unroll
        for (int l = 0; l < kI8Limbs; ++l) {
          a[l] = 0;
#pragma unroll
          for (int g = 0; g < 4; ++g) a[l] = dot4(qd[g], H[c][4 * l + g], a[l]);
        }
        // each limb sum is exact in float32 (|a| <= 16*127*128 < 2^24) and so
        // is its scaling; the float32 sum of the scaled limbs rounds
        float p = static_cast<float>(a[kI8Limbs - 1]);
#pragma unroll
        for (int l = kI8Limbs - 2; l >= 0; --l) p = fmaf(p, 256.0f, static_cast<float>(a[l]));
        part += ldexpf(p, Ec[c]);
      }
      const float total = group_sum<64>(part);
      if (r + u < r1) {
        const float logit = sv[u] * total;
        if (logits != nullptr && lane == 0) logits[r + u] = logit;
        if (logit > best) {  // rows ascend within a wave: ties keep the lower index
          best = logit;
          best_idx = static_cast<unsigned>(r + u);
        }
      }
    }
  };

  u32x4 A[U][C], B[U][C];
  float sA[U], sB[U];
  long r = r0;
  if (r < r1) load(r, A, sA);
  while (r < r1) {
    const long rn = r + U;
    if (rn < r1) load(rn, B, sB);
    compute(r, A, sA);
    r = rn;
    if (r >= r1) break;
    const long rnn = r + U;
    if (rnn < r1) load(rnn, A, sA);
    compute(r, B, sB);
    r = rnn;
  }

  // workgroup (max, lowest index) -> one key
  __shared__ unsigned long long wkeys[WPB];
  if (lane == 0) wkeys[wave] = best_idx == 0xFFFFFFFFu ? 0ull : argmax_key(best, best_idx);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long k = 0ull;
    for (int i = 0; i < WPB; ++i) k = wkeys[i] > k ? wkeys[i] : k;
    partials[blockIdx.x] = k;
  }
}

__global__ __launch_bounds__(256) void argmax_reduce_kernel(const unsigned long long* __restrict__ partials, int n,
                                                            int32_t* __restrict__ token) {
  unsigned long long k = 0ull;
  for (int i = threadIdx.x; i < n; i += 256) k = partials[i] > k ? partials[i] : k;
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(k, off, kWave);
    k = o > k ? o : k;
  }
  __shared__ unsigned long long wk[4];
  if ((threadIdx.x & 63) == 0) wk[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = wk[0];
    for (int i = 1; i < 4; ++i) m = wk[i] > m ? wk[i] : m;
    token[0] = static_cast<int32_t>(argmax_key_index(m));
  }
}

// Stage 2 for several vectors: block b reduces vector b's keys.
__global__ __launch_bounds__(256) void argmax_reduce_batch_kernel(const unsigned long long* __restrict__ partials,
                                                                  int n, size_t nparts, int32_t* __restrict__ token) {
  const unsigned long long* pb = partials + static_cast<size_t>(blockIdx.x) * nparts;
  unsigned long long k = 0ull;
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + static_cast<int>(threadIdx.x);
    if (i < n) k = pb[i] > k ? pb[i] : k;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(k, off, kWave);
    k = o > k ? o : k;
  }
  __shared__ unsigned long long wk[4];
  if ((threadIdx.x & 63) == 0) wk[threadIdx.x >> 6] = k;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = wk[0];
    for (int i = 1; i < 4; ++i) m = wk[i] > m ? wk[i] : m;
    token[blockIdx.x] = static_cast<int32_t>(argmax_key_index(m));
  }
}

// One workgroup per id; 16-byte copies; invalid ids give a zero row and NaN.
__global__ __launch_bounds__(256) void embed_gather_kernel(const u32x4* __restrict__ table,
                                                           const float* __restrict__ scale, int rows, int cols,
                                                           const int32_t* __restrict__ ids,
                                                           u32x4* __restrict__ rows_out, float* __restrict__ scales_out,
                                                           float4* __restrict__ deq_out) {
  const int i = blockIdx.x;
  const int id = ids[i];
  const bool ok = id >= 0 && id < rows;
  const int nchunks = cols >> 4;
  const float s = ok ? scale[id] : __builtin_nanf("");
  if (threadIdx.x == 0) scales_out[i] = s;
  for (int c = threadIdx.x; c < nchunks; c += 256) {
    const u32x4 v = ok ? table[static_cast<size_t>(id) * nchunks + c] : u32x4{0u, 0u, 0u, 0u};
    rows_out[static_cast<size_t>(i) * nchunks + c] = v;
    if (deq_out != nullptr) {
      const unsigned wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = ok ? make_float4(static_cast<float>(static_cast<int8_t>(wd[q] & 0xFF)) * s,
                                          static_cast<float>(static_cast<int8_t>((wd[q] >> 8) & 0xFF)) * s,
                                          static_cast<float>(static_cast<int8_t>((wd[q] >> 16) & 0xFF)) * s,
                                          static_cast<float>(static_cast<int8_t>(wd[q] >> 24)) * s)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        deq_out[(static_cast<size_t>(i) * nchunks + c) * 4 + q] = f;
      }
    }
  }
}

struct I8Instance {
  const void* fn;
  int wpb;
  int max_active;
};

template <int C, int U, int WPB>
I8Instance make_i8() {
  return I8Instance{reinterpret_cast<const void*>(&int8_gemv_argmax_kernel<C, U, WPB>), WPB, 0};
}

I8Instance* pick_i8(int cols) {
  static I8Instance c1 = make_i8<1, 4, 16>(), c2 = make_i8<2, 4, 16>(), c4 = make_i8<4, 2, 8>(),
                    c8 = make_i8<8, 1, 8>();
  const int nchunks = cols / 16;
  if (nchunks <= 64) return &c1;
  if (nchunks <= 128) return &c2;
  if (nchunks <= 256) return &c4;
  return &c8;  // cols <= kMaxInt8Cols
}

int cu_count() {
  static int cus = -1;
  if (cus < 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
  }
  return cus;
}

unsigned i8_grid(I8Instance* in, int64_t rows, size_t lds) {
  if (in->max_active == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, in->fn, in->wpb * 64, lds) != hipSuccess || n < 1) n = 1;
    in->max_active = n;
  }
  const long want = (rows + in->wpb - 1) / in->wpb;
  const long cap = static_cast<long>(cu_count()) * in->max_active;
  return static_cast<unsigned>(want < cap ? want : cap);
}

}  // namespace

size_t i8_lds_bytes(int64_t cols) { return static_cast<size_t>(cols / 16) * (kI8ChunkDwords + 1) * 4; }

// Upper bound of stage-1 workgroups for `rows` (the workspace holds one key
// each).  A fixed cap keeps workspace sizes independent of the device.
size_t int8_partials(int64_t rows) {
  constexpr long kCap = 4096;
  return static_cast<size_t>(rows < kCap ? rows : kCap);
}

int launch_int8_gemv_argmax(const int8_t* table, const float* s, int64_t rows, int64_t cols, const float* h,
                            int32_t batch, void* ws, int32_t* token, float* logits, void* stream) {
  if (batch > 1 && i8b_supported(cols, batch)) {
    const size_t nparts = int8_partials(rows);
    auto* parts = static_cast<unsigned long long*>(ws);
    return launch_i8b(table, false, s, rows, cols, h, batch, parts, nparts,
                      static_cast<unsigned char*>(ws) + nparts * sizeof(unsigned long long) * batch, logits, token, stream);
  }
  I8Instance* in = pick_i8(static_cast<int>(cols));
  const size_t lds = i8_lds_bytes(cols);
  unsigned grid = i8_grid(in, rows, lds);
  const size_t nparts = int8_partials(rows);
  if (grid > nparts) grid = static_cast<unsigned>(nparts);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  for (int b = 0; b < batch; ++b) {
    const u32x4* tp = reinterpret_cast<const u32x4*>(table);
    const float* sp = s;
    int r32 = static_cast<int>(rows), c32 = static_cast<int>(cols);
    const float* hb = h + static_cast<size_t>(b) * cols;
    float* lb = logits ? logits + static_cast<size_t>(b) * rows : nullptr;
    unsigned long long* parts = static_cast<unsigned long long*>(ws) + static_cast<size_t>(b) * nparts;
    void* args[] = {&tp, &sp, &r32, &c32, &hb, &lb, &parts};
    hipError_t e = hipLaunchKernel(in->fn, dim3(grid), dim3(in->wpb * 64), args, lds, st);
    if (e != hipSuccess) return fail(PWG_ERR_HIP, "int8_gemv_argmax launch: %s", hipGetErrorString(e));
    int n = static_cast<int>(grid);
    int32_t* tb = token + b;
    void* args2[] = {&parts, &n, &tb};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&argmax_reduce_kernel), dim3(1), dim3(256), args2, 0, st);
    if (e != hipSuccess) return fail(PWG_ERR_HIP, "argmax_reduce launch: %s", hipGetErrorString(e));
  }
  return PWG_OK;
}

int launch_argmax_reduce_batch(const unsigned long long* partials, int n, size_t nparts, int32_t batch, int32_t* token,
                               void* stream) {
  void* args[] = {const_cast<unsigned long long**>(&partials), &n, &nparts, &token};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&argmax_reduce_batch_kernel), dim3(batch), dim3(256),
                                       args, 0, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "argmax_reduce (batch) launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

int launch_embed_gather(const int8_t* table, const float* s, int64_t rows, int64_t cols, const int32_t* ids, int32_t n,
                        int8_t* rows_out, float* scales_out, float* deq_out, void* stream) {
  if (n == 0) return PWG_OK;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(embed_gather_kernel, dim3(n), dim3(256), 0, st, reinterpret_cast<const u32x4*>(table), s,
                     static_cast<int>(rows), static_cast<int>(cols), ids, reinterpret_cast<u32x4*>(rows_out),
                     scales_out, reinterpret_cast<float4*>(deq_out));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "embed_gather launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

}  // namespace pwg
