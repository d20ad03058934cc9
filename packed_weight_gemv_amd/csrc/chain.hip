// Input formation of a chained step on the levels schedule, as a kernel of
// its own: it forms an input vector (RMSNorm with a gain, one-position
// grouped-query attention or SwiGLU, with the residual sum) and writes it to
// its x before the consumer runs (page "The Neutrino Engine", section "A 104
// microsecond floor inside a 694 microsecond step": each projection waits for
// the activations of the one before it).  The levels schedule runs it for the
// output projection's input h; the ternary levels form theirs inside their
// GEMV kernel.
#include "chain_input.h"
#include "device_common.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

constexpr int kChainThreads = 512;  // the persistent kernel's workgroup size: both schedules reduce in one order

// Workgroup b writes elements [b * kChainThreads, (b + 1) * kChainThreads)
// of the formed vector; for a norm it forms all of it (the sum of squares
// needs every element), for the other ops only its own elements.
__global__ __launch_bounds__(kChainThreads) void chain_input_kernel(chain::DevInput in, int n, float* x,
                                                                    chain::EmbedSrc e) {
  extern __shared__ __align__(16) float v[];
  float* red = v + n;
  const int lo = blockIdx.x * kChainThreads, hi = lo + kChainThreads < n ? lo + kChainThreads : n;
  chain::form_input<kChainThreads>(in, n, v, red, e, lo, hi);
  chain::store_formed(in, n, v, x, e, lo, hi, threadIdx.x, kChainThreads);
}

}  // namespace

int launch_chain_input(const pwg_input& in, int64_t n, float* x, const pwg_step_desc* d, void* stream) {
  const chain::DevInput di = chain::from_abi(in);
  const chain::EmbedSrc e{d->emb_table, d->emb_scale, d->token_in, static_cast<long>(d->vocab)};
  const size_t lds = static_cast<size_t>(n) * 4 + (kChainThreads / 64 + 1) * 4;
  const unsigned grid = static_cast<unsigned>((n + kChainThreads - 1) / kChainThreads);
  hipLaunchKernelGGL(chain_input_kernel, dim3(grid), dim3(kChainThreads), lds, reinterpret_cast<hipStream_t>(stream), di,
                     static_cast<int>(n), x, e);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return fail(PWG_ERR_HIP, "chain input launch: %s", hipGetErrorString(err));
  return PWG_OK;
}

}  // namespace pwg
