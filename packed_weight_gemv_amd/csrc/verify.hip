// Acceptance of drafted tokens after a batched verify pass, on the device.
//
// Page "The Neutrino Engine", section "The 0.6B model does not get to
// decide": drafted tokens are scored by the large model in one batched
// forward pass and kept only while its own greedy choice agrees, so the
// output equals the large model's greedy decode.  With position 0 fed the
// last accepted token and position i fed draft i, draft i + 1 is accepted
// while targets[i] == tokens_in[i + 1] for every earlier i; the step then
// emits the accepted drafts and targets[k].  One wave: lane i compares
// position i, a ballot finds the first disagreement.
#include "device_common.h"
#include "pwg_internal.h"

namespace pwg {
namespace {

__global__ __launch_bounds__(64) void verify_accept_kernel(const int* __restrict__ tokens_in,
                                                           const int* __restrict__ targets, int n_drafts,
                                                           int* accepted, int* next_token) {
  const int lane = threadIdx.x;
  const bool agree = lane < n_drafts && targets[lane] == tokens_in[lane + 1];
  const unsigned long long ok = __ballot(agree);
  // k = number of leading agreeing positions (the first zero bit of ok)
  const int k = static_cast<int>(__builtin_ctzll(~ok));
  if (lane == 0) {
    const int kk = k < n_drafts ? k : n_drafts;
    *accepted = kk;
    *next_token = targets[kk];
  }
}

}  // namespace

int launch_verify_accept(const int32_t* tokens_in, const int32_t* targets, int32_t n_drafts, int32_t* accepted,
                         int32_t* next_token, void* stream) {
  hipLaunchKernelGGL(verify_accept_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), tokens_in,
                     targets, n_drafts, accepted, next_token);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "verify accept launch: %s", hipGetErrorString(e));
  return PWG_OK;
}

}  // namespace pwg
