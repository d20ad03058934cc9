// pwg_int8_gemv_argmax without a caller-provided workspace and without any
// allocation: its scratch (the per-workgroup (max, index) keys of every
// vector and, for batch 4, 8, 16, the matrix-core operands of h) lives in a
// fixed device array of this library, one per GPU, held until the process
// ends.  For callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
#include <hip/hip_runtime.h>

#include <mutex>

#include "pwg_internal.h"

namespace pwg {
namespace {

constexpr size_t kScratchBytes = size_t{1} << 20;  // 1 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device; in host code the array's name is not a device address).
int scratch_ptr(void** out, const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PWG_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PWG_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PWG_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array: %s", fn, hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return PWG_OK;
}

}  // namespace

}  // namespace pwg

using namespace pwg;

extern "C" int pwg_int8_gemv_argmax_noalloc(const int8_t* table, const float* row_scale, int64_t rows, int64_t cols,
                                           const float* h, int32_t batch, int32_t* token_out, float* logits_out,
                                           void* stream) {
  const char* fn = "pwg_int8_gemv_argmax_noalloc";
  if (!valid_batch(batch)) return fail(PWG_ERR_ARG, "%s: batch must be 1, 4, 8 or 16 (got %d)", fn, batch);
  if (rows < 1) return fail(PWG_ERR_ARG, "%s: rows must be >= 1", fn);
  const size_t need = pwg_argmax_workspace_bytes(rows, batch);
  if (need > kScratchBytes)
    return fail(PWG_ERR_SIZE,
                "%s: %lld rows at batch %d need %zu bytes of scratch; the fixed scratch array holds %zu (use "
                "pwg_int8_gemv_argmax with a workspace)",
                fn, static_cast<long long>(rows), batch, need, kScratchBytes);
  void* ws = nullptr;
  TRY(scratch_ptr(&ws, fn));
  return pwg_int8_gemv_argmax(table, row_scale, rows, cols, h, batch, ws, need, token_out, logits_out, stream);
}
