// The forward for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// scratch the forward's kernels need (the prefill path's split partial sums
// of H = X A^T, H itself and bf16 s H; the decode path's partial sums of H
// for ranks above the fused limit) lives in a fixed device array owned by
// the library instead of a caller workspace.
//
// The array below is a device symbol: its name in host code is only a
// stand-in, so the device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and that address is what
// reaches the kernels. Each device holds its own copy until the process ends.
#include <mutex>

#include "internal.h"

namespace {

static_assert(QLORA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size is a multiple of its alignment");

static __device__ __align__(256) unsigned char scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call on that device.
qlora_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QLORA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QLORA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return QLORA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight* w, const uint16_t* x, int64_t m,
                                                 const uint16_t* a, const uint16_t* b, int r, float alpha,
                                                 uint16_t* y, float* h_out, hipStream_t stream) {
  // arguments and sizes first: a call that is invalid or does not fit is
  // rejected before the device is touched
  const qlora_status chk = qlora::linear_fwd_check(w, x, m, a, b, r, y, h_out);
  if (chk != QLORA_OK || m == 0) return chk;
  if (qlora::linear_fwd_scratch_bytes(m, w->n, w->k, r) > QLORA_NOALLOC_SCRATCH_BYTES) return QLORA_ERR_WORKSPACE;
  void* ptr = nullptr;
  const qlora_status st = scratch_on_current_device(&ptr);
  if (st != QLORA_OK) return st;
  return qlora::linear_fwd_scratch(w, x, m, a, b, r, alpha, y, h_out, ptr, QLORA_NOALLOC_SCRATCH_BYTES, stream);
}
