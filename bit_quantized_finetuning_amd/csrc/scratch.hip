// qlora_forward without a workspace argument, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc), in the weight-streaming regime (T <= 16). The kernel is the same
// as qlora_forward's; only the scratch memory differs: one static device array
// per GPU (the counter region and the tagged exchange of the adapter
// intermediate) instead of the caller's workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is ever handed to
// a kernel.
#include <mutex>

#include "kernels.h"

namespace qlora {
namespace {

static __device__ __align__(256) uint8_t scratch[QLORA_STATIC_SCRATCH_BYTES];


struct DeviceScratch {
  std::once_flag once;
  hipError_t status = hipSuccess;
  void *ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

// Zero the array (a plain fill kernel: no memset node is recorded when the
// first call is being captured into a graph).
__global__ void k_zero_words(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The device address of the current device's array, cleared by a fill kernel
// enqueued on `stream` at the first call on that device.
hipError_t device_scratch(void **out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch &d = g_scratch[dev];
  std::call_once(d.once, [&] {
    void *p = nullptr;
    d.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.status != hipSuccess) return;
    constexpr int n = QLORA_STATIC_SCRATCH_BYTES / 4;
    k_zero_words<<<dim3(n / 256), dim3(256), 0, stream>>>(static_cast<uint32_t *>(p), n);
    d.status = hipGetLastError();
    if (d.status == hipSuccess) d.ptr = p;
  });
  if (d.status != hipSuccess) return d.status;
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace
}  // namespace qlora

using namespace qlora;

extern "C" int qlora_forward_noalloc(const qlora_nf4_weight *W, const uint16_t *x, int64_t T, const uint16_t *A,
                                     const uint16_t *B, int32_t r, float alpha, uint16_t *h, float *u_out,
                                     hipStream_t stream) {
  const int s = validate_forward(W, x, T, A, B, r, h, u_out);
  if (s) return s;
  if (!A && !B) r = 0;
  // the weight-streaming kernel only (its scratch is a few hundred KB)
  if (T > 16 || !gemv_supported(W->d_out, W->d_in, T)) return QLORA_ERR_SCRATCH;
  if (forward_workspace_need(W->d_out, W->d_in, T, r) > (size_t)QLORA_STATIC_SCRATCH_BYTES) return QLORA_ERR_SCRATCH;
  void *ws = nullptr;
  if (device_scratch(&ws, stream) != hipSuccess) return QLORA_ERR_HIP;
  return enqueue_forward(W, x, T, A, B, r, alpha, h, u_out, ws, stream);
}
