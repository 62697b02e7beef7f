// ssm_ssd_fwd_noalloc: the Mamba-2 (SSD) forward with its workspace in a static device
// buffer, for callers that cannot allocate (declared in include/ssm_ssd.h).
//
// The buffer is a file-scope __device__ array. In host code its name only stands in for the
// symbol: the device address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is ever passed to a kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "scan_launch.h"
#include "ssm_ssd.h"

namespace {

constexpr int64_t kScratchBytes = SSM_SSD_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (nullptr if the runtime refuses).
// Two threads racing on the first lookup store the same address.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

const ssm::SsdScratch kStatic = {kScratchBytes, &scratch_on_current_device};

}  // namespace

extern "C" {

int ssm_ssd_fwd_noalloc(const void* x, const void* dt, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* dt_bias,
                        const uint8_t* mask, uint32_t flags, void* out, float* final_state,
                        int64_t batch, int64_t nheads, int64_t headdim, int64_t dstate,
                        int64_t seqlen, void* stream) {
  return ssm::ssd_fwd_impl(x, dt, A, B, C, D, z, dt_bias, mask, flags, out, final_state,
                           nullptr, 0, batch, nheads, headdim, dstate, seqlen, stream, &kStatic);
}

}  // extern "C"
