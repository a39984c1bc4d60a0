// The whole forward pass for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): ssd_forward with its workspace taken from a fixed device array
// the library owns, one copy per GPU, instead of from the caller or from a
// stream-ordered allocation.
//
// The array is a file-scope __device__ variable. In host code its name is
// only a stand-in (passing it to a kernel would hand the kernel a host
// address), so its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// used afterwards. Every call on a GPU shares that GPU's array and finds it
// as the last call left it: the kernels clear what must start at zero (the
// one-pass kernel's hand-over counters and ticket, the segmented state
// passing's flags, the status record) in their own launches, so no memset is
// enqueued. Calls that overlap in time on one GPU (other streams, other host
// threads) race on the array; callers must order them.
#include "../../include/ssd.h"

#include <mutex>

#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;  // 256 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array; looked up on the
// first call on each device.
hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace ssd

extern "C" ssd_status_t ssd_forward_noalloc(const ssd_desc_t* desc, const void* x, const float* dt, const float* A,
                                            const void* B, const void* C, const float* D, const float* init_state,
                                            void* y, float* final_state, void* stream) {
  size_t need = 0;
  const ssd_status_t st = ssd_workspace_bytes(desc, &need);  // validates the descriptor
  if (st != SSD_OK) return st;
  if (need > ssd::kScratchBytes) return SSD_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (ssd::scratch_for_current_device(&ws) != hipSuccess) return SSD_ERR_HIP;
  // a workspace is given, so ssd_forward allocates nothing
  return ssd_forward(desc, x, dt, A, B, C, D, init_state, y, final_state, ws, ssd::kScratchBytes, stream);
}
