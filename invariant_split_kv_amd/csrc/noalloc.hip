// Workspace of isk_attn_decode_static: a device array of fixed size in the
// library's own code object, for callers that cannot allocate device memory.
// Every GPU the library runs on holds one copy, from the first use of the
// library on that GPU until the process ends; every call on a GPU shares it.

#include <mutex>

#include "isk_internal.hpp"

namespace isk {
namespace {

constexpr size_t kScratchBytes = 64u << 20;   // 64 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device

}  // namespace

size_t static_workspace_bytes() { return kScratchBytes; }

// The array's device address on the current device, looked up once per
// device (each device has its own copy at its own address).  Host code uses
// only this address: the array's name denotes a host-side stand-in.
hipError_t static_workspace(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
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
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace isk
