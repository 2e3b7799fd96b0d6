// Static device scratch for the entry point that allocates nothing
// (nc_attn_fwd_noalloc): callers under HIP graph capture, tight serving loops,
// or harnesses that forbid hipMalloc pass only their inputs and outputs, and
// the forward's workspace (the (cos, sin) table, k', slice partials) lives in
// this array instead.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, from module load until the process ends. Its name on
// the host is only a stand-in for the symbol, never a device address: the
// address is looked up with hipGetSymbolAddress once per device (with that
// device current) and kept per device; every use goes through that pointer.
// Calls that overlap in time on one GPU share the array and so race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

static constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

namespace nc {

size_t scratch_capacity() { return kScratchBytes; }

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace nc
