// Fixed device workspace of the single launch for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): a file-scope device
// array, its address looked up once per device at set-up, and handed to the kernels like the
// runtime's grown workspace.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "pr_internal.h"

namespace pr {
namespace {

constexpr int kMaxScratchDevices = 64;

// Row-partial slots first (kNoallocSlotWords 64-bit words), then kNoallocSyncWords 32-bit
// words: status bits, finished workgroups, the last launch's epoch, one completion counter
// per tile row.  Every GPU the library runs on holds its own copy until the process ends.  In
// host code this name is only a handle for the symbol lookup, never a device address.
static __device__ __align__(256) unsigned long long
    scratch[kNoallocSlotWords + kNoallocSyncWords / 2];

unsigned long long* g_scratch[kMaxScratchDevices] = {};
std::mutex g_scratch_mu;

__global__ void zero_words_kernel(unsigned long long* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

}  // namespace

int noalloc_setup() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices) return fail(PR_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] != nullptr) return PR_OK;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return fail(PR_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                hipGetErrorString(e));
  // Everything the launches need at zero starts at zero: counters, finished count, epoch (a
  // zero epoch tag matches no launch).  Each launch's last workgroup returns the counters to
  // zero, so later calls need no clearing.
  const size_t n = kNoallocSlotWords + kNoallocSyncWords / 2;
  hipLaunchKernelGGL(zero_words_kernel, dim3(1024), dim3(256), 0, nullptr,
                     static_cast<unsigned long long*>(ptr), n);
  e = hipGetLastError();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess)
    return fail(PR_ERR_HIP, "clearing the fixed workspace on device %d: %s", dev,
                hipGetErrorString(e));
  g_scratch[dev] = static_cast<unsigned long long*>(ptr);
  return PR_OK;
}

int noalloc_workspace(SingleWs* ws) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PR_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  unsigned long long* p = nullptr;
  if (dev >= 0 && dev < kMaxScratchDevices) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev];
  }
  if (p == nullptr)
    return fail(PR_ERR_UNSUPPORTED,
                "the fixed workspace of device %d is not set up: call pr_init() on the device "
                "first", dev);
  ws->slots = p;
  ws->slot_words = kNoallocSlotWords;
  ws->sync = reinterpret_cast<unsigned*>(p + kNoallocSlotWords);
  ws->pwords = nullptr;
  ws->pword_words = 0;
  ws->xbuf = nullptr;
  ws->xbuf_words = 0;
  return PR_OK;
}

}  // namespace pr
