// static_scratch.hip -- the library-owned scratch buffer of the entry point
// that allocates nothing (quest_decode_step_noalloc): a file-scope device
// array holding the decode's split partials, so a caller that cannot
// allocate device memory (graph capture, tight serving loops) needs no
// workspace.  Each GPU holds its own copy of the array from the library's
// load until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept; kernels receive that address, never the name.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "quest.h"
#include "quest_launch.h"

namespace quest {

static_assert(QUEST_STATIC_SCRATCH_BYTES % 256 == 0, "whole 256-byte lines");

namespace {

static __device__ __align__(256) float scratch[QUEST_STATIC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_lookup;

}  // namespace

hipError_t static_scratch(void **ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace quest
