// abi_sanitize_stubs.cpp -- host stand-ins for the kernel launchers of
// libquest (the functions quest_launch.h declares), so the C ABI's host code
// (quest_abi.cpp, plan.cpp) can be built with g++ under the address and
// undefined-behaviour sanitizers and driven without a GPU
// (tests/test_abi_sanitize.py).  Each stand-in records that it was reached
// and what it was asked to launch, and returns hipSuccess; nothing is
// dereferenced.  Test infrastructure only.
#include <stdint.h>

#include "quest_launch.h"

extern "C" {
int stub_launches = 0;           // launchers reached since the last reset
int stub_last_batch = -1;        // batch of the last launch
int stub_last_max_k = -1;        // max_k of the last decode / top-k launch
void *stub_last_workspace = nullptr;
}

namespace quest {

static hipError_t reached(int batch, int max_k = -1, void *ws = nullptr) {
  ++stub_launches;
  stub_last_batch = batch;
  stub_last_max_k = max_k;
  stub_last_workspace = ws;
  return hipSuccess;
}

hipError_t launch_append(const Dims &, int batch, const void *, const void *, const int32_t *,
                         const int32_t *, int, const int32_t *, void *, void *, void *,
                         hipStream_t) {
  return reached(batch);
}

hipError_t launch_page_scores(const Dims &, int batch, const void *, const void *,
                              const int32_t *, const int32_t *, int, float *, hipStream_t) {
  return reached(batch);
}

hipError_t launch_append_scores(const Dims &, int batch, const void *, const void *,
                                const void *, const int32_t *, const int32_t *, int,
                                const int32_t *, void *, void *, void *, int, float *,
                                hipStream_t) {
  return reached(batch);
}

hipError_t launch_topk(const Dims &, int batch, const float *, const int32_t *,
                       const int32_t *, int max_k, int, int, int32_t *, int32_t *,
                       hipStream_t) {
  return reached(batch, max_k);
}

hipError_t launch_decode(const Dims &, int batch, const void *, const void *, const void *,
                         const int32_t *, const int32_t *, const int32_t *, const int32_t *,
                         int max_k, float, void *, float *workspace, hipStream_t) {
  return reached(batch, max_k, workspace);
}

hipError_t launch_topk_decode(const Dims &, int batch, const void *, const void *,
                              const void *, const int32_t *, const int32_t *, const float *,
                              const int32_t *, int max_k, int, int, float, int32_t *,
                              int32_t *, void *, float *workspace, hipStream_t) {
  return reached(batch, max_k, workspace);
}

hipError_t launch_decode_step(const Dims &, int batch, const void *, const void *, const void *,
                              const int32_t *, const int32_t *, int, const int32_t *, void *,
                              void *, void *, int, const int32_t *, const int32_t *, int max_k,
                              int, int, float, float *, int32_t *, int32_t *, void *,
                              float *workspace, hipStream_t) {
  return reached(batch, max_k, workspace);
}

// The library's scratch array lives on the device; a host build hands out a
// fixed, never dereferenced address.
hipError_t static_scratch(void **ptr) {
  *ptr = reinterpret_cast<void *>(static_cast<uintptr_t>(0x7f0000000000ull));
  return hipSuccess;
}

}  // namespace quest
