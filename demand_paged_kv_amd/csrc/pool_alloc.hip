// Physically contiguous device memory for the K/V pools (a deployment helper, not part of
// the boundary path).  The boundary kernels address pool pages at random, and the row
// moves of a compaction run at one of a few speeds set by the physical pages behind the
// pools (on MI355X the slower placements wait longer for DRAM read credits); contiguity
// did not reliably change which speed a placement gets.  The two functions have the
// signatures of a PyTorch pluggable allocator.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "growpage.h"

extern "C" {

void* gp_contiguous_malloc(int64_t size, int32_t device, void* stream) {
  (void)stream;
  if (size <= 0) return nullptr;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != device && hipSetDevice(device) != hipSuccess) return nullptr;
  void* p = nullptr;
  if (hipExtMallocWithFlags(&p, (size_t)size, hipDeviceMallocContiguous) != hipSuccess) p = nullptr;
  if (cur != device) (void)hipSetDevice(cur);
  return p;
}

void gp_contiguous_free(void* ptr, int64_t size, int32_t device, void* stream) {
  (void)size;
  (void)stream;
  if (!ptr) return;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return;
  if (cur != device) (void)hipSetDevice(device);
  (void)hipFree(ptr);
  if (cur != device) (void)hipSetDevice(cur);
}

}  // extern "C"
