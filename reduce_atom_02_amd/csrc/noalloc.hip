// The collective entry point that allocates nothing: its flag block, staging
// slot flags and staging rings live in one fixed device array per GPU.
//
// For callers that cannot allocate device memory on the call path (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The array below is a file-scope device variable: in host
// code its name stands for a host-side shadow, not for device memory, so
// host code never passes it to a kernel, a memset or a copy.  Its device
// address is looked up once per device with hipGetSymbolAddress (each GPU
// holds its own copy at its own address) and only that address is used.
#include <hip/hip_runtime.h>

#include <vector>

#include "collective.hpp"
#include "plan.hpp"

namespace purlin {
namespace {

// Layout of the array: the flag block, the staging slot flags (256 bytes per
// slot: 1024 slots), the staging rings.
constexpr int64_t kScratchFlagBytes = 8192;
constexpr int64_t kScratchSlotFlagBytes = int64_t(256) << 10;
constexpr int64_t kScratchRingBytes = int64_t(32) << 20;
constexpr int64_t kScratchBytes = kScratchFlagBytes + kScratchSlotFlagBytes + kScratchRingBytes;
static_assert(int64_t(kFlagWords) * 4 <= kScratchFlagBytes, "flag block fits its region");

}  // namespace

// Zero-initialized when the code object is loaded; every later state is
// restored by the kernels themselves (exit counters are reset by each
// launch's last workgroup, flags carry launch epochs, the status word is
// cleared by purlin_check).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on each device (index = device), looked up
// on the first call on that device.
std::vector<unsigned char *> &scratch_ptrs() {
  static std::vector<unsigned char *> v;
  return v;
}

purlin_status scratch_of_current_device(FixedWorkspace *w) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PURLIN_ERR_HIP;
  auto &ptrs = scratch_ptrs();
  if (int(ptrs.size()) <= dev) ptrs.resize(dev + 1, nullptr);
  if (!ptrs[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PURLIN_ERR_HIP;
    ptrs[dev] = static_cast<unsigned char *>(p);
  }
  unsigned char *base = ptrs[dev];
  w->flags = reinterpret_cast<uint32_t *>(base);
  w->slot_flags = reinterpret_cast<uint64_t *>(base + kScratchFlagBytes);
  w->slot_flag_bytes = kScratchSlotFlagBytes;
  w->ring = reinterpret_cast<char *>(base + kScratchFlagBytes + kScratchSlotFlagBytes);
  w->ring_bytes = kScratchRingBytes;
  return PURLIN_OK;
}

}  // namespace

uint32_t *scratch_status_word() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  auto &ptrs = scratch_ptrs();
  if (int(ptrs.size()) <= dev || !ptrs[dev]) return nullptr;
  return reinterpret_cast<uint32_t *>(ptrs[dev]) + kFlagStatus;
}

}  // namespace purlin

extern "C" PURLIN_API purlin_status purlin_collective_noalloc(
    const purlin_layout *in, const purlin_layout *out, purlin_op op, purlin_dtype dtype, int P,
    const int64_t *counts, const int64_t *displs, hipStream_t stream) {
  return purlin::collective_impl(in, out, op, dtype, P, counts, displs, stream,
                                 purlin::scratch_of_current_device);
}
