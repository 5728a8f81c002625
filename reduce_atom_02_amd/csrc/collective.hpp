// Internal interface between the C ABI's collective entry points.
#pragma once
#include <stdint.h>

#include "../../include/purlin.h"

namespace purlin {

// Device memory a call takes its flag block, staging slot flags and staging
// rings from instead of its stream's workspace (the no-allocation entry
// point's fixed scratch array).  Staged plans are shrunk to fit it.
struct FixedWorkspace {
  uint32_t *flags;
  uint64_t *slot_flags;
  int64_t slot_flag_bytes;
  char *ring;
  int64_t ring_bytes;
};

// Fills a FixedWorkspace for the current device.
typedef purlin_status (*FixedWorkspaceFn)(FixedWorkspace *w);

// purlin_collective with fixed == nullptr.  With a fixed workspace (fetched
// through `fixed` once the arguments have been checked) it never allocates,
// and returns PURLIN_ERR_NO_MEMORY when the staged plan the policy fixes
// cannot fit it.
purlin_status collective_impl(const purlin_layout *in, const purlin_layout *out, purlin_op op,
                              purlin_dtype dtype, int P, const int64_t *counts,
                              const int64_t *displs, hipStream_t stream, FixedWorkspaceFn fixed);

// The fixed scratch array's status word on the current device, or nullptr
// while no call on this device has used the array.
uint32_t *scratch_status_word();

}  // namespace purlin
