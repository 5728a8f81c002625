// Host-side entry points of the kernels in kernels.hip.
#pragma once
#include <hip/hip_runtime_api.h>

#include "plan.hpp"

namespace purlin {

enum class KernelKind { kCopy, kSumF32, kSumBf16 };

// nt: bit 0 = nontemporal loads, bit 1 = nontemporal stores.
hipError_t launch_zs(const LaunchPlan &p, KernelKind kind, int nt, int grid, hipStream_t stream);
hipError_t launch_staged(const StagedPlan &p, KernelKind kind, int nt, hipStream_t stream);
hipError_t launch_stream_copy(void *dst, const void *src, int64_t bytes, int grid,
                              hipStream_t stream);
hipError_t max_resident_per_cu(KernelKind kind, bool staged, int nt, int *blocks);

}  // namespace purlin
