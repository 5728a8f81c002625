// Host-side entry points of the kernels in kernels.hip.
#pragma once
#include <hip/hip_runtime_api.h>

#include "plan.hpp"

namespace purlin {

enum class KernelKind { kCopy, kSumF32, kSumBf16 };

// nt: nontemporal loads and stores.  unroll_sel picks one of three unroll
// depths (units in flight per lane and source): copy 4 / 8 / 16, sum 1 / 2 / 4.
// rows = false: the kernel built without the row bodies, for launches whose
// every job has its sources on its destinations' 16-byte phase.  one = true:
// the kernel built for launches whose every job has a single destination
// rank (no broadcast), whose destination loops fold to one store.  wide =
// true: the latency-regime build with the wide element pass (row bodies of
// the default nontemporal form and unroll only; ignored otherwise).  bcast =
// true: a launch with broadcast jobs, whose body stores are plain (same
// forms only).  dstore = true: broadcast jobs stored at device scope (the
// forms dstore_build accepts).
hipError_t launch_zs(const LaunchPlan &p, KernelKind kind, bool nt, int unroll_sel, bool rows,
                     bool one, bool wide, bool bcast, bool dstore, int grid, hipStream_t stream);
hipError_t launch_staged(const StagedPlan &p, KernelKind kind, bool nt, hipStream_t stream);
// The zero-staging build with the LDS-staged aligned body (launches whose
// every job is aligned; one: single-destination jobs; bcast: plain stores).
hipError_t launch_zs_lds(const LaunchPlan &p, KernelKind kind, bool one, bool bcast, int grid,
                         hipStream_t stream);
hipError_t zs_lds_resident_per_cu(KernelKind kind, bool one, bool bcast, int *blocks);
int unroll_of(KernelKind kind, int unroll_sel);
// Whether a launch whose jobs all have one destination rank (single_dst) runs
// the single-destination build (the `one` argument of launch_zs).
bool one_build(KernelKind kind, bool nt, bool rows, bool single_dst);
// Whether a broadcast launch of this form has a build with device-scope
// stores: the default unroll and loads, aligned, or a copy on the wide row
// body.
bool dstore_build(KernelKind kind, bool nt, int unroll_sel, bool rows, bool wide);
hipError_t launch_stream_copy(void *dst, const void *src, int64_t bytes, int grid,
                              hipStream_t stream);
// The bare access pattern of a collective (n_src, n_dst in {0, 1, 8}, not
// both 0): `tile_bytes` per tile (a multiple of 16, below 4 GiB), `unroll`
// units per lane in flight (2, 4 or 8), nontemporal loads (ntl), store mode
// smode (atom::kStorePlain / kStoreNT / kStoreDevice).
hipError_t launch_pattern(const void *const *srcs, int n_src, void *const *dsts, int n_dst,
                          int64_t bytes, int grid, int64_t tile_bytes, int unroll, bool ntl,
                          int smode, hipStream_t stream);
hipError_t max_resident_per_cu(KernelKind kind, bool staged, bool nt, int unroll_sel, bool rows,
                               bool one, bool wide, bool bcast, bool dstore, int *blocks);

// MoE dispatch one row at a time (rows: the build with the realigning row
// bodies), the inverse-map pass, dispatch one token at a time (after the
// inverse pass) and the combine's folding pass.
enum class MoeKernel { kDispatch, kInverse, kDispatchTokens, kCombine };
hipError_t launch_moe(const MoePlan &m, MoeKernel which, bool rows, int grid, hipStream_t stream);
hipError_t moe_resident_per_cu(MoeKernel which, bool rows, int *blocks);

// Strided-row exchange in units of `unit` bytes (16, 8, 4 or 2); plain:
// plain instead of nontemporal stores.
hipError_t launch_strided(const StridedPlan &sp, int unit, bool plain, int grid,
                          hipStream_t stream);
hipError_t strided_resident_per_cu(int unit, bool plain, int *blocks);

}  // namespace purlin
