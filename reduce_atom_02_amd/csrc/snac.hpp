// SNAC device protocol: notify flags, credits and the watchdog.
//
// Purlin's middle layer is Stage, Notify, And Consume (abstract): a producer
// stages a chunk, notifies, and a consumer consumes it.  Here every flag is
// a word in HBM.  Costs on a multi-XCD gfx950 shape the protocol:
//  * an agent-scope acquire invalidates the XCD's L2 and an agent-scope
//    release writes it back, so neither may sit inside a spin loop;
//  * a wait therefore polls with relaxed agent-scope loads (which bypass the
//    non-coherent caches) and issues one acquire fence once the value is
//    seen, and only when it is about to read data the flag publishes; a
//    wait for "done reading" (credits, exit counts, entry) orders later
//    stores only and takes no acquire;
//  * a notify that publishes data ("ready") is a release store, so the
//    chunk written by one workgroup is visible on every XCD;
//  * a notify that only says "I have finished reading" (a credit, the exit
//    count) is a relaxed add issued after every wavefront's loads have
//    returned their data (s_waitcnt 0, then a barrier): once the data is in
//    registers, the writer may overwrite the source.
// Flag values carry the launch epoch in their high bits, so a flag is never
// reset between launches; a consumer waits for the value it expects.
//
// Every wait is bounded by a wall-clock watchdog.  On expiry the workgroup
// sets the device status word and the launch's abort epoch; every other
// wait of the same launch then gives up at once, so each wavefront exits
// and the host reads PURLIN_ERR_TIMEOUT from purlin_check.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace purlin {
namespace snac {

__device__ __forceinline__ uint32_t load_rlx(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_rlx(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void acquire_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void store_rel(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_rel(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_rlx(uint32_t *p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_rlx(uint64_t *p, uint64_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wavefront of the workgroup has its loads back (and its stores
// acknowledged); call from all threads.  After it, a relaxed notify may say
// "done reading".
__device__ __forceinline__ void drain_workgroup() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

__device__ __forceinline__ bool aborted(const LaunchPlan &p) {
  return __hip_atomic_load(&p.flags[kFlagAbort], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
         p.epoch;
}

__device__ __forceinline__ void raise_timeout(const LaunchPlan &p) {
  __hip_atomic_fetch_or(&p.flags[kFlagStatus], kStatusTimeout, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p.flags[kFlagAbort], p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Spin until *f - target >= 0 (wrap-aware), then acquire (kAcquire) ;
// false if the watchdog expired or the launch was aborted.  A wait that only
// orders this workgroup's later accesses after another's earlier *reads*
// (a credit-like "done reading" flag) needs no acquire: no store is issued
// before the load that saw the flag has returned.
template <class W, bool kAcquire = true>
__device__ __forceinline__ bool wait_geq(const W *f, W target, const LaunchPlan &p) {
  using S = typename std::conditional<sizeof(W) == 8, int64_t, int32_t>::type;
  const uint64_t t0 = wall_clock64();
  while (true) {
    if (S(load_rlx(f) - target) >= 0) {
      if (kAcquire) acquire_fence();
      return true;
    }
    if (aborted(p)) return false;
    if (wall_clock64() - t0 > p.watchdog_ticks) {
      raise_timeout(p);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Entry notify: rank r may let peers read its input and write its output
// once every reader of the previous collective is done (its exit counters),
// and announces that with entry[r] = epoch.  Every workgroup then waits for
// the entry flag of every rank before its first access.  Workgroup b
// announces ranks b, b + grid, ...; all workgroups are resident at once (the
// grid never exceeds what the device holds), so the announcements always
// happen.  Both waits order later writes after earlier reads only (the data
// a collective reads reaches it through stream order), so they poll without
// an acquire: an acquire here would invalidate the XCD's L2 once per
// workgroup and rank, thousands of times per launch.
__device__ __forceinline__ bool entry(const LaunchPlan &p) {
  __shared__ int ok;
  if (threadIdx.x == 0) ok = 1;
  __syncthreads();
  uint32_t *f = p.flags;
  const bool announcer = int(blockIdx.x) < p.P;
  if (announcer && int(threadIdx.x) < kExitSlots) {
    const uint32_t prev = (p.epoch - 1u) & 1u;
    if (!wait_geq<uint32_t, false>(&f[exit_word(prev, threadIdx.x)], p.exit_expect[threadIdx.x], p))
      ok = 0;
  }
  __syncthreads();
  if (announcer && threadIdx.x == 0 && ok) {
    for (int r = blockIdx.x; r < p.P; r += gridDim.x) store_rel(&f[kFlagEntry + r * kFlagStride], p.epoch);
  }
  __syncthreads();
  if (int(threadIdx.x) < p.P && ok) {
    if (!wait_geq<uint32_t, false>(&f[kFlagEntry + threadIdx.x * kFlagStride], p.epoch, p)) ok = 0;
  }
  __syncthreads();
  return ok != 0;
}

// Exit notify: this workgroup has finished reading every input of this
// launch.  (Its outputs reach the next launch through stream order; ranks on
// separate GPUs would need a system-scope release here.)
__device__ __forceinline__ void exit_notify(const LaunchPlan &p) {
  drain_workgroup();
  if (threadIdx.x == 0) add_rlx(&p.flags[exit_word(p.epoch & 1u, blockIdx.x % kExitSlots)], 1u);
}

}  // namespace snac
}  // namespace purlin
