// SNAC device protocol: notify flags, credits, launch epochs and the watchdog.
//
// Purlin's middle layer is Stage, Notify, And Consume (abstract): a producer
// stages a chunk, notifies, and a consumer consumes it.  Here every flag is
// a word in HBM, in the flag block of the stream the launch runs on (each
// stream has its own, so launches on different streams never share a flag).
// Costs on a multi-XCD gfx950 shape the protocol:
//  * an agent-scope acquire invalidates the XCD's L2 and an agent-scope
//    release writes its dirty lines back, so neither may sit inside a spin
//    loop, and the release is the dear one;
//  * a wait therefore polls with relaxed agent-scope loads (which bypass the
//    non-coherent caches) and issues one acquire fence once the value is
//    seen, and only when it is about to read data the flag publishes; a
//    wait for "done reading" (credits, entry) orders later stores only and
//    takes no acquire;
//  * a notify that publishes data ("ready") follows data written with
//    device-scope stores, which are counted as done only once every XCD
//    would read them: each wavefront waits for its store counter, the
//    workgroup meets at a barrier, and a relaxed store of the flag then
//    publishes the chunk (a release store would first write back every
//    dirty line of the XCD's L2, other workgroups' outputs among them, and
//    made a handoff of a 32-256 KiB chunk 1.5-4 times slower); the
//    consumer's acquire fence, a cheap invalidate, keeps it from reading a
//    stale copy;
//  * a notify that only says "I have finished reading" (a credit, the exit
//    count) is a relaxed add issued after every wavefront's loads have
//    returned their data (s_waitcnt 0, then a barrier): once the data is in
//    registers, the writer may overwrite the source.
//
// Launch epochs live in device memory, not in the kernel arguments: every
// workgroup reads the stream's epoch word when it starts, and the last
// workgroup of the launch to count itself out advances it.  Launches on one
// stream run one after another, so each launch that counts its exit sees a
// fresh epoch, including every replay of a captured HIP graph, whose kernel
// arguments are fixed at capture.  Flag values carry the epoch in their high
// bits, so a flag is never reset between launches; a consumer waits for the
// value it expects.
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
__device__ __forceinline__ void store_rlx(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_rlx(uint32_t *p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_rlx(uint64_t *p, uint64_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wavefront of the workgroup has its loads back (and its stores
// acknowledged); call from all threads.  After it, a relaxed notify may say
// "done reading", or publish what the workgroup wrote with device-scope
// stores (publish()).
__device__ __forceinline__ void drain_workgroup() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Ready notify of data the workgroup wrote with device-scope stores, by one
// thread after drain_workgroup(): every such store is then visible on every
// XCD, so the flag needs no release ordering of its own.
__device__ __forceinline__ void publish(uint64_t *p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// This launch's epoch: the stream's epoch word plus one (the block starts
// zeroed, so the first epoch is 1; 0 is never an epoch).  The word changes
// only when the last workgroup of a launch counts itself out, after every
// workgroup of that launch has read it, so all workgroups read one value.
__device__ __forceinline__ uint32_t launch_epoch(const LaunchPlan &p) {
  const uint32_t w = load_rlx(&p.flags[kFlagEpoch]);
  return uint32_t(__builtin_amdgcn_readfirstlane(int(w))) + 1u;
}

__device__ __forceinline__ bool aborted(const LaunchPlan &p, uint32_t e) {
  return load_rlx(&p.flags[kFlagAbort]) == e;
}

__device__ __forceinline__ void raise_timeout(const LaunchPlan &p, uint32_t e) {
  __hip_atomic_fetch_or(&p.flags[kFlagStatus], kStatusTimeout, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
  store_rel(&p.flags[kFlagAbort], e);
}

// Spin until *f - target >= 0 (wrap-aware), then acquire (kAcquire) ;
// false if the watchdog expired or launch e was aborted.  A wait that only
// orders this workgroup's later accesses after another's earlier *reads*
// (a credit-like "done reading" flag) needs no acquire: no store is issued
// before the load that saw the flag has returned.
template <class W, bool kAcquire = true>
__device__ __forceinline__ bool wait_geq(const W *f, W target, const LaunchPlan &p, uint32_t e) {
  using S = typename std::conditional<sizeof(W) == 8, int64_t, int32_t>::type;
  const uint64_t t0 = wall_clock64();
  while (true) {
    if (S(load_rlx(f) - target) >= 0) {
      if (kAcquire) acquire_fence();
      return true;
    }
    if (aborted(p, e)) return false;
    if (wall_clock64() - t0 > p.watchdog_ticks) {
      raise_timeout(p, e);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Entry notify: rank r announces "my input is ready, epoch e" with
// entry[r] = e, and every workgroup waits for the entry flag of every rank
// before its first access.  Workgroup b announces ranks b, b + grid, ...;
// workgroups are dispatched in ascending order, so every waiting workgroup's
// announcers are already running.  The epoch a launch reads was published by
// the last exit of the stream's previous counting launch, so every reader of
// that launch has finished before any rank announces again.  The waits order
// later writes after earlier reads only (the data a collective reads reaches
// it through stream order), so they poll without an acquire: an acquire here
// would invalidate the XCD's L2 once per workgroup and rank, thousands of
// times per launch.
__device__ __forceinline__ bool entry(const LaunchPlan &p, uint32_t e) {
  __shared__ int ok;
  if (threadIdx.x == 0) ok = 1;
  uint32_t *f = p.flags;
  if (threadIdx.x == 0)
    for (int r = blockIdx.x; r < p.P; r += gridDim.x) store_rel(&f[kFlagEntry + r * kFlagStride], e);
  __syncthreads();
  if (int(threadIdx.x) < p.P) {
    if (!wait_geq<uint32_t, false>(&f[kFlagEntry + threadIdx.x * kFlagStride], e, p, e)) ok = 0;
  }
  __syncthreads();
  return ok != 0;
}

// Exit notify: this workgroup has finished reading every input of launch e.
// Workgroup b adds one to counter b % kExitSlots; the workgroup completing a
// counter resets it and adds one to the second-level counter, and the one
// completing that (the launch's last) resets it and advances the stream's
// epoch word, which the next launch reads.  Every add follows the drain, so
// it is issued after this workgroup's epoch read and all its loads have
// returned.  (Outputs reach the next launch through stream order; ranks on
// separate GPUs would need a system-scope release here.)
__device__ __forceinline__ void exit_notify(const LaunchPlan &p, uint32_t e) {
  drain_workgroup();
  if (threadIdx.x == 0) {
    const uint32_t G = gridDim.x;
    const uint32_t s = blockIdx.x % uint32_t(kExitSlots);
    const uint32_t want = G / kExitSlots + (s < G % kExitSlots ? 1u : 0u);
    const uint32_t nslots = G < uint32_t(kExitSlots) ? G : uint32_t(kExitSlots);
    uint32_t *slot = &p.flags[exit_word(int(s))];
    if (__hip_atomic_fetch_add(slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == want) {
      store_rlx(slot, 0u);
      uint32_t *top = &p.flags[kFlagExitTop];
      if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) + 1u == nslots) {
        store_rlx(top, 0u);
        // the word holds the next epoch minus one; after 0xffffffff comes 1
        store_rel(&p.flags[kFlagEpoch], e == 0xffffffffu ? 0u : e);
      }
    }
  }
}

}  // namespace snac
}  // namespace purlin
