// The collective kernels: zero-staging (ZS) and staged SNAC pipelines built
// from the Atom copy / reduce tiles, plus the plain streaming copy used to
// calibrate HBM counters.
#include <hip/hip_runtime.h>

#include "atom.hpp"
#include "kernels.hpp"
#include "snac.hpp"

namespace purlin {

// Where a read-only pattern's folded loads go, so that they are not dead:
// written only when the fold hits one value.  External linkage: a global
// no code could read would let the compiler drop the store and every load.
__device__ atom::u32x4 g_pattern_sink;

namespace {

__device__ __forceinline__ void job_srcs(const LaunchPlan &p, const Job &jb, atom::Srcs &s) {
  if (jb.src < 0) {
    s.n = p.P;
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i)
      s.a[i] = uint64_t(p.in[i < p.P ? i : 0]) + uint64_t(jb.src_off);
  } else {
    s.n = 1;
    const uint64_t a = uint64_t(p.in[jb.src]) + uint64_t(jb.src_off);
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) s.a[i] = a;
  }
}

// Index of the job holding tile t: the last j with tile_begin[j] <= t
// (binary search over the prefix table, so a workgroup far down the list
// does not walk it one dependent load at a time).
__device__ __forceinline__ int job_of_tile(const LaunchPlan &p, int t) {
  int lo = 0, hi = p.njobs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (p.tile_begin[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Job byte range of tile tl (of ntl) of a job of n bytes whose lines follow
// address ref (its first destination byte, or atom::line_ref): tile 0 also
// takes the bytes before the first 128-byte boundary, so every later tile
// starts on a line.
__device__ __forceinline__ void tile_bounds(uint64_t ref, int64_t n, int64_t C, int tl, int ntl,
                                            int64_t &x0, int64_t &x1) {
  int64_t h = int64_t((128u - uint32_t(ref & 127u)) & 127u);
  if (h > n) h = n;
  x0 = tl == 0 ? 0 : h + int64_t(tl) * C;
  x1 = tl == ntl - 1 ? n : h + int64_t(tl + 1) * C;
  if (x0 > n) x0 = n;
  if (x1 > n) x1 = n;
}

// ---- zero staging --------------------------------------------------------
// The zero-staging variant has no staging step (Figure 10 caption): every
// workgroup reads the inputs of all ranks directly and writes each result
// unit straight from registers to every destination (Figure 6: the reduced
// chunk of piece k reaches all ranks without a second pass).  Tiles are dealt to a resident
// grid in grid-stride order; the tile list holds the share of rank 0, then
// rank 1, and so on.
// kWide: the build for the latency regime, whose small misaligned tiles may
// take the wide element pass; the others leave that pass out, whose
// registers would cost a row-body kernel a workgroup per CU.
template <class Op, int kU, bool kNTL, int kNTS, bool kRows, bool kOne, bool kWide = false>
__global__ void __launch_bounds__(kThreads) zs_kernel(const LaunchPlan p) {
  // With the handshake on, a workgroup whose entry wait failed skips its
  // tiles but still counts itself out, so the stream's epoch advances.
  uint32_t e = 0;
  bool run = true;
  if (p.sync) {
    e = snac::launch_epoch(p);
    run = snac::entry(p, e);
  }
  int t = run ? int(blockIdx.x) : p.total_tiles;
  int j = t < p.total_tiles ? job_of_tile(p, t) : 0;
  for (; t < p.total_tiles; t += gridDim.x) {
    if (t >= p.tile_begin[j + 1]) j = job_of_tile(p, t);
    const Job jb = p.jobs[j];
    atom::Srcs s;
    job_srcs(p, jb, s);
    atom::Dsts d;
    // kOne: built for launches whose every job has one destination rank, so
    // every destination loop below folds to a single store
    if (kOne && jb.dst < 0) continue;
    if (!kOne && jb.dst < 0) {
      d.n = p.P;
#pragma unroll
      for (int k = 0; k < kMaxRanks; ++k)
        d.b[k] = uint64_t(p.out[k < p.P ? k : 0]) + uint64_t(jb.dst_off);
    } else {
      d.n = 1;
#pragma unroll
      for (int k = 0; k < kMaxRanks; ++k) d.b[k] = uint64_t(p.out[jb.dst]) + uint64_t(jb.dst_off);
    }
    d.b[kMaxRanks] = d.b[0];
    int64_t x0, x1;
    tile_bounds(atom::line_ref<Op>(s, d, p.shift_stores != 0), jb.nbytes, p.chunk_bytes,
                t - p.tile_begin[j], p.tile_begin[j + 1] - p.tile_begin[j], x0, x1);
    atom::tile<Op, kU, kNTL, true, kRows, kOne, kWide, kNTS>(s, d, x0, x1, p.nt_any_phase != 0,
                                                  p.wide_max, p.shift_stores != 0, nullptr,
                                                  p.unaligned_loads != 0, p.shift_stores == 2);
  }
  if (p.sync) snac::exit_notify(p, e);
}

// The zero-staging kernel for launches whose every job is aligned, with the
// LDS-staged body (kLdsRows rows of 64 units per wavefront and batch): an
// experimental build, selected with PURLIN_LDS=1.
template <class Op, int kU, bool kNTS, bool kOne, int kLdsRows>
__global__ void __launch_bounds__(kThreads) zs_lds_kernel(const LaunchPlan p) {
  constexpr int kS = Op::kSum ? kMaxRanks : 1;
  constexpr int kSlice = kS * kLdsRows * 64;  // 16-byte units per wavefront
  __shared__ atom::u32x4 lds[4 * kSlice];
  atom::lds_u32x4 *slice =
      (atom::lds_u32x4 *)(&lds[0]) + int(__builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6))) * kSlice;
  uint32_t e = 0;
  bool run = true;
  if (p.sync) {
    e = snac::launch_epoch(p);
    run = snac::entry(p, e);
  }
  int t = run ? int(blockIdx.x) : p.total_tiles;
  int j = t < p.total_tiles ? job_of_tile(p, t) : 0;
  for (; t < p.total_tiles; t += gridDim.x) {
    if (t >= p.tile_begin[j + 1]) j = job_of_tile(p, t);
    const Job jb = p.jobs[j];
    atom::Srcs s;
    job_srcs(p, jb, s);
    atom::Dsts d;
    if (kOne && jb.dst < 0) continue;
    if (!kOne && jb.dst < 0) {
      d.n = p.P;
#pragma unroll
      for (int k = 0; k < kMaxRanks; ++k)
        d.b[k] = uint64_t(p.out[k < p.P ? k : 0]) + uint64_t(jb.dst_off);
    } else {
      d.n = 1;
#pragma unroll
      for (int k = 0; k < kMaxRanks; ++k) d.b[k] = uint64_t(p.out[jb.dst]) + uint64_t(jb.dst_off);
    }
    d.b[kMaxRanks] = d.b[0];
    int64_t x0, x1;
    tile_bounds(d.b[0], jb.nbytes, p.chunk_bytes, t - p.tile_begin[j],
                p.tile_begin[j + 1] - p.tile_begin[j], x0, x1);
    atom::tile<Op, kU, true, true, false, kOne, false, kNTS, kLdsRows>(
        s, d, x0, x1, p.nt_any_phase != 0, 0, false, slice);
  }
  if (p.sync) snac::exit_notify(p, e);
}

// ---- staged SNAC pipeline --------------------------------------------------
// Each job runs on `lanes` parallel pipelines; chunk c goes to lane c % lanes.
// Per lane the job has three kinds of workgroup, numbered in this order (so
// that the dispatcher, which starts workgroups in ascending order, starts a
// chunk's producers before its consumers, and every job's workgroups are
// contiguous: the jobs before the one being dispatched are wholly resident
// and finish without it, whatever else occupies the device):
//   stager   (one per source rank other than the owner) copies its rank's
//            chunk into a ring slot, then notifies (Stage, Notify).
//   owner    combines chunk c: its own rank's input read directly, every other
//            source taken from that source's staging ring after its ready
//            notify, in ascending rank; writes the owner's output and, when
//            other ranks need the result, stages it in the scatter ring.  A
//            reduction has a team of owners per lane, each combining its own
//            slice of the chunk (whole 128-byte lines of the destination), so
//            that the owners, who read every source, keep pace with the
//            stagers, who copy one; each owner notifies on its own ready word
//            and returns its own credit to every stager.
//   scatter  (one per destination rank other than the owner) waits for the
//            owner's notify and copies the slot into its rank's output
//            (Consume), then returns a credit for the slot.
// A ring has `depth` slots; a producer reuses a slot only after its consumers'
// credits for the previous round arrived.  No workgroup touches another
// rank's input or output buffer: cross-rank bytes travel through the rings.
// Producers write slots with device-scope stores, so a ready notify is a
// drain and a relaxed flag store, and a consumer's acquire is an L2
// invalidate only; with that, chunks of 32-64 KiB on many lanes are the
// fastest shape (the ring then stays small).
struct SlotRef {
  uint64_t data;
  uint64_t *ready;
  uint64_t *credit;
};

__device__ __forceinline__ SlotRef slot_ref(const StagedPlan &sp, int ring, int slot) {
  const int64_t g = int64_t(ring) * sp.depth + slot;
  SlotRef r;
  r.data = uint64_t(sp.ring) + uint64_t(g * sp.slot_stride);
  r.ready = sp.slot_flags + g * 32;        // + t for owner t of a team
  r.credit = sp.slot_flags + g * 32 + 16;
  return r;
}

// Base address such that job byte x of chunk [x0, x1) lands at base + x,
// keeping the destination's phase modulo 128 inside the slot.
__device__ __forceinline__ uint64_t slot_base(uint64_t slot, uint64_t b0, int64_t x0) {
  return slot + ((b0 + uint64_t(x0)) & 127u) - uint64_t(x0);
}

__device__ __forceinline__ uint64_t tag(uint32_t epoch, uint64_t v) {
  return (uint64_t(epoch) << 32) | v;
}

// ---- protocol checks (built with PURLIN_DEBUG_PROTOCOL) ---------------------
// A producer writes, after a slot's data and before its ready notify, a
// header (the launch epoch and the chunk index) and a canary word at byte
// chunk_bytes + 128 of the slot, past every byte a chunk can occupy (the
// data starts at most 127 bytes into the slot); a consumer checks both after
// its wait.  A consumer also checks that the flag it waited for holds exactly
// the value it waited for, and a producer that its credits are exactly the
// round's: with the protocol right, no producer can run a round ahead.  A
// failed check sets the status bit that purlin_check reports as
// PURLIN_ERR_PROTOCOL.
#ifdef PURLIN_DEBUG_PROTOCOL
constexpr bool kCheckProtocol = true;
#else
constexpr bool kCheckProtocol = false;
#endif
constexpr uint64_t kSlotCanary = 0xc0ffee5a5aa5f00dull;

[[maybe_unused]] __device__ __forceinline__ void flag_protocol(const LaunchPlan &p) {
  __hip_atomic_fetch_or(&p.flags[kFlagStatus], kStatusProtocol, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
}

[[maybe_unused]] __device__ __forceinline__ uint64_t *slot_header(const StagedPlan &sp,
                                                                   uint64_t slot_data) {
  return reinterpret_cast<uint64_t *>(slot_data + uint64_t(sp.base.chunk_bytes) + 128u);
}

// thread 0 of a producer, after its drain and before its ready notify
__device__ __forceinline__ void write_header(const StagedPlan &sp, uint64_t slot_data, uint32_t e,
                                             int chunk) {
  if constexpr (kCheckProtocol) {
    uint64_t *h = slot_header(sp, slot_data);
    // device scope, like the slot's data, and done before the notify
    __hip_atomic_store(&h[0], tag(e, uint64_t(chunk) + 1u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&h[1], kSlotCanary, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// thread 0 of a consumer, after its wait (and acquire)
__device__ __forceinline__ void check_header(const StagedPlan &sp, uint64_t slot_data, uint32_t e,
                                             int chunk) {
  if constexpr (kCheckProtocol) {
    const uint64_t *h = slot_header(sp, slot_data);
    if (__hip_atomic_load(&h[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
            tag(e, uint64_t(chunk) + 1u) ||
        __hip_atomic_load(&h[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != kSlotCanary)
      flag_protocol(sp.base);
  }
}

// thread 0, after a wait that saw *f reach `target`: it must not be past it
__device__ __forceinline__ void check_exact(const LaunchPlan &p, const uint64_t *f, uint64_t target) {
  if constexpr (kCheckProtocol)
    if (snac::load_rlx(f) != target) flag_protocol(p);
}

template <class Op, int kU, bool kNTL, bool kNTS>
__global__ void __launch_bounds__(kThreads) staged_kernel(const StagedPlan sp) {
  const LaunchPlan &p = sp.base;
  __shared__ int ok;
  // job of this workgroup: the last j with role_begin[j] <= blockIdx.x
  int j = 0;
  {
    int hi = p.njobs - 1;
    while (j < hi) {
      const int mid = (j + hi + 1) >> 1;
      if (sp.sj[mid].role_begin <= int(blockIdx.x)) j = mid;
      else hi = mid - 1;
    }
  }
  const StagedJob sj = sp.sj[j];
  const Job jb = p.jobs[j];
  const int L = sp.lanes;
  const int r = int(blockIdx.x) - sj.role_begin;
  const int lane = r % L;
  const int team = sj.team;
  const int kind = r / L;  // 0..n_stage-1 stagers, then team owners, then scatter
  const int owner = sj.owner;
  const int rings_per_lane = sj.n_stage + (sj.n_scatter > 0 ? 1 : 0);
  const int ring0 = sj.ring_begin + lane * rings_per_lane;
  const int ntl = p.tile_begin[j + 1] - p.tile_begin[j];
  const int D = sp.depth;
  const uint32_t e = snac::launch_epoch(p);

  // first destination address of the job (alignment reference for the slots)
  const uint64_t b0 =
      uint64_t(p.out[jb.dst < 0 ? 0 : jb.dst]) + uint64_t(jb.dst_off);
  // Entry notify as in the zero-staging kernel; a workgroup whose entry wait
  // failed skips its role but still counts itself out at the end.
  const bool run = !p.sync || snac::entry(p, e);
  if (threadIdx.x == 0) ok = run ? 1 : 0;
  __syncthreads();

  if (!run) {
    // nothing: fall through to the exit count
  } else if (kind < sj.n_stage) {
    // ---------------- stager ----------------
    const int k = kind;
    const int src = jb.src >= 0 ? jb.src : (k < owner ? k : k + 1);
    const int ring = ring0 + k;
    for (int m = 0;; ++m) {
      const int c = lane + L * m;
      if (c >= ntl) break;
      const int slot = m % D;
      const uint64_t round = uint64_t(m / D);
      const SlotRef o = slot_ref(sp, ring, slot);
      if (threadIdx.x == 0) {
        // every owner of the team returns one credit per round
        if (round == 0) {
          __hip_atomic_store(o.credit, tag(e, 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (!snac::wait_geq<uint64_t, false>(o.credit, tag(e, round * uint64_t(team)), p, e)) {
          ok = 0;
        } else {
          check_exact(p, o.credit, tag(e, round * uint64_t(team)));
        }
      }
      __syncthreads();
      if (!ok) break;
      int64_t x0, x1;
      tile_bounds(b0, jb.nbytes, p.chunk_bytes, c, ntl, x0, x1);
      atom::Srcs s;
      s.n = 1;
      const uint64_t a = uint64_t(p.in[src]) + uint64_t(jb.src_off);
#pragma unroll
      for (int i = 0; i < kMaxRanks; ++i) s.a[i] = a;
      atom::Dsts d;
      d.n = 1;
#pragma unroll
      for (int q = 0; q < kMaxRanks + 1; ++q) d.b[q] = slot_base(o.data, b0, x0);
      // the slot is written with device-scope stores
      atom::tile<atom::CopyOp, kU, kNTL, true, true, false, false, atom::kStoreDevice>(s, d, x0, x1);
      // Every wavefront's stores must be acknowledged before thread 0
      // publishes the slot: a workgroup barrier alone does not wait for
      // other wavefronts' global stores (their head and tail element passes
      // run on wavefronts 2 and 3), so the notify could overtake them and
      // the owner read a stale line.
      snac::drain_workgroup();
      if (threadIdx.x == 0) {
        write_header(sp, o.data, e, c);
        const bool withhold = sp.withhold > 0 && ring == 0 && m + 1 == sp.withhold;
        if (!withhold) snac::publish(o.ready, tag(e, round + 1));
      }
    }
  } else if (kind < sj.n_stage + team) {
    // ---------------- owner (member t of the lane's team) ----------------
    const int t = kind - sj.n_stage;
    for (int m = 0;; ++m) {
      const int c = lane + L * m;
      if (c >= ntl) break;
      const int slot = m % D;
      const uint64_t round = uint64_t(m / D);
      int64_t x0, x1;
      tile_bounds(b0, jb.nbytes, p.chunk_bytes, c, ntl, x0, x1);
      // wait for every staged source chunk, and for the scatter slot's credits
      if (threadIdx.x == 0) {
        // relaxed polls, then one acquire for all of them: the chunks were
        // written with device-scope stores and drained before each notify,
        // and the acquire (an invalidate of the XCD's L2) keeps this
        // workgroup from reading a stale copy of any of them
        for (int k = 0; k < sj.n_stage && ok; ++k)
          if (!snac::wait_geq<uint64_t, false>(slot_ref(sp, ring0 + k, slot).ready, tag(e, round + 1), p, e))
            ok = 0;
        if (sj.n_stage > 0 && ok) snac::acquire_fence();
        if (kCheckProtocol && ok) {
          for (int k = 0; k < sj.n_stage; ++k) {
            const SlotRef o = slot_ref(sp, ring0 + k, slot);
            check_exact(p, o.ready, tag(e, round + 1));
            check_header(sp, o.data, e, c);
          }
        }
        if (sj.n_scatter > 0 && ok) {
          const SlotRef o = slot_ref(sp, ring0 + sj.n_stage, slot);
          if (round == 0) {
            __hip_atomic_store(o.credit, tag(e, 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          } else if (!snac::wait_geq<uint64_t, false>(o.credit, tag(e, round * sj.n_scatter), p, e)) {
            ok = 0;
          } else {
            check_exact(p, o.credit, tag(e, round * sj.n_scatter));
          }
        }
      }
      __syncthreads();
      if (!ok) break;
      atom::Srcs s;
      if (jb.src < 0) {
        s.n = p.P;
#pragma unroll
        for (int i = 0; i < kMaxRanks; ++i) {
          const int src = i < p.P ? i : 0;
          if (src == owner) {
            s.a[i] = uint64_t(p.in[owner]) + uint64_t(jb.src_off);
          } else {
            const int k = src < owner ? src : src - 1;
            s.a[i] = slot_base(slot_ref(sp, ring0 + k, slot).data, b0, x0);
          }
        }
      } else {
        s.n = 1;
        const uint64_t a = jb.src == owner
                               ? uint64_t(p.in[owner]) + uint64_t(jb.src_off)
                               : slot_base(slot_ref(sp, ring0, slot).data, b0, x0);
#pragma unroll
        for (int i = 0; i < kMaxRanks; ++i) s.a[i] = a;
      }
      // destinations: the owner's output (when it is one) and the scatter slot
      atom::Dsts d;
      const bool to_own = jb.dst < 0 || jb.dst == owner;
      const uint64_t own = uint64_t(p.out[owner]) + uint64_t(jb.dst_off);
      const uint64_t scat =
          sj.n_scatter > 0 ? slot_base(slot_ref(sp, ring0 + sj.n_stage, slot).data, b0, x0) : own;
      d.n = (to_own ? 1 : 0) + (sj.n_scatter > 0 ? 1 : 0);
      d.b[0] = to_own ? own : scat;
#pragma unroll
      for (int k = 1; k < kMaxRanks + 1; ++k) d.b[k] = scat;
      // this owner's slice: split points on the destination's 128-byte lines
      // (32-bit offsets, made wavefront-uniform again after the division,
      // which the compiler expands on the vector unit: tile bounds held in
      // vector registers would cost the kernel a workgroup per CU)
      int64_t y0 = x0, y1 = x1;
      if (team > 1) {
        const uint32_t len = uint32_t(x1 - x0);  // a tile is at most 64 MiB + 128 bytes
        const uint32_t part = ((len + uint32_t(team) - 1u) / uint32_t(team) + 127u) & ~127u;
        auto split = [&](int q) -> uint32_t {
          if (q == 0) return 0u;
          uint32_t y = uint32_t(q) * part;
          y += (128u - uint32_t((b0 + uint64_t(x0) + y) & 127u)) & 127u;
          return y < len ? y : len;
        };
        const uint32_t a = uint32_t(__builtin_amdgcn_readfirstlane(int(split(t))));
        const uint32_t z = t + 1 == team ? len
                                         : uint32_t(__builtin_amdgcn_readfirstlane(int(split(t + 1))));
        y0 = x0 + int64_t(a);
        y1 = x0 + int64_t(z);
      }
      // device-scope stores: the scatter slot (and the owner's output with it)
      atom::tile<Op, kU, kNTL, false, true, false, false, atom::kStoreDevice>(s, d, y0, y1);
      snac::drain_workgroup();
      if (threadIdx.x == 0) {
        for (int k = 0; k < sj.n_stage; ++k)
          snac::add_rlx(slot_ref(sp, ring0 + k, slot).credit, uint64_t(1));
        if (sj.n_scatter > 0) {
          // the team's last member writes the scatter slot's header
          if (t + 1 == team) write_header(sp, slot_ref(sp, ring0 + sj.n_stage, slot).data, e, c);
          snac::publish(slot_ref(sp, ring0 + sj.n_stage, slot).ready + t, tag(e, round + 1));
        }
      }
    }
  } else {
    // ---------------- scatter consumer ----------------
    const int k = kind - team - sj.n_stage;
    const int dst = k < owner ? k : k + 1;
    const int ring = ring0 + sj.n_stage;
    for (int m = 0;; ++m) {
      const int c = lane + L * m;
      if (c >= ntl) break;
      const int slot = m % D;
      const uint64_t round = uint64_t(m / D);
      const SlotRef o = slot_ref(sp, ring, slot);
      // the chunk is whole once every owner of the team has notified;
      // relaxed polls, then one acquire (as in the owner)
      if (threadIdx.x == 0) {
        for (int q = 0; q < team && ok; ++q)
          if (!snac::wait_geq<uint64_t, false>(o.ready + q, tag(e, round + 1), p, e)) ok = 0;
        if (ok) snac::acquire_fence();
        if (kCheckProtocol && ok) {
          for (int q = 0; q < team; ++q) check_exact(p, o.ready + q, tag(e, round + 1));
          check_header(sp, o.data, e, c);
        }
      }
      __syncthreads();
      if (!ok) break;
      int64_t x0, x1;
      tile_bounds(b0, jb.nbytes, p.chunk_bytes, c, ntl, x0, x1);
      atom::Srcs s;
      s.n = 1;
      const uint64_t a = slot_base(o.data, b0, x0);
#pragma unroll
      for (int i = 0; i < kMaxRanks; ++i) s.a[i] = a;
      atom::Dsts d;
      d.n = 1;
#pragma unroll
      for (int q = 0; q < kMaxRanks + 1; ++q) d.b[q] = uint64_t(p.out[dst]) + uint64_t(jb.dst_off);
      atom::tile<atom::CopyOp, kU, kNTS>(s, d, x0, x1);
      snac::drain_workgroup();
      if (threadIdx.x == 0) snac::add_rlx(o.credit, uint64_t(1));
    }
  }
  snac::exit_notify(p, e);
}

// ---- MoE dispatch / combine --------------------------------------------------
// Expert-parallel dispatch and combine are among the inference call sites of
// Purlin's AllToAll (Table 2).  Here the token permutation is folded into the
// exchange: dispatch reads each send row by its token index (no permuted send
// buffer), and combine reads the returned rows and folds them per token.

__device__ __forceinline__ void flag_bad_arg(const LaunchPlan &p) {
  __hip_atomic_fetch_or(&p.flags[kFlagStatus], kStatusBadArg, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
}

// One row per tile: row k of pair (i, j) is row idx[i][group j + k] of x[i],
// written to row pos_ij + k of y[j]; an index outside x[i] is skipped and
// reported through the status word.
template <int kU, bool kNT, bool kRows>
__global__ void __launch_bounds__(kThreads) moe_dispatch_kernel(const MoePlan m) {
  const LaunchPlan &p = m.base;
  uint32_t e = 0;
  bool run = true;
  if (p.sync) {
    e = snac::launch_epoch(p);
    run = snac::entry(p, e);
  }
  int t = run ? int(blockIdx.x) : p.total_tiles;
  int q = t < p.total_tiles ? job_of_tile(p, t) : 0;
  for (; t < p.total_tiles; t += gridDim.x) {
    if (t >= p.tile_begin[q + 1]) q = job_of_tile(p, t);
    const Job jb = p.jobs[q];
    const int64_t k = t - p.tile_begin[q];
    const int64_t tok = m.idx[jb.src][jb.src_off + k];
    if (tok < 0 || tok >= m.x_rows[jb.src]) {
      if (threadIdx.x == 0) flag_bad_arg(p);
      continue;
    }
    atom::Srcs s;
    s.n = 1;
    const uint64_t a = uint64_t(p.in[jb.src]) + uint64_t(tok) * uint64_t(m.row_bytes);
#pragma unroll
    for (int r = 0; r < kMaxRanks; ++r) s.a[r] = a;
    atom::Dsts d;
    d.n = 1;
    const uint64_t b = uint64_t(p.out[jb.dst]) + uint64_t(jb.dst_off) + uint64_t(k) * uint64_t(m.row_bytes);
#pragma unroll
    for (int r = 0; r < kMaxRanks + 1; ++r) d.b[r] = b;
    atom::tile<atom::CopyOp, kU, kNT, true, kRows>(s, d, 0, m.row_bytes, true);
  }
  if (p.sync) snac::exit_notify(p, e);
}

// Dispatch with one row per (token, destination rank), after the inverse
// pass below: one tile per token row, read once and written to every rank
// the token goes to (a broadcast with the token's own destination set).
// Rows and buffers are 16-byte aligned, so the destinations are congruent.
// It reads the epoch the inverse pass wrote its entries with, and its last
// workgroup advances it, so the next call's entries carry a new one.
template <int kU, bool kNT>
__global__ void __launch_bounds__(kThreads) moe_dispatch_tokens_kernel(const MoePlan m) {
  const LaunchPlan &p = m.base;
  const uint32_t e = snac::launch_epoch(p);
  const bool run = !p.sync || snac::entry(p, e);
  const int64_t rows = m.inv_base[p.P];
  for (int64_t r = run ? int64_t(blockIdx.x) : rows; r < rows; r += gridDim.x) {
    int i = 0;
    for (int q = 1; q < kMaxRanks; ++q)
      if (q < p.P && m.inv_base[q] <= r) i = q;
    const int64_t t = r - m.inv_base[i];
    atom::Dsts d;
    d.n = 0;
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) {
      d.b[j] = 0;
      if (j < p.P) {
        const uint64_t v = m.inv[(m.inv_base[i] + t) * p.P + j];
        if (uint32_t(v >> 32) == e) {
          const int64_t k = int64_t(uint32_t(v)) - 1;
          d.b[j] = uint64_t(p.out[j]) + uint64_t(p.jobs[i * p.P + j].dst_off) +
                   uint64_t(k) * uint64_t(m.row_bytes);
        }
      }
    }
    // compact the present destinations to the front (unrolled, so the
    // array stays in registers)
    uint64_t b[kMaxRanks + 1];
#pragma unroll
    for (int j = 0; j < kMaxRanks + 1; ++j) b[j] = 0;
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) {
      if (d.b[j]) {
#pragma unroll
        for (int q = 0; q < kMaxRanks; ++q)
          if (q == d.n) b[q] = d.b[j];
        ++d.n;
      }
    }
    if (d.n == 0) continue;
#pragma unroll
    for (int j = 0; j < kMaxRanks + 1; ++j) d.b[j] = j < d.n ? b[j] : b[0];
    atom::Srcs s;
    s.n = 1;
    const uint64_t a = uint64_t(p.in[i]) + uint64_t(t) * uint64_t(m.row_bytes);
#pragma unroll
    for (int q = 0; q < kMaxRanks; ++q) s.a[q] = a;
    atom::tile<atom::CopyOp, kU, kNT, true, false>(s, d, 0, m.row_bytes, true);
  }
  snac::exit_notify(p, e);
}

// Combine, first pass: for every entry (i, j, k) the slot (token, j) of
// rank i's table gets (epoch, k + 1).  Entries of earlier launches carry an
// older epoch, so the table is never cleared; a slot already holding this
// launch's epoch is a token twice in one group, which is reported.  The
// pass does not count its exit: the kernel after it reads the same epoch
// and advances it.
__global__ void __launch_bounds__(kThreads) moe_inverse_kernel(const MoePlan m) {
  const LaunchPlan &p = m.base;
  const uint32_t epoch = snac::launch_epoch(p);
  const int64_t total = m.ent_base[p.P];
  for (int64_t e = int64_t(blockIdx.x) * kThreads + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * kThreads) {
    int i = 0;
    for (int r = 1; r < kMaxRanks; ++r)
      if (r < p.P && m.ent_base[r] <= e) i = r;
    const int64_t ei = e - m.ent_base[i];
    int j = 0;
    for (int r = 1; r < kMaxRanks; ++r)
      if (r < p.P && p.jobs[i * p.P + r].src_off <= ei) j = r;
    const int64_t k = ei - p.jobs[i * p.P + j].src_off;
    const int64_t tok = m.idx[i][ei];
    if (tok < 0 || tok >= m.x_rows[i]) {
      flag_bad_arg(p);
      continue;
    }
    const uint64_t v = (uint64_t(epoch) << 32) | uint64_t(k + 1);
    const uint64_t old = __hip_atomic_exchange(&m.inv[(m.inv_base[i] + tok) * p.P + j], v,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (uint32_t(old >> 32) == epoch) flag_bad_arg(p);
  }
}

// Combine, second pass: one token row per tile.  The row's contributions
// are the table's slots of this epoch, in ascending destination rank; each
// lane folds its 16-byte units as acc = acc + w * y from +0 in fp32, every
// product rounded before the add (no contraction), then rounds once to
// bf16.  Rows and buffers are 16-byte aligned (checked by the host).
template <int kU, bool kNT>
__global__ void __launch_bounds__(kThreads) moe_combine_kernel(const MoePlan m) {
#pragma clang fp contract(off)
  const LaunchPlan &p = m.base;
  const uint32_t e = snac::launch_epoch(p);
  const bool run = !p.sync || snac::entry(p, e);
  const int64_t rows = m.inv_base[p.P];
  const uint32_t nunits = uint32_t(m.row_bytes >> 4);
  for (int64_t r = run ? int64_t(blockIdx.x) : rows; r < rows; r += gridDim.x) {
    int i = 0;
    for (int q = 1; q < kMaxRanks; ++q)
      if (q < p.P && m.inv_base[q] <= r) i = q;
    const int64_t t = r - m.inv_base[i];
    const uint64_t dst = uint64_t(p.out[i]) + uint64_t(t) * uint64_t(m.row_bytes);
    uint64_t src[kMaxRanks];
    float wt[kMaxRanks];
    bool on[kMaxRanks];
#pragma unroll
    for (int j = 0; j < kMaxRanks; ++j) {
      on[j] = false;
      src[j] = dst;
      wt[j] = 0.0f;
      if (j < p.P) {
        const uint64_t v = m.inv[(m.inv_base[i] + t) * p.P + j];
        if (uint32_t(v >> 32) == e) {
          const int64_t k = int64_t(uint32_t(v)) - 1;
          const Job jb = p.jobs[i * p.P + j];
          on[j] = true;
          src[j] = uint64_t(p.in[j]) + uint64_t(jb.dst_off) + uint64_t(k) * uint64_t(m.row_bytes);
          wt[j] = m.w[i][jb.src_off + k];
        }
      }
    }
    for (uint32_t u0 = 0; u0 < nunits; u0 += kThreads * kU) {
      atom::u32x4 x[kU][kMaxRanks];
#pragma unroll
      for (int kk = 0; kk < kU; ++kk) {
        uint32_t u = u0 + uint32_t(kk) * kThreads + threadIdx.x;
        if (u >= nunits) u = nunits - 1;
        // absent contributions load nothing (the branch is the same in every lane)
#pragma unroll
        for (int j = 0; j < kMaxRanks; ++j)
          x[kk][j] = on[j] ? atom::ld16<kNT>(src[j] + uint64_t(u) * 16u) : atom::u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int kk = 0; kk < kU; ++kk) {
        const uint32_t u = u0 + uint32_t(kk) * kThreads + threadIdx.x;
        if (u >= nunits) continue;
        float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kMaxRanks; ++j) {
          if (on[j]) {
            const atom::u32x4 v = x[kk][j];
            const float w = wt[j];
            a[0] = a[0] + w * atom::bf16_lo(v.x); a[1] = a[1] + w * atom::bf16_hi(v.x);
            a[2] = a[2] + w * atom::bf16_lo(v.y); a[3] = a[3] + w * atom::bf16_hi(v.y);
            a[4] = a[4] + w * atom::bf16_lo(v.z); a[5] = a[5] + w * atom::bf16_hi(v.z);
            a[6] = a[6] + w * atom::bf16_lo(v.w); a[7] = a[7] + w * atom::bf16_hi(v.w);
          }
        }
        atom::u32x4 o;
        o.x = atom::bf16x2_rne(a[0], a[1]);
        o.y = atom::bf16x2_rne(a[2], a[3]);
        o.z = atom::bf16x2_rne(a[4], a[5]);
        o.w = atom::bf16x2_rne(a[6], a[7]);
        atom::st16<kNT>(dst + uint64_t(u) * 16u, o);
      }
    }
  }
  snac::exit_notify(p, e);
}

// ---- Ulysses strided exchange -----------------------------------------------
// Ulysses sequence parallelism is one of the call sites of Purlin's AllToAll
// (Table 2, the diffusion workload): each pair of ranks exchanges the rows of
// one attention-head group, which are strided in the sequence-sharded layout
// and contiguous in the head-sharded one.  No intermediate packed buffer:
// lanes walk the pair's rows laid end to end in units of kUnit bytes, and each
// unit finds its row with one multiply-high (the host's magic divisor), so
// consecutive lanes read and write consecutive bytes of a row and a wavefront
// crosses row ends without idle lanes, whatever the row size.

template <int kUnit> struct UnitOf;
template <> struct UnitOf<16> { typedef atom::u32x4 T; };
template <> struct UnitOf<8> { typedef uint32_t T __attribute__((ext_vector_type(2))); };
template <> struct UnitOf<4> { typedef uint32_t T; };
template <> struct UnitOf<2> { typedef uint16_t T; };

// kNTS: nontemporal stores (large exchanges); small ones, whose bytes stay
// largely in the caches between the producing and the consuming kernel,
// store plainly.
template <class T, bool kNTS>
__device__ __forceinline__ void strided_store(uint64_t addr, T v) {
  if constexpr (kNTS) __builtin_nontemporal_store(v, atom::gp<T>(addr));
  else *atom::gp<T>(addr) = v;
}

template <int kUnit, int kU, bool kNTS = true>
__global__ void __launch_bounds__(kThreads) strided_kernel(const StridedPlan sp) {
  typedef typename UnitOf<kUnit>::T T;
  const LaunchPlan &p = sp.base;
  uint32_t e = 0;
  bool run = true;
  if (p.sync) {
    e = snac::launch_epoch(p);
    run = snac::entry(p, e);
  }
  const uint32_t per_row = uint32_t(sp.row_bytes / kUnit);
  const int64_t per_tile = p.chunk_bytes / kUnit;
  int t = run ? int(blockIdx.x) : p.total_tiles;
  int q = t < p.total_tiles ? job_of_tile(p, t) : 0;
  for (; t < p.total_tiles; t += gridDim.x) {
    if (t >= p.tile_begin[q + 1]) q = job_of_tile(p, t);
    const Job jb = p.jobs[q];
    const uint64_t sb = uint64_t(p.in[jb.src]) + uint64_t(jb.src_off);
    const uint64_t db = uint64_t(p.out[jb.dst]) + uint64_t(jb.dst_off);
    const int64_t u0 = int64_t(t - p.tile_begin[q]) * per_tile;
    const int64_t n = jb.nbytes / kUnit;
    // units of the pair are < 2^31 (checked by the host)
    const uint32_t u1 = uint32_t(u0 + per_tile < n ? u0 + per_tile : n);
    // full passes: every load and store unconditional (no pass waits for
    // the previous pass's stores); then one guarded pass for the rest
    uint32_t p0 = uint32_t(u0);
    for (; p0 + kThreads * kU <= u1; p0 += kThreads * kU) {
      T v[kU];
      uint64_t dst[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const uint32_t uk = p0 + uint32_t(k) * kThreads + threadIdx.x;
        const uint32_t r = uint32_t((uint64_t(uk) * sp.magic) >> sp.shift);
        const uint32_t c = uk - r * per_row;
        v[k] = __builtin_nontemporal_load(atom::gp<const T>(
            sb + uint64_t(r) * uint64_t(sp.src_stride) + uint64_t(c) * kUnit));
        dst[k] = db + uint64_t(r) * uint64_t(sp.dst_stride) + uint64_t(c) * kUnit;
      }
#pragma unroll
      for (int k = 0; k < kU; ++k) strided_store<T, kNTS>(dst[k], v[k]);
    }
    if (p0 < u1) {
      T v[kU];
      uint64_t dst[kU];
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const uint32_t uk = p0 + uint32_t(k) * kThreads + threadIdx.x;
        if (uk < u1) {
          const uint32_t r = uint32_t((uint64_t(uk) * sp.magic) >> sp.shift);
          const uint32_t c = uk - r * per_row;
          v[k] = __builtin_nontemporal_load(atom::gp<const T>(
              sb + uint64_t(r) * uint64_t(sp.src_stride) + uint64_t(c) * kUnit));
          dst[k] = db + uint64_t(r) * uint64_t(sp.dst_stride) + uint64_t(c) * kUnit;
        }
      }
#pragma unroll
      for (int k = 0; k < kU; ++k)
        if (p0 + uint32_t(k) * kThreads + threadIdx.x < u1)
          strided_store<T, kNTS>(dst[k], v[k]);
      atom::drain_vm();
    }
  }
  if (p.sync) snac::exit_notify(p, e);
}

// ---- calibration copy ------------------------------------------------------
// A plain streaming copy with the same access style as the collectives (16-byte
// nontemporal loads and stores, 4 per lane in flight): the reference for HBM
// counters and the copy ceiling the collectives are compared with.
__global__ void __launch_bounds__(kThreads) stream_copy_kernel(atom::u32x4 *dst,
                                                                const atom::u32x4 *src,
                                                                int64_t n16) {
  constexpr int kU = 4;
  const int64_t stride = int64_t(gridDim.x) * kThreads * kU;
  for (int64_t b = int64_t(blockIdx.x) * kThreads * kU + threadIdx.x; b < n16; b += stride) {
    atom::u32x4 v[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int64_t i = b + int64_t(k) * kThreads;
      if (i < n16) v[k] = atom::ld16<true>(uint64_t(src + i));
    }
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int64_t i = b + int64_t(k) * kThreads;
      if (i < n16) atom::st16<true>(uint64_t(dst + i), v[k]);
    }
  }
}

// Bare access pattern of a collective (ceiling measurement): kR sources
// (0: write-only) added as integers, written to kW destinations (0:
// read-only), the same offset everywhere, with no planning or flags.  Tiles
// of `tile16` units are dealt in grid-stride order as the collectives deal
// theirs; full passes of kU units per lane are unguarded, the tile's last
// pass is guarded.  kNTL: nontemporal loads; kNTS: the store mode (plain,
// nontemporal or device scope, atom::kStore*).
struct PatternPtrs {
  const atom::u32x4 *src[kMaxRanks];
  atom::u32x4 *dst[kMaxRanks];
};


// One pass of kU units per lane from unit b (this lane's first) of the
// tile that starts at unit tb; with kGuard, units at or past `end` are
// neither loaded (clamped) nor stored.
template <int kR, int kW, int kU, bool kNTL, int kNTS, bool kGuard>
__device__ __forceinline__ void pattern_pass(const PatternPtrs &p, int64_t tb, int64_t b,
                                             int64_t end, atom::u32x4 &acc) {
  atom::u32x4 v[kU][kR > 0 ? kR : 1];
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    int64_t i = b + int64_t(k) * kThreads;
    if (kGuard && i >= end) i = end - 1;
#pragma unroll
    for (int r = 0; r < kR; ++r) v[k][r] = atom::ld16<kNTL>(uint64_t(p.src[r] + i));
  }
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    const int64_t i = b + int64_t(k) * kThreads;
    atom::u32x4 a;
    if constexpr (kR == 0) {
      a = atom::u32x4{uint32_t(i), uint32_t(i >> 32), 0x5a5a5a5au, 0xa5a5a5a5u};
    } else {
      a = v[k][0];
#pragma unroll
      for (int r = 1; r < kR; ++r) a += v[k][r];
    }
    if constexpr (kW == 0) {
      acc ^= a;
    } else if (!kGuard || i < end) {
#pragma unroll
      for (int w = 0; w < kW; ++w)
        atom::stm<kNTS>(uint64_t(p.dst[w] + tb), uint32_t(i - tb) * 16u, a);
    }
  }
}

template <int kR, int kW, int kU, bool kNTL, int kNTS>
__global__ void __launch_bounds__(kThreads) pattern_kernel(PatternPtrs p, int64_t n16, int64_t tile16) {
  constexpr int64_t kPass = int64_t(kThreads) * kU;
  const int64_t ntiles = (n16 + tile16 - 1) / tile16;
  atom::u32x4 acc{0u, 0u, 0u, 0u};
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t end = (t + 1) * tile16 < n16 ? (t + 1) * tile16 : n16;
    const int64_t tb = t * tile16;
    int64_t b = tb;
    // full passes: every unit lies inside the tile, no guard
    for (; b + kPass <= end; b += kPass)
      pattern_pass<kR, kW, kU, kNTL, kNTS, false>(p, tb, b + threadIdx.x, end, acc);
    if (b < end) {
      pattern_pass<kR, kW, kU, kNTL, kNTS, true>(p, tb, b + threadIdx.x, end, acc);
      atom::drain_vm();
    }
  }
  if constexpr (kW == 0)
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) g_pattern_sink = acc;
}

template <int kR, int kW, int kU, bool kNTL>
const void *pattern_fn_s(int smode) {
  if constexpr (kW > 0)
    if (smode == atom::kStoreDevice)
      return reinterpret_cast<const void *>(&pattern_kernel<kR, kW, kU, kNTL, atom::kStoreDevice>);
  return smode == atom::kStorePlain
             ? reinterpret_cast<const void *>(&pattern_kernel<kR, kW, kU, kNTL, atom::kStorePlain>)
             : reinterpret_cast<const void *>(&pattern_kernel<kR, kW, kU, kNTL, atom::kStoreNT>);
}

template <int kR, int kW, int kU>
const void *pattern_fn_u(bool ntl, int smode) {
  return ntl ? pattern_fn_s<kR, kW, kU, true>(smode) : pattern_fn_s<kR, kW, kU, false>(smode);
}

// Eight sources keep at most four units per lane in flight (eight would
// hold 256 VGPRs of loads and spill).
template <int kR, int kW>
const void *pattern_fn_rw(int unroll, bool ntl, int smode) {
  switch (unroll) {
    case 2: return pattern_fn_u<kR, kW, 2>(ntl, smode);
    case 8:
      if constexpr (kR < 8) return pattern_fn_u<kR, kW, 8>(ntl, smode);
      else return pattern_fn_u<kR, kW, 4>(ntl, smode);
    default: return pattern_fn_u<kR, kW, 4>(ntl, smode);
  }
}

const void *pattern_fn(int n_src, int n_dst, int unroll, bool ntl, int smode) {
  if (n_src == 0 && n_dst == 1) return pattern_fn_rw<0, 1>(unroll, ntl, smode);
  if (n_src == 0 && n_dst == 8) return pattern_fn_rw<0, 8>(unroll, ntl, smode);
  if (n_src == 1 && n_dst == 0) return pattern_fn_rw<1, 0>(unroll, ntl, smode);
  if (n_src == 8 && n_dst == 0) return pattern_fn_rw<8, 0>(unroll, ntl, smode);
  if (n_src == 1 && n_dst == 1) return pattern_fn_rw<1, 1>(unroll, ntl, smode);
  if (n_src == 1 && n_dst == 8) return pattern_fn_rw<1, 8>(unroll, ntl, smode);
  if (n_src == 8 && n_dst == 1) return pattern_fn_rw<8, 1>(unroll, ntl, smode);
  if (n_src == 8 && n_dst == 8) return pattern_fn_rw<8, 8>(unroll, ntl, smode);
  return nullptr;
}

}  // namespace

hipError_t launch_pattern(const void *const *srcs, int n_src, void *const *dsts, int n_dst,
                          int64_t bytes, int grid, int64_t tile_bytes, int unroll, bool ntl,
                          int smode, hipStream_t stream) {
  PatternPtrs p{};
  for (int r = 0; r < kMaxRanks; ++r) {
    p.src[r] = n_src ? static_cast<const atom::u32x4 *>(srcs[r < n_src ? r : 0]) : nullptr;
    p.dst[r] = n_dst ? static_cast<atom::u32x4 *>(dsts[r < n_dst ? r : 0]) : nullptr;
  }
  int64_t n16 = bytes / 16;
  int64_t tile16 = tile_bytes / 16;
  const void *fn = pattern_fn(n_src, n_dst, unroll, ntl, smode);
  if (!fn) return hipErrorInvalidValue;
  void *args[] = {&p, &n16, &tile16};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, stream);
}

namespace {

// The single-destination builds exist for the default (nontemporal) form,
// without row bodies, and with row bodies for sums; one_build says which
// launches get one.  The wide builds (latency regime) exist for the row
// bodies of the default form and unroll, and so do the builds for large copy
// broadcasts, whose stores are plain (bcast; sums are never asked for one),
// and the broadcast builds with device-scope stores (dstore: aligned sums,
// and copies aligned or on the wide row body; dstore_build says which).
template <class Op, int kU, bool kNT, bool kWideOk = false>
void *zs_fn(bool rows, bool one, bool wide, bool bcast, bool dstore) {
  if constexpr (kNT && kWideOk) {
    if (dstore && !one) {
      if (!rows) return reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, atom::kStoreDevice, false, false>);
      if constexpr (!Op::kSum)
        if (wide) return reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, atom::kStoreDevice, true, false, true>);
    }
  }
  if constexpr (kNT) {
    if (one && !rows) return reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, kNT, false, true>);
    if constexpr (Op::kSum)
      if (one && rows) {
        if constexpr (kWideOk)
          if (wide) return reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, kNT, true, true, true>);
        return reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, kNT, true, true>);
      }
    if constexpr (kWideOk && !Op::kSum) {
      if (bcast) {
        if (!rows) return reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, false, false, false>);
        return wide ? reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, false, true, false, true>)
                    : reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, false, true, false>);
      }
    }
    if constexpr (kWideOk)
      if (rows && wide) return reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, kNT, true, false, true>);
  }
  return rows ? reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, kNT, true, false>)
              : reinterpret_cast<void *>(&zs_kernel<Op, kU, kNT, kNT, false, false>);
}
template <class Op, int kU, bool kNT>
void *st_fn() { return reinterpret_cast<void *>(&staged_kernel<Op, kU, kNT, kNT>); }

// Unroll depth: 16-byte units each lane keeps in flight per source.
template <class Op, int kU0, int kU1, int kU2>
void *pick(bool staged, bool nt, int unroll_sel, bool rows, bool one, bool wide, bool bcast,
           bool dstore) {
  if (staged) return nt ? st_fn<Op, kU1, true>() : st_fn<Op, kU1, false>();
  switch (unroll_sel) {
    case 0:
      return nt ? zs_fn<Op, kU0, true, true>(rows, one, wide, bcast, dstore)
                : zs_fn<Op, kU0, false>(rows, one, false, false, false);
    case 2:
      return nt ? zs_fn<Op, kU2, true>(rows, one, false, false, false)
                : zs_fn<Op, kU2, false>(rows, one, false, false, false);
    default:
      return nt ? zs_fn<Op, kU1, true>(rows, one, false, false, false)
                : zs_fn<Op, kU1, false>(rows, one, false, false, false);
  }
}

}  // namespace

bool dstore_build(KernelKind kind, bool nt, int unroll_sel, bool rows, bool wide) {
  return nt && unroll_sel == 0 && (!rows || (kind == KernelKind::kCopy && wide));
}

bool one_build(KernelKind kind, bool nt, bool rows, bool single_dst) {
  // measured: the single-destination build of the copy with row bodies is
  // 1.5% slower on AllToAllV at 64 MiB per rank than the general one
  return single_dst && nt && (!rows || kind != KernelKind::kCopy);
}

int unroll_of(KernelKind kind, int unroll_sel) {
  static const int copy_u[3] = {4, 8, 16};
  static const int sum_u[3] = {1, 2, 4};
  const int sel = unroll_sel < 0 || unroll_sel > 2 ? 1 : unroll_sel;
  return kind == KernelKind::kCopy ? copy_u[sel] : sum_u[sel];
}

void *kernel_fn(KernelKind kind, bool staged, bool nt, int unroll_sel, bool rows, bool one,
                bool wide = false, bool bcast = false, bool dstore = false) {
  switch (kind) {
    case KernelKind::kCopy:
      return pick<atom::CopyOp, 4, 8, 16>(staged, nt, unroll_sel, rows, one, wide, bcast, dstore);
    case KernelKind::kSumF32:
      return pick<atom::SumF32, 1, 2, 4>(staged, nt, unroll_sel, rows, one, wide, bcast, dstore);
    default:
      return pick<atom::SumBf16, 1, 2, 4>(staged, nt, unroll_sel, rows, one, wide, bcast, dstore);
  }
}

hipError_t launch_zs(const LaunchPlan &p, KernelKind kind, bool nt, int unroll_sel, bool rows,
                     bool one, bool wide, bool bcast, bool dstore, int grid, hipStream_t stream) {
  void *args[] = {const_cast<LaunchPlan *>(&p)};
  return hipLaunchKernel(kernel_fn(kind, false, nt, unroll_sel, rows, one, wide, bcast, dstore), dim3(grid),
                         dim3(kThreads), args, 0, stream);
}

static void *zs_lds_fn(KernelKind kind, bool one, bool bcast) {
  switch (kind) {
    case KernelKind::kCopy:
      if (one) return reinterpret_cast<void *>(&zs_lds_kernel<atom::CopyOp, 4, true, true, 8>);
      return bcast ? reinterpret_cast<void *>(&zs_lds_kernel<atom::CopyOp, 4, false, false, 8>)
                   : reinterpret_cast<void *>(&zs_lds_kernel<atom::CopyOp, 4, true, false, 8>);
    case KernelKind::kSumF32:
      return one ? reinterpret_cast<void *>(&zs_lds_kernel<atom::SumF32, 1, true, true, 2>)
                 : reinterpret_cast<void *>(&zs_lds_kernel<atom::SumF32, 1, true, false, 2>);
    default:
      return one ? reinterpret_cast<void *>(&zs_lds_kernel<atom::SumBf16, 1, true, true, 2>)
                 : reinterpret_cast<void *>(&zs_lds_kernel<atom::SumBf16, 1, true, false, 2>);
  }
}

hipError_t launch_zs_lds(const LaunchPlan &p, KernelKind kind, bool one, bool bcast, int grid,
                         hipStream_t stream) {
  void *args[] = {const_cast<LaunchPlan *>(&p)};
  return hipLaunchKernel(zs_lds_fn(kind, one, bcast), dim3(grid), dim3(kThreads), args, 0, stream);
}

hipError_t zs_lds_resident_per_cu(KernelKind kind, bool one, bool bcast, int *blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, zs_lds_fn(kind, one, bcast), kThreads, 0);
}

hipError_t launch_staged(const StagedPlan &p, KernelKind kind, bool nt, hipStream_t stream) {
  void *args[] = {const_cast<StagedPlan *>(&p)};
  return hipLaunchKernel(kernel_fn(kind, true, nt, 1, true, false), dim3(p.total_roles), dim3(kThreads),
                         args, 0, stream);
}

void *moe_kernel_fn(MoeKernel which, bool rows) {
  switch (which) {
    case MoeKernel::kDispatch:
      return rows ? reinterpret_cast<void *>(&moe_dispatch_kernel<4, true, true>)
                  : reinterpret_cast<void *>(&moe_dispatch_kernel<4, true, false>);
    case MoeKernel::kInverse: return reinterpret_cast<void *>(&moe_inverse_kernel);
    case MoeKernel::kDispatchTokens:
      return reinterpret_cast<void *>(&moe_dispatch_tokens_kernel<4, true>);
    default: return reinterpret_cast<void *>(&moe_combine_kernel<2, true>);
  }
}

hipError_t launch_moe(const MoePlan &m, MoeKernel which, bool rows, int grid, hipStream_t stream) {
  void *args[] = {const_cast<MoePlan *>(&m)};
  return hipLaunchKernel(moe_kernel_fn(which, rows), dim3(grid), dim3(kThreads), args, 0, stream);
}

hipError_t moe_resident_per_cu(MoeKernel which, bool rows, int *blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, moe_kernel_fn(which, rows), kThreads, 0);
}

// Units in flight per lane: 16 KiB per workgroup pass for 16-byte units.
template <bool kNTS>
static void *strided_fn_of(int unit) {
  switch (unit) {
    case 16: return reinterpret_cast<void *>(&strided_kernel<16, 4, kNTS>);
    case 8: return reinterpret_cast<void *>(&strided_kernel<8, 8, kNTS>);
    case 4: return reinterpret_cast<void *>(&strided_kernel<4, 8, kNTS>);
    default: return reinterpret_cast<void *>(&strided_kernel<2, 16, kNTS>);
  }
}
static void *strided_fn(int unit, bool plain) {
  return plain ? strided_fn_of<false>(unit) : strided_fn_of<true>(unit);
}

hipError_t launch_strided(const StridedPlan &sp, int unit, bool plain, int grid,
                          hipStream_t stream) {
  void *args[] = {const_cast<StridedPlan *>(&sp)};
  return hipLaunchKernel(strided_fn(unit, plain), dim3(grid), dim3(kThreads), args, 0, stream);
}

hipError_t strided_resident_per_cu(int unit, bool plain, int *blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, strided_fn(unit, plain), kThreads, 0);
}

hipError_t launch_stream_copy(void *dst, const void *src, int64_t bytes, int grid,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_copy_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     reinterpret_cast<atom::u32x4 *>(dst),
                     reinterpret_cast<const atom::u32x4 *>(src), bytes / 16);
  return hipGetLastError();
}

hipError_t max_resident_per_cu(KernelKind kind, bool staged, bool nt, int unroll_sel, bool rows,
                               bool one, bool wide, bool bcast, bool dstore, int *blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks,
      kernel_fn(kind, staged, nt, staged ? 1 : unroll_sel, staged || rows, !staged && one,
                !staged && wide, !staged && bcast, !staged && dstore),
      kThreads, 0);
}

}  // namespace purlin
