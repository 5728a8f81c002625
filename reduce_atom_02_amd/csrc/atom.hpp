// Atom: the datapath primitives, copy and reduce, for gfx950.
//
// Purlin keeps the hardware-specific movement of bytes in a layer of its own
// with two primitives, copy and reduce (abstract; Figure 1 caption).
// This is that layer for one CDNA4 GPU, where every byte moves through HBM:
//
//  * 16-byte global loads and stores (dwordx4), 64 lanes x 16 B = 1 KiB per
//    wavefront instruction, 4 KiB per 256-thread workgroup pass, with kU
//    independent units per lane in flight;
//  * a tile whose sources sit on its destinations' 16-byte phase moves
//    aligned units; otherwise it takes one of these forms, chosen per
//    launch by measurement: the row body (units aligned to the destination,
//    each source read in aligned 16-byte blocks and shifted into place in
//    registers with a lane shuffle and v_alignbyte); for sums whose sources
//    share one phase, source-aligned units with misaligned 16-byte stores,
//    or the same units folded and shifted into aligned stores across rows
//    each wavefront carries (body_carry); for copy broadcasts,
//    destination-aligned units with misaligned 16-byte loads.  Rows follow
//    the sources' 128-byte lines for a sum with one destination, so none of
//    its eight sources' lines is loaded by two rows (a second nontemporal
//    load of a line fetches it from HBM again, while split destination
//    lines merge in L2), and the destinations' lines for copies, which read
//    one stream;
//  * stores are nontemporal, plain, or at device scope (written through the
//    L2: the staged pipeline's ring slots, and broadcasts where that
//    measured faster);
//  * the reduce is a per-lane fold over the sources in ascending rank, in
//    fp32 (bf16 widened exactly), with one final round to nearest even for
//    a bf16 output; there is no cross-lane tree, so the summation order is
//    the same for every element.
//
// Reading an aligned 16-byte block that contains at least one byte of a
// buffer never touches an unmapped page (pages are 16-byte aligned), so the
// realigning reads at the ends of a source stay inside mapped memory.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace purlin {
namespace atom {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every access names the global address space explicitly, so the compiler
// emits global_* instructions (scalar base + lane offset) instead of flat_*
// ones, which would also occupy the counter that scalar loads wait on.
template <class T>
using gptr = __attribute__((address_space(1))) T *;

template <class T>
__device__ __forceinline__ gptr<T> gp(uint64_t addr) {
  return reinterpret_cast<gptr<T>>(addr);
}

template <bool kNT>
__device__ __forceinline__ u32x4 ld16(uint64_t addr) {
  gptr<const u32x4> p = gp<const u32x4>(addr);
  if constexpr (kNT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool kNT>
__device__ __forceinline__ void st16(uint64_t addr, u32x4 v) {
  gptr<u32x4> p = gp<u32x4>(addr);
  if constexpr (kNT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// A 16-byte store to an address that is only 2-byte aligned: one
// global_store_dwordx4 (gfx950 under the HSA runtime serves misaligned
// global accesses; the compiler emits this form for any 2-byte-aligned
// 16-byte access).  The memory system splits it at 16-byte boundaries.
typedef u32x4 u32x4_a2 __attribute__((aligned(2)));
template <bool kNT>
__device__ __forceinline__ void st16u(uint64_t addr, u32x4 v) {
  gptr<u32x4_a2> p = gp<u32x4_a2>(addr);
  if constexpr (kNT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// A 16-byte load from an address that is only 2-byte aligned (as st16u).
template <bool kNT>
__device__ __forceinline__ u32x4 ld16u(uint64_t addr) {
  gptr<const u32x4_a2> p = gp<const u32x4_a2>(addr);
  if constexpr (kNT) return __builtin_nontemporal_load(p);
  else return *p;
}

// kUL: the source is off the 16-byte grid (misaligned loads).
template <bool kNT, bool kUL>
__device__ __forceinline__ u32x4 ld16x(uint64_t addr) {
  if constexpr (kUL) return ld16u<kNT>(addr);
  else return ld16<kNT>(addr);
}

// kUS: the destination is off the 16-byte grid (misaligned stores).
template <bool kNT, bool kUS>
__device__ __forceinline__ void st16x(uint64_t addr, u32x4 v) {
  if constexpr (kUS) st16u<kNT>(addr, v);
  else st16<kNT>(addr, v);
}

// Store modes of the tile bodies: plain, nontemporal, or device scope.  A
// device-scope store (the sc1 cache policy) is written through the XCD's L2
// and counted as done only once every XCD would read it, so bytes that one
// workgroup hands to another through HBM are published by a wait for the
// store counter and a relaxed flag store: no writeback of the L2's dirty
// lines, which is what a release costs on a multi-XCD gfx950 (measured: a
// handoff of a 32-256 KiB chunk 1.5-4 times slower with it).  The staged
// pipeline writes its ring slots this way.
constexpr int kStorePlain = 0;
constexpr int kStoreNT = 1;
constexpr int kStoreDevice = 2;

// The sc1 bit of a buffer instruction's cache-policy operand.
constexpr int kCpolSc1 = 16;

// Device-scope 16-byte store to base + off (base the same in every lane: it
// becomes a buffer resource in scalar registers; the range is left open,
// the caller keeps off inside the buffer).
__device__ __forceinline__ void st16_device(uint64_t base, uint32_t off, u32x4 v) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(base), 0, -1, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kCpolSc1);
}

// 16-byte store of a tile body in store mode kM (an aligned destination).
template <int kM>
__device__ __forceinline__ void stm(uint64_t base, uint32_t off, u32x4 v) {
  if constexpr (kM == kStoreDevice) st16_device(base, off, v);
  else st16<kM == kStoreNT>(base + off, v);
}

// Element store (2 or 4 bytes), device scope when kDev.
template <class T, bool kDev>
__device__ __forceinline__ void ste(uint64_t addr, T v) {
  if constexpr (kDev) __hip_atomic_store(gp<T>(addr), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *gp<T>(addr) = v;
}

// The 16 bytes that start `sh` bytes into the 32-byte pair (lo, hi);
// sh in [0, 16) is the same for every lane.
__device__ __forceinline__ u32x4 funnel(u32x4 lo, u32x4 hi, uint32_t sh) {
  uint32_t w0 = lo.x, w1 = lo.y, w2 = lo.z, w3 = lo.w;
  uint32_t w4 = hi.x, w5 = hi.y, w6 = hi.z, w7 = hi.w;
  if (sh & 8) { w0 = w2; w1 = w3; w2 = w4; w3 = w5; w4 = w6; w5 = w7; }
  if (sh & 4) { w0 = w1; w1 = w2; w2 = w3; w3 = w4; w4 = w5; }
  const uint32_t r = sh & 3;  // bytes still to shift inside a dword
  u32x4 o;
  o.x = __builtin_amdgcn_alignbyte(w1, w0, r);
  o.y = __builtin_amdgcn_alignbyte(w2, w1, r);
  o.z = __builtin_amdgcn_alignbyte(w3, w2, r);
  o.w = __builtin_amdgcn_alignbyte(w4, w3, r);
  return o;
}

// Wait until every vector memory access of this wave has completed.  Put at
// the end of a guarded pass (whose stores may be skipped, leaving their loads
// unconsumed), it lets the compiler's wait insertion know that no load is
// still pending there, so the unguarded loops of the next tile issue their
// loads without first draining the stores of this one.
__device__ __forceinline__ void drain_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- bf16 <-> fp32 -------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// IEEE round to nearest, ties to even, of two fp32 values to bf16 (lo in
// the low half, hi in the high half), with gfx950's one packed conversion
// instruction (v_cvt_pk_bf16_f32) instead of six integer operations per
// value.  Its results were compared on the device with the integer rule
// (add 0x7fff plus the lowest kept bit, keep the top half) for every one of
// the 2^32 fp32 patterns: identical for every non-NaN input (subnormals,
// ties, overflow to inf, signed zeros), and every NaN input gives a NaN.  A
// NaN result of a sum may carry any payload (IEEE leaves it open).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t bf16_rne(float f) { return bf16x2_rne(f, 0.0f) & 0xffffu; }

// ---- element operations (head and tail of a tile, < 16 bytes) -------------

// Elements per thread of the wide element pass that small misaligned tiles
// take instead of a row body: enough for a 4 KiB tile plus the bytes before
// its first line (4224 bytes of 2-byte elements).
constexpr int kWideElems = 9;

// Copy moves 2-byte elements: every offset of an fp32 or bf16 buffer is a
// multiple of 2.
struct CopyOp {
  static constexpr bool kSum = false;
  static constexpr int kElem = 2;
};
struct SumF32 {
  static constexpr bool kSum = true;
  static constexpr int kElem = 4;
};
struct SumBf16 {
  static constexpr bool kSum = true;
  static constexpr int kElem = 2;
};

// Sources: byte x of the job lives at a[i] + x.  Entries past n repeat
// source 0, so reads of them are harmless and need no branch.
struct Srcs {
  uint64_t a[kMaxRanks];
  int n;
};
// Destinations: byte x of the job goes to b[d] + x; all congruent mod 16.
struct Dsts {
  uint64_t b[kMaxRanks + 1];
  int n;
};

// Element-wise [y0, y1) of a job, one element per thread from thread t0
// on (at most kThreads - t0 elements).  Every source is loaded before any is
// added (entries past n repeat source 0, so the loads need no guard), so
// the loads are in flight together: one memory round trip.
template <class Op, bool kDevStore = false>
__device__ __forceinline__ void elements(const Srcs &s, const Dsts &d, int64_t y0, int64_t y1,
                                         int t0 = 0) {
  const int64_t n = (y1 - y0) / Op::kElem;
  const int idx = int(threadIdx.x) - t0;
  if (idx < 0 || idx >= n) return;
  const int64_t x = y0 + int64_t(idx) * Op::kElem;
  // Loops over sources and destinations are fully unrolled with a guard so
  // that the pointer arrays stay in registers.
  if constexpr (!Op::kSum) {
    const uint16_t v = *gp<const uint16_t>(s.a[0] + x);
#pragma unroll
    for (int k = 0; k < kMaxRanks + 1; ++k)
      if (k < d.n) ste<uint16_t, kDevStore>(d.b[k] + x, v);
  } else if constexpr (Op::kElem == 4) {
    float v[kMaxRanks];
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) v[i] = *gp<const float>(s.a[i] + x);
    float acc = v[0];
#pragma unroll
    for (int i = 1; i < kMaxRanks; ++i)
      if (i < s.n) acc = acc + v[i];
#pragma unroll
    for (int k = 0; k < kMaxRanks + 1; ++k)
      if (k < d.n) ste<float, kDevStore>(d.b[k] + x, acc);
  } else {
    uint16_t v[kMaxRanks];
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) v[i] = *gp<const uint16_t>(s.a[i] + x);
    float acc = bf16_lo(v[0]);
#pragma unroll
    for (int i = 1; i < kMaxRanks; ++i)
      if (i < s.n) acc = acc + bf16_lo(v[i]);
    const uint16_t r = uint16_t(bf16_rne(acc));
#pragma unroll
    for (int k = 0; k < kMaxRanks + 1; ++k)
      if (k < d.n) ste<uint16_t, kDevStore>(d.b[k] + x, r);
  }
}

// Element-wise [y0, y1) of a job with kE elements per thread (element
// t + e * kThreads for e < kE): every load of every element is issued before
// any is used (indexes past the end are clamped to the last element, so the
// loads need no branch), so the whole range is one memory round trip.  The
// caller guarantees 0 < (y1 - y0) / kElem <= kE * kThreads.
template <class Op, int kE, bool kDevStore = false>
__device__ __forceinline__ void elements_wide(const Srcs &s, const Dsts &d, int64_t y0, int64_t y1) {
  const int64_t n = (y1 - y0) / Op::kElem;
  const int64_t tid = int64_t(threadIdx.x);
  if constexpr (!Op::kSum) {
    uint16_t v[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t i = tid + e * kThreads;
      v[e] = *gp<const uint16_t>(s.a[0] + y0 + (i < n ? i : n - 1) * 2);
    }
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t i = tid + e * kThreads;
      if (i < n) {
#pragma unroll
        for (int k = 0; k < kMaxRanks + 1; ++k)
          if (k < d.n) ste<uint16_t, kDevStore>(d.b[k] + y0 + i * 2, v[e]);
      }
    }
  } else if constexpr (Op::kElem == 4) {
    float v[kE][kMaxRanks];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t i = tid + e * kThreads;
      const int64_t x = y0 + (i < n ? i : n - 1) * 4;
#pragma unroll
      for (int r = 0; r < kMaxRanks; ++r) v[e][r] = *gp<const float>(s.a[r] + x);
    }
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t i = tid + e * kThreads;
      float acc = v[e][0];
#pragma unroll
      for (int r = 1; r < kMaxRanks; ++r)
        if (r < s.n) acc = acc + v[e][r];
      if (i < n) {
#pragma unroll
        for (int k = 0; k < kMaxRanks + 1; ++k)
          if (k < d.n) ste<float, kDevStore>(d.b[k] + y0 + i * 4, acc);
      }
    }
  } else {
    uint16_t v[kE][kMaxRanks];
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t i = tid + e * kThreads;
      const int64_t x = y0 + (i < n ? i : n - 1) * 2;
#pragma unroll
      for (int r = 0; r < kMaxRanks; ++r) v[e][r] = *gp<const uint16_t>(s.a[r] + x);
    }
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      const int64_t i = tid + e * kThreads;
      float acc = bf16_lo(v[e][0]);
#pragma unroll
      for (int r = 1; r < kMaxRanks; ++r)
        if (r < s.n) acc = acc + bf16_lo(v[e][r]);
      const uint16_t o = uint16_t(bf16_rne(acc));
      if (i < n) {
#pragma unroll
        for (int k = 0; k < kMaxRanks + 1; ++k)
          if (k < d.n) ste<uint16_t, kDevStore>(d.b[k] + y0 + i * 2, o);
      }
    }
  }
}

// ---- 16-byte unit operations ----------------------------------------------

// Fold of one unit over the sources, in ascending rank, fp32 accumulator.
__device__ __forceinline__ u32x4 fold_f32(const u32x4 *x, int n) {
  float a0 = __uint_as_float(x[0].x), a1 = __uint_as_float(x[0].y);
  float a2 = __uint_as_float(x[0].z), a3 = __uint_as_float(x[0].w);
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i) {
    if (i < n) {
      a0 = a0 + __uint_as_float(x[i].x);
      a1 = a1 + __uint_as_float(x[i].y);
      a2 = a2 + __uint_as_float(x[i].z);
      a3 = a3 + __uint_as_float(x[i].w);
    }
  }
  u32x4 o;
  o.x = __float_as_uint(a0); o.y = __float_as_uint(a1);
  o.z = __float_as_uint(a2); o.w = __float_as_uint(a3);
  return o;
}

__device__ __forceinline__ u32x4 fold_bf16(const u32x4 *x, int n) {
  float a[8];
  a[0] = bf16_lo(x[0].x); a[1] = bf16_hi(x[0].x);
  a[2] = bf16_lo(x[0].y); a[3] = bf16_hi(x[0].y);
  a[4] = bf16_lo(x[0].z); a[5] = bf16_hi(x[0].z);
  a[6] = bf16_lo(x[0].w); a[7] = bf16_hi(x[0].w);
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i) {
    if (i < n) {
      a[0] = a[0] + bf16_lo(x[i].x); a[1] = a[1] + bf16_hi(x[i].x);
      a[2] = a[2] + bf16_lo(x[i].y); a[3] = a[3] + bf16_hi(x[i].y);
      a[4] = a[4] + bf16_lo(x[i].z); a[5] = a[5] + bf16_hi(x[i].z);
      a[6] = a[6] + bf16_lo(x[i].w); a[7] = a[7] + bf16_hi(x[i].w);
    }
  }
  u32x4 o;
  o.x = bf16x2_rne(a[0], a[1]);
  o.y = bf16x2_rne(a[2], a[3]);
  o.z = bf16x2_rne(a[4], a[5]);
  o.w = bf16x2_rne(a[6], a[7]);
  return o;
}

// One pass of the aligned body: kU units per lane, loaded before any is
// stored.  kGuard = false for passes that lie wholly inside the tile: then
// the pass is straight-line code, so the compiler keeps every load in
// flight until its data is needed instead of draining at guard branches.
template <class Op, int kU, bool kNTL, int kNTS, bool kGuard, bool kUS = false, bool kUL = false>
__device__ __forceinline__ void pass_aligned(const uint64_t *sa, int ns, const uint64_t *db,
                                             int nd, uint32_t nunits, uint32_t u0) {
  constexpr int kS = Op::kSum ? kMaxRanks : 1;
  const uint32_t tid = threadIdx.x;
  u32x4 x[kU][kS];
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    uint32_t u = u0 + uint32_t(k) * kThreads + tid;
    // The tail pass loads a clamped unit instead of branching around the
    // load: a branch per load would make every load wait for the previous.
    if (kGuard && u >= nunits) u = nunits - 1;
    const uint64_t o = uint64_t(u * 16u);
#pragma unroll
    for (int i = 0; i < kS; ++i) x[k][i] = ld16x<kNTL, kUL>(sa[i] + o);
  }
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    const uint32_t u = u0 + uint32_t(k) * kThreads + tid;
    if (!kGuard || u < nunits) {
      u32x4 v;
      if constexpr (!Op::kSum) v = x[k][0];
      else if constexpr (Op::kElem == 4) v = fold_f32(x[k], ns);
      else v = fold_bf16(x[k], ns);
#pragma unroll
      for (int j = 0; j < kMaxRanks + 1; ++j) {
        if (j < nd) {
          if constexpr (kUS) st16u<kNTS == kStoreNT>(db[j] + uint64_t(u * 16u), v);
          else stm<kNTS>(db[j], u * 16u, v);
        }
      }
    }
  }
}

// Body of a tile, all sources aligned like the destinations: units
// [0, nunits) of 16 bytes, where every destination db[d] is 16-byte
// aligned.  Each lane handles units tid, tid + 256, ...  Addresses are a
// uniform 64-bit base per buffer plus one 32-bit lane offset shared by all
// buffers, so the loads use the scalar-base form and the sources cost no
// per-lane address registers.
// kUS: the destinations are off the 16-byte grid (every source on one
// 16-byte phase, the destinations on another): units follow the sources and
// every store is a misaligned 16-byte store.
template <class Op, int kU, bool kNTL, int kNTS, bool kOne = false, bool kUS = false,
          bool kUL = false>
__device__ __forceinline__ void body_aligned(const uint64_t *sa, int ns, const uint64_t *db,
                                             int nd, uint32_t nunits) {
  static_assert(!kUS || kNTS != kStoreDevice, "misaligned stores have no device-scope form");
  constexpr uint32_t kPass = uint32_t(kThreads) * kU;
  uint32_t u0 = 0;
  if constexpr (!Op::kSum && kOne) {
    if (nd == 1) {
      // One destination: every store of a full pass is unconditional, so
      // each load is consumed in its own pass and a wave's next loads go
      // out while its stores drain (measured +4-5% on AllToAll at 64-256
      // MiB per rank).  Only in the single-destination build: elsewhere the
      // extra path measured slower on AllToAllV and AllGather.
      const uint32_t tid = threadIdx.x;
      for (; u0 + kPass <= nunits; u0 += kPass) {
        u32x4 x[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k)
          x[k] = ld16x<kNTL, kUL>(sa[0] + uint64_t((u0 + uint32_t(k) * kThreads + tid) * 16u));
#pragma unroll
        for (int k = 0; k < kU; ++k) {
          const uint32_t o = (u0 + uint32_t(k) * kThreads + tid) * 16u;
          if constexpr (kUS) st16u<kNTS == kStoreNT>(db[0] + uint64_t(o), x[k]);
          else stm<kNTS>(db[0], o, x[k]);
        }
      }
      if (u0 < nunits) {
        pass_aligned<Op, kU, kNTL, kNTS, true, kUS, kUL>(sa, ns, db, nd, nunits, u0);
        drain_vm();
      }
      return;
    }
  }
  for (; u0 + kPass <= nunits; u0 += kPass)
    pass_aligned<Op, kU, kNTL, kNTS, false, kUS, kUL>(sa, ns, db, nd, nunits, u0);
  if (u0 < nunits) pass_aligned<Op, kU, kNTL, kNTS, true, kUS, kUL>(sa, ns, db, nd, nunits, u0);
}

// ---- LDS-staged body (experimental build) ----------------------------------
// Aligned jobs staged through LDS with gfx950's 16-byte global-to-LDS loads.
// The workgroup's rows (64 units = 1 KiB of each source) go in batches of
// 4 * kR rows; wavefront w takes rows w, w + 4, ... of a batch, loads every
// source row of them straight into its own LDS slice (no VGPR holds data in
// flight), waits once for all of them, reads each lane's units back, folds
// them (sums) and stores them: per wavefront a burst of loads, then a burst
// of stores.  The units after the last whole batch take the register
// passes.  `slice` is this wavefront's kS * kR KiB of LDS.
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

template <class Op, int kR, int kU, bool kNTL, int kNTS>
__device__ __forceinline__ void body_lds(const uint64_t *sa, int ns, const uint64_t *db, int nd,
                                         uint32_t nunits, lds_u32x4 *slice) {
  constexpr int kS = Op::kSum ? kMaxRanks : 1;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = uint32_t(__builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)));
  const uint32_t nrows = nunits >> 6;
  constexpr uint32_t kBatch = 4u * kR;
  uint32_t r0 = 0;
  for (; r0 + kBatch <= nrows; r0 += kBatch) {
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const uint64_t off = (uint64_t(r0 + wave + 4u * uint32_t(k)) * 64u + lane) * 16u;
#pragma unroll
      for (int i = 0; i < kS; ++i)
        __builtin_amdgcn_global_load_lds(gp<const void>(sa[i] + off),
                                         reinterpret_cast<__attribute__((address_space(3))) void *>(
                                             slice + (k * kS + i) * 64),
                                         16, 0, kNTL ? 2 : 0);
    }
    drain_vm();  // every row of the batch is in LDS
    u32x4 v[kR];
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      u32x4 x[kS];
#pragma unroll
      for (int i = 0; i < kS; ++i) x[i] = slice[(k * kS + i) * 64 + int(lane)];
      if constexpr (!Op::kSum) v[k] = x[0];
      else if constexpr (Op::kElem == 4) v[k] = fold_f32(x, ns);
      else v[k] = fold_bf16(x, ns);
    }
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const uint64_t off = (uint64_t(r0 + wave + 4u * uint32_t(k)) * 64u + lane) * 16u;
#pragma unroll
      for (int j = 0; j < kMaxRanks + 1; ++j)
        if (j < nd) stm<kNTS>(db[j], uint32_t(off), v[k]);
    }
  }
  constexpr uint32_t kPass = uint32_t(kThreads) * kU;
  uint32_t u0 = r0 * 64u;
  for (; u0 + kPass <= nunits; u0 += kPass)
    pass_aligned<Op, kU, kNTL, kNTS, false>(sa, ns, db, nd, nunits, u0);
  if (u0 < nunits) pass_aligned<Op, kU, kNTL, kNTS, true>(sa, ns, db, nd, nunits, u0);
}

// Lane l receives lane l + 1's value (lane 63: unspecified).  kDpp: a DPP
// wavefront shift (wave_shl:1), a plain VALU move; else __shfl_down, which
// goes through the LDS crossbar (ds_bpermute).  Copies take the DPP move;
// a sum row keeps the VALU busy (eight sources widened, added and rounded),
// so there the crossbar, which runs beside it, measured faster.
template <bool kDpp>
__device__ __forceinline__ uint32_t next_lane(uint32_t v) {
  if constexpr (kDpp) return uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), 0x130, 0xF, 0xF, false));
  else return __shfl_down(v, 1);
}

template <bool kDpp>
__device__ __forceinline__ u32x4 next_lane(u32x4 v) {
  u32x4 o;
  o.x = next_lane<kDpp>(v.x);
  o.y = next_lane<kDpp>(v.y);
  o.z = next_lane<kDpp>(v.z);
  o.w = next_lane<kDpp>(v.w);
  return o;
}

__device__ __forceinline__ u32x4 lane0(u32x4 v) {
  u32x4 o;
  o.x = __builtin_amdgcn_readfirstlane(v.x);
  o.y = __builtin_amdgcn_readfirstlane(v.y);
  o.z = __builtin_amdgcn_readfirstlane(v.z);
  o.w = __builtin_amdgcn_readfirstlane(v.w);
  return o;
}

// One pass of the row body (see body_rows).  kOne: a single destination
// (a store without the guarded loop over destinations).  kFold (sums whose
// sources all share one 16-byte phase): a block of every source then holds
// the same elements at the same places, so the raw blocks are folded first
// and only the folded block is shifted into place: one shift per unit
// instead of one per source, and the same rounded values.
template <class Op, int kU, bool kNTL, int kNTS, bool kGuard, bool kOne, bool kFold>
__device__ __forceinline__ void pass_rows(const uint64_t *base, const uint32_t *lim, int ns,
                                          const uint64_t *db, int nd, uint32_t nunits,
                                          const uint32_t *sh, uint32_t u0) {
  constexpr int kS = Op::kSum ? kMaxRanks : 1;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = threadIdx.x >> 6;
  const uint32_t r0 = u0 + wave * kU * 64u;  // this wavefront's rows start here
  u32x4 edge[kS];
  u32x4 x[kU][kS];
  // The block after the wavefront's last row, the same address in every
  // lane, first and through the cache (see body_rows).
#pragma unroll
  for (int i = 0; i < kS; ++i) {
    uint32_t b = r0 + uint32_t(kU) * 64u;
    if (b >= lim[i]) b = lim[i] - 1;
    edge[i] = ld16<false>(base[i] + uint64_t(b) * 16u);
  }
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    const uint32_t u = r0 + uint32_t(k) * 64u + lane;
#pragma unroll
    for (int i = 0; i < kS; ++i) {
      const uint32_t b = (kGuard && u >= lim[i]) ? lim[i] - 1 : u;
      x[k][i] = ld16<kNTL>(base[i] + uint64_t(b) * 16u);
    }
  }
  if constexpr (kFold) {
    static_assert(Op::kSum, "folding first applies to sums");
    u32x4 f[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k) f[k] = Op::kElem == 4 ? fold_f32(x[k], ns) : fold_bf16(x[k], ns);
    const u32x4 fe = Op::kElem == 4 ? fold_f32(edge, ns) : fold_bf16(edge, ns);
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const uint32_t u = r0 + uint32_t(k) * 64u + lane;
      const u32x4 after = k + 1 < kU ? lane0(f[k + 1 < kU ? k + 1 : k]) : fe;
      u32x4 hi = next_lane<false>(f[k]);
      if (lane == 63u) hi = after;
      const u32x4 v = funnel(f[k], hi, sh[0]);
      if (!kGuard || u < nunits) {
        const uint32_t o = u * 16u;
        if constexpr (kOne) {
          stm<kNTS>(db[0], o, v);
        } else {
#pragma unroll
          for (int j = 0; j < kMaxRanks + 1; ++j)
            if (j < nd) stm<kNTS>(db[j], o, v);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < kU; ++k) {
    const uint32_t u = r0 + uint32_t(k) * 64u + lane;
    u32x4 y[kS];
#pragma unroll
    for (int i = 0; i < kS; ++i) {
      // lane 63's right neighbour: the next row's first block, or the edge
      const u32x4 after = k + 1 < kU ? lane0(x[k + 1 < kU ? k + 1 : k][i]) : edge[i];
      u32x4 hi = next_lane<!Op::kSum>(x[k][i]);
      if (lane == 63u) hi = after;
      y[i] = funnel(x[k][i], hi, sh[i]);
    }
    if (!kGuard || u < nunits) {
      u32x4 v;
      if constexpr (!Op::kSum) v = y[0];
      else if constexpr (Op::kElem == 4) v = fold_f32(y, ns);
      else v = fold_bf16(y, ns);
      const uint32_t o = u * 16u;
      if constexpr (kOne) {
        stm<kNTS>(db[0], o, v);
      } else {
#pragma unroll
        for (int j = 0; j < kMaxRanks + 1; ++j)
          if (j < nd) stm<kNTS>(db[j], o, v);
      }
    }
  }
}

// Body of a tile when some source is not on the destinations' 16-byte
// phase (variable-length partitions at arbitrary element offsets).  Each
// source is read as aligned 16-byte blocks; a wavefront row loads 64
// consecutive blocks, one per lane, and each lane shifts its block and its
// right neighbour's into place in registers (lane shuffle + v_alignbyte),
// producing the 64 destination units the row covers; each wavefront takes
// kU consecutive rows.  Lane 63 of a row needs one block past the row: the
// next row's first block, read from lane 0, or after the wavefront's last
// row one extra block, which lies in a line another wavefront streams: it
// is loaded first and as an ordinary (cached) load, which measured fewer
// HBM bytes and more bandwidth than a nontemporal one or a hand-over in LDS
// behind a barrier.
// Rows start on a 128-byte line of source 0 for a sum with one destination,
// and on a destination line otherwise.  One side's lines are then split
// between neighbouring rows.  Two nontemporal loads of one line fetch it
// from HBM twice (measured: one line in eight more read traffic for
// ReduceScatterV, even when one wavefront takes both rows back to back),
// while two partial stores to one line mostly merge in L2; so a sum with
// one destination, whose eight source streams are almost all its traffic,
// gets source-aligned rows (ReduceScatterV).  A copy reads one stream, and
// whole-line stores measured faster there: destination-aligned rows for
// AllToAllV (+2-4% at 64 MiB - 1 GiB per rank, paired on the same
// buffers) and for broadcasts (AllGatherV).
// sa[] holds the sources at the first unit; block b of source i is at
// sa[i] - sh[i] + 16 b, and a source with sh[i] > 0 needs block nunits too,
// which holds its last unit's last bytes.  An unguarded pass reads blocks
// up to u0 + kPass, so it needs u0 + kPass < nunits.
template <class Op, int kU, bool kNTL, int kNTS, bool kOne, bool kFoldOk>
__device__ __forceinline__ void body_rows(const uint64_t *sa, int ns, const uint64_t *db, int nd,
                                          uint32_t nunits, const uint32_t *sh) {
  constexpr int kS = Op::kSum ? kMaxRanks : 1;
  constexpr uint32_t kPass = 64u * (kThreads / 64) * kU;
  uint64_t base[kS];
  uint32_t lim[kS];
#pragma unroll
  for (int i = 0; i < kS; ++i) {
    base[i] = sa[i] - sh[i];
    lim[i] = nunits + (sh[i] ? 1u : 0u);
  }
  uint32_t same = 1;
#pragma unroll
  for (int i = 1; i < kS; ++i) same &= sh[i] == sh[0] ? 1u : 0u;
  // Offset of this wavefront's first row in a pass.  The last pass (at most
  // one is guarded) is skipped by a wavefront whose rows all lie past the
  // body, which then issues no loads at all.
  const uint32_t first = uint32_t(__builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6))) * 64u * kU;
  uint32_t u0 = 0;
  if (kFoldOk && Op::kSum && same) {
    constexpr bool kF = kFoldOk && Op::kSum;
    for (; u0 + kPass < nunits; u0 += kPass)
      pass_rows<Op, kU, kNTL, kNTS, false, kOne, kF>(base, lim, ns, db, nd, nunits, sh, u0);
    if (u0 + first < nunits)
      pass_rows<Op, kU, kNTL, kNTS, true, kOne, kF>(base, lim, ns, db, nd, nunits, sh, u0);
    return;
  }
  for (; u0 + kPass < nunits; u0 += kPass)
    pass_rows<Op, kU, kNTL, kNTS, false, kOne, false>(base, lim, ns, db, nd, nunits, sh, u0);
  if (u0 + first < nunits)
    pass_rows<Op, kU, kNTL, kNTS, true, kOne, false>(base, lim, ns, db, nd, nunits, sh, u0);
}

// Body of a sum tile whose sources share one 16-byte phase and whose
// destinations (congruent) sit on another, with aligned stores and no
// block read twice: source-aligned units are loaded and folded, and each
// destination unit is shifted together from a folded unit and the next
// (lane shuffle + v_alignbyte).  Each wavefront takes a contiguous block of
// rows (64 units) and carries a row's folded units until the next row is
// folded, whose first unit lane 63 needs; the unit after a wavefront's last
// row is the first of the next wavefront's block, handed over in LDS behind
// a barrier once per tile.  sa[] / db[]: sources and destinations at the
// body's first source byte (16-byte aligned sources); n16 source units;
// sig = (16 - (db - sa)) % 16, the source offset of the first destination
// unit boundary.  Destination unit k (source bytes 16k + sig ..) is stored
// for k + 1 < n16.  The bytes before unit 0 (source bytes [0, sig)) and
// after unit n16 - 2 (bytes [16 (n16 - 1) + sig, 16 n16)) are written from
// the folded units 0 and n16 - 1 with 2-byte stores when `edges` is set (a
// tile whose source range is whole units: no block is then read again);
// otherwise the caller's element passes cover them.  Every wavefront of the
// workgroup calls it.
template <class Op, bool kNTL, int kNTS, bool kOne>
__device__ __forceinline__ void body_carry(const uint64_t *sa, int ns, const uint64_t *db, int nd,
                                           uint32_t n16, uint32_t sig, bool edges) {
  static_assert(Op::kSum, "the carried row body folds sums");
  __shared__ u32x4 handover[kThreads / 64];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = uint32_t(__builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)));
  constexpr uint32_t kWaves = kThreads / 64;
  const uint32_t nrows = (n16 + 63u) >> 6;
  const uint32_t per = (nrows + kWaves - 1u) / kWaves;
  const uint32_t r0 = wave * per < nrows ? wave * per : nrows;
  const uint32_t r1 = r0 + per < nrows ? r0 + per : nrows;
  auto fold_row = [&](uint32_t r) -> u32x4 {
    uint32_t u = (r << 6) + lane;
    if (u >= n16) u = n16 - 1u;   // past the body: a unit inside it, never stored
    u32x4 x[kMaxRanks];
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) x[i] = ld16<kNTL>(sa[i] + uint64_t(u) * 16u);
    return Op::kElem == 4 ? fold_f32(x, ns) : fold_bf16(x, ns);
  };
  // bytes [b0, b1) of a folded unit (2-byte steps) to destination offset
  // `at` + b of every destination
  auto bytes_of = [&](u32x4 v, uint32_t b0, uint32_t b1, uint32_t at) {
    for (uint32_t b = b0; b < b1; b += 2u) {
      const uint32_t w = b < 4u ? v.x : b < 8u ? v.y : b < 12u ? v.z : v.w;
      const uint16_t h = uint16_t(w >> ((b & 3u) * 8u));
#pragma unroll
      for (int j = 0; j < kMaxRanks + 1; ++j)
        if (j < (kOne ? 1 : nd)) ste<uint16_t, kNTS == kStoreDevice>(db[j] + at + b, h);
    }
  };
  auto emit = [&](uint32_t r, u32x4 v) {
    const uint32_t k = (r << 6) + lane;
    if (k + 1u < n16) {
      const uint32_t o = k * 16u + sig;
      if constexpr (kOne) {
        stm<kNTS>(db[0], o, v);
      } else {
#pragma unroll
        for (int j = 0; j < kMaxRanks + 1; ++j)
          if (j < nd) stm<kNTS>(db[j], o, v);
      }
    }
  };
  // the previous tile's last reads of the handover are done
  __syncthreads();
  u32x4 cur{0u, 0u, 0u, 0u};
  if (r0 < r1) {
    cur = fold_row(r0);
    if (lane == 0u) handover[wave] = cur;
    if (edges && r0 == 0u && lane == 0u) bytes_of(cur, 0u, sig, 0u);   // head
    for (uint32_t r = r0; r + 1u < r1; ++r) {
      const u32x4 nxt = fold_row(r + 1u);
      // read lane 0 with every lane active (under lane == 63 alone, the
      // first active lane would be lane 63)
      const u32x4 first = lane0(nxt);
      u32x4 hi = next_lane<false>(cur);
      if (lane == 63u) hi = first;
      emit(r, funnel(cur, hi, sig));
      cur = nxt;
    }
  }
  __syncthreads();   // every wavefront's first unit is in LDS
  if (r0 < r1) {
    // the unit after this block: the next block's first (a wavefront whose
    // block is last stores no unit that needs it)
    const uint32_t w1 = wave + 1u < kWaves ? wave + 1u : wave;
    u32x4 hi = next_lane<false>(cur);
    if (lane == 63u) hi = handover[w1];
    emit(r1 - 1u, funnel(cur, hi, sig));
    // tail: the block holding the last unit writes its bytes past sig
    if (edges && r1 == nrows && lane == ((n16 - 1u) & 63u))
      bytes_of(cur, sig, 16u, (n16 - 1u) * 16u);
  }
}

// Whether a job's rows are aligned to its sources: a sum with one
// destination, and some source off the destination's 16-byte phase (the
// offset between a source and the destination is the same at every byte of
// a job).
template <class Op>
__device__ __forceinline__ bool src_rows(const Srcs &s, const Dsts &d) {
  if constexpr (!Op::kSum) return false;
  if (d.n != 1) return false;
  uint32_t any = 0;
#pragma unroll
  for (int i = 0; i < kMaxRanks; ++i) any |= uint32_t(s.a[i] - d.b[0]) & 15u;
  return any != 0;
}

// The address whose 128-byte lines a job's tile boundaries follow (a
// boundary x satisfies (line_ref + x) % 128 == 0): the destination's, or for
// rows aligned to the sources the destination shifted so that at a boundary the
// destination is on a 16-byte unit and source 0's block containing it
// starts a 128-byte line.  Then a full tile is whole source-aligned rows
// with no head pass.  With e = (dst - src0) mod 128 the boundary sits where
// the destination is at ceil16(e) mod 128, and src0 there is < 16 bytes
// past a line start.
// Whether a job's tiles take source-aligned units with misaligned stores
// (the launch allows it, every source sits on one 16-byte phase and the
// destinations on another).
__device__ __forceinline__ bool shifted_stores(const Srcs &s, const Dsts &d, bool allow) {
  if (!allow) return false;
  uint32_t spread = 0;
#pragma unroll
  for (int i = 1; i < kMaxRanks; ++i) spread |= uint32_t(s.a[i] - s.a[0]) & 15u;
  return spread == 0 && (uint32_t(d.b[0] - s.a[0]) & 15u) != 0;
}

template <class Op>
__device__ __forceinline__ uint64_t line_ref(const Srcs &s, const Dsts &d, bool shift_stores = false) {
  if (shifted_stores(s, d, shift_stores)) return s.a[0];
  if (!src_rows<Op>(s, d)) return d.b[0];
  const uint32_t e = uint32_t(d.b[0] - s.a[0]) & 127u;
  return d.b[0] - uint64_t((e + 15u) & 112u);
}

// One tile: job bytes [x0, x1).  kFoldOk: sum rows whose sources share one
// phase may fold before shifting (more registers; the staged kernel, whose
// owner mixes its own input with staging slots, leaves it out).  kRows =
// false builds the tile without the row bodies, for launches whose every
// job is aligned: a smaller kernel.  kNTS: nontemporal stores in the body
// (kNT by default; broadcasts store plainly).  kWide builds in the wide element pass
// for small misaligned tiles (its registers would cost the staged kernel,
// which never takes it, a workgroup per CU of occupancy).  x0 is 0 or on a 128-byte boundary of the
// job's line_ref, x1 is the job's end or on such a boundary.  Layout:
//   [x0, xh)   the head, < 128 bytes: the bytes before the first 16-byte
//              unit of the destination and the units before the first row
//              start (a destination line, or with rows aligned to the
//              sources a unit whose source-0 block starts a line); element
//              operations on wavefront 0, or on wavefront 2 when a row body
//              leaves it idle
//   [xh, xb)   the body: whole units, nontemporal stores when kNT
//   [xb, x1)   < 16 bytes of tail: element operations on wavefront 3, in
//              parallel with the head
// A tile of at most one element per thread is one element pass.  Loads are
// nontemporal when every source sits on the destinations' 128-byte phase,
// or when nt_any_phase asks for it (measured faster for misaligned
// variable-length partitions too).  A tile spans less than 4 GiB.
template <class Op, int kU, bool kNT, bool kFoldOk = true, bool kRows = true, bool kOne = false,
          bool kWide = false, int kNTS = kNT, int kLdsRows = 0>
__device__ __forceinline__ void tile(const Srcs &s, const Dsts &d, int64_t x0, int64_t x1,
                                     bool nt_any_phase = false, int64_t wide_max = 0,
                                     bool shift_stores = false, lds_u32x4 *lds_slice = nullptr,
                                     bool unaligned_loads = false, bool carry_rows = false) {
  constexpr bool kDev = kNTS == kStoreDevice;
  static_assert(!(kDev && kLdsRows > 0), "the LDS body has no device-scope stores");
  if (x1 <= x0) return;
  if (x1 - x0 <= int64_t(kThreads) * Op::kElem) {
    elements<Op, kDev>(s, d, x0, x1);
    return;
  }
  if constexpr (kRows && !kDev) {
    if (shifted_stores(s, d, shift_stores)) {
      // Every source on one 16-byte phase, the destinations on another:
      // units follow the sources (the loads are the aligned body's, with no
      // realignment in registers) and the stores are misaligned.  Head and
      // tail (< 16 bytes each) are element passes.
      const int64_t xs =
          x0 + int64_t((16u - uint32_t((s.a[0] + uint64_t(x0)) & 15u)) & 15u);
      const uint32_t n16 = uint32_t((x1 - xs) >> 4);
      const int64_t xe = xs + int64_t(n16) * 16;
      uint64_t sa[kMaxRanks], db[kMaxRanks + 1];
#pragma unroll
      for (int i = 0; i < kMaxRanks; ++i) sa[i] = s.a[i] + uint64_t(xs);
#pragma unroll
      for (int j = 0; j < kMaxRanks + 1; ++j) db[j] = d.b[j] + uint64_t(xs);
      if constexpr (Op::kSum) {
        if (carry_rows && n16 >= 2u) {
          // aligned stores from carried rows: the element passes take the
          // bytes before the first destination unit and after the last
          const uint32_t sig = (16u - uint32_t(db[0] & 15u)) & 15u;
          // a tile whose source range is whole units (every tile but a
          // job's ragged first and last) writes its edges from registers
          const bool edges = xs == x0 && xe == x1;
          if (!edges) {
            elements<Op>(s, d, x0, xs + int64_t(sig));
            elements<Op>(s, d, xs + int64_t(n16 - 1u) * 16 + int64_t(sig), x1, kThreads - 64);
          }
          if (kNT && nt_any_phase) body_carry<Op, true, kNTS, kOne>(sa, s.n, db, d.n, n16, sig, edges);
          else body_carry<Op, false, kNTS, kOne>(sa, s.n, db, d.n, n16, sig, edges);
          return;
        }
      }
      elements<Op>(s, d, x0, xs);
      elements<Op>(s, d, xe, x1, kThreads - 64);
      if (kNT && nt_any_phase) body_aligned<Op, kU, true, kNTS, kOne, true>(sa, s.n, db, d.n, n16);
      else body_aligned<Op, kU, false, kNTS, kOne, true>(sa, s.n, db, d.n, n16);
      return;
    }
  }
  if constexpr (kRows && kWide) {
    // In the latency regime (the launch sets wide_max), a single-
    // destination tile that would take a row body (some source off the
    // destination's 16-byte phase) is one wide element pass instead: one
    // round trip, and none of the row body's much larger code to fetch.
    // A broadcast would store every element to each destination
    // separately, and at larger sizes the 2-byte accesses cost more than
    // the row body's 16-byte ones: those keep the row body.
    uint32_t off = 0;
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i) off |= uint32_t(s.a[i] - d.b[0]) & 15u;
    if (off != 0 && d.n == 1 && x1 - x0 <= wide_max &&
        x1 - x0 <= int64_t(kThreads) * Op::kElem * kWideElems) {
      elements_wide<Op, kWideElems, kDev>(s, d, x0, x1);
      return;
    }
  }
  // from here on the tile holds more than 16 units, so the head (< 8 units
  // past x16) leaves a non-empty body
  const uint64_t b0 = d.b[0];
  const int64_t x16 = x0 + int64_t((16u - uint32_t((b0 + uint64_t(x0)) & 15u)) & 15u);
  const uint32_t nall = uint32_t((x1 - x16) >> 4);
  const int64_t xb = x16 + int64_t(nall) * 16;
  uint64_t sa[kMaxRanks];
  uint64_t db[kMaxRanks + 1];
  uint32_t sh[kMaxRanks];
  uint32_t any = 0, phase = 0;
#pragma unroll
  for (int i = 0; i < kMaxRanks; ++i) {
    sa[i] = s.a[i] + uint64_t(x16);
    sh[i] = uint32_t(sa[i] & 15u);
    any |= sh[i];
    phase |= uint32_t((s.a[i] - b0) & 127u);
  }
  const bool srows = src_rows<Op>(s, d);
  // units before the first row start
  const uint64_t line = srows ? sa[0] - sh[0] : b0 + uint64_t(x16);
  uint32_t nh = ((128u - uint32_t(line & 127u)) & 127u) >> 4;
  if (nh > nall) nh = nall;
  const int64_t xh = x16 + int64_t(nh) * 16;
  const uint32_t nbody = nall - nh;
  // a sum holds eight sources per row, so two rows per wavefront (more
  // measured slower); a copy holds one and takes the tile's unroll
#ifndef PURLIN_SUM_ROWS
#define PURLIN_SUM_ROWS 2
#endif
  constexpr int kUr = Op::kSum ? PURLIN_SUM_ROWS : kU;
  // The head goes to wavefront 2 when the row body leaves wavefronts 2 and
  // 3 without rows (small tiles, the latency regime), so that no wavefront
  // makes two round trips; otherwise to wavefront 0.
  const int t_head = (kRows && any != 0 && nbody <= 2u * uint32_t(kUr) * 64u) ? 128 : 0;
  elements<Op, kDev>(s, d, x0, xh, t_head);
  elements<Op, kDev>(s, d, xb, x1, kThreads - 64);
  if (nbody == 0) return;
#pragma unroll
  for (int i = 0; i < kMaxRanks; ++i) sa[i] += uint64_t(nh) * 16u;
#pragma unroll
  for (int j = 0; j < kMaxRanks + 1; ++j) db[j] = d.b[j] + uint64_t(xh);
  const bool ntl = kNT && (phase == 0 || nt_any_phase);
  if (any == 0) {
    if constexpr (kLdsRows > 0) {
      if (ntl) body_lds<Op, kLdsRows, kU, true, kNTS>(sa, s.n, db, d.n, nbody, lds_slice);
      else body_lds<Op, kLdsRows, kU, false, kNTS>(sa, s.n, db, d.n, nbody, lds_slice);
      return;
    }
    if (ntl) body_aligned<Op, kU, true, kNTS, kOne>(sa, s.n, db, d.n, nbody);
    else body_aligned<Op, kU, false, kNTS, kOne>(sa, s.n, db, d.n, nbody);
    return;
  }
  if constexpr (kRows) {
    if (unaligned_loads) {
      // Destination-aligned units whose sources are read with misaligned
      // 16-byte loads (no lane shuffles, no block past a row; lines at the
      // ends of a wavefront's range may be read twice).
      if (ntl) body_aligned<Op, kU, true, kNTS, kOne, false, true>(sa, s.n, db, d.n, nbody);
      else body_aligned<Op, kU, false, kNTS, kOne, false, true>(sa, s.n, db, d.n, nbody);
      return;
    }
  }
  if constexpr (!kRows) {
    // Built without the row bodies (the launch checked that every job is
    // aligned); should a misaligned tile arrive anyway, it is still right,
    // element by element.
    for (int64_t y = xh; y < xb; y += int64_t(kThreads) * Op::kElem)
      elements<Op, kDev>(s, d, y, y + int64_t(kThreads) * Op::kElem < xb ? y + int64_t(kThreads) * Op::kElem : xb);
    return;
  }
  if (d.n == 1) {
    if (ntl) body_rows<Op, kUr, true, kNTS, true, kFoldOk>(sa, s.n, db, 1, nbody, sh);
    else body_rows<Op, kUr, false, kNTS, true, kFoldOk>(sa, s.n, db, 1, nbody, sh);
  } else {
    if (ntl) body_rows<Op, kUr, true, kNTS, false, kFoldOk>(sa, s.n, db, d.n, nbody, sh);
    else body_rows<Op, kUr, false, kNTS, false, kFoldOk>(sa, s.n, db, d.n, nbody, sh);
  }
}

}  // namespace atom
}  // namespace purlin
