// Launch plan shared by the host planner and the device kernels.
//
// A collective (Purlin, abstract: input naming, output naming, copy or sum)
// is derived into at most P*P jobs.  A job produces `nbytes` bytes: byte x of
// it is op(src_i[x] for each source i in ascending rank) written to every
// destination.  Sources are one rank or every rank (a sum in rank order);
// destinations are one rank or every rank (a broadcast).  Each job is cut
// into chunks ("tiles") of chunk_bytes of destination bytes; chunk
// boundaries sit on 16-byte boundaries of the destination so that every
// chunk body is whole 16-byte units.
#pragma once
#include <stdint.h>

namespace purlin {

constexpr int kMaxRanks = 8;
constexpr int kMaxJobs = kMaxRanks * kMaxRanks;
constexpr int kThreads = 256;           // 4 wavefronts of 64
constexpr int kFlagStride = 32;          // u32 words between flags (128 bytes)
// The exit count of a launch is spread over this many counters (workgroup b
// counts on b % kExitSlots): one counter taking an atomic add from each of
// ~1000 workgroups serialises them, measured at ~18 us per launch.  The
// workgroup that completes a counter then adds one to a second-level
// counter, and the one that completes that is the launch's last.
constexpr int kExitSlots = 32;

// Flag block of one stream's workspace (u32 words, each flag on its own
// 128-byte line).  The block starts zeroed.
enum FlagWord : int {
  kFlagEntry = 0,                                         // kMaxRanks entry epochs
  kFlagExit = kMaxRanks * kFlagStride,                    // kExitSlots exit counters
  kFlagExitTop = (kMaxRanks + kExitSlots) * kFlagStride,  // completed exit counters
  kFlagEpoch = (kMaxRanks + kExitSlots + 1) * kFlagStride,   // epoch of the next launch, minus one
  kFlagStatus = (kMaxRanks + kExitSlots + 2) * kFlagStride,  // sticky device status bits
  kFlagAbort = (kMaxRanks + kExitSlots + 3) * kFlagStride,   // epoch of an aborted launch
  kFlagWords = (kMaxRanks + kExitSlots + 4) * kFlagStride,
};

// Word of exit counter `slot`.
constexpr int exit_word(int slot) { return kFlagExit + slot * kFlagStride; }
constexpr uint32_t kStatusTimeout = 1u;
constexpr uint32_t kStatusBadArg = 2u;   // a device-side argument check failed (MoE indices)
constexpr uint32_t kStatusProtocol = 4u; // a protocol check of the debug build failed

struct Job {
  int64_t src_off;  // byte offset into in[src] (into every in[i] when src < 0)
  int64_t dst_off;  // byte offset into out[dst] (into every out[j] when dst < 0)
  int64_t nbytes;
  int32_t src;      // source rank, or -1: every rank, summed in ascending order
  int32_t dst;      // destination rank, or -1: every rank
};

// Staged (SNAC) role layout: for each job, per lane, one owner workgroup,
// one stager per source other than the owner, and one scatter consumer per
// destination other than the owner.
struct StagedJob {
  int16_t owner;        // rank that combines the chunk (reducer / root)
  int16_t n_stage;      // sources other than the owner (0 or P-1)
  int16_t n_scatter;    // destinations other than the owner (0 or P-1)
  int16_t team;         // owner workgroups per lane, each combining 1/team of a chunk
  int32_t role_begin;   // first workgroup of this job
  int32_t ring_begin;   // first ring of this job
};

struct LaunchPlan {
  const char *in[kMaxRanks];
  char *out[kMaxRanks];
  uint32_t *flags;          // the stream's flag block (kFlagWords u32 words), or null for a
                            // launch that uses no flag (zero staging without the handshake)
  int32_t P;
  int32_t njobs;
  int32_t total_tiles;
  int32_t sync;             // 1: entry / exit notify (the full per-rank handshake)
  int64_t chunk_bytes;      // bytes per tile (multiple of 4096)
  uint64_t watchdog_ticks;  // bound of every spin wait, in wall-clock ticks
  int32_t nt_any_phase;     // 1: nontemporal loads even for sources off the line phase
  int32_t wide_max;         // tiles up to this many bytes that would take a row body
                            // take one wide element pass instead (0: never)
  int32_t shift_stores;     // 1: jobs whose sources share a 16-byte phase off their
                            // destinations' take source-aligned units, misaligned stores;
                            // 2: the same units shifted into aligned stores (body_carry)
  int32_t unaligned_loads;  // 1: jobs with a source off their destinations' 16-byte phase take
                            // destination-aligned units, misaligned loads
  int32_t tile_begin[kMaxJobs + 1];
  Job jobs[kMaxJobs];
};

struct StagedPlan {
  LaunchPlan base;
  char *ring;               // staging rings
  uint64_t *slot_flags;     // per slot (256 bytes): ready words at [32*s + t] (one per owner
                            // of the team), credit at [32*s + 16] (u64)
  int64_t slot_stride;      // bytes per slot (chunk_bytes + 256)
  int32_t depth;            // slots per ring
  int32_t lanes;            // parallel rings per (job, source)
  int32_t total_roles;      // grid size
  int32_t withhold;         // test only: > 0 withholds that ready notify of ring 0
  StagedJob sj[kMaxJobs];
};

// MoE dispatch / combine (expert parallelism, Table 2 of the Purlin pages):
// AllToAllV whose rows are gathered by token index, and its reverse with a
// weighted sum per token.  base.jobs[i * P + j] is the pair (source rank i,
// destination rank j): src_off = first entry of group j in idx[i], dst_off =
// byte offset of the pair's rows in y[j], nbytes = rows * row_bytes;
// base.tile_begin is the row prefix over the pairs (a tile is one row).
struct MoePlan {
  LaunchPlan base;               // in = x (dispatch) or y (combine), out = y or out
  const int32_t *idx[kMaxRanks]; // token index of each entry, grouped by destination
  const float *w[kMaxRanks];     // combine weight of each entry
  uint64_t *inv;                 // combine: (token, destination rank) -> tagged entry
  int64_t inv_base[kMaxRanks + 1];  // first token row of rank i in inv (prefix of x_rows)
  int64_t ent_base[kMaxRanks + 1];  // first entry of rank i in the entry numbering
  int64_t x_rows[kMaxRanks];
  int64_t row_bytes;
};

// Strided-row AllToAll: the Ulysses exchange between sequence-sharded and
// head-sharded activations (Table 2 of the Purlin pages, the diffusion
// workload).  base.jobs[q] moves rows of row_bytes bytes from rank jobs[q].src
// to rank jobs[q].dst: row k is read at in[src] + src_off + k * src_stride and
// written at out[dst] + dst_off + k * dst_stride, nbytes = rows * row_bytes.
// Work is counted in units of `unit` bytes, the largest power of two up to 16
// that divides every row size, stride, offset and buffer address; a tile is
// chunk_bytes of the pair's rows laid end to end.
struct StridedPlan {
  LaunchPlan base;
  int64_t row_bytes;
  int64_t src_stride;
  int64_t dst_stride;
  uint32_t magic;   // row of unit u (u < 2^31) = (u * magic) >> shift
  int32_t shift;
};

static_assert(sizeof(LaunchPlan) <= 3072, "launch plan must fit in kernel arguments");
static_assert(sizeof(MoePlan) <= 3840, "MoE plan must fit in kernel arguments");
static_assert(sizeof(StridedPlan) <= 3840, "strided plan must fit in kernel arguments");
static_assert(sizeof(StagedPlan) <= 3840, "staged plan must fit in kernel arguments");

}  // namespace purlin
