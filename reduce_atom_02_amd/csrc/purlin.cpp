// C ABI of the collective library: argument checks, policy, workspace and
// launch.  Semantics are documented in include/purlin.h.
#include "../../include/purlin.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <vector>

#include "collective.hpp"
#include "kernels.hpp"
#include "planner.hpp"

namespace purlin {
namespace {

constexpr int64_t kDefaultWatchdogNs = 2000000000;  // 2 s
constexpr int kMaxLanes = 256;
// Owner workgroups per lane of a staged reduction (PURLIN_OWNER_TEAM
// overrides, 1 - kMaxTeam): each combines a slice of every chunk.
constexpr int kOwnerTeam = 8;
constexpr int kMaxTeam = 8;

// Library workspace of one stream: the flag block (entry flags, exit
// counters, epoch, status, abort) and, when a call needs them, the staging
// rings with their slot flags and the MoE inverse table.  Calls on one
// stream run one after another (stream order), so they may share it; calls
// on different streams use different workspaces and never wait for each
// other.
struct StreamCtx {
  hipStream_t stream = nullptr;
  uint32_t *flags = nullptr;
  char *ring = nullptr;
  int64_t ring_bytes = 0;
  uint64_t *slot_flags = nullptr;
  int64_t slot_flag_bytes = 0;
  uint64_t *inv = nullptr;     // MoE: (token, destination rank) -> tagged entry
  int64_t inv_bytes = 0;
};

struct DeviceState {
  bool ready = false;
  int cus = 0;
  uint64_t wall_khz = 0;
  std::vector<std::unique_ptr<StreamCtx>> ctx;
  // Outgrown workspace: launches enqueued earlier, or HIP graphs captured
  // earlier, may still use it, so it is freed only by purlin_release.
  std::vector<void *> retired;
  int occ[3][2][2][3][2][2][2][2][2] = {};  // resident workgroups per CU, by kernel; 0 = not asked yet
};

std::vector<DeviceState> &devices() {
  static std::vector<DeviceState> d;
  return d;
}

purlin_policy &user_policy() {
  static purlin_policy p{};
  return p;
}
bool g_user_policy_set = false;
// What the calling host thread launched last (purlin_last_launch).
thread_local purlin_launch_info g_last{};
thread_local bool g_have_last = false;

// One lock over the library's host state (device and stream workspace, the
// plan cache, the policy, the fixed scratch's addresses): calls from several
// host threads are serialized here; the launches stay asynchronous.
std::recursive_mutex &api_mutex() {
  static std::recursive_mutex m;
  return m;
}

int64_t env_i64(const char *name, int64_t dflt) {
  const char *v = std::getenv(name);
  if (!v || !*v) return dflt;
  char *end = nullptr;
  long long x = std::strtoll(v, &end, 0);
  return (end && *end == 0) ? int64_t(x) : dflt;
}

bool policy_valid(const purlin_policy &p) {
  if (p.chunk_bytes < 0 || (p.chunk_bytes % 4096) != 0 || p.chunk_bytes > (int64_t(64) << 20))
    return false;
  if (p.depth < 0 || p.depth > 8) return false;
  if (p.wgs_per_rank < 0 || p.wgs_per_rank > 4096) return false;
  if (p.zero_staging < 0 || p.zero_staging > 2) return false;
  if (p.sync < 0 || p.sync > 2) return false;
  if (p.watchdog_ns < 0 || p.test_withhold < 0) return false;
  if (p.engine < PURLIN_ENGINE_AUTO || p.engine > PURLIN_ENGINE_COPY) return false;
  return true;
}

// Defaults, then environment overrides, then purlin_set_policy fields.
purlin_policy effective_policy() {
  purlin_policy p{};
  p.chunk_bytes = env_i64("PURLIN_CHUNK_BYTES", 0);
  p.depth = int32_t(env_i64("PURLIN_DEPTH", 0));
  p.wgs_per_rank = int32_t(env_i64("PURLIN_WGS_PER_RANK", 0));
  const int64_t zs = env_i64("PURLIN_ZS", -1);
  p.zero_staging = zs < 0 ? PURLIN_STAGING_AUTO : (zs ? PURLIN_STAGING_ZS : PURLIN_STAGING_STAGED);
  const int64_t sy = env_i64("PURLIN_SYNC", -1);
  p.sync = sy < 0 ? 0 : (sy ? 1 : 2);
  p.watchdog_ns = env_i64("PURLIN_WATCHDOG_NS", 0);
  p.engine = int32_t(env_i64("PURLIN_ENGINE", 0));
  if (!policy_valid(p)) p = purlin_policy{};
  if (g_user_policy_set) {
    const purlin_policy &u = user_policy();
    if (u.chunk_bytes) p.chunk_bytes = u.chunk_bytes;
    if (u.depth) p.depth = u.depth;
    if (u.wgs_per_rank) p.wgs_per_rank = u.wgs_per_rank;
    if (u.zero_staging) p.zero_staging = u.zero_staging;
    if (u.sync) p.sync = u.sync;
    if (u.watchdog_ns) p.watchdog_ns = u.watchdog_ns;
    if (u.engine) p.engine = u.engine;
    p.test_withhold = u.test_withhold;
  }
  return p;
}

bool nt_env(bool dflt) {
  const int64_t v = env_i64("PURLIN_NT", -1);
  return v < 0 ? dflt : v != 0;
}
int unroll_env() { return int(env_i64("PURLIN_UNROLL", -1)); }

purlin_status device_state(DeviceState **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PURLIN_ERR_HIP;
  auto &all = devices();
  if (int(all.size()) <= dev) all.resize(dev + 1);
  DeviceState &s = all[dev];
  if (!s.ready) {
    int cus = 0, khz = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
      return PURLIN_ERR_HIP;
    s.cus = cus;
    s.wall_khz = uint64_t(khz > 0 ? khz : 100000);
    s.ready = true;
  }
  *out = &s;
  return PURLIN_OK;
}

// Nothing is allocated or cleared on a stream that is being captured into a
// HIP graph: a call that would need that returns UNSUPPORTED.
purlin_status refuse_if_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return PURLIN_ERR_HIP;
  return cs == hipStreamCaptureStatusNone ? PURLIN_OK : PURLIN_ERR_UNSUPPORTED;
}

StreamCtx *find_ctx(DeviceState &ds, hipStream_t stream) {
  for (auto &c : ds.ctx)
    if (c->stream == stream) return c.get();
  return nullptr;
}

// The stream's workspace, created on its first call that needs one: the flag
// block is allocated and cleared in stream order (no device synchronization).
purlin_status stream_ctx(DeviceState &ds, hipStream_t stream, StreamCtx **out) {
  if ((*out = find_ctx(ds, stream))) return PURLIN_OK;
  purlin_status st = refuse_if_capturing(stream);
  if (st != PURLIN_OK) return st;
  void *f = nullptr;
  const size_t bytes = size_t(kFlagWords) * sizeof(uint32_t);
  if (hipMalloc(&f, bytes) != hipSuccess) return PURLIN_ERR_NO_MEMORY;
  if (hipMemsetAsync(f, 0, bytes, stream) != hipSuccess) {
    ds.retired.push_back(f);
    return PURLIN_ERR_HIP;
  }
  auto c = std::make_unique<StreamCtx>();
  c->stream = stream;
  c->flags = static_cast<uint32_t *>(f);
  ds.ctx.push_back(std::move(c));
  *out = ds.ctx.back().get();
  return PURLIN_OK;
}

// Grow a workspace buffer to `want` bytes: a new allocation (cleared in
// stream order when `zero`), the old one retired.
purlin_status grow(DeviceState &ds, hipStream_t stream, void **buf, int64_t *have, int64_t want,
                   bool zero) {
  if (want <= *have) return PURLIN_OK;
  purlin_status st = refuse_if_capturing(stream);
  if (st != PURLIN_OK) return st;
  void *b = nullptr;
  if (hipMalloc(&b, size_t(want)) != hipSuccess) return PURLIN_ERR_NO_MEMORY;
  if (zero && hipMemsetAsync(b, 0, size_t(want), stream) != hipSuccess) {
    ds.retired.push_back(b);
    return PURLIN_ERR_HIP;
  }
  if (*buf) ds.retired.push_back(*buf);
  *buf = b;
  *have = want;
  return PURLIN_OK;
}

int occupancy(DeviceState &s, KernelKind kind, bool staged, bool nt, int unroll_sel, bool rows,
              bool one, bool wide, bool bcast, bool dstore = false) {
  int &o = s.occ[int(kind)][staged ? 1 : 0][nt ? 1 : 0][unroll_sel][rows ? 1 : 0][one ? 1 : 0]
                [wide ? 1 : 0][bcast ? 1 : 0][dstore ? 1 : 0];
  if (o == 0) {
    int b = 0;
    if (max_resident_per_cu(kind, staged, nt, unroll_sel, rows, one, wide, bcast, dstore, &b) !=
            hipSuccess ||
        b < 1)
      b = 1;
    o = b;
  }
  return o;
}

purlin_status ensure_staging(DeviceState &ds, StreamCtx &c, int64_t ring_bytes, int64_t flag_bytes) {
  purlin_status st = grow(ds, c.stream, reinterpret_cast<void **>(&c.ring), &c.ring_bytes,
                          ring_bytes, false);
  if (st != PURLIN_OK) return st;
  return grow(ds, c.stream, reinterpret_cast<void **>(&c.slot_flags), &c.slot_flag_bytes,
              flag_bytes, true);
}

// The MoE inverse table, cleared when (re)allocated; its entries carry the
// launch epoch, so it is never cleared again.
purlin_status ensure_inverse(DeviceState &ds, StreamCtx &c, int64_t bytes) {
  return grow(ds, c.stream, reinterpret_cast<void **>(&c.inv), &c.inv_bytes, bytes, true);
}

KernelKind kind_of(purlin_op op, purlin_dtype dtype) {
  if (op == PURLIN_OP_COPY) return KernelKind::kCopy;
  return dtype == PURLIN_F32 ? KernelKind::kSumF32 : KernelKind::kSumBf16;
}

// Policy table (Figure 1 caption: policies chosen with the hardware in mind
// decide how a collective runs), from sweeps of grid, chunk and unroll at
// 1 MiB - 1 GiB per rank on MI355X (256 CUs), the policies alternated call
// by call on the same buffers.  Large messages
// want two workgroups per CU (fewer concurrent DRAM streams), smaller ones
// four (each workgroup has few tiles, so more of them overlap more round
// trips); the crossover, in bytes of jobs per launch (the per-rank size T
// for the reductions and broadcasts, P x T for AllToAll), differs by kind:
//   reductions  16 KiB chunks; four per CU below 16 MiB (AllReduce 5-8%,
//               ReduceScatter 5-6% faster at 4-8 MiB per rank), two from
//               there (at 16-32 MiB the two grids traded places between
//               sweeps; ReduceScatter 2.5% faster on two at 64 MiB);
//   broadcasts  16 KiB chunks; four per CU below 16 MiB (AllGather 12-16%,
//               AllGatherV 8-15% faster at 4-8 MiB), two from there
//               (AllGatherV 4% faster at 16 MiB, AllGather 1-4% at 32-64);
//   copies      32 KiB chunks; four per CU below 32 MiB (1 MiB per rank:
//               14 us against 17 us), two from there (AllToAll +2-3%,
//               AllToAllV +4-9% at 64 MiB - 1 GiB per rank).
// Grids of 1.5 or 2.5 workgroups per CU measured 2-8% slower than either
// neighbour.  The grid is a whole-device figure (all P ranks share one
// GPU), so it does not shrink for P < 8; it is given in workgroups per CU.
struct AutoPolicy {
  int grid;
  int64_t chunk;
  int unroll_sel;
};

AutoPolicy auto_policy(KernelKind kind, bool broadcast, int64_t job_bytes, int cus) {
  const int64_t MiB = int64_t(1) << 20;
  if (kind != KernelKind::kCopy) return {(job_bytes >= 16 * MiB ? 2 : 4) * cus, 16 << 10, 0};
  if (broadcast) return {(job_bytes >= 16 * MiB ? 2 : 4) * cus, 16 << 10, 0};
  return {(job_bytes >= 32 * MiB ? 2 : 4) * cus, 32 << 10, 0};
}

// Small messages get smaller chunks, so that the default grid still sees
// about four chunks per workgroup; never below 4 KiB.
int64_t fit_chunk(int64_t chunk, int64_t job_bytes, int64_t grid, int64_t per_wg = 4,
                  int64_t floor = 4096) {
  while (chunk > floor && job_bytes / chunk < grid * per_wg) chunk /= 2;
  return chunk;
}

// Chunk of a zero-staging launch below the large-message regime, from grid
// x chunk sweeps at 1 - 32 MiB per rank (then paired on the same buffers):
// point-to-point copies (AllToAll(V)) with less than 32 MiB of jobs take
// one tile per workgroup, up to the 32 KiB chunk, instead of four (AllToAll
// 17-38%, AllToAllV 20-51% faster at 1-2 MiB per rank: fewer, longer
// tiles); copy broadcasts (AllGather(V)) of 2 - 16 MiB of jobs take no
// chunk below 8 KiB (AllGatherV 4-16% faster at 4-8 MiB per rank).  The
// sums keep four tiles per workgroup down to 4 KiB.
int64_t auto_chunk(KernelKind kind, bool broadcast, int64_t job_bytes, int64_t chunk,
                   int64_t grid) {
  const int64_t MiB = int64_t(1) << 20;
  const bool mid = env_i64("PURLIN_MID_CHUNKS", 1) != 0;
  if (mid && kind == KernelKind::kCopy && !broadcast && job_bytes < 32 * MiB)
    return fit_chunk(chunk, job_bytes, grid, 1, job_bytes > MiB / 2 ? 16384 : 4096);
  if (mid && kind == KernelKind::kCopy && broadcast && job_bytes >= 2 * MiB &&
      job_bytes < 16 * MiB)
    return fit_chunk(chunk, job_bytes, grid, 4, 8192);
  return fit_chunk(chunk, job_bytes, grid);
}

void fill_tiles(LaunchPlan &lp, const std::vector<Job> &jobs, int64_t chunk) {
  lp.njobs = int32_t(jobs.size());
  int64_t t = 0;
  for (size_t k = 0; k < jobs.size(); ++k) {
    lp.jobs[k] = jobs[k];
    lp.tile_begin[k] = int32_t(t);
    t += std::max<int64_t>(1, (jobs[k].nbytes + chunk - 1) / chunk);
  }
  lp.tile_begin[jobs.size()] = int32_t(t);
  for (size_t k = jobs.size() + 1; k <= size_t(kMaxJobs); ++k) lp.tile_begin[k] = int32_t(t);
  lp.total_tiles = int32_t(t);
}

// Shared argument checks and plan of the MoE entry points.  counts[i * P + j]
// rows go from rank i to rank j; rank i's entries (idx[i], w[i]) are the
// groups j = 0 .. P-1 in turn; pair (i, j)'s rows sit in the exchanged
// buffer of rank j after those of ranks 0 .. i-1.
purlin_status moe_plan(void *const *rowsrc, void *const *rowdst, int P, int64_t row_bytes,
                       const int32_t *const *idx, const int64_t *counts, const int64_t *x_rows,
                       bool combine, MoePlan *m, int64_t *total_rows, int64_t *y_rows_out) {
  // a row is one tile, and a tile spans less than 4 GiB (rows up to 1 GiB)
  if (!rowsrc || !rowdst || !idx || !counts || !x_rows || P < 1 || P > kMaxRanks ||
      row_bytes <= 0 || (row_bytes & 1) || row_bytes > (int64_t(1) << 30))
    return PURLIN_ERR_INVALID_ARG;
  int64_t n_ent[kMaxRanks] = {}, y_rows[kMaxRanks] = {};
  int64_t total = 0, x_total = 0;
  for (int i = 0; i < P; ++i) {
    if (x_rows[i] < 0) return PURLIN_ERR_INVALID_ARG;
    x_total += x_rows[i];
    for (int j = 0; j < P; ++j) {
      const int64_t c = counts[i * P + j];
      if (c < 0) return PURLIN_ERR_INVALID_ARG;
      n_ent[i] += c;
      y_rows[j] += c;
      total += c;
    }
  }
  if (total >= (int64_t(1) << 31) || x_total >= (int64_t(1) << 40)) return PURLIN_ERR_INVALID_ARG;
  // x: token rows (dispatch input, combine output); y: exchanged rows
  void *const *x = combine ? rowdst : rowsrc;
  void *const *y = combine ? rowsrc : rowdst;
  std::vector<std::pair<uintptr_t, uintptr_t>> xr, yr;
  for (int i = 0; i < P; ++i) {
    if (n_ent[i] > 0 && (!idx[i] || x_rows[i] == 0)) return PURLIN_ERR_INVALID_ARG;
    const int64_t xb = x_rows[i] * row_bytes, yb = y_rows[i] * row_bytes;
    if ((combine ? x_rows[i] : n_ent[i]) > 0 || xb > 0) {
      if (!x[i] || (uintptr_t(x[i]) & 1)) return PURLIN_ERR_INVALID_ARG;
      if (xb > 0) xr.push_back({uintptr_t(x[i]), uintptr_t(x[i]) + uintptr_t(xb)});
    }
    if (yb > 0) {
      if (!y[i] || (uintptr_t(y[i]) & 1)) return PURLIN_ERR_INVALID_ARG;
      yr.push_back({uintptr_t(y[i]), uintptr_t(y[i]) + uintptr_t(yb)});
    }
  }
  if (!(combine ? ranges_disjoint(yr, xr) : ranges_disjoint(xr, yr))) return PURLIN_ERR_INVALID_ARG;

  MoePlan &mp = *m;
  mp = MoePlan{};
  LaunchPlan &lp = mp.base;
  for (int r = 0; r < kMaxRanks; ++r) {
    lp.in[r] = r < P ? static_cast<const char *>(rowsrc[r]) : nullptr;
    lp.out[r] = r < P ? static_cast<char *>(rowdst[r]) : nullptr;
    mp.idx[r] = r < P ? idx[r] : nullptr;
    mp.x_rows[r] = r < P ? x_rows[r] : 0;
  }
  lp.P = P;
  lp.njobs = P * P;
  int64_t t = 0;
  int64_t pos[kMaxRanks] = {};
  for (int i = 0; i < P; ++i) {
    int64_t off = 0;
    for (int j = 0; j < P; ++j) {
      const int q = i * P + j;
      const int64_t c = counts[q];
      lp.jobs[q] = Job{off, pos[j] * row_bytes, c * row_bytes, int32_t(i), int32_t(j)};
      lp.tile_begin[q] = int32_t(t);
      t += c;
      off += c;
      pos[j] += c;
    }
  }
  for (int q = P * P; q <= kMaxJobs; ++q) lp.tile_begin[q] = int32_t(t);
  lp.total_tiles = int32_t(t);
  for (int i = 0; i < P; ++i) {
    mp.ent_base[i + 1] = mp.ent_base[i] + n_ent[i];
    mp.inv_base[i + 1] = mp.inv_base[i] + x_rows[i];
  }
  for (int i = P; i < kMaxRanks; ++i) {
    mp.ent_base[i + 1] = mp.ent_base[i];
    mp.inv_base[i + 1] = mp.inv_base[i];
  }
  mp.row_bytes = row_bytes;
  *total_rows = total;
  *y_rows_out = 0;
  for (int j = 0; j < P; ++j) *y_rows_out += y_rows[j];
  return PURLIN_OK;
}

// The launch-wide fields: flag block, watchdog and handshake.  The
// handshake (entry / exit notify) is off unless the policy asks for it:
// calls on one stream are already ordered by the stream.
void launch_fields(const DeviceState &ds, LaunchPlan &lp, const purlin_policy &pol,
                   uint32_t *flags) {
  lp.flags = flags;
  const int64_t wd_ns = pol.watchdog_ns ? pol.watchdog_ns : kDefaultWatchdogNs;
  lp.watchdog_ticks = uint64_t(wd_ns) * ds.wall_khz / 1000000u + 1;
  lp.sync = pol.sync == 1 ? 1 : 0;
}

// Divisor d of the strided kernel's row lookup: floor(u / d) = (u * m) >> s
// for every 0 <= u < 2^31, with l = ceil(log2 d), s = 31 + l and
// m = ceil(2^s / d) (Granlund and Montgomery, "Division by invariant integers
// using multiplication", 1994, Theorem 4.2 with N = 31: m * d - 2^s < d <= 2^l).
// m < 2^32 for every d < 2^31.
void magic_divisor(uint32_t d, uint32_t *m, int32_t *s) {
  int l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t two_s = uint64_t(1) << (31 + l);
  *m = uint32_t((two_s + d - 1) / d);
  *s = 31 + l;
}

// Plan of the Ulysses exchange.  Sequence layout: rank i holds
// [seq[i], heads, head_bytes]; head layout: rank j holds [S, heads / P,
// head_bytes], the tokens of rank 0 first.  Pair (i, j) moves rank i's
// tokens' slice of head group j.
purlin_status ulysses_plan(void *const *in, void *const *out, int P, const int64_t *seq,
                           int64_t heads, int64_t head_bytes, int to_sequence, StridedPlan *sp,
                           int *unit_out, int64_t *total_out) {
  if (!in || !out || !seq || P < 1 || P > kMaxRanks || heads < 1 || heads % P ||
      head_bytes <= 0 || (head_bytes & 1) || (to_sequence != 0 && to_sequence != 1))
    return PURLIN_ERR_INVALID_ARG;
  const int64_t kLimit = int64_t(1) << 40;
  if (heads > kLimit / head_bytes) return PURLIN_ERR_INVALID_ARG;
  const int64_t token_bytes = heads * head_bytes;        // one token, all heads
  const int64_t row = token_bytes / P;                   // one token, one head group
  int64_t S = 0;
  int64_t off[kMaxRanks + 1] = {};
  for (int i = 0; i < P; ++i) {
    if (seq[i] < 0 || seq[i] > kLimit) return PURLIN_ERR_INVALID_ARG;
    S += seq[i];
    off[i + 1] = S;
  }
  if (S > kLimit / token_bytes) return PURLIN_ERR_INVALID_ARG;
  // seq-layout and head-layout buffers of each rank
  void *const *sq = to_sequence ? out : in;
  void *const *hd = to_sequence ? in : out;
  std::vector<std::pair<uintptr_t, uintptr_t>> sr, hr;
  uint64_t align = uint64_t(row) | uint64_t(token_bytes) | 16u;
  for (int r = 0; r < P; ++r) {
    const int64_t sb = seq[r] * token_bytes, hb = S * row;
    if (sb > 0) {
      if (!sq[r]) return PURLIN_ERR_INVALID_ARG;
      sr.push_back({uintptr_t(sq[r]), uintptr_t(sq[r]) + uintptr_t(sb)});
      align |= uint64_t(uintptr_t(sq[r]));
    }
    if (hb > 0) {
      if (!hd[r]) return PURLIN_ERR_INVALID_ARG;
      hr.push_back({uintptr_t(hd[r]), uintptr_t(hd[r]) + uintptr_t(hb)});
      align |= uint64_t(uintptr_t(hd[r]));
    }
  }
  if (align & 1) return PURLIN_ERR_INVALID_ARG;
  if (!(to_sequence ? ranges_disjoint(hr, sr) : ranges_disjoint(sr, hr)))
    return PURLIN_ERR_INVALID_ARG;
  const int unit = int(align & (~align + 1));   // lowest set bit, at most 16
  // every pair's units must stay below 2^31
  for (int i = 0; i < P; ++i)
    if (seq[i] * row / unit >= (int64_t(1) << 31)) return PURLIN_ERR_INVALID_ARG;

  *sp = StridedPlan{};
  LaunchPlan &lp = sp->base;
  for (int r = 0; r < kMaxRanks; ++r) {
    lp.in[r] = r < P ? static_cast<const char *>(in[r]) : nullptr;
    lp.out[r] = r < P ? static_cast<char *>(out[r]) : nullptr;
  }
  lp.P = P;
  lp.njobs = P * P;
  int64_t total = 0;
  for (int a = 0; a < P; ++a) {      // source rank
    for (int b = 0; b < P; ++b) {    // destination rank
      // i: the sequence rank of the pair, j: its head group
      const int i = to_sequence ? b : a, j = to_sequence ? a : b;
      const int64_t seq_off = int64_t(j) * row;      // head group j inside a token
      const int64_t head_off = off[i] * row;         // rank i's tokens in the head layout
      lp.jobs[a * P + b] = Job{to_sequence ? head_off : seq_off, to_sequence ? seq_off : head_off,
                               seq[i] * row, int32_t(a), int32_t(b)};
      total += seq[i] * row;
    }
  }
  sp->row_bytes = row;
  sp->src_stride = to_sequence ? row : token_bytes;
  sp->dst_stride = to_sequence ? token_bytes : row;
  magic_divisor(uint32_t(row / unit), &sp->magic, &sp->shift);
  *unit_out = unit;
  *total_out = total;
  return PURLIN_OK;
}

// Workgroups of an MoE launch: the policy's wgs_per_rank when set, else
// `cap`; never more than the work or than the device holds resident.
int moe_grid(DeviceState &ds, MoeKernel which, bool rows, int64_t work, int64_t cap) {
  const purlin_policy pol = effective_policy();
  if (pol.wgs_per_rank && which != MoeKernel::kInverse) cap = int64_t(pol.wgs_per_rank) * kMaxRanks;
  int b = 0;
  if (moe_resident_per_cu(which, rows, &b) != hipSuccess || b < 1) b = 1;
  return int(std::max<int64_t>(1, std::min<int64_t>({work, cap, int64_t(ds.cus) * b})));
}

}  // namespace

purlin_status collective_impl(const purlin_layout *in, const purlin_layout *out, purlin_op op,
                              purlin_dtype dtype, int P, const int64_t *counts,
                              const int64_t *displs, hipStream_t stream, FixedWorkspaceFn fixed_fn) {
  if (!in || !out || !in->bufs || !out->bufs) return PURLIN_ERR_INVALID_ARG;
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  const Derived *d = nullptr;
  purlin_status st = derive_cached(in->naming, out->naming, op, dtype, P, counts, displs, &d);
  if (st != PURLIN_OK) return st;
  // The overlap checks sort every partition; skip them when the plan and the
  // buffers are those of the previous successful call.
  static uint64_t last_id = 0;
  static void *last_ptrs[2 * kMaxRanks];
  void *ptrs[2 * kMaxRanks] = {};
  for (int r = 0; r < P; ++r) {
    ptrs[r] = in->bufs[r];
    ptrs[kMaxRanks + r] = out->bufs[r];
  }
  const bool same_call = d->id == last_id && std::memcmp(ptrs, last_ptrs, sizeof(ptrs)) == 0;
  if (!same_call) {
    st = check_pointers(*d, in->bufs, out->bufs);
    if (st != PURLIN_OK) return st;
  }
  if (d->jobs.empty()) return PURLIN_OK;  // every partition is empty

  std::vector<Job> jobs;
  std::vector<int> owners;
  st = launch_jobs(*d, reinterpret_cast<char *const *>(out->bufs), &jobs, &owners);
  if (st != PURLIN_OK) return st;
  if (!same_call) {
    last_id = d->id;
    std::memcpy(last_ptrs, ptrs, sizeof(ptrs));
  }
  FixedWorkspace fixed_ws{};
  const FixedWorkspace *fixed = nullptr;
  if (fixed_fn) {
    st = fixed_fn(&fixed_ws);
    if (st != PURLIN_OK) return st;
    fixed = &fixed_ws;
  }

  const purlin_policy pol = effective_policy();
  if (op == PURLIN_OP_COPY && pol.engine == PURLIN_ENGINE_COPY) {
    // The copy engines: one stream-ordered DMA transfer per (job,
    // destination rank), no kernel and no compute unit.
    purlin_launch_info info{};
    info.bytes_min = d->bytes_min;
    info.njobs = int32_t(jobs.size());
    for (const Job &jb : jobs) {
      const char *src = static_cast<const char *>(in->bufs[jb.src]) + jb.src_off;
      for (int r = jb.dst < 0 ? 0 : jb.dst; r < (jb.dst < 0 ? P : jb.dst + 1); ++r) {
        char *dst = static_cast<char *>(out->bufs[r]) + jb.dst_off;
        if (hipMemcpyAsync(dst, src, size_t(jb.nbytes), hipMemcpyDeviceToDeviceNoCU, stream) !=
            hipSuccess)
          return PURLIN_ERR_HIP;
        ++info.engine_copies;
      }
    }
    info.tiles = info.engine_copies;
    g_last = info;
    g_have_last = true;
    return PURLIN_OK;
  }
  DeviceState *ds = nullptr;
  st = device_state(&ds);
  if (st != PURLIN_OK) return st;
  const KernelKind kind = kind_of(op, dtype);
  const bool nt = nt_env(true);

  const bool staged = pol.zero_staging == PURLIN_STAGING_STAGED;
  bool broadcast = false;
  int64_t job_bytes = 0;
  for (const Job &jb : jobs) {
    job_bytes += jb.nbytes;
    broadcast |= jb.dst < 0;
  }
  AutoPolicy ap = auto_policy(kind, broadcast, job_bytes, ds->cus);
  int unroll_sel = unroll_env();
  if (unroll_sel < 0 || unroll_sel > 2) unroll_sel = ap.unroll_sel;
  // Whether some job has a source off its destinations' 16-byte phase and
  // so needs the kernel with the row bodies.  (Broadcast destinations are
  // congruent modulo 16 once launch_jobs has split the others.)
  bool rows = false;
  for (const Job &jb : jobs) {
    const uint64_t d0 = uint64_t(reinterpret_cast<uintptr_t>(out->bufs[jb.dst < 0 ? 0 : jb.dst])) +
                        uint64_t(jb.dst_off);
    for (int i = jb.src < 0 ? 0 : jb.src; i < (jb.src < 0 ? P : jb.src + 1); ++i) {
      const uint64_t a = uint64_t(reinterpret_cast<uintptr_t>(in->bufs[i])) + uint64_t(jb.src_off);
      rows |= ((a - d0) & 15u) != 0;
    }
  }
  // every job writes one destination rank (no broadcast): the build whose
  // destination loops fold to a single store
  bool single_dst = true;
  for (const Job &jb : jobs) single_dst &= jb.dst >= 0;
  const bool one = !staged && one_build(kind, nt, rows, single_dst);
  // The build with the wide element pass (for small misaligned single-
  // destination tiles, taken in the latency regime only: at most 512 KiB of
  // jobs).  Larger reductions run the build without it, whose row bodies
  // keep a workgroup per CU more (ReduceScatterV 4-11% faster at 2-8 MiB per
  // rank, 2% at 16).  Copies run the wide build at every size: its row body
  // measured 2-3% faster on AllToAllV at 8 MiB - 1 GiB per rank (paired on
  // the same buffers; the pass itself is not taken there, so this is the
  // compiled code, not the pass).
  const bool small = job_bytes <= (int64_t(512) << 10);
  const bool wide = !staged && rows && (small || kind == KernelKind::kCopy);
  // Point-to-point copies on the row body (AllToAllV) from 256 MiB of jobs
  // keep eight units per lane in flight (the build without the wide pass):
  // +3-9% at 32-512 MiB per rank and +1.1-1.6% at 1 GiB, paired on the
  // same buffers with both placements (at 16 MiB -1.6%; the aligned
  // AllToAll 2-6% slower with it).
  if (!staged && unroll_env() < 0 && kind == KernelKind::kCopy && !broadcast && rows &&
      job_bytes >= (int64_t(256) << 20))
    unroll_sel = 1;
  // Aligned single-destination sums (ReduceScatter) with 16 - 256 MiB of
  // jobs keep two units per lane in flight (sixteen loads): +1.4-3.8% at
  // 16 - 64 MiB per rank and -0.3 to +1.1% at 96 - 192 MiB (paired, buffers
  // placed three ways); from 256 MiB 1-3% slower.  AllReduce (broadcast
  // sums, which would give up their device-scope stores for it) moved -7 to
  // +2.6% at 16 MiB - 1 GiB per rank with box and placement, so it keeps one.
  if (!staged && unroll_env() < 0 && kind != KernelKind::kCopy && single_dst && !rows &&
      job_bytes >= (int64_t(16) << 20) && job_bytes < (int64_t(256) << 20))
    unroll_sel = 1;
  // Point-to-point copies on the row body (AllToAllV) with 32 - 256 MiB of
  // jobs run as many workgroups as are resident (five per CU) on 16 KiB
  // chunks: AllToAllV 21 / 12 / 9 / 4% faster at 4 / 8 / 16 / 32 MiB per
  // rank than on two per CU and 32 KiB chunks (paired on the same buffers);
  // the aligned AllToAll gains nothing there and keeps the table's.
  // Reductions on the row build (ReduceScatterV) with 16 - 128 MiB of jobs
  // run three workgroups per CU (as many as are resident) on 8 KiB chunks:
  // 6-9 / 3 / 2-5% faster at 16 / 32 / 64 MiB per rank (three paired runs
  // on two boxes), 4-5% slower from 256 MiB.  Copy broadcasts (AllGather(V))
  // keep four workgroups per CU and 8 KiB chunks up to 32 MiB of jobs:
  // 4-11% faster at 16-24 MiB per rank (three runs), even at 32.  Each rule
  // held with the buffers allocated three ways (exactly, and as prefixes of
  // 256 MiB and 1 GiB allocations).  AllReduce keeps the table's: four
  // workgroups per CU on 4 KiB chunks at 16-48 MiB per rank measured 7-11%
  // faster with exactly sized buffers and 6-9% slower with the others.
  const bool mid_rules = env_i64("PURLIN_MID_CHUNKS", 1) != 0;
  const int64_t MiB = int64_t(1) << 20;
  bool chunk_fixed = false;
  if (mid_rules && kind == KernelKind::kCopy && !broadcast && rows && job_bytes >= 32 * MiB &&
      job_bytes < 256 * MiB) {
    ap.grid = 5 * ds->cus;
    ap.chunk = 16 << 10;
    chunk_fixed = true;
  } else if (mid_rules && kind != KernelKind::kCopy && rows && job_bytes >= 16 * MiB &&
             job_bytes < 128 * MiB) {
    ap.grid = 3 * ds->cus;
    ap.chunk = 8 << 10;
    chunk_fixed = true;
  } else if (mid_rules && kind == KernelKind::kCopy && broadcast && job_bytes >= 16 * MiB &&
             (job_bytes < 32 * MiB || (rows && job_bytes < 64 * MiB))) {
    // (AllGatherV keeps it up to 64 MiB of jobs: +2-5% at 32-48 MiB per
    // rank, paired with both placements; AllGather gains nothing there)
    ap.grid = 4 * ds->cus;
    ap.chunk = 8 << 10;
    chunk_fixed = true;
  }
  // Aligned copy broadcasts (AllGather) from 64 MiB of jobs run four
  // workgroups per CU on 4 KiB chunks with device-scope stores (below), from
  // grid x chunk sweeps at 64 MiB - 1 GiB per rank: +7-8% at 128 MiB -
  // 1 GiB, +0.7% at 64 MiB, paired against the table's two per CU, 16 KiB
  // chunks and plain stores on two boxes with both placements (at 32 MiB
  // -4%).  One workgroup per CU and 32 KiB chunks for AllReduce measured
  // +1-2% on one box and -3 to -7% on another, so AllReduce keeps the
  // table's.
  // Aligned point-to-point copies (AllToAll) from 1 GiB of jobs run one
  // workgroup per CU: +1.6-2.2% at 256 - 512 MiB per rank, +0.2-0.7% at
  // 128 MiB and 1 GiB (paired, two boxes, both placements); at 64 MiB 3-4.5%
  // slower, and AllToAllV on the row body 9-17% slower with it.
  if (mid_rules && kind == KernelKind::kCopy && !broadcast && !rows &&
      job_bytes >= (int64_t(1) << 30))
    ap.grid = ds->cus;
  const bool large_bcast = env_i64("PURLIN_LARGE_BCAST", 1) != 0;
  const bool large_copy_bcast = large_bcast && broadcast && !rows && kind == KernelKind::kCopy &&
                                job_bytes >= 64 * MiB && !chunk_fixed;
  if (large_copy_bcast) {
    ap.grid = 4 * ds->cus;
    ap.chunk = 4 << 10;
    chunk_fixed = true;
  }
  // Copy broadcasts of 16 MiB of jobs or more store plainly (where they do
  // not store at device scope, below): AllGather 5-8%,
  // AllGatherV 4-8% faster at 64 MiB - 1 GiB per rank than with nontemporal
  // stores (paired on the same buffers, both orders).  Nontemporal stores
  // stay for smaller broadcasts (AllGather 6% faster with them at 4 MiB),
  // for AllReduce's broadcast sums (2-4% faster with them at 64 MiB -
  // 1 GiB) and for single-destination copies (AllToAllV 3-5%).
  const bool bcast = !staged && broadcast && kind == KernelKind::kCopy &&
                     job_bytes >= (int64_t(16) << 20) && env_i64("PURLIN_BCAST_PLAIN", 1) != 0;
  // Broadcast jobs store at device scope (written through the L2 as they
  // go, instead of left dirty in it for eviction to write back) in the
  // windows where that measured faster, paired on the same buffers with
  // both placements (exactly sized, and prefixes of 1 GiB allocations):
  //   AllReduce   256 KiB - 128 MiB per rank: 3-8% (16-32 MiB: 5-15%), even
  //               at 4 MiB and from 256 MiB;
  //   AllGather   16 - 64 MiB: 1-7%; below 16 MiB up to -5%; from 128 MiB
  //               0 to -2.4% on the table's grid, the gains above on the
  //               grid and chunk of the large copy broadcasts;
  //   AllGatherV  16 MiB - 1 GiB: 1-8% (32 MiB even); below, -3 to -6%.
  const int64_t dstore_env = env_i64("PURLIN_DEVICE_STORES", -1);
  const bool dstore_auto =
      kind != KernelKind::kCopy ? job_bytes >= 256 * 1024 && job_bytes < 256 * MiB
                                : job_bytes >= 16 * MiB &&
                                      (rows || large_copy_bcast || job_bytes < 128 * MiB);
  const bool dstore = !staged && broadcast && !one && dstore_build(kind, nt, unroll_sel, rows, wide) &&
                      (dstore_env < 0 ? dstore_auto : dstore_env != 0);
  const int capacity =
      ds->cus * occupancy(*ds, kind, staged, nt, unroll_sel, rows, one, wide, bcast && !dstore, dstore);

  // The stream's flag block: for the staged kernel and for the handshake;
  // a zero-staging launch without the handshake touches no flag at all.
  StreamCtx *ctx = nullptr;
  uint32_t *flags = nullptr;
  if (fixed && (staged || pol.sync == 1)) {
    flags = fixed->flags;
  } else if (staged || pol.sync == 1) {
    st = stream_ctx(*ds, stream, &ctx);
    if (st != PURLIN_OK) return st;
    flags = ctx->flags;
  }

  LaunchPlan lp{};
  for (int r = 0; r < kMaxRanks; ++r) {
    lp.in[r] = r < P ? static_cast<const char *>(in->bufs[r]) : nullptr;
    lp.out[r] = r < P ? static_cast<char *>(out->bufs[r]) : nullptr;
  }
  lp.P = P;
  launch_fields(*ds, lp, pol, flags);

  purlin_launch_info info{};
  info.threads = kThreads;
  info.bytes_min = d->bytes_min;
  info.njobs = int32_t(jobs.size());

  hipError_t err;
  if (!staged) {
    const int64_t want_grid = std::min<int64_t>(
        capacity, pol.wgs_per_rank ? int64_t(P) * pol.wgs_per_rank : int64_t(ap.grid));
    const int64_t chunk =
        pol.chunk_bytes ? pol.chunk_bytes
        : chunk_fixed   ? ap.chunk
                        : auto_chunk(kind, broadcast, job_bytes, ap.chunk, want_grid);
    lp.chunk_bytes = chunk;
    fill_tiles(lp, jobs, chunk);
    const int grid = int(std::max<int64_t>(1, std::min<int64_t>(lp.total_tiles, want_grid)));
    // Nontemporal loads pay off for sources off the destination's line
    // phase too (variable-length partitions), measured at 16 MiB - 1 GiB.
    lp.nt_any_phase = env_i64("PURLIN_NT_ANY_PHASE", 1) ? 1 : 0;
    // Latency regime (the wide build, 4 KiB tiles): small misaligned
    // single-destination tiles take one wide element pass instead of a row
    // body (ReduceScatterV at 8 - 16 KiB per rank: 8.9 us against 10.3 us);
    // from 1 MiB per rank on, the row body is faster.
    lp.wide_max = (wide && small && chunk <= 4096) ? int32_t(chunk + 128) : 0;
    // Reductions whose sources share a 16-byte phase off the destination's
    // (ReduceScatterV) take source-aligned units with misaligned stores:
    // their loads are then the aligned body's (eight source streams for one
    // written), 5-8% faster than the realigning row body at 64 MiB - 1 GiB
    // per rank (paired on the same buffers).  Copies keep the row bodies,
    // whose stores are whole lines: misaligned stores measured 2-11% slower
    // on AllGatherV and 4-11% on AllToAllV.
    // From 32 MiB of jobs the same units are folded and then shifted into
    // destination-aligned stores across rows each wavefront carries
    // (body_carry, shift_stores 2): ReduceScatterV +0.1-0.7% at 32 MiB,
    // +1.5-3.9% at 48-512 MiB and +0.6-1.3% at 1 GiB per rank (paired, both
    // placements), traffic 1.012 x B_min against 1.014; at 16 MiB -0.3 to
    // +1.3%, at 1-8 MiB 5-12% slower.  PURLIN_SHIFT_STORES: 0 row body, 1
    // misaligned stores, 2 carried rows.
    const int64_t shift_env = env_i64("PURLIN_SHIFT_STORES", -1);
    const int shift_auto = kind == KernelKind::kCopy ? 0 : job_bytes >= 32 * MiB ? 2 : 1;
    lp.shift_stores = shift_env < 0    ? shift_auto
                      : shift_env == 2 ? (kind != KernelKind::kCopy ? 2 : 0)
                                       : (shift_env != 0 ? 1 : 0);
    // Copy broadcasts whose source is off the destinations' phase
    // (AllGatherV) from 32 MiB of jobs take destination-aligned units with
    // misaligned source loads instead of the row body: +2-4% at 64 and
    // 256 MiB per rank (paired, two runs), +1.4-2.1% at 768 MiB - 1 GiB with
    // the device-scope stores they take there (even with plain stores); at
    // 16 MiB -3%, in the latency regime slower.  The other copies keep the
    // row body (AllToAllV 4-9% slower with misaligned loads), and
    // reductions their misaligned stores.
    const int64_t ul_env = env_i64("PURLIN_UNALIGNED_LOADS", -1);
    const bool ul_auto = kind == KernelKind::kCopy && broadcast && job_bytes >= (int64_t(32) << 20);
    lp.unaligned_loads = (ul_env < 0 ? ul_auto : ul_env != 0) ? 1 : 0;
    const bool lds = !rows && nt && env_i64("PURLIN_LDS", 0) != 0;
    if (lds) {
      int b = 0;
      if (zs_lds_resident_per_cu(kind, single_dst, bcast, &b) != hipSuccess || b < 1) b = 1;
      const int g = std::min(grid, ds->cus * b);
      err = launch_zs_lds(lp, kind, single_dst, bcast, g, stream);
    } else {
      err = launch_zs(lp, kind, nt, unroll_sel, rows, one, wide, bcast && !dstore, dstore, grid, stream);
    }
    info.grid = grid;
    info.zero_staging = 1;
    info.rows = rows ? 1 : 0;
    info.one = one ? 1 : 0;
    info.plain_stores = bcast && !dstore ? 1 : 0;
    info.device_stores = dstore ? 1 : 0;
    info.shift_stores = lp.shift_stores;
    info.unaligned_loads = lp.unaligned_loads;
    info.unroll = unroll_of(kind, unroll_sel);
    info.chunk_bytes = chunk;
    info.tiles = lp.total_tiles;
    info.sync = lp.sync;
  } else {
    StagedPlan sp{};
    sp.base = lp;
    sp.withhold = pol.test_withhold;
    int64_t max_job = 0;
    for (const Job &jb : jobs) max_job = std::max(max_job, jb.nbytes);
    int depth = pol.depth ? pol.depth : 2;
    // roles per lane of each job
    const int owner_team = int(std::min<int64_t>(kMaxTeam, std::max<int64_t>(1, env_i64("PURLIN_OWNER_TEAM", kOwnerTeam))));
    int roles_per_lane = 0;
    std::vector<StagedJob> sj(jobs.size());
    for (size_t k = 0; k < jobs.size(); ++k) {
      const Job &jb = jobs[k];
      const int owner = jb.dst >= 0 ? jb.dst : (jb.src >= 0 ? jb.src : owners[k]);
      sj[k].owner = int16_t(owner);
      sj[k].n_stage = int16_t(jb.src < 0 ? P - 1 : (jb.src != owner ? 1 : 0));
      sj[k].n_scatter = int16_t(jb.dst < 0 ? P - 1 : 0);
      // A reduction's owner reads every source of a chunk while a stager
      // copies one: a team of owners, each combining a slice of the chunk,
      // keeps pace with the stagers.
      sj[k].team = int16_t(kind != KernelKind::kCopy && sj[k].n_stage > 0 ? owner_team : 1);
      roles_per_lane += sj[k].team + sj[k].n_stage + sj[k].n_scatter;
    }
    if (roles_per_lane > capacity) return PURLIN_ERR_UNSUPPORTED;  // cannot be co-resident
    int lane_cap = pol.wgs_per_rank ? pol.wgs_per_rank : capacity / std::max(1, roles_per_lane);
    // Default shape, from the depth x chunk x lanes sweep at 256 MiB per
    // rank: a ring two slots deep (deeper measured no faster), as many lanes
    // as fit, and 64 KiB chunks for copies, 256 KiB for reductions (whose
    // team of owners splits each chunk eight ways); a handoff is a drain and
    // a flag store (the slots take device-scope stores), so short chunks
    // pay.  A job shorter than eight chunks takes shorter ones, down to
    // 16 KiB.
    int64_t chunk = pol.chunk_bytes;
    if (!chunk) {
      chunk = int64_t(kind == KernelKind::kCopy ? 64 : 256) << 10;
      while (chunk > (int64_t(16) << 10) && chunk * 8 > max_job) chunk /= 2;
    }
    int64_t ring_bytes = 0, flag_bytes = 0;
    // Lay out tiles, lanes, roles and rings for (chunk, depth, lane_cap).
    auto layout = [&]() {
      sp.base.chunk_bytes = chunk;
      fill_tiles(sp.base, jobs, chunk);
      sp.slot_stride = chunk + 256;
      int max_tiles = 1;
      for (size_t k = 0; k < jobs.size(); ++k)
        max_tiles = std::max(max_tiles, sp.base.tile_begin[k + 1] - sp.base.tile_begin[k]);
      int lanes = std::max(1, std::min({lane_cap, kMaxLanes, max_tiles}));
      while (lanes > 1 && lanes * roles_per_lane > capacity) --lanes;
      sp.lanes = lanes;
      // a default ring is no deeper than the chunks a lane carries
      sp.depth = pol.depth ? depth : std::min(depth, (max_tiles + lanes - 1) / lanes);
      int role = 0, ring = 0;
      for (size_t k = 0; k < jobs.size(); ++k) {
        sj[k].role_begin = role;
        sj[k].ring_begin = ring;
        role += (sj[k].team + sj[k].n_stage + sj[k].n_scatter) * lanes;
        ring += (sj[k].n_stage + (sj[k].n_scatter > 0 ? 1 : 0)) * lanes;
        sp.sj[k] = sj[k];
      }
      for (size_t k = jobs.size(); k < size_t(kMaxJobs); ++k) sp.sj[k].role_begin = role;
      sp.total_roles = role;
      ring_bytes = std::max<int64_t>(1, int64_t(ring) * sp.depth * sp.slot_stride);
      flag_bytes = std::max<int64_t>(256, int64_t(ring) * sp.depth * 256);
    };
    layout();
    if (fixed) {
      // The fixed scratch: shrink what the policy leaves open until the rings
      // fit (depth down to 2, which the pipeline sweep measured as fast as
      // deeper rings, then fewer lanes, then shorter chunks).
      while (ring_bytes > fixed->ring_bytes || flag_bytes > fixed->slot_flag_bytes) {
        if (!pol.depth && depth > 2) --depth;
        else if (!pol.wgs_per_rank && sp.lanes > 1) lane_cap = sp.lanes / 2;
        else if (!pol.chunk_bytes && chunk > 4096) chunk /= 2;
        else return PURLIN_ERR_NO_MEMORY;  // the policy fixes a plan too large for the scratch
        layout();
      }
      sp.ring = fixed->ring;
      sp.slot_flags = fixed->slot_flags;
    } else {
      st = ensure_staging(*ds, *ctx, ring_bytes, flag_bytes);
      if (st != PURLIN_OK) return st;
      sp.ring = ctx->ring;
      sp.slot_flags = ctx->slot_flags;
    }
    err = launch_staged(sp, kind, nt, stream);
    info.grid = sp.total_roles;
    info.zero_staging = 0;
    info.rows = 1;
    info.unroll = unroll_of(kind, 1);
    info.depth = sp.depth;
    info.chunk_bytes = sp.base.chunk_bytes;
    info.tiles = sp.base.total_tiles;
    info.sync = sp.base.sync;
  }
  if (err != hipSuccess) return PURLIN_ERR_HIP;
  g_last = info;
  g_have_last = true;
  return PURLIN_OK;
}

}  // namespace purlin

using namespace purlin;

extern "C" {

const char *purlin_strerror(purlin_status s) {
  switch (s) {
    case PURLIN_OK: return "ok";
    case PURLIN_ERR_INVALID_ARG: return "invalid argument";
    case PURLIN_ERR_UNSUPPORTED: return "unsupported collective";
    case PURLIN_ERR_NO_MEMORY: return "out of device memory";
    case PURLIN_ERR_HIP: return "HIP error";
    case PURLIN_ERR_TIMEOUT: return "device wait timed out";
    case PURLIN_ERR_PROTOCOL: return "protocol check failed";
  }
  return "unknown status";
}

purlin_status purlin_set_policy(const purlin_policy *p) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  if (!p) {
    g_user_policy_set = false;
    user_policy() = purlin_policy{};
    return PURLIN_OK;
  }
  if (!policy_valid(*p)) return PURLIN_ERR_INVALID_ARG;
  user_policy() = *p;
  g_user_policy_set = true;
  return PURLIN_OK;
}

purlin_status purlin_get_policy(purlin_policy *p) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  if (!p) return PURLIN_ERR_INVALID_ARG;
  *p = effective_policy();
  return PURLIN_OK;
}

purlin_status purlin_plan_describe(const purlin_layout *in, const purlin_layout *out,
                                   purlin_op op, purlin_dtype dtype, int P,
                                   const int64_t *counts, const int64_t *displs,
                                   purlin_segment *segs, int64_t *n_segs) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  if (!in || !out || !in->bufs || !out->bufs || !n_segs) return PURLIN_ERR_INVALID_ARG;
  const Derived *d = nullptr;
  purlin_status s = derive_cached(in->naming, out->naming, op, dtype, P, counts, displs, &d);
  if (s != PURLIN_OK) return s;
  s = check_pointers(*d, in->bufs, out->bufs);
  if (s != PURLIN_OK) return s;
  if (!d->jobs.empty()) {
    std::vector<Job> jobs;
    std::vector<int> owners;
    s = launch_jobs(*d, reinterpret_cast<char *const *>(out->bufs), &jobs, &owners);
    if (s != PURLIN_OK) return s;
  }
  const int64_t n = int64_t(d->segs.size());
  if (segs) {
    const int64_t m = std::min<int64_t>(*n_segs, n);
    for (int64_t k = 0; k < m; ++k) segs[k] = d->segs[size_t(k)];
  }
  *n_segs = n;
  return PURLIN_OK;
}

purlin_status purlin_collective(const purlin_layout *in, const purlin_layout *out,
                                purlin_op op, purlin_dtype dtype, int P,
                                const int64_t *counts, const int64_t *displs,
                                hipStream_t stream) {
  return collective_impl(in, out, op, dtype, P, counts, displs, stream, nullptr);
}

purlin_status purlin_moe_dispatch(void *const *x, void *const *y, int P, int64_t row_bytes,
                                  const int32_t *const *idx, const int64_t *counts,
                                  const int64_t *x_rows, int unique, hipStream_t stream) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  MoePlan m;
  int64_t total = 0, y_total = 0;
  purlin_status st = moe_plan(x, y, P, row_bytes, idx, counts, x_rows, false, &m, &total, &y_total);
  if (st != PURLIN_OK) return st;
  if (total == 0) return PURLIN_OK;
  DeviceState *ds = nullptr;
  st = device_state(&ds);
  if (st != PURLIN_OK) return st;
  StreamCtx *ctx = nullptr;  // the status word for index errors, epochs, the table
  st = stream_ctx(*ds, stream, &ctx);
  if (st != PURLIN_OK) return st;
  launch_fields(*ds, m.base, effective_policy(), ctx->flags);
  bool rows = (row_bytes & 15) != 0;
  for (int r = 0; r < P; ++r)
    rows |= ((uintptr_t(x[r]) | uintptr_t(y[r])) & 15) != 0;
  m.base.chunk_bytes = row_bytes;
  int grid = 0;
  const bool by_token = unique && !rows;
  if (by_token) {
    // each token row read once and written to all its ranks: the (token,
    // rank) -> entry table first
    st = ensure_inverse(*ds, *ctx, m.inv_base[P] * P * int64_t(sizeof(uint64_t)));
    if (st != PURLIN_OK) return st;
    m.inv = ctx->inv;
    const int g0 = moe_grid(*ds, MoeKernel::kInverse, false, (total + kThreads - 1) / kThreads,
                            int64_t(ds->cus) * 8);
    if (launch_moe(m, MoeKernel::kInverse, false, g0, stream) != hipSuccess) return PURLIN_ERR_HIP;
    // one workgroup per CU: at 4096 x 7168 per rank, top-8 of 256, 569 us
    // against 649 us with four per CU (two: 660 us, three: 650 us; 0.75 or
    // 1.25 per CU: 713 / 728 us), the calls alternated on the same buffers
    grid = moe_grid(*ds, MoeKernel::kDispatchTokens, false, m.inv_base[P], int64_t(ds->cus));
    if (launch_moe(m, MoeKernel::kDispatchTokens, false, grid, stream) != hipSuccess)
      return PURLIN_ERR_HIP;
  } else {
    // the copy policy's grid: four workgroups per CU
    grid = moe_grid(*ds, MoeKernel::kDispatch, rows, total, int64_t(ds->cus) * 4);
    if (launch_moe(m, MoeKernel::kDispatch, rows, grid, stream) != hipSuccess) return PURLIN_ERR_HIP;
  }
  purlin_launch_info info{};
  info.grid = grid;
  info.threads = kThreads;
  info.zero_staging = 1;
  info.chunk_bytes = row_bytes;
  info.tiles = by_token ? m.inv_base[P] : total;
  // rows written, plus rows read: one per entry, or (by token) at most one
  // per token row
  info.bytes_min = (total + (by_token ? std::min(total, m.inv_base[P]) : total)) * row_bytes;
  info.njobs = P * P;
  info.sync = m.base.sync;
  info.rows = rows ? 1 : 0;
  g_last = info;
  g_have_last = true;
  return PURLIN_OK;
}

purlin_status purlin_moe_combine(void *const *y, void *const *out, int P, int64_t row_bytes,
                                 const int32_t *const *idx, const float *const *w,
                                 const int64_t *counts, const int64_t *x_rows, hipStream_t stream) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  MoePlan m;
  int64_t total = 0, y_total = 0;
  purlin_status st = moe_plan(y, out, P, row_bytes, idx, counts, x_rows, true, &m, &total, &y_total);
  if (st != PURLIN_OK) return st;
  if (!w || (row_bytes & 15)) return PURLIN_ERR_INVALID_ARG;
  for (int r = 0; r < P; ++r) {
    if (m.ent_base[r + 1] > m.ent_base[r] && !w[r]) return PURLIN_ERR_INVALID_ARG;
    if ((uintptr_t(y[r]) | uintptr_t(out[r])) & 15) return PURLIN_ERR_INVALID_ARG;
    m.w[r] = w[r];
  }
  const int64_t out_rows = m.inv_base[P];
  if (out_rows == 0) return PURLIN_OK;
  DeviceState *ds = nullptr;
  st = device_state(&ds);
  if (st != PURLIN_OK) return st;
  StreamCtx *ctx = nullptr;
  st = stream_ctx(*ds, stream, &ctx);
  if (st != PURLIN_OK) return st;
  st = ensure_inverse(*ds, *ctx, out_rows * P * int64_t(sizeof(uint64_t)));
  if (st != PURLIN_OK) return st;
  m.inv = ctx->inv;
  launch_fields(*ds, m.base, effective_policy(), ctx->flags);
  m.base.chunk_bytes = row_bytes;
  if (total > 0) {
    const int g0 = moe_grid(*ds, MoeKernel::kInverse, false, (total + kThreads - 1) / kThreads,
                            int64_t(ds->cus) * 8);
    if (launch_moe(m, MoeKernel::kInverse, false, g0, stream) != hipSuccess) return PURLIN_ERR_HIP;
  }
  const int grid = moe_grid(*ds, MoeKernel::kCombine, false, out_rows, int64_t(ds->cus) * 4);
  if (launch_moe(m, MoeKernel::kCombine, false, grid, stream) != hipSuccess) return PURLIN_ERR_HIP;
  purlin_launch_info info{};
  info.grid = grid;
  info.threads = kThreads;
  info.zero_staging = 1;
  info.chunk_bytes = row_bytes;
  info.tiles = out_rows;
  info.bytes_min = (y_total + out_rows) * row_bytes;
  info.njobs = P * P;
  info.sync = m.base.sync;
  g_last = info;
  g_have_last = true;
  return PURLIN_OK;
}

purlin_status purlin_ulysses(void *const *in, void *const *out, int P, const int64_t *seq,
                             int64_t heads, int64_t head_bytes, int to_sequence,
                             hipStream_t stream) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  StridedPlan sp;
  int unit = 16;
  int64_t total = 0;
  purlin_status st = ulysses_plan(in, out, P, seq, heads, head_bytes, to_sequence, &sp, &unit, &total);
  if (st != PURLIN_OK) return st;
  if (total == 0) return PURLIN_OK;
  DeviceState *ds = nullptr;
  st = device_state(&ds);
  if (st != PURLIN_OK) return st;
  const purlin_policy pol = effective_policy();
  StreamCtx *ctx = nullptr;
  if (pol.sync == 1) {
    st = stream_ctx(*ds, stream, &ctx);
    if (st != PURLIN_OK) return st;
  }
  launch_fields(*ds, sp.base, pol, ctx ? ctx->flags : nullptr);
  // four workgroups per CU (two or three measured within 1% at the
  // Qwen-Image and 64 MiB shapes), 32 KiB tiles, smaller tiles for small
  // exchanges
  const int64_t cap = pol.wgs_per_rank ? int64_t(pol.wgs_per_rank) * kMaxRanks : int64_t(ds->cus) * 4;
  // at least one full 16 KiB pass per tile: a tile shorter than a pass
  // takes the guarded path only, measured slower at the Qwen-Image sizes
  const int64_t chunk = pol.chunk_bytes
                            ? pol.chunk_bytes
                            : std::max<int64_t>(int64_t(16) << 10, fit_chunk(int64_t(32) << 10, total, cap));
  sp.base.chunk_bytes = chunk;
  int64_t t = 0;
  for (int q = 0; q < P * P; ++q) {
    sp.base.tile_begin[q] = int32_t(t);
    t += (sp.base.jobs[q].nbytes + chunk - 1) / chunk;
  }
  for (int q = P * P; q <= kMaxJobs; ++q) sp.base.tile_begin[q] = int32_t(t);
  sp.base.total_tiles = int32_t(t);
  // Exchanges of at most 128 MiB each way store plainly: at the Qwen-Image
  // 1024x1024 shape (80 MB / 27 MB each way) 11% / up to 7% faster than with
  // nontemporal stores, paired on the same buffers in both orders; at 64
  // MiB per rank (537 MB each way) nontemporal stores are 4-8% faster.
  const bool plain = total <= (int64_t(128) << 20);
  int b = 0;
  if (strided_resident_per_cu(unit, plain, &b) != hipSuccess || b < 1) b = 1;
  const int grid = int(std::max<int64_t>(1, std::min<int64_t>({t, cap, int64_t(ds->cus) * b})));
  if (launch_strided(sp, unit, plain, grid, stream) != hipSuccess) return PURLIN_ERR_HIP;
  purlin_launch_info info{};
  info.grid = grid;
  info.threads = kThreads;
  info.zero_staging = 1;
  info.chunk_bytes = chunk;
  info.tiles = t;
  info.bytes_min = 2 * total;
  info.njobs = P * P;
  info.sync = sp.base.sync;
  info.unit = unit;
  info.plain_stores = plain ? 1 : 0;
  g_last = info;
  g_have_last = true;
  return PURLIN_OK;
}

purlin_status purlin_check(hipStream_t stream) {
  if (hipStreamSynchronize(stream) != hipSuccess) return PURLIN_ERR_HIP;
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PURLIN_ERR_HIP;
  auto &all = devices();
  // the stream's flag block, and the fixed scratch's (no-allocation calls)
  uint32_t *words[2] = {nullptr, scratch_status_word()};
  if (int(all.size()) > dev)
    if (StreamCtx *c = find_ctx(all[dev], stream)) words[0] = c->flags + kFlagStatus;
  uint32_t status = 0;
  for (uint32_t *word : words) {
    if (!word) continue;
    uint32_t v = 0;
    if (hipMemcpy(&v, word, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return PURLIN_ERR_HIP;
    if (v && hipMemset(word, 0, sizeof(uint32_t)) != hipSuccess) return PURLIN_ERR_HIP;
    status |= v;
  }
  if (status == 0) return PURLIN_OK;
  if (status & kStatusTimeout) return PURLIN_ERR_TIMEOUT;
  if (status & kStatusProtocol) return PURLIN_ERR_PROTOCOL;
  return (status & kStatusBadArg) ? PURLIN_ERR_INVALID_ARG : PURLIN_ERR_HIP;
}

purlin_status purlin_last_launch(purlin_launch_info *info) {
  if (!info) return PURLIN_ERR_INVALID_ARG;
  if (!g_have_last) return PURLIN_ERR_INVALID_ARG;
  *info = g_last;
  return PURLIN_OK;
}

purlin_status purlin_stream_copy(void *dst, const void *src, int64_t bytes, hipStream_t stream) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  if (!dst || !src || bytes < 0 || (bytes & 15) || (uintptr_t(dst) & 15) || (uintptr_t(src) & 15))
    return PURLIN_ERR_INVALID_ARG;
  if (bytes == 0) return PURLIN_OK;
  DeviceState *ds = nullptr;
  purlin_status st = device_state(&ds);
  if (st != PURLIN_OK) return st;
  const int grid = ds->cus * 2;
  return launch_stream_copy(dst, src, bytes, grid, stream) == hipSuccess ? PURLIN_OK
                                                                           : PURLIN_ERR_HIP;
}

purlin_status purlin_stream_pattern(const void *const *srcs, int n_src, void *const *dsts,
                                    int n_dst, int64_t bytes, int grid, int64_t tile_bytes,
                                    int unroll, int access, hipStream_t stream) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  const bool ok_n = (n_src == 0 || n_src == 1 || n_src == 8) && (n_dst == 0 || n_dst == 1 || n_dst == 8) &&
                    (n_src + n_dst) > 0;
  if (!ok_n || (n_src && !srcs) || (n_dst && !dsts) || bytes < 0 || (bytes & 15) || grid < 0 ||
      grid > 65536 || tile_bytes < 0 || (tile_bytes & 15) || tile_bytes >= (int64_t(1) << 32) ||
      (unroll != 0 && unroll != 2 && unroll != 4 && unroll != 8) || access < 0 || access > 7)
    return PURLIN_ERR_INVALID_ARG;
  for (int r = 0; r < n_src; ++r)
    if (!srcs[r] || (uintptr_t(srcs[r]) & 15)) return PURLIN_ERR_INVALID_ARG;
  for (int r = 0; r < n_dst; ++r)
    if (!dsts[r] || (uintptr_t(dsts[r]) & 15)) return PURLIN_ERR_INVALID_ARG;
  if (bytes == 0) return PURLIN_OK;
  DeviceState *ds = nullptr;
  purlin_status st = device_state(&ds);
  if (st != PURLIN_OK) return st;
  return launch_pattern(srcs, n_src, dsts, n_dst, bytes, grid ? grid : ds->cus * 4,
                        tile_bytes ? tile_bytes : int64_t(16) << 10, unroll ? unroll : 4,
                        (access & 1) != 0, (access & 4) ? 2 : (access & 2) ? 1 : 0,
                        stream) == hipSuccess
             ? PURLIN_OK
             : PURLIN_ERR_HIP;
}

void purlin_release(void) {
  std::lock_guard<std::recursive_mutex> lock(api_mutex());
  auto &all = devices();
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (size_t dev = 0; dev < all.size(); ++dev) {
    DeviceState &s = all[dev];
    if (s.ctx.empty() && s.retired.empty()) continue;
    if (hipSetDevice(int(dev)) != hipSuccess) continue;
    (void)hipDeviceSynchronize();
    for (auto &c : s.ctx) {
      for (void *b : {static_cast<void *>(c->flags), static_cast<void *>(c->ring),
                      static_cast<void *>(c->slot_flags), static_cast<void *>(c->inv)})
        if (b) (void)hipFree(b);
    }
    for (void *b : s.retired) (void)hipFree(b);
    s.ctx.clear();
    s.retired.clear();
  }
  if (have_cur) (void)hipSetDevice(cur);
}

}  // extern "C"
