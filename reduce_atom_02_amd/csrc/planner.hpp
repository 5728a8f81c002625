// Host planner: argument validation and derivation of a collective's jobs
// from its specification (no HIP call in here, so it runs without a GPU).
#pragma once
#include <utility>
#include <vector>

#include "../../include/purlin.h"
#include "plan.hpp"

namespace purlin {

struct ByteRange {
  int rank;
  int64_t off, len;  // bytes within that rank's buffer
};

// What a (naming, naming, op, dtype, P, counts, displs) specification
// derives into.  It depends on no pointer, so it is cached across calls.
struct Derived {
  uint64_t id = 0;                   // unique per cached derivation (never reused)
  int P = 0;
  int esz = 0;
  purlin_op op = PURLIN_OP_COPY;
  std::vector<purlin_segment> segs;  // every (output partition, matched input) pair
  std::vector<Job> jobs;             // bytes; grouped by owner rank
  std::vector<int> owner;            // owner rank of each job
  std::vector<ByteRange> in_ranges, out_ranges;
  int64_t bytes_min = 0;             // every input byte read once, every output byte written once
};

// Structural checks and derivation.  Returns PURLIN_OK, INVALID_ARG or UNSUPPORTED.
purlin_status derive(purlin_naming in_naming, purlin_naming out_naming, purlin_op op,
                     purlin_dtype dtype, int P, const int64_t *counts,
                     const int64_t *displs, Derived *d);

// Pointer checks of one call: NULL and misaligned buffers, overlapping output
// partitions, input bytes overlapping output bytes.
purlin_status check_pointers(const Derived &d, void *const *in, void *const *out);

// Byte ranges [first, second): the outputs pairwise disjoint and no input
// overlapping an output.  Empty ranges are ignored by construction.
bool ranges_disjoint(const std::vector<std::pair<uintptr_t, uintptr_t>> &ins,
                     std::vector<std::pair<uintptr_t, uintptr_t>> outs);

// Cached derive(): same result, reused when the specification repeats.
purlin_status derive_cached(purlin_naming in_naming, purlin_naming out_naming, purlin_op op,
                            purlin_dtype dtype, int P, const int64_t *counts,
                            const int64_t *displs, const Derived **d);

// The jobs of one launch: broadcast jobs whose destinations are not all
// congruent modulo 16 bytes are split into one job per destination.
// UNSUPPORTED (and no jobs) when the split would exceed kMaxJobs.
purlin_status launch_jobs(const Derived &d, char *const *out, std::vector<Job> *jobs,
                          std::vector<int> *owner);

int name_count(purlin_naming n, int P);

}  // namespace purlin
