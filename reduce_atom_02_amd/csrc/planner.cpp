// Host planner: derives the jobs of a collective from its specification.
//
// In Purlin the coordination of a collective follows from its specification,
// with no communication schedule written by hand (abstract; the
// derivability column of Table 1).  Here that derivation is the naming rule itself: every
// output partition takes the input partitions with the same name, in
// ascending source rank (Figure 4 caption gives the three layouts this
// reproduces).  Output partitions that take the same source bytes and sit at
// the same offset in every rank's output become one broadcast job, which is
// how AllGather and the gather half of the composed AllReduce (Figure 6
// caption) write a chunk to every rank from registers.
#include "planner.hpp"

#include <algorithm>
#include <cstring>
#include <map>
#include <tuple>

namespace purlin {

namespace {

constexpr int64_t kMaxCount = int64_t(1) << 40;  // elements per partition

struct Part {
  int name;
  int64_t off, cnt;  // elements
};

bool valid_naming(int n) { return n >= PURLIN_NAME_WHOLE && n <= PURLIN_NAME_BY_INDEX_RANK; }

// Components of a naming's names: () for WHOLE, (r) or (q), (r, q) or (q, r).
// Names of different lengths never match, even where their numbers in the
// counts array coincide (P = 1).
int name_arity(purlin_naming n) {
  switch (n) {
    case PURLIN_NAME_WHOLE: return 0;
    case PURLIN_NAME_BY_RANK:
    case PURLIN_NAME_BY_INDEX: return 1;
    default: return 2;
  }
}

// Partitions of rank r's buffer under naming n; displs_side may be null (packed).
int parts_of(purlin_naming n, int r, int P, const int64_t *counts, const int64_t *displs_side,
             Part *out) {
  int np = 0;
  auto add = [&](int name, int64_t packed) {
    out[np].name = name;
    out[np].cnt = counts[name];
    out[np].off = displs_side ? displs_side[name] : packed;
    ++np;
  };
  int64_t packed = 0;
  switch (n) {
    case PURLIN_NAME_WHOLE: add(0, 0); break;
    case PURLIN_NAME_BY_RANK: add(r, 0); break;
    case PURLIN_NAME_BY_INDEX:
      for (int q = 0; q < P; ++q) { add(q, packed); packed += counts[q]; }
      break;
    case PURLIN_NAME_BY_RANK_INDEX:
      for (int q = 0; q < P; ++q) { add(r * P + q, packed); packed += counts[r * P + q]; }
      break;
    case PURLIN_NAME_BY_INDEX_RANK:
      for (int q = 0; q < P; ++q) { add(q * P + r, packed); packed += counts[q * P + r]; }
      break;
  }
  return np;
}

bool ranges_overlap(std::vector<std::pair<uintptr_t, uintptr_t>> &v) {
  std::sort(v.begin(), v.end());
  for (size_t k = 1; k < v.size(); ++k)
    if (v[k].first < v[k - 1].second) return true;
  return false;
}

}  // namespace

int name_count(purlin_naming n, int P) {
  switch (n) {
    case PURLIN_NAME_WHOLE: return 1;
    case PURLIN_NAME_BY_RANK:
    case PURLIN_NAME_BY_INDEX: return P;
    default: return P * P;
  }
}

purlin_status derive(purlin_naming in_naming, purlin_naming out_naming, purlin_op op,
                     purlin_dtype dtype, int P, const int64_t *counts,
                     const int64_t *displs, Derived *d) {
  if (P < 1 || P > kMaxRanks) return PURLIN_ERR_INVALID_ARG;
  if (!valid_naming(in_naming) || !valid_naming(out_naming)) return PURLIN_ERR_INVALID_ARG;
  if (op != PURLIN_OP_COPY && op != PURLIN_OP_SUM) return PURLIN_ERR_INVALID_ARG;
  if (dtype != PURLIN_F32 && dtype != PURLIN_BF16) return PURLIN_ERR_INVALID_ARG;
  if (!counts) return PURLIN_ERR_INVALID_ARG;
  const int nn = name_count(in_naming, P);
  const int nn_out = name_count(out_naming, P);
  // counts has one entry per name of the input naming; check it before the
  // name sets are compared so that a bad count is always INVALID_ARG.
  for (int k = 0; k < nn; ++k)
    if (counts[k] < 0 || counts[k] > kMaxCount) return PURLIN_ERR_INVALID_ARG;
  if (displs)
    for (int k = 0; k < 2 * std::min(nn, nn_out); ++k)
      if (displs[k] < 0 || displs[k] > kMaxCount) return PURLIN_ERR_INVALID_ARG;
  // no name can match
  if (nn_out != nn || name_arity(in_naming) != name_arity(out_naming)) return PURLIN_ERR_UNSUPPORTED;

  const int esz = dtype == PURLIN_F32 ? 4 : 2;
  const int64_t *in_d = displs ? displs : nullptr;
  const int64_t *out_d = displs ? displs + nn : nullptr;

  d->P = P;
  d->esz = esz;
  d->op = op;
  d->segs.clear();
  d->jobs.clear();
  d->owner.clear();
  d->in_ranges.clear();
  d->out_ranges.clear();
  d->bytes_min = 0;

  // name -> (rank, element offset) of every input partition, ascending rank
  std::vector<std::vector<std::pair<int, int64_t>>> sources(nn);
  Part parts[kMaxRanks];
  for (int i = 0; i < P; ++i) {
    const int np = parts_of(in_naming, i, P, counts, in_d, parts);
    for (int k = 0; k < np; ++k) {
      sources[parts[k].name].push_back({i, parts[k].off});
      if (parts[k].cnt) d->in_ranges.push_back({i, parts[k].off * esz, parts[k].cnt * esz});
    }
  }

  // Output partitions with the same (source, source offset, size, output
  // offset) in every rank's buffer form one broadcast job.
  using Key = std::tuple<int, int64_t, int64_t, int64_t>;  // src, soff, cnt, doff
  std::map<Key, std::vector<int>> groups;
  std::vector<Key> order;
  for (int j = 0; j < P; ++j) {
    const int np = parts_of(out_naming, j, P, counts, out_d, parts);
    for (int k = 0; k < np; ++k) {
      const Part &p = parts[k];
      const auto &m = sources[p.name];
      if (op == PURLIN_OP_COPY && m.size() != 1) return PURLIN_ERR_UNSUPPORTED;
      if (op == PURLIN_OP_SUM && m.empty()) return PURLIN_ERR_UNSUPPORTED;
      for (const auto &s : m) d->segs.push_back({s.first, j, s.second, p.off, p.cnt});
      if (p.cnt == 0) continue;
      d->out_ranges.push_back({j, p.off * esz, p.cnt * esz});
      int src;
      int64_t soff = m[0].second;
      if (m.size() == 1) {
        src = m[0].first;
      } else {
        // a sum over every rank: all partitions must sit at one offset
        if ((int)m.size() != P) return PURLIN_ERR_UNSUPPORTED;
        for (int i = 0; i < P; ++i)
          if (m[i].first != i || m[i].second != soff) return PURLIN_ERR_UNSUPPORTED;
        src = -1;
      }
      Key key{src, soff, p.cnt, p.off};
      auto it = groups.find(key);
      if (it == groups.end()) {
        groups[key] = {j};
        order.push_back(key);
      } else {
        it->second.push_back(j);
      }
    }
  }

  // Jobs, each with the rank that owns it: the reducer of a sum (ReduceScatter
  // y_k belongs to rank k), the root of a broadcast (AllGather y_k is pushed
  // by rank k), the destination of a point-to-point copy (AllToAll).
  struct Pending { Job job; int owner; };
  std::vector<Pending> pend;
  for (const Key &key : order) {
    const auto &dsts = groups[key];
    const int src = std::get<0>(key);
    Job base{std::get<1>(key) * esz, std::get<3>(key) * esz, std::get<2>(key) * esz, src, 0};
    const int nsrc = src < 0 ? P : 1;
    if ((int)dsts.size() == P && P > 1) {
      base.dst = -1;
      d->bytes_min += base.nbytes * (nsrc + P);
      if (src >= 0) {
        pend.push_back({base, src});
      } else {
        // AllReduce (Figure 6): rank k reduces piece k of the buffer and
        // writes it to every rank.  Pieces start on 16-byte boundaries.
        const int64_t n = base.nbytes;
        for (int k = 0; k < P; ++k) {
          const int64_t b0 = (n * k / P) & ~int64_t(15);
          const int64_t b1 = k + 1 == P ? n : (n * (k + 1) / P) & ~int64_t(15);
          if (b1 <= b0) continue;
          Job piece = base;
          piece.src_off += b0;
          piece.dst_off += b0;
          piece.nbytes = b1 - b0;
          pend.push_back({piece, k});
        }
      }
    } else {
      for (int j : dsts) {
        Job one = base;
        one.dst = j;
        d->bytes_min += base.nbytes * (nsrc + 1);
        pend.push_back({one, j});
      }
    }
  }
  std::stable_sort(pend.begin(), pend.end(),
                   [](const Pending &a, const Pending &b) { return a.owner < b.owner; });
  if ((int)pend.size() > kMaxJobs) return PURLIN_ERR_UNSUPPORTED;
  for (const auto &p : pend) {
    d->jobs.push_back(p.job);
    d->owner.push_back(p.owner);
  }
  return PURLIN_OK;
}

purlin_status check_pointers(const Derived &d, void *const *in, void *const *out) {
  const uintptr_t a = uintptr_t(d.esz) - 1;
  std::vector<std::pair<uintptr_t, uintptr_t>> outs, ins;
  for (const auto &r : d.out_ranges) {
    const uintptr_t b = uintptr_t(out[r.rank]);
    if (!b || (b & a)) return PURLIN_ERR_INVALID_ARG;
    outs.push_back({b + r.off, b + r.off + r.len});
  }
  for (const auto &r : d.in_ranges) {
    const uintptr_t b = uintptr_t(in[r.rank]);
    if (!b || (b & a)) return PURLIN_ERR_INVALID_ARG;
    ins.push_back({b + r.off, b + r.off + r.len});
  }
  return ranges_disjoint(ins, outs) ? PURLIN_OK : PURLIN_ERR_INVALID_ARG;
}

bool ranges_disjoint(const std::vector<std::pair<uintptr_t, uintptr_t>> &ins,
                     std::vector<std::pair<uintptr_t, uintptr_t>> outs) {
  if (ranges_overlap(outs)) return false;  // sorts outs
  for (const auto &r : ins) {
    // first output range ending after r starts
    auto it = std::lower_bound(outs.begin(), outs.end(), r,
                               [](const std::pair<uintptr_t, uintptr_t> &o,
                                  const std::pair<uintptr_t, uintptr_t> &x) {
                                 return o.second <= x.first;
                               });
    if (it != outs.end() && it->first < r.second) return false;
  }
  return true;
}

namespace {

struct CacheEntry {
  int in_n, out_n, op, dtype, P, has_displs;
  std::vector<int64_t> counts, displs;
  Derived d;
};

std::vector<CacheEntry> &cache() {
  static std::vector<CacheEntry> c;
  return c;
}

}  // namespace

purlin_status derive_cached(purlin_naming in_naming, purlin_naming out_naming, purlin_op op,
                            purlin_dtype dtype, int P, const int64_t *counts,
                            const int64_t *displs, const Derived **out) {
  if (P < 1 || P > kMaxRanks || !valid_naming(in_naming) || !valid_naming(out_naming) ||
      !counts)
    return PURLIN_ERR_INVALID_ARG;
  const int nn = name_count(in_naming, P);
  const int nd = displs ? 2 * std::min(nn, name_count(out_naming, P)) : 0;
  auto &c = cache();
  for (size_t k = 0; k < c.size(); ++k) {
    const CacheEntry &e = c[k];
    if (e.in_n == in_naming && e.out_n == out_naming && e.op == op && e.dtype == dtype &&
        e.P == P && e.has_displs == (displs != nullptr) && (int)e.counts.size() == nn &&
        std::memcmp(e.counts.data(), counts, nn * sizeof(int64_t)) == 0 &&
        (int)e.displs.size() == nd &&
        (nd == 0 || std::memcmp(e.displs.data(), displs, nd * sizeof(int64_t)) == 0)) {
      if (k) std::swap(c[k], c[0]);  // most recent first
      *out = &c[0].d;
      return PURLIN_OK;
    }
  }
  CacheEntry e;
  purlin_status s = derive(in_naming, out_naming, op, dtype, P, counts, displs, &e.d);
  if (s != PURLIN_OK) return s;
  static uint64_t next_id = 0;
  e.d.id = ++next_id;
  e.in_n = in_naming; e.out_n = out_naming; e.op = op; e.dtype = dtype; e.P = P;
  e.has_displs = displs != nullptr;
  e.counts.assign(counts, counts + nn);
  if (nd) e.displs.assign(displs, displs + nd);
  if (c.size() >= 32) c.pop_back();
  c.insert(c.begin(), std::move(e));
  *out = &c[0].d;
  return PURLIN_OK;
}

purlin_status launch_jobs(const Derived &d, char *const *out, std::vector<Job> *jobs,
                          std::vector<int> *owner) {
  jobs->clear();
  owner->clear();
  for (size_t k = 0; k < d.jobs.size(); ++k) {
    const Job &jb = d.jobs[k];
    bool congruent = true;
    if (jb.dst < 0) {
      const uintptr_t m0 = (uintptr_t(out[0]) + jb.dst_off) & 15;
      for (int j = 1; j < d.P; ++j)
        if (((uintptr_t(out[j]) + jb.dst_off) & 15) != m0) congruent = false;
    }
    if (congruent) {
      jobs->push_back(jb);
      owner->push_back(d.owner[k]);
    } else {
      for (int j = 0; j < d.P; ++j) {
        Job one = jb;
        one.dst = j;
        jobs->push_back(one);
        owner->push_back(d.owner[k]);
      }
    }
  }
  // A launch plan holds kMaxJobs jobs.  The seven collectives stay within it
  // (at most P * P after the split); a sum of P partitions broadcast to every
  // rank (by_index -> by_index) with outputs off each other's 16-byte phase
  // would need P^3.
  if (jobs->size() > size_t(kMaxJobs)) {
    jobs->clear();
    owner->clear();
    return PURLIN_ERR_UNSUPPORTED;
  }
  return PURLIN_OK;
}

}  // namespace purlin
