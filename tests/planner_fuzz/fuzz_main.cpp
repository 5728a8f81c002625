// Driver of the host planner for the sanitizer fuzz test (test
// infrastructure).  Built with g++ and AddressSanitizer /
// UndefinedBehaviorSanitizer from the planner's own source; no HIP call.
//
// Reads cases from stdin, one per line:
//   in_naming out_naming op dtype P n_counts c_0 .. c_{n-1} n_displs d_0 .. d_{m-1} n_out o_0 ..
// (o_k: output buffer addresses for the launch split, decimal) and prints,
// per case, "status <s>" then "seg <src> <dst> <src_off> <dst_off> <len>" for
// every segment of the derivation, then "jobs <status> <count>" from the
// launch split with those output addresses, then "end".
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "../../reduce_atom_02_amd/csrc/planner.hpp"

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    if (line.empty()) continue;
    std::istringstream in(line);
    int in_n, out_n, op, dtype, P, nc, nd, no;
    in >> in_n >> out_n >> op >> dtype >> P >> nc;
    std::vector<int64_t> counts(size_t(nc > 0 ? nc : 0));
    for (auto &c : counts) in >> c;
    in >> nd;
    std::vector<int64_t> displs(size_t(nd > 0 ? nd : 0));
    for (auto &d : displs) in >> d;
    in >> no;
    std::vector<uint64_t> outs(size_t(no > 0 ? no : 0));
    for (auto &o : outs) in >> o;
    // counts and displs are exactly as long as the caller says: the
    // sanitizers catch a read past them
    purlin::Derived d;
    const purlin_status s =
        purlin::derive(purlin_naming(in_n), purlin_naming(out_n), purlin_op(op), purlin_dtype(dtype),
                       P, counts.empty() ? nullptr : counts.data(),
                       displs.empty() ? nullptr : displs.data(), &d);
    std::printf("status %d\n", int(s));
    if (s == PURLIN_OK) {
      for (const auto &g : d.segs)
        std::printf("seg %d %d %lld %lld %lld\n", g.src_rank, g.dst_rank, (long long)g.src_off,
                    (long long)g.dst_off, (long long)g.len);
      if (int(outs.size()) >= P) {
        std::vector<char *> ptrs(outs.size());
        for (size_t k = 0; k < outs.size(); ++k) ptrs[k] = reinterpret_cast<char *>(outs[k]);
        std::vector<purlin::Job> jobs;
        std::vector<int> owners;
        const purlin_status js = purlin::launch_jobs(d, ptrs.data(), &jobs, &owners);
        std::printf("jobs %d %zu\n", int(js), jobs.size());
      }
    }
    std::printf("end\n");
  }
  return 0;
}
