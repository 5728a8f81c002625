// CPU model of the staged SNAC protocol and of the entry / exit handshake,
// for ThreadSanitizer (test infrastructure; shares no code with the HIP
// kernels, which it models).
//
// Purlin's middle layer is Stage, Notify, And Consume (abstract).  The model
// runs the staged AllReduce of P ranks: piece k of the buffer is owned by
// rank k (Figure 6: the reduced chunk of piece k reaches every rank).  Per
// piece, one thread per role, as the kernel has one workgroup per role:
//   stager s   copies its rank's chunk m into slot m % D of its ring, after
//              the owner's credit for the slot's previous round, and
//              notifies "ready" with (epoch, round + 1);
//   owner t    (one of a team of T per piece and lane) waits for every
//              stager's ready, folds its own input and the staged chunks in
//              ascending rank into its own output and into slot m % D of its
//              scatter ring (after the scatter threads' credits for that
//              slot's previous round), for its slice t of the chunk only;
//              returns a credit to each stager's slot (a stager waits for T
//              per round) and notifies its own ready word of the scatter slot;
//   scatter d  waits for the notify of every owner of the team, copies the
//              slot into rank d's output and returns a credit.
// Flags are 64-bit words tagged with the launch epoch in the high half and
// are never reset; a waiter waits for (flag - target) >= 0.  Every wait has
// a wall-clock watchdog; on expiry it sets the status word and the launch's
// abort epoch, and every other wait of that launch then gives up.
//
// The launch epoch lives in shared memory, as on the device: every workgroup
// reads the epoch word when it starts (epoch = word + 1), and the last
// workgroup to count itself out advances it.  The exit count is spread over
// several counters (workgroup b adds 1 to counter b % S); the workgroup that
// completes a counter resets it and adds 1 to a second-level counter, and
// the one completing that resets it and stores the next epoch.  Launches run
// one after another (stream order), and the host checks that every launch
// advanced the epoch by exactly one.  Launches also run the handshake:
// announcer r publishes entry[r] = epoch, and every workgroup waits for all
// entry flags before it starts.  Workgroups are numbered as in the kernel:
// per piece and lane the stagers, then the owners, then the scatter
// consumers.
//
// Memory orders: a notify that publishes data is a release and its wait an
// acquire.  On the GPU the producer writes the slot with device-scope
// stores, waits for all of them to complete and then stores the flag
// relaxed, which orders the data before the flag the way a release does
// (without the release's writeback of the L2), and the consumer takes an
// acquire fence after its wait.  The GPU's "done reading" notifies (credits, exit
// counts) are relaxed adds issued after the workgroup's loads have returned,
// and their waits take no acquire; that ordering comes from the hardware (no
// store issues before the load that saw the flag returned).  C++ gives no
// such guarantee for plain memory, so the model uses release / acquire for
// those too; it checks the protocol's counting, tags and slot reuse, not
// the GPU memory model.
//
// Usage: snac_model P D lanes chunks chunk_elems launches seed
//                   [withhold_launch withhold_chunk] [watchdog_ms]
// SNAC_TEAM=T sets the owners per piece and lane (default 1).
// SNAC_MUTATION=n plants a protocol mistake, so a test can check that the
// model catches it: 1 a stager reuses a slot without its credit wait, 2 the
// owner notifies its scatter ring before writing the slot, 3 a scatter
// consumer returns its credit before copying the slot, 4 a scatter consumer
// waits for the first owner of the team only, 5 a stager waits for one
// owner's credit per round instead of the team's, 6 the workgroup completing
// an exit counter does not reset it (the next launch's count never
// completes, so the epoch stops advancing and the flags of two launches
// carry one epoch).
// Exit status 0: every launch correct, or with withholding: the withheld
// launch ended in TIMEOUT, every thread returned, and the launches after it
// are correct again.
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

namespace {

using Clock = std::chrono::steady_clock;

constexpr int kExitSlots = 4;

struct Flag {
  alignas(64) std::atomic<uint64_t> v{0};
};

uint64_t tag(uint32_t epoch, uint64_t v) { return (uint64_t(epoch) << 32) | v; }

struct Model {
  int P, D, L, chunks, C;
  int T = 1;  // owners per piece and lane
  long watchdog_ms;
  // buffers: in[r], out[r] of P * pieceN elements, piece k = [k * pieceN, (k+1) * pieceN)
  int pieceN;
  std::vector<std::vector<int64_t>> in, out;
  // rings: per piece k, per lane: (P-1) stage rings + 1 scatter ring, D slots of C elements
  int rings_per_lane;
  std::vector<int64_t> ring;  // [piece][lane][ring][slot][C]
  std::vector<Flag> ready, credit;
  std::vector<Flag> team_ready;  // scatter slots: one ready word per owner of the team
  Flag entry[64];
  Flag exits[kExitSlots];
  Flag exit_top;
  std::atomic<uint32_t> epoch_word{0};
  std::atomic<uint32_t> status{0};
  std::atomic<uint32_t> abort_epoch{0};
  int withhold_launch = -1, withhold_chunk = -1;
  int mutation = 0;

  int slot_index(int piece, int lane, int r, int slot) const {
    return ((piece * L + lane) * rings_per_lane + r) * D + slot;
  }
  int64_t *slot_data(int piece, int lane, int r, int slot) {
    return &ring[size_t(slot_index(piece, lane, r, slot)) * C];
  }

  // spin until flag - target >= 0 (wrap-aware); false on watchdog or abort
  bool wait_geq(std::atomic<uint64_t> &f, uint64_t target, uint32_t epoch, std::mt19937 &rng) {
    const auto t0 = Clock::now();
    for (;;) {
      if (int64_t(f.load(std::memory_order_acquire) - target) >= 0) return true;
      if (abort_epoch.load(std::memory_order_acquire) == epoch) return false;
      if (Clock::now() - t0 > std::chrono::milliseconds(watchdog_ms)) {
        status.fetch_or(1u, std::memory_order_relaxed);
        abort_epoch.store(epoch, std::memory_order_release);
        return false;
      }
      if (rng() % 4 == 0) std::this_thread::yield();
    }
  }

  static void jitter(std::mt19937 &rng) {
    const unsigned r = rng() % 16;
    if (r == 0) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 200));
    else if (r < 6) std::this_thread::yield();
  }

  // rank of stager k of piece `owner` (the sources other than the owner, in order)
  static int src_of(int k, int owner) { return k < owner ? k : k + 1; }

  // chunk m of a lane covers elements [x0, x1) of the piece
  void bounds(int lane, int m, int &x0, int &x1) const {
    const int c = lane + L * m;
    x0 = c * C;
    x1 = x0 + C < pieceN ? x0 + C : pieceN;
  }
  int lane_chunks(int lane) const {
    int n = 0;
    for (int c = lane; c < chunks; c += L) ++n;
    return n;
  }

  void stager(int piece, int lane, int k, uint32_t e, int launch, unsigned seed) {
    std::mt19937 rng(seed);
    const int src = src_of(k, piece);
    for (int m = 0; m < lane_chunks(lane); ++m) {
      const int slot = m % D;
      const uint64_t round = uint64_t(m / D);
      const int g = slot_index(piece, lane, k, slot);
      const uint64_t per_round = mutation == 5 ? 1 : uint64_t(T);
      if (round == 0) credit[g].v.store(tag(e, 0), std::memory_order_relaxed);
      else if (mutation != 1 && !wait_geq(credit[g].v, tag(e, round * per_round), e, rng)) return;
      int x0, x1;
      bounds(lane, m, x0, x1);
      int64_t *d = slot_data(piece, lane, k, slot);
      for (int x = x0; x < x1; ++x) d[x - x0] = in[src][piece * pieceN + x];
      jitter(rng);
      const bool withhold = launch == withhold_launch && piece == 0 && lane == 0 && k == 0 &&
                            lane + L * m == withhold_chunk;
      if (!withhold) ready[g].v.store(tag(e, round + 1), std::memory_order_release);
    }
  }

  void owner(int piece, int lane, int t, uint32_t e, unsigned seed) {
    std::mt19937 rng(seed);
    const int scat = P - 1;  // scatter ring index
    for (int m = 0; m < lane_chunks(lane); ++m) {
      const int slot = m % D;
      const uint64_t round = uint64_t(m / D);
      for (int k = 0; k < P - 1; ++k)
        if (!wait_geq(ready[slot_index(piece, lane, k, slot)].v, tag(e, round + 1), e, rng)) return;
      const int gs = slot_index(piece, lane, scat, slot);
      if (round == 0) credit[gs].v.store(tag(e, 0), std::memory_order_relaxed);
      else if (!wait_geq(credit[gs].v, tag(e, round * uint64_t(P - 1)), e, rng)) return;
      int c0, c1;
      bounds(lane, m, c0, c1);
      const int x0 = c0;
      int64_t *sd = slot_data(piece, lane, scat, slot);
      // this owner's slice of the chunk
      const int part = (c1 - c0 + T - 1) / T;
      const int lo = c0 + (t * part < c1 - c0 ? t * part : c1 - c0);
      const int hi = c0 + ((t + 1) * part < c1 - c0 ? (t + 1) * part : c1 - c0);
      std::atomic<uint64_t> &mine = team_ready[size_t(gs) * T + t].v;
      if (mutation == 2) mine.store(tag(e, round + 1), std::memory_order_release);
      for (int x = lo; x < hi; ++x) {
        int64_t acc = 0;
        for (int r = 0; r < P; ++r) {  // ascending rank: own input or staged chunk
          if (r == piece) acc += in[r][piece * pieceN + x];
          else acc += slot_data(piece, lane, r < piece ? r : r - 1, slot)[x - x0];
        }
        out[piece][piece * pieceN + x] = acc;
        sd[x - x0] = acc;
      }
      jitter(rng);
      for (int k = 0; k < P - 1; ++k)
        credit[slot_index(piece, lane, k, slot)].v.fetch_add(1, std::memory_order_release);
      if (mutation != 2) mine.store(tag(e, round + 1), std::memory_order_release);
    }
  }

  void scatter(int piece, int lane, int k, uint32_t e, unsigned seed) {
    std::mt19937 rng(seed);
    const int dst = src_of(k, piece);
    const int scat = P - 1;
    for (int m = 0; m < lane_chunks(lane); ++m) {
      const int slot = m % D;
      const uint64_t round = uint64_t(m / D);
      const int gs = slot_index(piece, lane, scat, slot);
      bool ok = true;
      for (int t = 0; t < (mutation == 4 ? 1 : T) && ok; ++t)
        ok = wait_geq(team_ready[size_t(gs) * T + t].v, tag(e, round + 1), e, rng);
      if (!ok) return;
      int x0, x1;
      bounds(lane, m, x0, x1);
      const int64_t *sd = slot_data(piece, lane, scat, slot);
      if (mutation == 3) credit[gs].v.fetch_add(1, std::memory_order_release);
      for (int x = x0; x < x1; ++x) out[dst][piece * pieceN + x] = sd[x - x0];
      jitter(rng);
      if (mutation != 3) credit[gs].v.fetch_add(1, std::memory_order_release);
    }
  }

  // the launch epoch a workgroup reads when it starts
  uint32_t launch_epoch() const { return epoch_word.load(std::memory_order_acquire) + 1u; }
  // handshake of one workgroup b of a grid of G
  bool entry_wait(int b, int G, uint32_t e, std::mt19937 &rng) {
    for (int r = b; r < P; r += G) entry[r].v.store(e, std::memory_order_release);
    for (int r = 0; r < P; ++r)
      if (!wait_geq(entry[r].v, e, e, rng)) return false;
    return true;
  }
  void exit_notify(int b, int G, uint32_t e) {
    const int s = b % kExitSlots;
    const uint64_t want = uint64_t(G / kExitSlots + (s < G % kExitSlots ? 1 : 0));
    const uint64_t nslots = uint64_t(G < kExitSlots ? G : kExitSlots);
    if (exits[s].v.fetch_add(1, std::memory_order_acq_rel) + 1 == want) {
      if (mutation != 6) exits[s].v.store(0, std::memory_order_relaxed);
      if (exit_top.v.fetch_add(1, std::memory_order_acq_rel) + 1 == nslots) {
        exit_top.v.store(0, std::memory_order_relaxed);
        epoch_word.store(e == 0xffffffffu ? 0u : e, std::memory_order_release);
      }
    }
  }
};

}  // namespace

int main(int argc, char **argv) {
  if (argc < 8) {
    std::fprintf(stderr, "usage: %s P D lanes chunks chunk_elems launches seed "
                         "[withhold_launch withhold_chunk] [watchdog_ms]\n", argv[0]);
    return 2;
  }
  Model M;
  M.P = std::atoi(argv[1]);
  M.D = std::atoi(argv[2]);
  M.L = std::atoi(argv[3]);
  M.chunks = std::atoi(argv[4]);
  M.C = std::atoi(argv[5]);
  const int launches = std::atoi(argv[6]);
  const unsigned seed = unsigned(std::atoi(argv[7]));
  if (argc >= 10) {
    M.withhold_launch = std::atoi(argv[8]);
    M.withhold_chunk = std::atoi(argv[9]);
  }
  M.watchdog_ms = argc >= 11 ? std::atol(argv[10]) : 20000;
  if (const char *mu = std::getenv("SNAC_MUTATION")) M.mutation = std::atoi(mu);
  if (const char *tm = std::getenv("SNAC_TEAM")) M.T = std::atoi(tm);
  if (M.P < 2 || M.P > 16 || M.D < 1 || M.L < 1 || M.chunks < 1 || M.C < 1 || launches < 1 ||
      M.T < 1 || M.T > 16)
    return 2;
  M.pieceN = M.chunks * M.C - M.C / 3;  // a ragged last chunk
  const int N = M.P * M.pieceN;
  M.in.assign(M.P, std::vector<int64_t>(N));
  M.out.assign(M.P, std::vector<int64_t>(N));
  M.rings_per_lane = M.P;  // P-1 stage rings + 1 scatter ring
  const size_t nslots = size_t(M.P) * M.L * M.rings_per_lane * M.D;
  M.ring.assign(nslots * M.C, 0);
  M.ready = std::vector<Flag>(nslots);
  M.credit = std::vector<Flag>(nslots);
  M.team_ready = std::vector<Flag>(nslots * size_t(M.T));

  std::mt19937 rng(seed);
  int bad = 0;
  uint32_t last_epoch = 0;
  for (int launch = 0; launch < launches; ++launch) {
    const uint32_t before = M.launch_epoch();
    if (before != last_epoch + 1) {
      std::fprintf(stderr, "launch %d: epoch %u after %u\n", launch, before, last_epoch);
      ++bad;
    }
    last_epoch = before;
    for (int r = 0; r < M.P; ++r)
      for (int x = 0; x < N; ++x) M.in[r][x] = int64_t(rng() % 1000003) - 500000 + launch;
    for (auto &o : M.out) std::fill(o.begin(), o.end(), int64_t(-1));
    // one workgroup per role, as in the kernel: per piece and lane P-1
    // stagers, T owners and P-1 scatter consumers
    std::vector<std::thread> th;
    const int roles = M.T + 2 * (M.P - 1);
    int G = M.P * M.L * roles;
    int b = 0;
    for (int piece = 0; piece < M.P; ++piece)
      for (int lane = 0; lane < M.L; ++lane)
        for (int role = 0; role < roles; ++role, ++b) {
          const unsigned s = unsigned(rng());
          th.emplace_back([&M, piece, lane, role, b, G, launch, s] {
            std::mt19937 r(s);
            const uint32_t epoch = M.launch_epoch();
            if (M.entry_wait(b, G, epoch, r)) {
              if (role < M.P - 1) M.stager(piece, lane, role, epoch, launch, s);
              else if (role < M.P - 1 + M.T) M.owner(piece, lane, role - (M.P - 1), epoch, s);
              else M.scatter(piece, lane, role - M.T - (M.P - 1), epoch, s);
            }
            M.exit_notify(b, G, epoch);
          });
        }
    for (auto &t : th) t.join();
    if (M.launch_epoch() != last_epoch + 1) {
      std::fprintf(stderr, "launch %d: the epoch did not advance\n", launch);
      ++bad;
    }
    const bool timed_out = (M.status.load() & 1u) != 0;
    if (launch == M.withhold_launch) {
      if (!timed_out) {
        std::fprintf(stderr, "launch %d: withheld notify did not time out\n", launch);
        ++bad;
      }
      M.status.store(0);  // the host reads and clears the status word
      continue;
    }
    if (timed_out) {
      std::fprintf(stderr, "launch %d: unexpected timeout\n", launch);
      ++bad;
      M.status.store(0);
      continue;
    }
    for (int j = 0; j < M.P; ++j)
      for (int x = 0; x < N; ++x) {
        int64_t want = 0;
        for (int r = 0; r < M.P; ++r) want += M.in[r][x];
        if (M.out[j][x] != want) {
          if (bad < 5)
            std::fprintf(stderr, "launch %d rank %d elem %d: got %lld want %lld\n", launch, j, x,
                         (long long)M.out[j][x], (long long)want);
          ++bad;
        }
      }
  }
  std::printf("%s P=%d D=%d lanes=%d team=%d chunks=%d C=%d launches=%d\n", bad ? "FAIL" : "ok",
              M.P, M.D, M.L, M.T, M.chunks, M.C, launches);
  return bad ? 1 : 0;
}
