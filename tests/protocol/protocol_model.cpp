// Host-thread model of the signal and work-queue protocol of the
// tile-signaled kernels, run on the CPU.
//
// Each device workgroup is a host thread; device memory words are
// std::atomic words; a workgroup's "coherent stores, wait for completion,
// barrier, then one lane publishes" is a release, and a poll followed by an
// acquire is an acquire.  Random delays and permuted arrival orders shuffle
// the interleavings, and every scenario is repeated over many calls (epochs)
// back to back on the same words, as the library does.  The model restates
// the logic of the device code (csrc/ag.hip: claim_unit, copy_unit's unit
// decode, leave_queue, SlabWait; csrc/tsg_device.hpp: sig_arrive_counted_*,
// wave_poll_ge, xcd_queue_claim; csrc/moe.hip and csrc/mlp2.hip: persistent
// queues and their last-one-out reset) and checks the properties the kernels
// rely on:
//   * every copy unit is moved exactly once per call, whoever claims it (the
//     copy kernel's workgroups or the GEMM's pulling workgroups), and the
//     unit decode is a bijection onto (slab, channel, chunk, piece);
//   * a signal completes only after all of its pieces, exactly once per
//     call, and its counter is back at zero afterwards;
//   * a consumer that passed its wait sees every byte its signal covers;
//   * a signal value of an earlier call never satisfies a later call's wait;
//   * ticket and exit counters are back at zero after every call, also when
//     a launch never ran;
//   * per-XCD phased claims hand out every item exactly once, and no worker
//     gets a phase-1 item while a phase-0 item is still unclaimed, so GEMM2
//     tiles (which wait for GEMM1 row blocks) never starve the producers;
//   * a withheld signal ends in a bounded wait that sets the error word, and
//     later waits of that call return at once;
//   * when the last GEMM workgroup of an AllGather call ends (the caller's
//     stream does not wait for the copy kernel), every row of every chunk,
//     the local chunk's included, holds the call's data and every arrival
//     counter is back at zero, while copy workgroups may still be leaving
//     their queue;
//   * when the last GEMM workgroup of a GEMM + ReduceScatter call ends (the
//     caller's stream does not wait for the reduce kernel), every output
//     word holds its final value (the peers' sum plus the local partial).
// Usage: protocol_model [iterations] [seed]; prints one "ok <scenario>" line
// per scenario and exits 0, or prints "FAIL ..." and exits 1.
// Built with -DMUTATION=m (m > 0) the model plants one mistake in its own
// restatement of the protocol, so that a test can show the checks catch it:
//   1: the last arriver does not reset the arrival counter;
//   2: a counted signal is published by its first arriver;
//   3: the last claimer to leave does not reset the ticket counter;
//   4: AllGather tiles inside the local chunk do not wait for its arrival at
//      their end;
//   5: the last GEMM + ReduceScatter GEMM workgroup does not wait for the
//      reduce's end signal.
#ifndef MUTATION
#define MUTATION 0
#endif
#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <functional>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

namespace {

int g_fail = 0;
std::mutex g_mu;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      std::lock_guard<std::mutex> lk_(g_mu);               \
      if (g_fail++ < 10) {                                 \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__);   \
        std::printf(__VA_ARGS__);                          \
        std::printf("\n");                                 \
      }                                                    \
    }                                                      \
  } while (0)

thread_local std::mt19937_64 t_rng{1};

void jitter(int max_us) {
  const int r = (int)(t_rng() % 8);
  if (r == 0) std::this_thread::sleep_for(std::chrono::microseconds(t_rng() % (max_us + 1)));
  else if (r < 3) std::this_thread::yield();
}

void run_threads(int n, uint64_t seed, const std::function<void(int)>& body) {
  std::vector<std::thread> th;
  th.reserve(n);
  for (int i = 0; i < n; ++i)
    th.emplace_back([&, i] {
      t_rng.seed(seed * 1000003u + (uint64_t)i);
      body(i);
    });
  for (auto& t : th) t.join();
}

uint64_t target(uint32_t epoch, uint32_t n) { return ((uint64_t)epoch << 32) | n; }

// ---------------------------------------------------------------- signals
struct Signals {
  std::vector<std::atomic<uint64_t>> sig;
  std::vector<std::atomic<uint32_t>> cnt;
  std::atomic<uint32_t> status{0};
  explicit Signals(size_t n) : sig(n), cnt(n) {
    for (auto& s : sig) s.store(0);
    for (auto& c : cnt) c.store(0);
  }
};

// One of n producers arrives; the last one resets the counter and publishes
// {epoch | n} (sig_arrive_counted_*).
void arrive_counted(Signals& S, size_t i, uint32_t n, uint32_t epoch) {
  const uint32_t old = S.cnt[i].fetch_add(1, std::memory_order_acq_rel);
  if (MUTATION == 2 && old == 0) S.sig[i].store(target(epoch, n), std::memory_order_release);
  if (old == n - 1) {
    if (MUTATION != 1) S.cnt[i].store(0, std::memory_order_relaxed);
    S.sig[i].store(target(epoch, n), std::memory_order_release);
  }
}

// Bounded wait (wave_poll_ge + acquire): true if satisfied.  A wait that
// finds the error word already set returns at once, as on the device.
bool wait_ge(Signals& S, size_t i, uint64_t tgt, int bound_ms) {
  if (S.sig[i].load(std::memory_order_acquire) >= tgt) return true;
  if (S.status.load(std::memory_order_relaxed) & 1u) return false;
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    std::this_thread::yield();
    if (S.sig[i].load(std::memory_order_acquire) >= tgt) return true;
    if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(bound_ms)) {
      S.status.fetch_or(1u, std::memory_order_relaxed);
      return false;
    }
  }
}

// -------------------------------------------------- AllGather copy queue
// The unit decode of copy_unit: slab-major; within a slab, channel 0 of
// every arrival position, then channel 1, ...; np[s] pieces per channel.
constexpr int kHead = 4;
struct Unit {
  int s, ch, p, j, npc;
};
struct AgShape {
  int R, C, n_slab;
  int np[kHead + 1];
  int ustart[kHead + 1];
  int n_units;
};
AgShape ag_shape(int R, int C, int n_slab, const int (&np)[kHead + 1]) {
  AgShape a{};
  a.R = R;
  a.C = C;
  a.n_slab = n_slab;
  int n = 0;
  for (int h = 0; h <= kHead; ++h) a.np[h] = np[h];
  for (int h = 0; h < kHead; ++h) {
    a.ustart[h] = n;
    if (h < n_slab) n += R * C * np[h];
  }
  a.ustart[kHead] = n;
  n += std::max(0, n_slab - kHead) * R * C * np[kHead];
  a.n_units = n;
  return a;
}
Unit decode(const AgShape& a, int u) {
  int s, rem, npc;
  if (u >= a.ustart[kHead]) {
    npc = a.np[kHead];
    const int v = u - a.ustart[kHead];
    const int per = a.R * a.C * npc;
    s = kHead + v / per;
    rem = v - (s - kHead) * per;
  } else {
    s = 0;
    while (u >= a.ustart[s + 1]) ++s;
    npc = a.np[s];
    rem = u - a.ustart[s];
  }
  const int cp = rem / npc;
  const int j = rem - cp * npc;
  const int ch = cp / a.R;
  const int p = cp - ch * a.R;
  return Unit{s, ch, p, j, npc};
}

void check_decode() {
  std::mt19937_64 rng(7);
  for (int it = 0; it < 200; ++it) {
    const int R = 1 + (int)(rng() % 8), C = 1 + (int)(rng() % 4), n_slab = 1 + (int)(rng() % 9);
    int np[kHead + 1];
    for (int h = 0; h <= kHead; ++h) np[h] = 1 + (int)(rng() % 5);
    const AgShape a = ag_shape(R, C, n_slab, np);
    std::vector<int> seen((size_t)n_slab * C * R * 8, 0);
    int prev_s = 0;
    for (int u = 0; u < a.n_units; ++u) {
      const Unit x = decode(a, u);
      CHECK(x.s >= 0 && x.s < n_slab && x.ch >= 0 && x.ch < C && x.p >= 0 && x.p < R && x.j >= 0 && x.j < x.npc,
            "decode out of range u=%d", u);
      CHECK(x.npc == np[std::min(x.s, kHead)], "pieces of slab %d", x.s);
      CHECK(x.s >= prev_s, "units not slab-major at u=%d", u);
      prev_s = x.s;
      seen[(((size_t)x.s * C + x.ch) * R + x.p) * 8 + x.j]++;
    }
    for (int s = 0; s < n_slab; ++s)
      for (int ch = 0; ch < C; ++ch)
        for (int p = 0; p < R; ++p)
          for (int j = 0; j < np[std::min(s, kHead)]; ++j)
            CHECK(seen[(((size_t)s * C + ch) * R + p) * 8 + j] == 1, "unit (%d,%d,%d,%d) seen %d times", s, ch, p, j,
                  seen[(((size_t)s * C + ch) * R + p) * 8 + j]);
  }
  std::printf("ok unit_decode\n");
}

// One call of the AllGather protocol: pulling consumer j moves unit j
// directly (no ticket), and the copy workers claim the other units from one
// ticket counter (ticket t is unit n_pull + t); every unit "moves" its rows
// (writes the call's epoch into each row word of its piece) and arrives on
// its (channel, slab) signal; consumer tiles wait for their channels' signals
// and check every row word they cover.  Tiles inside the local chunk (the
// last arrival position, moved last and slowly here) read it in place and
// wait for its signals only after computing.  The last copy worker to leave
// resets the ticket and exit counters.
struct AgCall {
  AgShape a;
  int chunk_rows, ch_rows;
  int n_copy, n_gemm, n_pull;  // n_pull <= n_gemm GEMM workgroups pull a unit each
  std::vector<int> order;      // chunk at arrival position p; the last is the local chunk
};

void ag_call(Signals& S, std::vector<std::atomic<uint32_t>>& rows, std::atomic<uint32_t> (&queue)[2],
             std::vector<std::atomic<int>>& moved, const AgCall& c, uint32_t epoch, uint64_t seed,
             uint32_t withheld, int bound_ms) {
  const AgShape& a = c.a;
  const int R = a.R, C = a.C, n_workers = c.n_copy;
  const int n_pull = std::min(c.n_pull, a.n_units);  // units taken without a ticket
  for (auto& m : moved) m.store(0);
  auto move_unit = [&](int u) {
    const Unit x = decode(a, u);
    const int chunk = c.order[x.p];
    if (x.p == R - 1) std::this_thread::sleep_for(std::chrono::microseconds(50));
    const int rp = (c.ch_rows + x.npc - 1) / x.npc;
    const int r0 = x.ch * c.ch_rows + x.j * rp;
    const int nr = std::min(rp, (x.ch + 1) * c.ch_rows - r0);
    for (int r = 0; r < nr; ++r)
      rows[((size_t)chunk * c.chunk_rows + r0 + r) * a.n_slab + x.s].store(epoch, std::memory_order_relaxed);
    jitter(20);
    moved[u].fetch_add(1);
    const int g = chunk * C + x.ch;
    if (!(g < 32 && ((withheld >> g) & 1u))) arrive_counted(S, (size_t)g * a.n_slab + x.s, (uint32_t)x.npc, epoch);
  };
  auto leave = [&] {
    if (queue[1].fetch_add(1, std::memory_order_acq_rel) == (uint32_t)n_workers - 1) {
      if (MUTATION != 3) queue[0].store(0, std::memory_order_relaxed);
      queue[1].store(0, std::memory_order_relaxed);
    }
  };
  const int M = R * c.chunk_rows;
  const int BM = std::max(8, c.ch_rows / 2 + 3);  // tiles straddle channel edges
  const int n_tiles = (M + BM - 1) / BM;
  std::atomic<int> tile_next{0}, gemm_done{0};
  const int local = c.order[R - 1];
  run_threads(c.n_copy + c.n_gemm, seed, [&](int w) {
    if (w < c.n_copy) {  // copy kernel workgroup: claim until none is left
      for (;;) {
        const int u = n_pull + (int)queue[0].fetch_add(1, std::memory_order_relaxed);
        if (u >= a.n_units) break;
        jitter(30);
        move_unit(u);
      }
      leave();
      return;
    }
    // GEMM workgroup j: move unit j, then compute tiles
    const int j = w - c.n_copy;
    if (j < n_pull) move_unit(j);
    for (int t = tile_next.fetch_add(1); t < n_tiles; t = tile_next.fetch_add(1)) {
      const int lo = t * BM, hi = std::min(M, lo + BM) - 1;
      auto wait_all = [&] {
        bool ok = true;
        for (int s = 0; s < a.n_slab && ok; ++s)
          for (int g = lo / c.ch_rows; g <= hi / c.ch_rows; ++g)
            ok = ok && wait_ge(S, (size_t)g * a.n_slab + s, target(epoch, 1), bound_ms);
        return ok;
      };
      if (lo / c.chunk_rows == local && hi / c.chunk_rows == local) {
        jitter(20);  // computes from the local shard in place
        if (MUTATION != 4) wait_all();
        continue;
      }
      if (!wait_all()) continue;  // timed out: the call reports an error
      for (int r = lo; r <= hi; ++r)
        for (int s = 0; s < a.n_slab; ++s)
          CHECK(rows[(size_t)r * a.n_slab + s].load(std::memory_order_relaxed) == epoch,
                "tile %d read row %d slab %d before its data (epoch %u)", t, r, s, epoch);
    }
    // The GEMM's end is where the caller's stream moves on: the gathered
    // buffer must be whole and the counters free for the next call's pulls.
    if (gemm_done.fetch_add(1, std::memory_order_acq_rel) == c.n_gemm - 1 && !withheld) {
      for (size_t i = 0; i < rows.size(); ++i)
        CHECK(rows[i].load(std::memory_order_relaxed) == epoch, "row word %zu incomplete when the GEMM ended",
              i);
      for (int g = 0; g < R * C; ++g)
        for (int s = 0; s < a.n_slab; ++s)
          CHECK(S.cnt[(size_t)g * a.n_slab + s].load(std::memory_order_relaxed) == 0,
                "counter (%d,%d) not reset when the GEMM ended", g, s);
    }
  });
  if (!withheld) {
    for (int u = 0; u < a.n_units; ++u) CHECK(moved[u].load() == 1, "unit %d moved %d times", u, moved[u].load());
    for (int g = 0; g < R * C; ++g)
      for (int s = 0; s < a.n_slab; ++s) {
        const size_t i = (size_t)g * a.n_slab + s;
        CHECK(S.sig[i].load() >> 32 == epoch, "signal (%d,%d) not published in epoch %u", g, s, epoch);
        CHECK(S.cnt[i].load() == 0, "counter (%d,%d) left at %u", g, s, S.cnt[i].load());
      }
  }
  CHECK(queue[0].load() == 0 && queue[1].load() == 0, "AG queue not reset (%u, %u)", queue[0].load(),
        queue[1].load());
}

void scenario_ag(int iters, uint64_t seed) {
  std::mt19937_64 rng(seed);
  std::atomic<uint32_t> queue[2];
  queue[0] = 0;
  queue[1] = 0;
  uint32_t epoch = 0;
  const int sig_cap = 8 * 4 * 9;
  Signals S(sig_cap);
  for (int it = 0; it < iters; ++it) {
    const int R = 2 + (int)(rng() % 6), C = 1 << (rng() % 3), n_slab = 1 + (int)(rng() % 6);
    const int ch_rows = 4 + (int)(rng() % 9);
    int np[kHead + 1];
    for (int h = 0; h <= kHead; ++h) np[h] = 1 + (int)(rng() % std::min(4, ch_rows));
    AgCall c;
    c.a = ag_shape(R, C, n_slab, np);
    c.ch_rows = ch_rows;
    c.chunk_rows = ch_rows * C;
    c.n_copy = 1 + (int)(rng() % 6);
    c.n_pull = (int)(rng() % 4);
    c.n_gemm = std::max(1, c.n_pull) + (int)(rng() % 2);
    c.order.resize(R);
    for (int p = 0; p < R; ++p) c.order[p] = p;
    std::shuffle(c.order.begin(), c.order.end(), rng);  // any arrival permutation
    std::vector<std::atomic<uint32_t>> rows((size_t)R * c.chunk_rows * n_slab);
    for (auto& r : rows) r.store(0);
    std::vector<std::atomic<int>> moved(c.a.n_units);
    ++epoch;
    ag_call(S, rows, queue, moved, c, epoch, seed + (uint64_t)it, 0u, 5000);
    CHECK(S.status.load() == 0, "status set in a complete call");
  }
  std::printf("ok ag_queue_counted_arrival_epochs (%d calls)\n", iters);

  // withheld signal: bounded waits, error word, later waits return at once;
  // the host then clears counters and status and the next call is clean
  for (int it = 0; it < std::max(2, iters / 10); ++it) {
    const int R = 3, C = 2, ch_rows = 6;
    int np[kHead + 1] = {2, 2, 1, 1, 1};
    AgCall c;
    c.a = ag_shape(R, C, 2, np);
    c.ch_rows = ch_rows;
    c.chunk_rows = ch_rows * C;
    c.n_copy = 3;
    c.n_pull = 2;
    c.n_gemm = 2;
    c.order = {2, 0, 1};
    std::vector<std::atomic<uint32_t>> rows((size_t)R * c.chunk_rows * 2);
    for (auto& r : rows) r.store(0);
    std::vector<std::atomic<int>> moved(c.a.n_units);
    ++epoch;
    ag_call(S, rows, queue, moved, c, epoch, seed + 77 + (uint64_t)it, 1u << 3, 20);
    CHECK(S.status.load() & 1u, "withheld signal did not time out");
    const auto t0 = std::chrono::steady_clock::now();
    CHECK(!wait_ge(S, 3 * 2, target(epoch, 1), 10000), "late wait satisfied");
    CHECK(std::chrono::steady_clock::now() - t0 < std::chrono::milliseconds(50), "late wait did not return at once");
    for (auto& x : S.cnt) x.store(0);  // tsg_check after a timeout
    S.status.store(0);
    ++epoch;
    ag_call(S, rows, queue, moved, c, epoch, seed + 99 + (uint64_t)it, 0u, 5000);
    CHECK(S.status.load() == 0, "call after recovery timed out");
  }
  std::printf("ok ag_withheld_signal_timeout_and_recovery\n");
}

// ------------------------------------------------ per-XCD phased queues
// xcd_queue_claim: phase p has n[p] items cut into 8 shares; a worker tries
// its XCD's share, then the shares whose counters still show tickets; it
// moves to phase p + 1 only after a failed claim on every share of phase p.
struct Claim {
  int phase, index;
};
Claim xcd_claim(std::atomic<uint32_t>* q, const int* n, int NP, int my_xcd, int from) {
  for (int ph = from; ph < NP; ++ph) {
    const int np = n[ph];
    int got = -1;
    auto claim = [&](int x) {
      const int lo = (int)((int64_t)np * x / 8), hi = (int)((int64_t)np * (x + 1) / 8);
      if (hi == lo) return;
      const uint32_t t = q[ph * 8 + x].fetch_add(1, std::memory_order_relaxed);
      if (t < (uint32_t)(hi - lo)) got = lo + (int)t;
    };
    claim(my_xcd);
    if (got < 0) {
      std::vector<int> open;
      for (int x = 0; x < 8; ++x) {
        if (x == my_xcd) continue;
        const int lo = (int)((int64_t)np * x / 8), hi = (int)((int64_t)np * (x + 1) / 8);
        if (q[ph * 8 + x].load(std::memory_order_relaxed) < (uint32_t)(hi - lo)) open.push_back(x);
      }
      for (size_t i = 0; i < open.size() && got < 0; ++i) claim(open[i]);
    }
    if (got >= 0) return Claim{ph, got};
  }
  return Claim{-1, 0};
}

void scenario_xcd_queues(int iters, uint64_t seed) {
  std::mt19937_64 rng(seed);
  std::atomic<uint32_t> q[17];
  for (auto& x : q) x.store(0);
  Signals S(64);
  uint32_t epoch = 0;
  for (int it = 0; it < iters; ++it) {
    // the fused MLP: phase 0 = GEMM1 tiles (n_rb row blocks x nt1 column
    // tiles, each arriving on its row block), phase 1 = GEMM2 tiles (each
    // waits for its row block)
    const int n_rb = 1 + (int)(rng() % 12), nt1 = 1 + (int)(rng() % 5), nt2 = 1 + (int)(rng() % 5);
    const int n[2] = {n_rb * nt1, n_rb * nt2};
    const int workers = 1 + (int)(rng() % 9);
    std::vector<std::atomic<int>> got0(n[0]), got1(n[1]);
    for (auto& x : got0) x.store(0);
    for (auto& x : got1) x.store(0);
    std::atomic<int> claimed0{0};
    ++epoch;
    run_threads(workers, seed + (uint64_t)it, [&](int w) {
      const int my_xcd = w % 8;
      int phase = 0;
      for (;;) {
        const Claim c = xcd_claim(q, n, 2, my_xcd, phase);
        if (c.phase < 0) break;
        phase = c.phase;
        jitter(20);
        if (c.phase == 0) {
          got0[c.index].fetch_add(1);
          claimed0.fetch_add(1);
          arrive_counted(S, (size_t)(c.index % n_rb), (uint32_t)nt1, epoch);
        } else {
          // no phase-1 item while a phase-0 item is unclaimed
          for (int x = 0; x < 8; ++x) {
            const int lo = (int)((int64_t)n[0] * x / 8), hi = (int)((int64_t)n[0] * (x + 1) / 8);
            CHECK(q[x].load() >= (uint32_t)(hi - lo), "phase-1 item taken while phase-0 share %d open", x);
          }
          got1[c.index].fetch_add(1);
          CHECK(wait_ge(S, (size_t)(c.index % n_rb), target(epoch, (uint32_t)nt1), 5000),
                "GEMM2 item %d starved (epoch %u)", c.index, epoch);
        }
      }
      // last one out resets every counter
      if (q[16].fetch_add(1, std::memory_order_acq_rel) == (uint32_t)workers - 1)
        for (int i = 0; i <= 16; ++i) q[i].store(0, std::memory_order_relaxed);
    });
    for (int i = 0; i < n[0]; ++i) CHECK(got0[i].load() == 1, "phase-0 item %d taken %d times", i, got0[i].load());
    for (int i = 0; i < n[1]; ++i) CHECK(got1[i].load() == 1, "phase-1 item %d taken %d times", i, got1[i].load());
    for (int i = 0; i <= 16; ++i) CHECK(q[i].load() == 0, "XCD queue word %d left at %u", i, q[i].load());
    for (int b = 0; b < n_rb; ++b) CHECK(S.cnt[b].load() == 0, "row-block counter %d left", b);
  }
  std::printf("ok xcd_phased_queues_mlp_dependencies (%d calls)\n", iters);
}

// ----------------------------------------------------- MoE producer queue
// One ticket counter over up tiles, down tiles (each waits for its row
// block's up tiles) and combine units (each waits for its down tile's ready
// signal); every workgroup ends with one failing ticket and the last one to
// leave resets the ticket and exit counters.
void moe_call(Signals& S, std::atomic<uint32_t> (&queue)[2], int n_rb, int nu, int nd, int workers,
              uint32_t epoch, uint64_t seed) {
  const int n_up = n_rb * nu, n_dn = n_rb * nd, n_items = n_up + 2 * n_dn;
  std::vector<std::atomic<int>> done(n_items);
  for (auto& d : done) d.store(0);
  std::vector<std::atomic<uint32_t>> h(n_rb), y(n_dn);
  for (auto& x : h) x.store(0);
  for (auto& x : y) x.store(0);
  run_threads(workers, seed, [&](int) {
    for (;;) {
      const int item = (int)queue[0].fetch_add(1, std::memory_order_relaxed);
      if (item >= n_items) break;
      jitter(20);
      if (item < n_up) {
        const int rb = item / nu;
        h[rb].store(epoch, std::memory_order_relaxed);
        arrive_counted(S, (size_t)rb, (uint32_t)nu, epoch);
      } else if (item < n_up + n_dn) {
        const int t = item - n_up, rb = t / nd;
        CHECK(wait_ge(S, (size_t)rb, target(epoch, (uint32_t)nu), 5000), "down tile %d starved", t);
        CHECK(h[rb].load(std::memory_order_relaxed) == epoch, "down tile %d read h before its signal", t);
        y[t].store(epoch, std::memory_order_relaxed);
        S.sig[1024 + t].store(target(epoch, 1), std::memory_order_release);
      } else {
        const int t = item - n_up - n_dn;
        CHECK(wait_ge(S, 1024 + (size_t)t, target(epoch, 1), 5000), "combine unit %d starved", t);
        CHECK(y[t].load(std::memory_order_relaxed) == epoch, "combine unit %d read y before ready", t);
      }
      done[item].fetch_add(1);
    }
    if (queue[1].fetch_add(1, std::memory_order_acq_rel) == (uint32_t)workers - 1) {
      queue[0].store(0, std::memory_order_relaxed);
      queue[1].store(0, std::memory_order_relaxed);
    }
  });
  for (int i = 0; i < n_items; ++i) CHECK(done[i].load() == 1, "MoE item %d done %d times", i, done[i].load());
}

void scenario_moe(int iters, uint64_t seed) {
  std::mt19937_64 rng(seed);
  std::atomic<uint32_t> queue[2];
  queue[0] = 0;
  queue[1] = 0;
  Signals S(2048);
  uint32_t epoch = 0;
  for (int it = 0; it < iters; ++it) {
    const int n_rb = 1 + (int)(rng() % 10), nu = 1 + (int)(rng() % 4), nd = 1 + (int)(rng() % 6);
    const int workers = 1 + (int)(rng() % 8);
    ++epoch;
    if (rng() % 5 == 0) {
      // a launch that never ran: the epoch advances, nothing is claimed,
      // and the counters stay at zero for the next call
      CHECK(queue[0].load() == 0 && queue[1].load() == 0, "queue not at zero before a failed launch");
      ++epoch;
    }
    moe_call(S, queue, n_rb, nu, nd, workers, epoch, seed + (uint64_t)it);
    CHECK(queue[0].load() == 0 && queue[1].load() == 0, "MoE queue not reset (%u, %u)", queue[0].load(),
          queue[1].load());
  }
  std::printf("ok moe_queue_reset_and_failed_launch (%d calls)\n", iters);
}

// --------------------------------------------------------------- epochs
// A signal left at {e-1 | n} by the previous call, or at {e | n-1} by an
// incomplete count, never satisfies a wait for {e | n}.
void scenario_epochs(uint64_t seed) {
  Signals S(4);
  std::mt19937_64 rng(seed);
  for (int it = 0; it < 1000; ++it) {
    const uint32_t e = 2 + (uint32_t)(rng() % 1000000), n = 1 + (uint32_t)(rng() % 64);
    S.status.store(1);  // waits return at once instead of spinning
    S.sig[0].store(target(e - 1, 0xFFFFFFFFu));
    CHECK(!wait_ge(S, 0, target(e, n), 1), "previous epoch satisfied a wait");
    S.sig[0].store(target(e, n - 1));
    CHECK(n == 1 || !wait_ge(S, 0, target(e, n), 1), "incomplete count satisfied a wait");
    S.sig[0].store(target(e, n));
    CHECK(wait_ge(S, 0, target(e, n), 1), "complete signal not accepted");
  }
  std::printf("ok epoch_tagging\n");
}

}  // namespace

// ------------------------------------------------- GEMM + ReduceScatter
// One call: GEMM workers take tiles from a counter, write the tile's partial
// words (the call's epoch) and publish its flag; the worker dispatched last
// then waits for the reduce's end signal.  Reduce workers own output words:
// phase 1 writes the peers' sum (2 e), phase 2 waits for the word's tile
// flag, reads the partial and writes 2 e + 1; then each arrives on the end
// signal (slowly, so that a GEMM that did not wait would end first).  When
// the last GEMM worker ends, every output word must be final.
void scenario_rs(int iters, uint64_t seed) {
  std::mt19937_64 rng(seed);
  uint32_t epoch = 1000;
  for (int it = 0; it < iters; ++it) {
    const int n_tiles = 1 + (int)(rng() % 12), per_tile = 1 + (int)(rng() % 4);
    const int n_gemm = 1 + (int)(rng() % 4), n_red = 1 + (int)(rng() % 4);
    Signals S((size_t)n_tiles + 1);  // tile flags, then the reduce's end signal
    const size_t done = (size_t)n_tiles;
    std::vector<std::atomic<uint32_t>> partial((size_t)n_tiles * per_tile), out((size_t)n_tiles * per_tile);
    for (auto& x : partial) x.store(0);
    for (auto& x : out) x.store(0);
    ++epoch;
    std::atomic<int> tile_next{0}, gemm_left{n_gemm};
    run_threads(n_gemm + n_red, seed + (uint64_t)it, [&](int w) {
      if (w < n_gemm) {
        for (int t = tile_next.fetch_add(1); t < n_tiles; t = tile_next.fetch_add(1)) {
          jitter(20);
          for (int i = 0; i < per_tile; ++i) partial[(size_t)t * per_tile + i].store(epoch, std::memory_order_relaxed);
          S.sig[t].store(target(epoch, 1), std::memory_order_release);
        }
        if (w == n_gemm - 1 && MUTATION != 5) wait_ge(S, done, target(epoch, (uint32_t)n_red), 5000);
        if (gemm_left.fetch_sub(1, std::memory_order_acq_rel) == 1)
          for (size_t i = 0; i < out.size(); ++i)
            CHECK(out[i].load(std::memory_order_relaxed) == 2 * epoch + 1,
                  "output word %zu not final when the GEMM ended (epoch %u)", i, epoch);
        return;
      }
      const int r = w - n_gemm;
      for (size_t i = (size_t)r; i < out.size(); i += (size_t)n_red) out[i].store(2 * epoch, std::memory_order_relaxed);
      for (size_t i = (size_t)r; i < out.size(); i += (size_t)n_red) {
        if (!wait_ge(S, i / (size_t)per_tile, target(epoch, 1), 5000)) continue;
        CHECK(partial[i].load(std::memory_order_relaxed) == epoch, "partial word %zu read before its flag", i);
        out[i].store(out[i].load(std::memory_order_relaxed) + 1, std::memory_order_relaxed);
      }
      std::this_thread::sleep_for(std::chrono::microseconds(200));
      arrive_counted(S, done, (uint32_t)n_red, epoch);
    });
    CHECK(S.status.load() == 0, "rs call timed out");
    CHECK(S.cnt[done].load() == 0, "end-signal counter left at %u", S.cnt[done].load());
  }
  std::printf("ok rs_end_signal_joins_through_the_gemm (%d calls)\n", iters);
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 200;
  const uint64_t seed = argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 12345;
  check_decode();
  scenario_epochs(seed);
  scenario_ag(iters, seed);
  scenario_xcd_queues(iters, seed + 1);
  scenario_moe(iters, seed + 2);
  scenario_rs(iters / 2, seed + 3);
  if (g_fail) {
    std::printf("FAIL: %d checks failed\n", g_fail);
    return 1;
  }
  return 0;
}
