// CPU model of the layer kernel's cross-workgroup protocols, one std::thread per
// workgroup, built with ThreadSanitizer by tests/test_host_sanitizers.py.
//
// The same counting rules as the kernel (the kernel's own code cannot run on a
// CPU), with C++ release/acquire atomics standing for the kernel's agent-scope
// write-backs and loads:
//   1. the two-level grid barrier: group counters that only grow by powers of
//      two (the first member of a short group adds the missing arrivals), the
//      last arrival of a group arriving on `top`, the last group leader
//      advancing `gen`; XCD groups (workgroup b in group b % 8) or groups of 16
//      consecutive workgroups with a short last group; counters started just
//      below 2^32 so they wrap; a bounded wait that sets the fault word, after
//      which every barrier returns false;
//   2. ticket-fed unit hand-out (workgroup b takes units b and b + nwg, then
//      units 2 nwg + 8 t + c from counter c, its own counter b % 8 first),
//      single units and pairs of units, and the down projection's variant
//      (a run of R consecutive units per workgroup, then tickets);
//   3. per-slot completion counters: units of a slot's producer phase write the
//      slot's rows and count themselves on the slot's counter; consumer units
//      wait (bounded) until the counter is full and then read the rows.
// Every unit must be processed exactly once, every value read must be the one
// written for it, and ThreadSanitizer must report no data race.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <thread>
#include <vector>

namespace {

int g_errors = 0;
std::atomic<int> g_err_atomic{0};
void fail(const char* what, long a, long b) {
  if (g_err_atomic.fetch_add(1) < 10) std::fprintf(stderr, "FAIL %s (%ld, %ld)\n", what, a, b);
}

uint32_t pow2_at_least(uint32_t n) { return n > 1 ? 1u << (32 - __builtin_clz(n - 1)) : 1u; }

// ------------------------------------------------------------------ 1. grid barrier
constexpr int kBarGroup = 16;
struct Barrier {
  std::atomic<uint32_t> gen{0}, fault{0}, top{0};
  std::atomic<uint32_t> grp[64];
};

// returns false once the fault word is set (by a timeout here or anyone else)
bool grid_barrier(Barrier& b, int blk, int nwg, bool xcd, long spin_limit) {
  if (b.fault.load(std::memory_order_acquire) != 0) return false;
  const uint32_t g = b.gen.load(std::memory_order_acquire);
  bool last = false;
  if (xcd) {
    const uint32_t grp = blk & 7, gsz = nwg / 8, gpow = pow2_at_least(gsz);
    const uint32_t add = blk < 8 ? gpow - gsz + 1 : 1u;
    if (((b.grp[grp].fetch_add(add, std::memory_order_acq_rel) + add) & (gpow - 1)) == 0)
      last = ((b.top.fetch_add(1u, std::memory_order_acq_rel) + 1u) & 7u) == 0;
  } else {
    const uint32_t grp = blk / kBarGroup, ngrp = (nwg + kBarGroup - 1) / kBarGroup;
    const uint32_t gsz = std::min<uint32_t>(kBarGroup, nwg - grp * kBarGroup);
    const uint32_t add = blk % kBarGroup == 0 ? kBarGroup - gsz + 1 : 1u;
    const uint32_t tpow = pow2_at_least(ngrp);
    const uint32_t tadd = grp == 0 ? tpow - ngrp + 1 : 1u;
    if (((b.grp[grp].fetch_add(add, std::memory_order_acq_rel) + add) & (kBarGroup - 1)) == 0)
      last = ((b.top.fetch_add(tadd, std::memory_order_acq_rel) + tadd) & (tpow - 1)) == 0;
  }
  if (last) {
    b.gen.fetch_add(1u, std::memory_order_release);
    return true;
  }
  long spins = 0;
  while (true) {
    const uint32_t gc = b.gen.load(std::memory_order_acquire);
    if (b.fault.load(std::memory_order_acquire) != 0) return false;
    if (gc != g) return true;
    if (++spins > spin_limit) {
      b.fault.store(1u, std::memory_order_release);
      return false;
    }
    std::this_thread::yield();
  }
}

// counters start just below 2^32 (each a multiple of its step) so that they wrap
void barrier_init_near_wrap(Barrier& b, int nwg, bool xcd) {
  b.gen.store(0xFFFFFFF0u);
  b.fault.store(0);
  const uint32_t gstep = xcd ? pow2_at_least(nwg / 8) : kBarGroup;
  const uint32_t tstep = xcd ? 8u : pow2_at_least((nwg + kBarGroup - 1) / kBarGroup);
  for (auto& c : b.grp) c.store(0u - 3u * gstep);
  b.top.store(0u - 5u * tstep);
}

void test_barrier(int nwg, bool xcd, int rounds) {
  Barrier b;
  barrier_init_near_wrap(b, nwg, xcd);
  std::vector<long> data(nwg, -1);   // plain memory: ordered only by the barrier
  std::vector<std::thread> th;
  for (int blk = 0; blk < nwg; ++blk)
    th.emplace_back([&, blk] {
      for (int k = 0; k < rounds; ++k) {
        data[blk] = (long)k * 100000 + blk;
        if (!grid_barrier(b, blk, nwg, xcd, 3000000)) { fail("barrier timed out", k, blk); return; }
        const int o = (blk * 7 + k + 1) % nwg;
        if (data[o] != (long)k * 100000 + o) fail("stale value after barrier", k, data[o]);
        if (!grid_barrier(b, blk, nwg, xcd, 3000000)) { fail("barrier timed out", k, blk); return; }
      }
    });
  for (auto& t : th) t.join();
  if (b.fault.load() != 0) fail("fault word set on a healthy run", nwg, xcd);
  std::printf("barrier nwg=%d %s: %d rounds ok\n", nwg, xcd ? "xcd groups" : "groups of 16", rounds);
}

// one workgroup never arrives at round `stuck_round`: everyone else's bounded
// wait gives up, the fault word is set and every later barrier returns false
void test_barrier_timeout(int nwg, bool xcd) {
  Barrier b;
  barrier_init_near_wrap(b, nwg, xcd);
  const int stuck = nwg / 3, stuck_round = 3;
  std::atomic<int> left{0};
  std::vector<std::thread> th;
  for (int blk = 0; blk < nwg; ++blk)
    th.emplace_back([&, blk] {
      for (int k = 0; k < 10; ++k) {
        if (blk == stuck && k == stuck_round) break;   // this workgroup leaves early
        if (!grid_barrier(b, blk, nwg, xcd, 20000)) break;
      }
      left.fetch_add(1);
    });
  for (auto& t : th) t.join();
  if (left.load() != nwg) fail("not every workgroup left", left.load(), nwg);
  if (b.fault.load() == 0) fail("no fault after a missing arrival", nwg, xcd);
  // a later launch (fault still set) returns at once
  if (grid_barrier(b, 0, nwg, xcd, 10)) fail("barrier passed with the fault word set", 0, 0);
  std::printf("barrier timeout nwg=%d %s: fault raised, all left\n", nwg, xcd ? "xcd" : "16");
}

// ------------------------------------------------------------------ 2. tickets
// run_stream_dyn's order: unit group cur, next group nxt; at the start of a
// group a ticket is drawn from counter cq, at its end turned into the group
// after nxt (moving to the next counter, at most 8 draws, while the counter's
// next group is past the end).
void test_tickets(int nwg, int U, int split, int reps) {
  for (int r = 0; r < reps; ++r) {
    const int UG = (U + split - 1) / split;
    std::atomic<uint32_t> ctr[8];
    for (auto& c : ctr) c.store(0);
    std::vector<std::atomic<int>> seen(U);
    for (auto& s : seen) s.store(0);
    std::vector<std::thread> th;
    for (int blk = 0; blk < nwg; ++blk)
      th.emplace_back([&, blk] {
        int cur = blk < UG ? blk : -1, nxt = blk + nwg < UG ? blk + nwg : -1;
        int cq = blk & 7;
        while (cur >= 0) {
          uint32_t tk = ctr[cq].fetch_add(1, std::memory_order_relaxed);
          for (int h = 0; h < split; ++h)
            if (cur * split + h < U) seen[cur * split + h].fetch_add(1);
          long long un2 = 2LL * nwg + 8LL * tk + cq;
          for (int tries = 1; un2 >= UG && tries < 8; ++tries) {
            cq = (cq + 1) & 7;
            tk = ctr[cq].fetch_add(1, std::memory_order_relaxed);
            un2 = 2LL * nwg + 8LL * tk + cq;
          }
          const int seq = un2 < UG ? (int)un2 : -1;
          cur = nxt;
          nxt = nxt >= 0 ? seq : -1;
        }
      });
    for (auto& t : th) t.join();
    for (int u = 0; u < U; ++u)
      if (seen[u].load() != 1) fail("unit not processed exactly once", u, seen[u].load());
  }
  std::printf("tickets nwg=%d units=%d split=%d: every unit once\n", nwg, U, split);
}

// phase_down_dyn's order: a run of R = min(8, U / nwg) consecutive units per
// workgroup (units b and b + nwg when R < 2), then tickets from RS * nwg on.
void test_down_tickets(int nwg, int U, int reps) {
  for (int r = 0; r < reps; ++r) {
    std::atomic<uint32_t> ctr[8];
    for (auto& c : ctr) c.store(0);
    std::vector<std::atomic<int>> seen(U);
    for (auto& s : seen) s.store(0);
    const int R = std::min(8, U / nwg), RS = R >= 2 ? R : 2;
    std::vector<std::thread> th;
    for (int blk = 0; blk < nwg; ++blk)
      th.emplace_back([&, blk] {
        auto static_unit = [&](int k) {
          const int u = R >= 2 ? blk * R + k : blk + k * nwg;
          return u < U ? u : -1;
        };
        int cur = static_unit(0), nxt = static_unit(1), kk = 0, cq = blk & 7;
        uint32_t tk = 0;
        while (cur >= 0) {
          if (kk + 2 >= RS) tk = ctr[cq].fetch_add(1, std::memory_order_relaxed);
          seen[cur].fetch_add(1);
          int seq;
          if (kk + 2 < RS) {
            seq = static_unit(kk + 2);
          } else {
            long long un2 = (long long)RS * nwg + 8LL * tk + cq;
            for (int tries = 1; un2 >= U && tries < 8; ++tries) {
              cq = (cq + 1) & 7;
              tk = ctr[cq].fetch_add(1, std::memory_order_relaxed);
              un2 = (long long)RS * nwg + 8LL * tk + cq;
            }
            seq = un2 < U ? (int)un2 : -1;
          }
          cur = nxt;
          nxt = nxt >= 0 ? seq : -1;
          ++kk;
        }
      });
    for (auto& t : th) t.join();
    for (int u = 0; u < U; ++u)
      if (seen[u].load() != 1) fail("down unit not processed exactly once", u, seen[u].load());
  }
  std::printf("down tickets nwg=%d units=%d: every unit once\n", nwg, U);
}

// ------------------------------------------------------------------ 3. slot counters
// Producer units (slot s, row block r) write rows[s][r]; after the write the
// unit counts itself on cnt[s].  Consumer units of slot s wait until cnt[s]
// equals the slot's producer count, then read every row block of the slot.
// Each workgroup first takes producer units by ticket, then consumer units by
// ticket, as the fused expert phases do.
void test_slots(int nwg, int slots, int per_slot, int consumers_per_slot) {
  const int P = slots * per_slot, C = slots * consumers_per_slot;
  std::vector<long> rows(P, -1);   // plain memory, ordered only by the counters
  std::vector<std::atomic<uint32_t>> cnt(slots);
  for (auto& c : cnt) c.store(0);
  std::atomic<int> pnext{0}, cnext{0}, cdone{0};
  std::vector<std::thread> th;
  for (int blk = 0; blk < nwg; ++blk)
    th.emplace_back([&] {
      for (int u; (u = pnext.fetch_add(1)) < P;) {
        rows[u] = 1000L * u + 7;
        cnt[u / per_slot].fetch_add(1, std::memory_order_release);
      }
      for (int u; (u = cnext.fetch_add(1)) < C;) {
        const int s = u / consumers_per_slot;
        long spins = 0;
        while (cnt[s].load(std::memory_order_acquire) < (uint32_t)per_slot) {
          if (++spins > 3000000) { fail("slot wait timed out", s, cnt[s].load()); return; }
          std::this_thread::yield();
        }
        for (int r = 0; r < per_slot; ++r) {
          const int pu = s * per_slot + r;
          if (rows[pu] != 1000L * pu + 7) fail("consumer read a row before it was written", pu, rows[pu]);
        }
        cdone.fetch_add(1);
      }
    });
  for (auto& t : th) t.join();
  if (cdone.load() != C) fail("consumer units missing", cdone.load(), C);
  std::printf("slot counters nwg=%d slots=%d: consumers saw every row\n", nwg, slots);
}

}  // namespace

int main(int argc, char** argv) {
  const int scale = argc > 1 ? std::atoi(argv[1]) : 1;
  test_barrier(64, true, 300 * scale);
  test_barrier(48, true, 300 * scale);      // XCD groups of 6 (counters step by 8)
  test_barrier(200, true, 100 * scale);     // XCD groups of 25 (counters step by 32)
  test_barrier(40, false, 300 * scale);     // a short last group of 8
  test_barrier(72, false, 200 * scale);     // 5 groups (top steps by 8)
  test_barrier(16, false, 300 * scale);     // one group
  test_barrier(8, true, 300 * scale);       // groups of one
  test_barrier_timeout(48, true);
  test_barrier_timeout(40, false);
  test_tickets(64, 1000, 1, 3 * scale);
  test_tickets(64, 129, 1, 3 * scale);      // fewer units than two per workgroup
  test_tickets(64, 1001, 2, 3 * scale);     // pairs of units, odd count
  test_tickets(40, 37, 1, 3 * scale);       // fewer units than workgroups
  test_down_tickets(64, 1485, 2 * scale);
  test_down_tickets(64, 100, 2 * scale);
  test_slots(48, 12, 16, 8);
  const int errs = g_err_atomic.load() + g_errors;
  std::printf(errs ? "FAILED (%d)\n" : "all protocol checks passed\n", errs);
  return errs ? 1 : 0;
}
