// Host-only checks of the plan code, built with sanitizers by
// tests/test_host_sanitizers.py from sta_plan.cpp and this file:
//   (default)           every host-side entry point of include/sta.h on fixed
//                       and seeded random plans, the error paths, allocation
//                       failure at every allocation of a plan build, and the
//                       STA_TEST_FAIL_ALLOC hook (run under ASan + UBSan);
//   -DHOST_CHECKS_THREADS  threads that take plans from the process-wide
//                       cache while another thread clears it (run under TSan).
// No HIP: plans built on the host never hold device tables, so releasing
// them is a no-op here.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "sta.h"
#include "sta_internal.h"

namespace sta {
void release_device_tables(sta_plan *) {}
}  // namespace sta

// ---- allocation-failure injection: operator new throws at the armed count
static std::atomic<long> g_allocs{0};
static std::atomic<long> g_fail_at{-1};

static void *counted_alloc(std::size_t n) {
  const long c = ++g_allocs;
  if (c == g_fail_at.load()) throw std::bad_alloc();
  void *p = std::malloc(n ? n : 1);
  if (!p) throw std::bad_alloc();
  return p;
}
void *operator new(std::size_t n) { return counted_alloc(n); }
void *operator new[](std::size_t n) { return counted_alloc(n); }
void *operator new(std::size_t n, const std::nothrow_t &) noexcept {
  try { return counted_alloc(n); } catch (...) { return nullptr; }
}
void *operator new[](std::size_t n, const std::nothrow_t &) noexcept {
  try { return counted_alloc(n); } catch (...) { return nullptr; }
}
void operator delete(void *p) noexcept { std::free(p); }
void operator delete[](void *p) noexcept { std::free(p); }
void operator delete(void *p, std::size_t) noexcept { std::free(p); }
void operator delete[](void *p, std::size_t) noexcept { std::free(p); }

static int g_checks = 0, g_fail = 0;
#define CHECK(c)                                                             \
  do {                                                                       \
    ++g_checks;                                                              \
    if (!(c)) {                                                              \
      ++g_fail;                                                              \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
    }                                                                        \
  } while (0)

static bool is_status(sta_status s) {
  return s == STA_OK || s == STA_ERR_ARG || s == STA_ERR_SHAPE || s == STA_ERR_UNSUPPORTED ||
         s == STA_ERR_ALLOC || s == STA_ERR_HIP;
}

// Every host query of a plan, with the invariants that need no oracle.
static void query_all(const sta_plan *p) {
  sta_plan_info info;
  CHECK(sta_plan_get_info(p, &info) == STA_OK);
  CHECK(sta_plan_get_info(p, nullptr) == STA_ERR_ARG);
  const int64_t N = (int64_t)info.T * info.H * info.W;
  std::vector<int32_t> perm((size_t)N);
  CHECK(sta_plan_perm(p, perm.data(), N - 1) == STA_ERR_ARG);
  if (sta_plan_perm(p, perm.data(), N) == STA_OK) {
    std::vector<char> seen((size_t)N, 0);
    bool ok = true;
    for (int32_t x : perm) {
      ok &= x >= 0 && x < N && !seen[(size_t)x];
      if (x >= 0 && x < N) seen[(size_t)x] = 1;
    }
    CHECK(ok);
  }
  for (int h = -1; h <= info.heads; ++h) {
    for (int t : {-1, 0, info.n_tiles / 2, info.n_tiles - 1, info.n_tiles}) {
      int cnt = -1;
      const sta_status s = sta_plan_kv_tiles(p, h, t, nullptr, 0, &cnt);
      const bool valid = h >= 0 && h < info.heads && t >= 0 && t < info.n_tiles;
      if (!valid) {
        CHECK(s == STA_ERR_ARG);
        continue;
      }
      if (info.swa) continue;
      CHECK(cnt >= 1 && cnt <= info.n_tiles);
      std::vector<int32_t> l((size_t)cnt);
      CHECK(sta_plan_kv_tiles(p, h, t, l.data(), cnt, &cnt) == STA_OK);
      bool ok = true;
      for (int32_t x : l) ok &= x >= 0 && x < info.n_tiles;
      CHECK(ok);
      if (cnt > 1) CHECK(sta_plan_kv_tiles(p, h, t, l.data(), cnt - 1, &cnt) == STA_ERR_ARG);
      int qc = -1;
      if (sta_plan_q_tiles(p, h, t, nullptr, 0, &qc) == STA_OK && qc > 0) {
        std::vector<int32_t> ql((size_t)qc);
        CHECK(sta_plan_q_tiles(p, h, t, ql.data(), qc, &qc) == STA_OK);
      }
    }
  }
  int64_t n = -1;
  CHECK(sta_plan_schedule(p, nullptr, 0, &n) == STA_OK || n >= 0);
  if (n > 0) {
    std::vector<int32_t> s((size_t)n);
    CHECK(sta_plan_schedule(p, s.data(), n, &n) == STA_OK);
  }
  for (int which = -1; which <= 2; ++which) {
    int64_t m = -1;
    const sta_status st = sta_plan_schedule_bwd(p, which, nullptr, 0, &m);
    CHECK(is_status(st));
    if (st == STA_OK && m > 0) {
      std::vector<int32_t> s((size_t)m);
      CHECK(sta_plan_schedule_bwd(p, which, s.data(), m, &m) == STA_OK);
    }
  }
  int64_t np = -1;
  CHECK(sta_plan_pieces(p, nullptr, 0, &np) == STA_OK || np >= 0);
  if (np > 0) {
    std::vector<int32_t> pc((size_t)np * 5);
    CHECK(sta_plan_pieces(p, pc.data(), np, &np) == STA_OK);
  }
}

static uint64_t g_rng = 0x9e3779b97f4a7c15ull;
static int rnd(int lo, int hi) {   // inclusive
  g_rng ^= g_rng << 13; g_rng ^= g_rng >> 7; g_rng ^= g_rng << 17;
  return lo + (int)(g_rng % (uint64_t)(hi - lo + 1));
}

static void fixed_and_random_plans() {
  struct Cfg { int b, h, T, H, W, t0, t1, t2, w0, w1, w2, d, flags; };
  const Cfg cfgs[] = {
      {1, 2, 6, 16, 16, 2, 4, 4, 3, 3, 3, 64, 0},      {1, 8, 12, 24, 24, 6, 8, 8, 3, 3, 3, 128, 0},
      {1, 24, 30, 48, 80, 6, 8, 8, 3, 3, 3, 128, 0},   {2, 3, 30, 45, 80, 6, 8, 8, 1, 2, 5, 128, 1},
      {1, 2, 5, 13, 11, 2, 4, 4, 3, 3, 3, 64, 1},      {1, 8, 1, 96, 96, 1, 16, 24, 1, 3, 3, 128, 0},
      {1, 4, 30, 48, 80, 6, 8, 8, 5, 6, 10, 128, 0},   {1, 2, 8, 16, 16, 2, 4, 8, 9, 9, 9, 128, 0},
  };
  for (const Cfg &c : cfgs) {
    std::vector<int> win((size_t)c.h * 3);
    for (int h = 0; h < c.h; ++h) { win[3 * h] = c.w0 + (h % 2); win[3 * h + 1] = c.w1; win[3 * h + 2] = c.w2; }
    const int tile[3] = {c.t0, c.t1, c.t2};
    sta_plan *p = nullptr;
    const sta_status s = sta_plan_create_ex(c.b, c.h, c.T, c.H, c.W, tile, win.data(), c.d, c.flags, &p);
    CHECK(s == STA_OK && p != nullptr);
    if (p) query_all(p);
    CHECK(sta_plan_destroy(p) == STA_OK);
  }
  for (int i = 0; i < 300; ++i) {
    const int heads = rnd(1, 4), d = rnd(0, 1) ? 64 : 128;
    const int tile[3] = {rnd(1, 6), rnd(1, 8), rnd(1, 8)};
    const int T = rnd(1, 24), H = rnd(1, 32), W = rnd(1, 32);
    std::vector<int> win((size_t)heads * 3);
    for (int &x : win) x = rnd(0, 7);
    const int flags = rnd(0, 2);   // 2 is an invalid flag
    sta_plan *p = nullptr;
    const sta_status s = sta_plan_create_ex(rnd(0, 2), heads, T, H, W, tile, win.data(), d, flags, &p);
    CHECK(is_status(s) && s != STA_ERR_HIP && s != STA_ERR_ALLOC);
    CHECK((s == STA_OK) == (p != nullptr));
    if (p) query_all(p);
    sta_plan_destroy(p);
    // token-wise SWA plans (windows in tokens)
    std::vector<int> wt((size_t)heads * 3);
    for (int &x : wt) x = rnd(0, 20);
    p = nullptr;
    const sta_status s2 = sta_swa_plan_create(1, heads, T, H, W, tile, wt.data(), d, &p);
    CHECK(is_status(s2) && s2 != STA_ERR_HIP && s2 != STA_ERR_ALLOC);
    if (p) query_all(p);
    sta_plan_destroy(p);
  }
}

static void error_paths() {
  const int tile[3] = {2, 4, 4}, win[6] = {3, 3, 3, 3, 3, 3};
  sta_plan *p = nullptr;
  CHECK(sta_plan_create(1, 2, 6, 16, 16, nullptr, win, 64, &p) == STA_ERR_ARG);
  CHECK(sta_plan_create(1, 2, 6, 16, 16, tile, nullptr, 64, &p) == STA_ERR_ARG);
  CHECK(sta_plan_create(1, 2, 6, 16, 16, tile, win, 64, nullptr) == STA_ERR_ARG);
  CHECK(sta_plan_create(1, 0, 6, 16, 16, tile, win, 64, &p) == STA_ERR_ARG);
  CHECK(sta_plan_create(1, 2, 7, 16, 16, tile, win, 64, &p) == STA_ERR_SHAPE);
  CHECK(sta_plan_create(1, 2, 6, 16, 16, tile, win, 96, &p) == STA_ERR_UNSUPPORTED);
  CHECK(sta_plan_create_ex(1, 2, 6, 16, 16, tile, win, 64, 4, &p) == STA_ERR_ARG);
  CHECK(p == nullptr);
  CHECK(sta_plan_destroy(nullptr) == STA_OK);
  CHECK(sta_plan_get_info(nullptr, nullptr) == STA_ERR_ARG);
  int grid[3] = {5, 6, 10}, cnt = 0;
  CHECK(sta_window_candidates(grid, nullptr, 0, &cnt) == STA_ERR_ARG || cnt > 0);
  std::vector<int> cand((size_t)cnt * 3);
  CHECK(sta_window_candidates(grid, cand.data(), cnt, &cnt) == STA_OK);
  std::vector<double> err((size_t)3 * cnt);
  for (double &e : err) e = rnd(0, 1000) / 1000.0;
  std::vector<int> out(9);
  CHECK(sta_window_select(3, grid, cand.data(), cnt, err.data(), 0.05, out.data()) == STA_OK);
  for (int h = 0; h < 3; ++h)
    for (int d = 0; d < 3; ++d) CHECK(out[3 * h + d] >= 1 && out[3 * h + d] <= grid[d]);
  CHECK(sta_window_select(0, grid, cand.data(), cnt, err.data(), 0.05, out.data()) == STA_ERR_ARG);
  CHECK(sta_window_select(3, grid, nullptr, cnt, err.data(), 0.05, out.data()) == STA_ERR_ARG);
  for (int s = -7; s <= 1; ++s) CHECK(sta_status_string((sta_status)s) != nullptr);
}

// The tables a host can read back from a plan (for comparing two plans).
static std::vector<int32_t> tables(const sta_plan *p) {
  std::vector<int32_t> out;
  sta_plan_info info;
  if (sta_plan_get_info(p, &info) != STA_OK) return out;
  for (int h = 0; h < info.heads; ++h)
    for (int t = 0; t < info.n_tiles; ++t) {
      int cnt = 0;
      sta_plan_kv_tiles(p, h, t, nullptr, 0, &cnt);
      std::vector<int32_t> l((size_t)cnt);
      sta_plan_kv_tiles(p, h, t, l.data(), cnt, &cnt);
      out.insert(out.end(), l.begin(), l.end());
    }
  int64_t n = 0;
  sta_plan_schedule(p, nullptr, 0, &n);
  std::vector<int32_t> s((size_t)n);
  sta_plan_schedule(p, s.data(), n, &n);
  out.insert(out.end(), s.begin(), s.end());
  for (int which = 0; which < 2; ++which) {
    int64_t m = 0;
    if (sta_plan_schedule_bwd(p, which, nullptr, 0, &m) != STA_OK) continue;
    std::vector<int32_t> b((size_t)m);
    sta_plan_schedule_bwd(p, which, b.data(), m, &m);
    out.insert(out.end(), b.begin(), b.end());
  }
  return out;
}

// Allocation failure at every allocation of a plan build: the build returns
// STA_ERR_ALLOC, or (where the standard library falls back, as stable_sort
// does without its temporary buffer) the same plan as without the failure;
// it never crashes, and LeakSanitizer finds nothing at exit.
static void allocation_failures() {
  const int tile[3] = {2, 4, 4}, win[6] = {3, 3, 3, 1, 2, 3};
  const long before = g_allocs.load();
  sta_plan *p = nullptr;
  CHECK(sta_plan_create_ex(1, 2, 6, 16, 16, tile, win, 64, 0, &p) == STA_OK);
  const long used = g_allocs.load() - before;
  const std::vector<int32_t> ref = tables(p);
  sta_plan_destroy(p);
  CHECK(used > 10 && !ref.empty());
  int failed = 0;
  for (long k = 1; k <= used; ++k) {
    p = nullptr;
    g_fail_at = g_allocs.load() + k;
    const sta_status s = sta_plan_create_ex(1, 2, 6, 16, 16, tile, win, 64, 0, &p);
    g_fail_at = -1;
    CHECK((s == STA_ERR_ALLOC && p == nullptr) || (s == STA_OK && p != nullptr && tables(p) == ref));
    failed += s == STA_ERR_ALLOC;
    sta_plan_destroy(p);
  }
  CHECK(failed > used / 2);
  // the query entry points allocate nothing: with every allocation failing
  // they still answer
  CHECK(sta_plan_create_ex(1, 2, 6, 16, 16, tile, win, 64, 0, &p) == STA_OK);
  int cnt = 0, grid[3] = {3, 4, 4};
  int32_t l[64];
  std::vector<int> cands(64 * 3);
  g_fail_at = g_allocs.load() + 1;
  const long mark = g_allocs.load();
  CHECK(sta_plan_kv_tiles(p, 1, 3, l, 64, &cnt) == STA_OK && cnt > 0);
  CHECK(sta_plan_q_tiles(p, 1, 3, l, 64, &cnt) == STA_OK && cnt > 0);
  CHECK(sta_window_candidates(grid, cands.data(), 64, &cnt) == STA_OK && cnt == 2 * 3 * 3);
  CHECK(g_allocs.load() == mark);
  g_fail_at = -1;
  sta_plan_destroy(p);
  // the environment hook, through the plan builders and the plan cache
  setenv("STA_TEST_FAIL_ALLOC", "1", 1);
  CHECK(sta_plan_create(1, 2, 6, 16, 16, tile, win, 64, &p) == STA_ERR_ALLOC && p == nullptr);
  CHECK(sta_swa_plan_create(1, 2, 6, 16, 16, tile, win, 64, &p) == STA_ERR_ALLOC && p == nullptr);
  sta_status st = STA_OK;
  CHECK(sta::cached_plan(1, 2, 6, 16, 16, tile, win, 64, &st) == nullptr && st == STA_ERR_ALLOC);
  setenv("STA_TEST_FAIL_ALLOC", "0", 1);
  CHECK(sta::cached_plan(1, 2, 6, 16, 16, tile, win, 64, &st) != nullptr && st == STA_OK);
  unsetenv("STA_TEST_FAIL_ALLOC");
  CHECK(sta_clear_plan_cache() == STA_OK);
}

#ifdef HOST_CHECKS_THREADS
// Threads take plans from the cache and read them while one thread keeps
// clearing it: no data race (TSan), no plan freed while in use.
static void cache_threads() {
  const int tile[3] = {2, 4, 4};
  const int wins[3][6] = {{3, 3, 3, 3, 3, 3}, {1, 2, 3, 3, 2, 1}, {2, 2, 2, 1, 1, 1}};
  std::atomic<bool> stop{false};
  std::atomic<int> bad{0};
  std::vector<std::thread> ts;
  for (int i = 0; i < 6; ++i) {
    ts.emplace_back([&, i]() {
      for (int it = 0; it < 150; ++it) {
        sta_status st = STA_OK;
        auto p = sta::cached_plan(1, 2, 6, 16, 16, tile, wins[(i + it) % 3], 64, &st);
        if (!p || st != STA_OK) { ++bad; continue; }
        sta_plan_info info;
        int cnt = 0;
        // (a count query: STA_ERR_ARG with the length in cnt)
        if (sta_plan_get_info(p.get(), &info) != STA_OK || info.heads != 2 ||
            sta_plan_kv_tiles(p.get(), 1, 5, nullptr, 0, &cnt) != STA_ERR_ARG || cnt < 1)
          ++bad;
      }
    });
  }
  std::thread clearer([&]() {
    while (!stop.load()) { sta_clear_plan_cache(); std::this_thread::yield(); }
  });
  for (auto &t : ts) t.join();
  stop = true;
  clearer.join();
  CHECK(bad.load() == 0);
  sta_clear_plan_cache();
}
#endif

int main() {
#ifdef HOST_CHECKS_THREADS
  cache_threads();
#else
  fixed_and_random_plans();
  error_paths();
  allocation_failures();
#endif
  std::printf("host checks: %d checks, %d failed\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
