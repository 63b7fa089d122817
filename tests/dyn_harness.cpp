// Host harness of the dynamic (push/pop) schedule's control logic.
//
// It compiles the very scheduler the kernels run (dynamic_moe_task_amd/
// csrc/dyn_sched.h: queue protocol, exit rule, notifies, pushes, task
// counts) with g++ and drives it with threads: each persistent workgroup is
// four threads, one per wave, meeting at a std::barrier wherever the kernel
// has a workgroup barrier.  The task bodies are stand-ins that check, when
// they start, that every task they depend on has finished (the MoE layer's
// graph: R -> K -> S -> G1 -> G2 -> C, and the split-K example's
// partial -> final), sleep a random time and mark themselves done.  A
// watchdog thread fails the run (exit status 3) if the workgroups have not
// all left in time, so a deadlock ends the test instead of hanging it.
//
// The host atomics are sequentially consistent; what this checks is the
// protocol (who pushes what when, which index waits on which slot, when a
// workgroup leaves, which barriers each path crosses), not the GPU's memory
// ordering.
//
//   dyn_harness moe T E k H I G seed [options]
//   dyn_harness splitk n nsplit G seed [options]
// options: --body-us N (task bodies sleep 0..N us), --scan-ms N (the scan
// task sleeps N ms, so pops land before the total is known), --late N
// (workgroups w >= N start 20 ms late, as if not yet resident),
// --skew (routing concentrated on few experts), --prefix-short (the router
// prefix counted with 32 experts a task while the bodies cover 16: the
// inconsistency the kernel had before the task counts came from
// launch_graph), --narrow (run the small-batch kernel variant whatever T
// is, as the dynamic kernel once did), --timeout-s N, --launches N (split-K:
// launches on the same control words).
#include <algorithm>
#include <atomic>
#include <barrier>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../dynamic_moe_task_amd/csrc/dyn_sched.h"

using namespace etc;
using namespace etc::dyn;

namespace {

struct Opts {
  int body_us = 20;
  int scan_ms = 0;
  int late = 1 << 30;
  bool skew = false;
  bool prefix_short = false;
  bool narrow = false;
  int timeout_s = 60;
  int launches = 1;
} opt;

struct WG {
  std::barrier<> bar{4};
  Shared sh{};
  int bcast = 0;  // a value wave 0 hands to the other waves (the scan's row-tile count)
};

thread_local int t_wave = 0;
thread_local WG* t_wg = nullptr;
thread_local uint64_t t_rng = 88172645463325252ull;

uint32_t rnd() {
  t_rng ^= t_rng << 13;
  t_rng ^= t_rng >> 7;
  t_rng ^= t_rng << 17;
  return (uint32_t)(t_rng >> 11);
}
void sleep_us(int us) {
  if (us > 0) std::this_thread::sleep_for(std::chrono::microseconds(us));
}

struct Host {
  static constexpr int kThreads = 4;
  static int tid() { return t_wave; }
  static uint32_t add(uint32_t* p, uint32_t v) { return std::atomic_ref<uint32_t>(*p).fetch_add(v); }
  static uint32_t load(const uint32_t* p) { return std::atomic_ref<uint32_t>(*const_cast<uint32_t*>(p)).load(); }
  static void put(uint32_t* p, uint32_t v) { std::atomic_ref<uint32_t>(*p).exchange(v); }
  static void orr(uint32_t* p, uint32_t v) { std::atomic_ref<uint32_t>(*p).fetch_or(v); }
  static uint64_t now() {
    return (uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(
               std::chrono::steady_clock::now().time_since_epoch()).count();
  }
  static void pause() {
    if (rnd() % 4 == 0) sleep_us(1 + (int)(rnd() % 20));
    else std::this_thread::yield();
  }
  static void barrier() { t_wg->bar.arrive_and_wait(); }
  static void publish() { barrier(); }
  static int lds_add(int* p, int v) { return std::atomic_ref<int>(*p).fetch_add(v); }
};

std::atomic<int> g_violations{0};
void violation(const char* what, int a, int b) {
  if (g_violations.fetch_add(1) < 20) std::fprintf(stderr, "violation: %s (%d, %d)\n", what, a, b);
}

// one task's run counter: must go 0 -> 1 exactly once
struct Runs {
  std::vector<std::atomic<int>> v;
  explicit Runs(size_t n = 0) : v(n) {}
  void resize(size_t n) { std::vector<std::atomic<int>> w(n); v.swap(w); }
  bool done(size_t i) const { return v[i].load() == 1; }
  void mark(size_t i, const char* what, int a, int b) {
    if (v[i].fetch_add(1) != 0) violation(what, a, b);
  }
  int count() const {
    int n = 0;
    for (auto& x : v) n += x.load();
    return n;
  }
  bool all_once() const {
    for (auto& x : v)
      if (x.load() != 1) return false;
    return true;
  }
};

// ------------------------------------------------------------- MoE layer --
struct MoeSim {
  MoeGraph g{};
  int T, E, k;
  // routing and row tiles, as S would compute them
  std::vector<int> ids;                  // [T*k]
  std::vector<int> row_token;            // grouped row -> token
  std::vector<int> slot;                 // pair -> grouped row
  std::vector<int> tile_r0, tile_n, row_tile;
  int nrt = 0;
  // events (the counter words the scheduler notifies)
  std::vector<uint32_t> ev_logit_w, ev_h_w, ev_y_w, ev_c_w;
  uint32_t ev_route_w = 0;
  Runs R, Kt, S, G1, G2, C;

  void build(int T_, int E_, int k_, int H, int I, int var, uint64_t seed) {
    T = T_;
    E = E_;
    k = k_;
    g = launch_graph(T, E, k, H, I, var);
    const int bm = var == kVarBig ? kBigBM : kBM;
    uint64_t s = seed * 2654435761ull + 12345;
    auto r = [&]() {
      s ^= s << 13;
      s ^= s >> 7;
      s ^= s << 17;
      return (uint32_t)(s >> 11);
    };
    ids.assign((size_t)T * k, 0);
    for (int t = 0; t < T; ++t) {
      std::vector<int> taken;
      for (int j = 0; j < k; ++j) {
        int e;
        do {
          e = opt.skew ? (int)(r() % (uint32_t)(k + 2 + (r() % 4 == 0 ? E : 0))) % E : (int)(r() % (uint32_t)E);
        } while (std::find(taken.begin(), taken.end(), e) != taken.end());
        taken.push_back(e);
        ids[(size_t)t * k + j] = e;
      }
    }
    // stable grouping by expert, row tiles of at most bm rows (the variant's)
    std::vector<int> cnt(E, 0), iptr(E + 1, 0);
    for (int e : ids) ++cnt[e];
    for (int e = 0; e < E; ++e) iptr[e + 1] = iptr[e] + cnt[e];
    row_token.assign((size_t)T * k, 0);
    slot.assign((size_t)T * k, 0);
    std::vector<int> fill(E, 0);
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const int rr = iptr[e] + fill[e]++;
        row_token[rr] = t;
        slot[(size_t)t * k + j] = rr;
      }
    row_tile.assign((size_t)T * k, 0);
    for (int e = 0; e < E; ++e)
      for (int m = 0; m * bm < cnt[e]; ++m) {
        const int r0 = iptr[e] + m * bm, n = std::min(bm, cnt[e] - m * bm);
        for (int q = 0; q < n; ++q) row_tile[r0 + q] = (int)tile_r0.size();
        tile_r0.push_back(r0);
        tile_n.push_back(n);
      }
    nrt = (int)tile_r0.size();
    ev_logit_w.assign(g.nTT, 0);
    ev_h_w.assign(nrt, 0);
    ev_y_w.assign(nrt, 0);
    ev_c_w.assign(g.nC, 0);
    R.resize(g.nR);
    Kt.resize(g.nK);
    S.resize(1);
    G1.resize((size_t)nrt * g.nN1);
    G2.resize((size_t)nrt * g.nN2);
    C.resize(g.nC);
  }
};
MoeSim sim;

// The task bodies: every wave enters and leaves through a barrier (the real
// bodies hold barriers of their own); wave 0 checks the dependencies, the
// body sleeps, wave 0 marks the task done.
struct MoeTasks {
  void body() { sleep_us(opt.body_us ? (int)(rnd() % (uint32_t)opt.body_us) : 0); }
  void router(int tt, int et) {
    Host::barrier();
    if (t_wave == 0) {
      if (tt >= sim.g.nTT || et >= sim.g.nET) violation("router tile outside the graph", tt, et);
      body();
      sim.R.mark((size_t)tt * sim.g.nET + et, "router ran twice", tt, et);
    }
    Host::barrier();
  }
  void topk(int tt) {
    Host::barrier();
    if (t_wave == 0) {
      for (int et = 0; et < sim.g.nET; ++et)
        if (!sim.R.done((size_t)tt * sim.g.nET + et)) violation("top-k before its router tasks", tt, et);
      body();
      sim.Kt.mark(tt, "top-k ran twice", tt, 0);
    }
    Host::barrier();
  }
  int scan() {
    Host::barrier();
    if (t_wave == 0) {
      for (int tt = 0; tt < sim.g.nK; ++tt)
        if (!sim.Kt.done(tt)) violation("scan before top-k", tt, 0);
      sleep_us(opt.scan_ms * 1000);
      body();
      sim.S.mark(0, "scan ran twice", 0, 0);
      t_wg->bcast = sim.nrt;
    }
    Host::barrier();
    return t_wg->bcast;
  }
  void g1(int rt, int nt) {
    Host::barrier();
    if (t_wave == 0) {
      if (rt >= sim.nrt || nt >= sim.g.nN1) violation("G1 tile outside the graph", rt, nt);
      else {
        if (!sim.S.done(0)) violation("G1 before the scan", rt, nt);
        body();
        sim.G1.mark((size_t)rt * sim.g.nN1 + nt, "G1 ran twice", rt, nt);
      }
    }
    Host::barrier();
  }
  void g2(int rt, int nt) {
    Host::barrier();
    if (t_wave == 0) {
      if (rt >= sim.nrt || nt >= sim.g.nN2) violation("G2 tile outside the graph", rt, nt);
      else {
        for (int j = 0; j < sim.g.nN1; ++j)
          if (!sim.G1.done((size_t)rt * sim.g.nN1 + j)) violation("G2 before its row tile's G1 tiles", rt, j);
        body();
        sim.G2.mark((size_t)rt * sim.g.nN2 + nt, "G2 ran twice", rt, nt);
      }
    }
    Host::barrier();
  }
  void combine(int ct) {
    Host::barrier();
    if (t_wave == 0) {
      if (ct >= sim.g.nC) violation("combine tile outside the graph", ct, 0);
      else {
        for (int t = ct * kCombineT; t < std::min(sim.T, (ct + 1) * kCombineT); ++t)
          for (int j = 0; j < sim.k; ++j) {
            const int rt = sim.row_tile[sim.slot[(size_t)t * sim.k + j]];
            for (int n = 0; n < sim.g.nN2; ++n)
              if (!sim.G2.done((size_t)rt * sim.g.nN2 + n)) violation("combine before a row tile's G2 tiles", ct, rt);
          }
        body();
        sim.C.mark(ct, "combine ran twice", ct, 0);
      }
    }
    Host::barrier();
  }
  uint32_t* ev_logit(int tt) { return &sim.ev_logit_w[tt]; }
  uint32_t* ev_route() { return &sim.ev_route_w; }
  uint32_t* ev_h(int rt) { return &sim.ev_h_w[rt]; }
  uint32_t* ev_y(int rt) { return &sim.ev_y_w[rt]; }
  uint32_t* ev_c(int ct) { return &sim.ev_c_w[ct]; }
  int tile_rows(int rt) { return sim.tile_n[rt]; }
  int row_ctile(int rt, int r) { return sim.row_token[sim.tile_r0[rt] + r] / kCombineT; }
  void trace_start() {}
  void trace_body() {}
  void trace_end(int, int, int) {}
};

// ------------------------------------------------------------- split-K --
struct SkSim {
  uint32_t n = 0, nsplit = 0;
  std::vector<uint32_t> ev;
  Runs P, F;
};
SkSim sk;

struct SkTasks {
  // the pages' wiring: out-edge "ij->i", in-edge "i->i"
  uint32_t notify_elem(uint32_t i, uint32_t) { return i; }
  uint32_t waiter(uint32_t e) { return e; }
  void partial(uint32_t i, uint32_t j) {
    Host::barrier();
    if (t_wave == 0) {
      if (i >= sk.n || j >= sk.nsplit) violation("partial sum outside the graph", (int)i, (int)j);
      else {
        sleep_us(opt.body_us ? (int)(rnd() % (uint32_t)opt.body_us) : 0);
        sk.P.mark((size_t)i * sk.nsplit + j, "partial sum ran twice", (int)i, (int)j);
      }
    }
    Host::barrier();
  }
  void final_sum(uint32_t i) {
    Host::barrier();
    if (t_wave == 0) {
      if (i >= sk.n) violation("final sum outside the graph", (int)i, 0);
      else {
        for (uint32_t j = 0; j < sk.nsplit; ++j)
          if (!sk.P.done((size_t)i * sk.nsplit + j)) violation("final sum before a partial sum", (int)i, (int)j);
        // sole waiter of event i: back to rest (the kernel does the same)
        Host::put(&sk.ev[i], 0u);
        sk.F.mark(i, "final sum ran twice", (int)i, 0);
      }
    }
    Host::barrier();
  }
};

// Runs `nwg` workgroups of four threads through fn(w); fails the process if
// they have not all left within the timeout.
template <class Fn>
void run_grid(int nwg, Fn fn) {
  std::vector<WG> wgs(nwg);
  std::vector<std::thread> th;
  std::atomic<int> left{nwg * 4};
  for (int w = 0; w < nwg; ++w)
    for (int v = 0; v < 4; ++v)
      th.emplace_back([&, w, v]() {
        t_wave = v;
        t_wg = &wgs[w];
        t_rng = 0x9E3779B97F4A7C15ull * (uint64_t)(w * 4 + v + 1);
        if (w >= opt.late) sleep_us(20000);
        fn(w);
        left.fetch_sub(1);
      });
  // the watchdog: poll (a condition variable's timed wait is not visible to
  // every thread sanitizer build)
  const auto deadline = std::chrono::steady_clock::now() + std::chrono::seconds(opt.timeout_s);
  while (left.load() > 0) {
    if (std::chrono::steady_clock::now() > deadline) {
      std::fprintf(stderr, "HANG: %d of %d threads still inside the schedule after %d s\n", left.load(), nwg * 4,
                   opt.timeout_s);
      std::fflush(stderr);
      std::_Exit(3);
    }
    std::this_thread::sleep_for(std::chrono::milliseconds(2));
  }
  for (auto& t : th) t.join();
}

void parse_opts(int i, int argc, char** argv) {
  for (; i < argc; ++i) {
    const std::string a = argv[i];
    auto next = [&]() { return std::atoi(argv[++i]); };
    if (a == "--body-us") opt.body_us = next();
    else if (a == "--scan-ms") opt.scan_ms = next();
    else if (a == "--late") opt.late = next();
    else if (a == "--skew") opt.skew = true;
    else if (a == "--prefix-short") opt.prefix_short = true;
    else if (a == "--narrow") opt.narrow = true;
    else if (a == "--timeout-s") opt.timeout_s = next();
    else if (a == "--launches") opt.launches = next();
    else {
      std::fprintf(stderr, "unknown option %s\n", a.c_str());
      std::exit(2);
    }
  }
}

int moe_main(int argc, char** argv) {
  if (argc < 9) return 2;
  const int T = std::atoi(argv[2]), E = std::atoi(argv[3]), k = std::atoi(argv[4]), H = std::atoi(argv[5]),
            I = std::atoi(argv[6]), G = std::atoi(argv[7]);
  const uint64_t seed = std::strtoull(argv[8], nullptr, 10);
  parse_opts(9, argc, argv);
  const int var = opt.narrow ? kVarSmall : launch_variant_of(T, k, H, I);
  sim.build(T, E, k, H, I, var, seed);
  const int64_t rows = (int64_t)T * k;
  const int64_t max_rt = (rows + kBM - 1) / kBM + (rows < E ? rows : E);
  Queue q{};
  std::vector<uint32_t> ctl(4 * 32, 0);
  const int64_t cap = moe_queue_capacity(T, max_rt, I, H, kBN1, kBN2, kRouterT, kCombineT);
  std::vector<uint32_t> slots((size_t)cap, 0);
  q.head = &ctl[0];
  q.tail = &ctl[32];
  q.total = &ctl[64];
  q.status = &ctl[96];
  q.slot = slots.data();
  q.cap = cap;
  q.prefix = (uint32_t)sim.g.nR;
  if (opt.prefix_short) q.prefix = (uint32_t)(sim.g.nTT * ((E + kRouterEXL - 1) / kRouterEXL));
  q.known_total = 0;
  q.budget = (uint64_t)std::max(2, opt.timeout_s / 3) * 1000000000ull;
  const uint32_t total = moe_total(sim.g, sim.nrt);
  if ((int64_t)total - sim.g.nR > cap) {
    std::fprintf(stderr, "queue capacity %lld below the %u queued tasks\n", (long long)cap, total - sim.g.nR);
    return 1;
  }
  run_grid(G, [&](int) {
    MoeTasks tk;
    run_moe<Host>(tk, q, sim.g, t_wg->sh);
  });
  const uint32_t st = ctl[96];
  const bool all = sim.R.all_once() && sim.Kt.all_once() && sim.S.all_once() && sim.G1.all_once() &&
                   sim.G2.all_once() && sim.C.all_once();
  std::printf("{\"T\": %d, \"E\": %d, \"k\": %d, \"G\": %d, \"variant\": %d, \"nrt\": %d, \"total\": %u, "
              "\"published_total\": %u, \"tail\": %u, \"head\": %u, \"cap\": %lld, \"status\": %u, "
              "\"violations\": %d, \"runs\": [%d, %d, %d, %d, %d, %d], \"all_once\": %d}\n",
              T, E, k, G, var, sim.nrt, total, ctl[64], ctl[32], ctl[0], (long long)cap, st,
              g_violations.load(), sim.R.count(), sim.Kt.count(), sim.S.count(), sim.G1.count(), sim.G2.count(),
              sim.C.count(), (int)all);
  const bool ok = all && st == 0 && g_violations.load() == 0 && ctl[64] == total && ctl[32] + sim.g.nR == total;
  return ok ? 0 : 1;
}

int splitk_main(int argc, char** argv) {
  if (argc < 6) return 2;
  sk.n = (uint32_t)std::atoi(argv[2]);
  sk.nsplit = (uint32_t)std::atoi(argv[3]);
  const int G = std::atoi(argv[4]);
  parse_opts(6, argc, argv);
  sk.ev.assign(sk.n, 0);
  const int64_t cap = sk.n > 4096 ? sk.n : 4096;
  std::vector<uint32_t> ctl(4 * 32, 0), slots((size_t)cap, 0);
  bool ok = true;
  for (int l = 0; l < opt.launches; ++l) {
    sk.P.resize((size_t)sk.n * sk.nsplit);
    sk.F.resize(sk.n);
    Queue q{};
    q.head = &ctl[0];
    q.tail = &ctl[32];
    q.total = &ctl[64];
    q.status = &ctl[96];
    q.slot = slots.data();
    q.cap = cap;
    q.prefix = sk.n * sk.nsplit;
    q.known_total = sk.n * (sk.nsplit + 1);
    q.budget = (uint64_t)std::max(2, opt.timeout_s / 3) * 1000000000ull;
    run_grid(G, [&](int) {
      SkTasks tk;
      run_splitk<Host>(tk, q, sk.nsplit, sk.nsplit, sk.ev.data(), t_wg->sh);
    });
    const uint32_t st = ctl[96];
    bool rest = true;  // everything the next launch reads is back at rest
    for (uint32_t v : slots) rest = rest && v == 0;
    for (uint32_t v : sk.ev) rest = rest && v == 0;
    const bool all = sk.P.all_once() && sk.F.all_once();
    std::printf("{\"launch\": %d, \"n\": %u, \"nsplit\": %u, \"G\": %d, \"status\": %u, \"violations\": %d, "
                "\"tail\": %u, \"all_once\": %d, \"at_rest\": %d}\n",
                l, sk.n, sk.nsplit, G, st, g_violations.load(), ctl[32], (int)all, (int)rest);
    ok = ok && all && rest && st == 0 && g_violations.load() == 0 && ctl[32] == sk.n;
    // the kernel's last workgroup returns the control words to rest
    splitk_reset<Host>(q);
  }
  return ok ? 0 : 1;
}

}  // namespace

// grouped_task (chunks of one and of two workgroups a CU) is a bijection of [0, R * C) onto the
// R x C tiles
int tilemap_main() {
  int bad = 0, checked = 0;
  for (int R = 1; R <= 70; ++R)
    for (int C = 1; C <= 40; ++C) {
      for (const int W : {kBigW, 2 * kBigW}) {
        std::vector<int> seen((size_t)R * C, 0);
        for (int i = 0; i < R * C; ++i) {
          const TileRC t = grouped_task(i, R, C, W);
          if (t.rt < 0 || t.rt >= R || t.nt < 0 || t.nt >= C || seen[(size_t)t.rt * C + t.nt]++) ++bad;
        }
        ++checked;
      }
    }
  for (const auto& rc : {std::pair<int, int>{32, 96}, {190, 6}, {194, 8}, {32, 16}, {32, 14}, {1000, 200}}) {
    const int R = rc.first, C = rc.second;
    std::vector<int> seen((size_t)R * C, 0);
    for (int i = 0; i < R * C; ++i) {
      const TileRC t = big_task(i, R, C);
      if (t.rt < 0 || t.rt >= R || t.nt < 0 || t.nt >= C || seen[(size_t)t.rt * C + t.nt]++) ++bad;
    }
    ++checked;
  }
  std::printf("{\"checked\": %d, \"bad\": %d}\n", checked, bad);
  return bad ? 1 : 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && std::strcmp(argv[1], "tilemap") == 0) return tilemap_main();
  if (argc >= 2 && std::strcmp(argv[1], "moe") == 0) return moe_main(argc, argv);
  if (argc >= 2 && std::strcmp(argv[1], "splitk") == 0) return splitk_main(argc, argv);
  std::fprintf(stderr, "usage: dyn_harness moe T E k H I G seed [options] | splitk n nsplit G seed [options]\n");
  return 2;
}
