// Control logic of the dynamic (push/pop) schedule, written once and
// compiled twice: by hipcc into the persistent kernel, and by g++ into a
// host harness in which threads play the workgroups' waves.  It holds only
// scheduling decisions: the queue protocol (reserve, publish, pop, the exit
// rule), the event notifies that release tasks, the pushes each completed
// event triggers, the task descriptors and the per-launch task counts.  The
// task bodies, the memory primitives and the workgroup barrier come from
// two template parameters:
//
//   P (platform):  tid(), kThreads, add(), load(), put(), orr(), now(),
//                  pause(), barrier(), publish(), lds_add()
//   K (tasks):     router(tt, et), topk(tt), scan() -> row tiles, g1(rt, nt),
//                  g2(rt, nt), combine(ct), the event element addresses and
//                  the row -> combine-tile map of a row tile
//
// The schedule follows the Event Tensor pages (arXiv 2604.13327, Figs. 8 and
// 9; podcast cue 11): when a notify completes an event, the notifier pushes
// the tasks that waited on it at once (early push), and idle workgroups pop
// ready tasks from one queue.  Tasks popped from the queue never wait.
//
// Queue.  A ring of 32-bit descriptors in memory, zero meaning "not yet
// written", with a head (pops taken) and a tail (slots reserved by pushes).
// The router tasks are ready at launch, so pop indices below `prefix` name
// them directly; index i >= prefix is slot i - prefix.  A push reserves its
// slots with one atomic on the tail and then writes them.  A workgroup pops
// by taking the next index and waiting until its slot is written, unless
// the total task count (published by the scan task once the row tiles are
// known) shows that no task will ever fill it: then it leaves.
//
// Deadlock freedom.  A workgroup holds at most one index it has not run
// (pop-ahead takes the next index while the current task runs, and a
// running task never waits).  Suppose every resident workgroup waits on an
// unwritten slot.  Then no task runs, and every slot reserved so far has
// been written (reservation and write happen inside one task), so each
// held slot lies at or past the tail.  Every task that has run has pushed
// the tasks its completed events released, and by induction over the
// graph every task has been pushed and run: the total is published and
// every held index is past it, so every waiter leaves.  Slots past `cap`
// are never written, so an index there leaves at once.
#pragma once
#include <stdint.h>

#ifndef ETC_HD
#define ETC_HD inline
#endif
#include "etc_tiles.h"

namespace etc {

// The kernel variant a launch of T tokens runs: the large-batch variant
// (column-split G tiles, eight-experts-a-wave router tiles) once T * k
// selects the column-split tiles.
ETC_HD bool wide_variant(int T, int k, int H, int I) { return g1_cols(T, k, H) > 2 * kBN1 || g2_cols(T, k, I) > kBN2; }
// the variant a launch runs: big tiles for the largest batches, else the
// large-batch variant once it is selected, else the small-batch one
ETC_HD int launch_variant_of(int T, int k, int H, int I) {
  return big_variant(T, k, H, I) ? kVarBig : (wide_variant(T, k, H, I) ? kVarWide : kVarSmall);
}

namespace dyn {

// status bits shared with the kernels' status word
constexpr uint32_t kStTimeout = 1u, kStOverNotify = 2u, kStOverflow = 8u, kStAbort = 0x80000000u;

// task types (the same numbers as the kernels' TaskType)
enum : int { T_R = 1, T_K = 2, T_S = 3, T_G1 = 5, T_G2 = 6, T_C = 7 };

// 32-bit descriptor: type in bits 29..31, a in bits 13..28, b in bits 0..12.
// Nonzero for every task (type >= 1), so zero marks an unwritten slot.
constexpr int kDescABits = 16, kDescBBits = 13;
ETC_HD uint32_t make_desc(int type, uint32_t a, uint32_t b) {
  return ((uint32_t)type << 29) | ((a & 0xffffu) << 13) | (b & 0x1fffu);
}
ETC_HD int desc_type(uint32_t d) { return (int)(d >> 29); }
ETC_HD int desc_a(uint32_t d) { return (int)((d >> 13) & 0xffffu); }
ETC_HD int desc_b(uint32_t d) { return (int)(d & 0x1fffu); }

// Per-launch task counts of the MoE layer graph, all derived from T (the
// symbolic batch dimension) and the tile widths the launch runs.
struct MoeGraph {
  int T, k;
  int nTT, nET, nR;  // router tasks: token tiles x expert tiles
  int nK;            // top-k tasks (one per token tile)
  int nC;            // combine tasks
  int nN1, nN2;      // G1 / G2 column tiles per row tile
  int ctok;          // tokens per combine task
};
ETC_HD MoeGraph moe_graph(int T, int E, int k, int H, int I, int router_tokens, int router_experts,
                          int combine_tokens, int bn1, int bn2) {
  MoeGraph g;
  g.T = T;
  g.k = k;
  g.nTT = (T + router_tokens - 1) / router_tokens;
  g.nET = (E + router_experts - 1) / router_experts;
  g.nR = g.nTT * g.nET;
  g.nK = g.nTT;
  g.nC = (T + combine_tokens - 1) / combine_tokens;
  g.nN1 = I / bn1;
  g.nN2 = H / bn2;
  g.ctok = combine_tokens;
  return g;
}
// Task counts of a launch of T tokens in variant `var` (kVarSmall, kVarWide
// or kVarBig).  The router tiles and G tile widths are those the variant's
// bodies run: the small-batch variant has no eight-experts-a-wave router
// tile and no column-split G tiles, so there the router task count follows
// four experts a wave and the G1 width stops at 32 columns; the big-tile
// variant runs the large-batch router and its own G tile widths.
ETC_HD MoeGraph launch_graph(int T, int E, int k, int H, int I, int var) {
  int re = router_experts(T);
  if (var == kVarSmall && re == kRouterEXL) re = kRouterEL;
  if (var == kVarBig) return moe_graph(T, E, k, H, I, kRouterT, re, kCombineT, kBigBN1, kBigBN2);
  int bn1 = g1_cols(T, k, H);
  if (var == kVarSmall && bn1 > 2 * kBN1) bn1 = 2 * kBN1;
  const int bn2 = var == kVarWide ? g2_cols(T, k, I) : kBN2;
  return moe_graph(T, E, k, H, I, kRouterT, re, kCombineT, bn1, bn2);
}
// every task a launch of nrt row tiles runs: the router prefix, then
// everything that goes through the queue
ETC_HD uint32_t moe_total(const MoeGraph& g, int nrt) {
  return (uint32_t)(g.nR + g.nK + 1 + g.nC) + (uint32_t)nrt * (uint32_t)(g.nN1 + g.nN2);
}
// rows of combine task ct (its tokens times k)
ETC_HD uint32_t ctile_rows(const MoeGraph& g, int ct) {
  const int t0 = ct * g.ctok;
  const int n = g.T - t0 < g.ctok ? g.T - t0 : g.ctok;
  return (uint32_t)(n * g.k);
}
// Queue slots a layer of at most T_max tokens can need: every task but the
// router prefix goes through the queue once, counted with the narrowest
// tiles (bn1, bn2) and the largest row-tile count (max_rt).
ETC_HD int64_t moe_queue_capacity(int64_t T_max, int64_t max_rt, int64_t I, int64_t H, int bn1, int bn2,
                                  int router_tokens, int combine_tokens) {
  const int64_t nK = (T_max + router_tokens - 1) / router_tokens;
  const int64_t nC = (T_max + combine_tokens - 1) / combine_tokens;
  return nK + 1 + max_rt * (I / bn1 + H / bn2) + nC + 64;
}

struct Queue {
  uint32_t* head;    // pop indices taken
  uint32_t* tail;    // slots reserved
  uint32_t* total;   // prefix + pushed tasks of the launch; 0 until known
  uint32_t* status;  // status word (abort, timeout, overflow bits)
  uint32_t* slot;    // [cap] descriptors
  int64_t cap;
  uint32_t prefix;   // tasks ready at launch (pop indices 0 .. prefix-1)
  uint32_t known_total;  // the total when it is known at launch (else 0: read *total)
  uint64_t budget;   // watchdog of one wait, in P::now() ticks
};

// Thread 0: the descriptor behind pop index idx >= prefix, or 0 when the
// workgroup should leave (no task will fill the slot, the launch aborts, or
// the watchdog expired).
template <class P>
ETC_HD uint32_t wait_slot(const Queue& q, uint32_t idx) {
  const int64_t s = (int64_t)idx - (int64_t)q.prefix;
  if (s >= q.cap || (q.known_total && idx >= q.known_total)) return 0u;
  const uint64_t t0 = P::now();
  for (uint32_t spins = 1;; ++spins) {
    const uint32_t v = P::load(q.slot + s);
    if (v) return v;
    if ((spins & 3u) == 0u) {
      const uint32_t tot = q.known_total ? q.known_total : P::load(q.total);
      if (tot && idx >= tot) return 0u;
      if (P::load(q.status) & kStAbort) return 0u;
      if (P::now() - t0 > q.budget) {
        P::orr(q.status, kStTimeout | kStAbort);
        return 0u;
      }
    }
    P::pause();
  }
}

// Thread 0: reserve n slots; returns the first, or -1 (overflow: the launch
// aborts, and the status word says why).
template <class P>
ETC_HD int64_t reserve(const Queue& q, uint32_t n) {
  const uint32_t base = P::add(q.tail, n);
  if ((int64_t)base + (int64_t)n > q.cap) {
    P::orr(q.status, kStOverflow | kStAbort);
    return -1;
  }
  return (int64_t)base;
}

// Notify one event element; true when this notify completed it.
template <class P>
ETC_HD bool notify(const Queue& q, uint32_t* ev, uint32_t target) {
  const uint32_t old = P::add(ev, 1u);
  if (old + 1u > target) P::orr(q.status, kStOverNotify | kStAbort);
  return old + 1u == target;
}

// Per-workgroup scratch of the runner (LDS on the device).
struct Shared {
  uint32_t desc;  // the popped descriptor, handed from thread 0 to the workgroup
  int flag;       // thread 0's notify completed its event
  int n;          // completed events collected by this task
  int base;       // first reserved slot
  int list[kBigBM];  // combine tasks released by a row tile (one per row at most; big tiles hold kBigBM rows)
};

// Pop index -> router task of the prefix
ETC_HD uint32_t router_desc(const MoeGraph& g, uint32_t idx) {
  return make_desc(T_R, idx / (uint32_t)g.nET, idx % (uint32_t)g.nET);
}

// The MoE layer under the dynamic schedule, run by every thread of one
// workgroup until the queue is drained.
//   R(tt, et) -> ev_logit[tt] (nET arrivals) -> push K(tt)
//   K(tt)     -> ev_route (nK arrivals)      -> push S
//   S         -> publish the total, push every G1(rt, nt)
//   G1(rt, nt)-> ev_h[rt] (nN1 arrivals)     -> push G2(rt, 0..nN2-1)
//   G2(rt, nt)-> ev_y[rt] (nN2 arrivals)     -> one arrival on ev_c[ct] per
//                row of the tile, ct its token's combine task
//   ev_c[ct] (its 2k rows)                   -> push C(ct)
// A producer's data is complete before its notify (P::publish waits for
// the workgroup's stores and then synchronises it), and a pushed task's
// descriptor is written after the notify that released it, so a task popped
// from the queue finds its inputs written.
template <class P, class K>
ETC_HD void run_moe(K& tk, const Queue& q, const MoeGraph& g, Shared& sh) {
  const int tid = P::tid();
  uint32_t idx = 0;
  if (tid == 0) idx = P::add(q.head, 1u);
  for (;;) {
    if (tid == 0) {
      const uint32_t d = idx < q.prefix ? router_desc(g, idx) : wait_slot<P>(q, idx);
      sh.desc = d;
      // pop-ahead: the next index is taken while this task runs, so the
      // head's round trip overlaps the task body
      if (d) idx = P::add(q.head, 1u);
    }
    P::barrier();
    const uint32_t d = sh.desc;
    P::barrier();
    if (!d) return;
    const int a = desc_a(d), b = desc_b(d);
    tk.trace_start();
    switch (desc_type(d)) {
      case T_R:
        tk.router(a, b);
        tk.trace_body();
        P::publish();
        if (tid == 0 && notify<P>(q, tk.ev_logit(a), (uint32_t)g.nET)) {
          const int64_t s = reserve<P>(q, 1u);
          if (s >= 0) P::put(q.slot + s, make_desc(T_K, (uint32_t)a, 0u));
        }
        break;
      case T_K:
        tk.topk(a);
        tk.trace_body();
        P::publish();
        if (tid == 0 && notify<P>(q, tk.ev_route(), (uint32_t)g.nK)) {
          const int64_t s = reserve<P>(q, 1u);
          if (s >= 0) P::put(q.slot + s, make_desc(T_S, 0u, 0u));
        }
        break;
      case T_S: {
        const int nrt = tk.scan();
        tk.trace_body();
        P::publish();
        if (tid == 0) {
          // the total goes out before the G1 slots are reserved: an index
          // past it can then leave as soon as it sees it
          P::put(q.total, moe_total(g, nrt));
          const uint32_t n1 = (uint32_t)nrt * (uint32_t)g.nN1;
          sh.n = (int)n1;
          sh.base = (int)reserve<P>(q, n1);
        }
        P::barrier();
        const int n1 = sh.n, base = sh.base;
        if (base >= 0)
          for (int i = tid; i < n1; i += P::kThreads)
            P::put(q.slot + base + i, make_desc(T_G1, (uint32_t)(i / g.nN1), (uint32_t)(i % g.nN1)));
        break;
      }
      case T_G1:
        tk.g1(a, b);
        tk.trace_body();
        P::publish();
        if (tid == 0) {
          sh.base = -1;
          if (notify<P>(q, tk.ev_h(a), (uint32_t)g.nN1)) sh.base = (int)reserve<P>(q, (uint32_t)g.nN2);
        }
        P::barrier();
        if (sh.base >= 0)
          for (int i = tid; i < g.nN2; i += P::kThreads)
            P::put(q.slot + sh.base + i, make_desc(T_G2, (uint32_t)a, (uint32_t)i));
        break;
      case T_G2: {
        tk.g2(a, b);
        tk.trace_body();
        P::publish();
        if (tid == 0) {
          sh.n = 0;
          sh.flag = notify<P>(q, tk.ev_y(a), (uint32_t)g.nN2) ? 1 : 0;
        }
        P::barrier();
        if (sh.flag) {
          // the row tile is complete: each of its rows arrives at its
          // token's combine event
          const int nrows = tk.tile_rows(a);
          for (int r = tid; r < nrows; r += P::kThreads) {
            const int ct = tk.row_ctile(a, r);
            if (notify<P>(q, tk.ev_c(ct), ctile_rows(g, ct))) sh.list[P::lds_add(&sh.n, 1)] = ct;
          }
          P::barrier();
          const int n = sh.n;
          if (n) {
            if (tid == 0) sh.base = (int)reserve<P>(q, (uint32_t)n);
            P::barrier();
            if (sh.base >= 0)
              for (int i = tid; i < n; i += P::kThreads)
                P::put(q.slot + sh.base + i, make_desc(T_C, (uint32_t)sh.list[i], 0u));
          }
        }
        break;
      }
      case T_C:
        tk.combine(a);
        tk.trace_body();
        break;
      default:
        if (tid == 0) P::orr(q.status, kStOverflow | kStAbort);
        return;
    }
    tk.trace_end(desc_type(d), a, b);
  }
}


// The split-K row-sum example (Event Tensor pages, Fig. 3; podcast cue 3)
// under the same queue: partial_sum(i, j) for every (i, j) is the ready
// prefix (pop index i * nsplit + j); it notifies the event element its
// out-edge maps (i, j) to (tk.notify_elem), and the notify that completes an
// element (wait_count arrivals) pushes the final_sum that waits on it
// (tk.waiter, the inverse of the in-edge).  The total n * (nsplit + 1) is
// known at launch.  Each popped slot is cleared again, so the ring is at
// rest for the next launch once the control words are reset.  Descriptors:
// type in bits 29..31, the 29-bit row or pair index below.
enum : int { T_SK_PART = 1, T_SK_FINAL = 2 };
// the last workgroup of a launch returns the control words to rest
template <class P>
ETC_HD void splitk_reset(const Queue& q) {
  P::put(q.status, 0u);
  P::put(q.head, 0u);
  P::put(q.tail, 0u);
}
ETC_HD uint32_t sk_desc(int type, uint32_t v) { return ((uint32_t)type << 29) | (v & 0x1fffffffu); }

template <class P, class K>
ETC_HD void run_splitk(K& tk, const Queue& q, uint32_t nsplit, uint32_t wait_count, uint32_t* ev, Shared& sh) {
  const int tid = P::tid();
  uint32_t idx = 0;
  if (tid == 0) idx = P::add(q.head, 1u);
  for (;;) {
    if (tid == 0) {
      uint32_t d;
      if (idx < q.prefix) {
        d = sk_desc(T_SK_PART, idx);
      } else {
        d = wait_slot<P>(q, idx);
        if (d) P::put(q.slot + (idx - q.prefix), 0u);  // slot back to rest
      }
      sh.desc = d;
      if (d) idx = P::add(q.head, 1u);
    }
    P::barrier();
    const uint32_t d = sh.desc;
    P::barrier();
    if (!d) return;
    const uint32_t v = d & 0x1fffffffu;
    if ((int)(d >> 29) == T_SK_PART) {
      const uint32_t i = v / nsplit, j = v % nsplit;
      tk.partial(i, j);
      P::publish();
      if (tid == 0) {
        const uint32_t e = tk.notify_elem(i, j);
        if (notify<P>(q, ev + e, wait_count)) {
          const int64_t s = reserve<P>(q, 1u);
          if (s >= 0) P::put(q.slot + s, sk_desc(T_SK_FINAL, tk.waiter(e)));
        }
      }
    } else {
      tk.final_sum(v);
    }
  }
}

}  // namespace dyn
}  // namespace etc
