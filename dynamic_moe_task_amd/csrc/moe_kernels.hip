// One MoE layer as a graph of tiled tasks inside one persistent HIP kernel
// for gfx950 (MI355X), plus the kernel-by-kernel comparator built from the
// same task bodies.
//
// Task graph (Event Tensor, arXiv 2604.13327: Fig. 2 and Fig. 5b; podcast
// cues 7 and 9):
//   R(tt, et)  router logits for a tile of tokens x experts (fixed-order fp32)
//   K(tt)      top-k + routing weights for the tile's tokens; notifies
//              ev_exp[e] once per routed (token, slot)           waits ev_logit[tt]
//   S          counts, exp_indptr, stable permutation, row tiles   waits ev_route
//   G1(rt, nt) gate/up GEMM + SwiGLU for one row tile of one expert, its
//              rows gathered from x through the permutation   waits ev_scan and
//              ev_exp[e] (released after counts[e] arrivals: the data-dependent
//              update; expert e's tiles cover grouped rows
//              [exp_indptr[e], exp_indptr[e+1]): the data-dependent trigger)
//   G2(rt, nt) down projection; notifies ev_y[rt]                 waits ev_h[rt]
//   C(ct)      weighted combine of the k expert rows per token: waits ev_y of
//              every row tile that holds one of its rows (DYNAMIC: ev_c[ct],
//              one arrival per row and G2 column tile)
//
// Schedules: STATIC (closed-form phase-ordered per-workgroup lists, notify /
// wait; Figs. 6-7), DYNAMIC (early push onto one HBM queue when a notify
// completes an event, pop by idle workgroups; Figs. 8-9), BARRIER (same
// lists, grid barriers instead of events), KBK (one launch per task type).
// T is a kernel argument; every event shape and task count below is derived
// from it in the kernel (Fig. 4: one template, instantiated per launch).
//
// Data that one workgroup writes and another reads (logits, routing tensors,
// intermediate Hmid, expert outputs Y) moves through
// device-coherent loads and stores (etc_rt.h); weights and input tokens are
// read through the caches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include "etc_internal.h"
#include "etc_rt.h"

namespace etc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum Mode : int { MODE_STATIC = ETC_SCHED_STATIC, MODE_DYNAMIC = ETC_SCHED_DYNAMIC,
                  MODE_KBK = ETC_SCHED_KBK, MODE_BARRIER = ETC_SCHED_BARRIER,
                  MODE_ORDERED = ETC_SCHED_ORDERED };

// ------------------------------------------------------------- helpers --
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ uint32_t f2bf(float f) {
  // fp32 -> bf16, round to nearest even: gfx950's conversion instruction
  // (v_cvt_pk_bf16_f32).  For every non-NaN fp32 value it gives the same
  // bits as (u + 0x7fff + ((u >> 16) & 1)) >> 16 on the value's bits u
  // (checked on MI355X over all 2^32 patterns); a NaN stays a quiet NaN.
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// The same rounding in integer arithmetic (the big tiles' epilogue, whose
// kernels sit at the register file's limit: the conversion instruction's
// pairing of values there costs registers).
__device__ __forceinline__ uint32_t f2bf_int(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ u32x4_t ld4(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st4(uint16_t* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ bf16x8_t as_bf(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ void unpack8(u32x4_t v, float* f) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}
__device__ __forceinline__ int first_of(int w, int64_t off, int G) {
  int o = (int)(off % G);
  return (w - o + G) % G;
}

// device-coherent resources of the arrays that cross workgroups
__device__ __forceinline__ rsrc_t r_logits(const MoeParams& p) { return make_rsrc(p.logits, p.logits_bytes); }
__device__ __forceinline__ rsrc_t r_ids(const MoeParams& p) { return make_rsrc(p.ids, p.rows_bytes); }
__device__ __forceinline__ rsrc_t r_topw(const MoeParams& p) { return make_rsrc(p.topw, p.rows_bytes); }
__device__ __forceinline__ rsrc_t r_perm(const MoeParams& p) { return make_rsrc(p.perm, p.rows_bytes); }
__device__ __forceinline__ rsrc_t r_slot(const MoeParams& p) { return make_rsrc(p.slot, p.rows_bytes); }
__device__ __forceinline__ rsrc_t r_counts(const MoeParams& p) { return make_rsrc(p.counts, (uint32_t)p.E * 4u); }
__device__ __forceinline__ rsrc_t r_indptr(const MoeParams& p) { return make_rsrc(p.indptr, (uint32_t)(p.E + 1) * 4u); }
__device__ __forceinline__ rsrc_t r_rtinfo(const MoeParams& p) { return make_rsrc(p.rt_info, (uint32_t)p.max_rt * 16u); }
__device__ __forceinline__ rsrc_t r_rowrt(const MoeParams& p) { return make_rsrc(p.row_rt, p.rows_bytes); }
__device__ __forceinline__ rsrc_t r_hh(const MoeParams& p) { return make_rsrc(p.hh, p.hh_bytes); }
__device__ __forceinline__ rsrc_t r_y(const MoeParams& p) { return make_rsrc(p.y, p.y_bytes); }
__device__ __forceinline__ rsrc_t r_ccnt(const MoeParams& p) { return make_rsrc(p.ccnt, p.ccnt_bytes); }

struct RowTile {
  int e, r0, nrows;
};
__device__ __forceinline__ RowTile load_rowtile(const MoeParams& p, int rt) {
  const u32x4_t v = co_ld128(r_rtinfo(p), (uint32_t)rt * 16u);
  RowTile r;
  r.e = (int)v.x;
  r.r0 = (int)v.y;
  r.nrows = (int)v.z;
  return r;
}

// Routing tables of a small batch, rebuilt by every persistent workgroup in
// its own LDS once all top-k tasks are done (see run_lists): G1 then starts
// without waiting for S, and the G runners read tile descriptors and the
// permutation from LDS instead of memory.
struct LocalRoute {
  uint32_t tile[kLocalTiles];  // expert | rows << 9 | first grouped row << 16
  uint16_t perm[kLocalRows];   // grouped row -> flat pair index t * k + j
  uint16_t cnt[kMaxE];         // rows per expert
};
__device__ __forceinline__ RowTile get_tile(const MoeParams& p, const LocalRoute* lr, int rt) {
  if (!lr) return load_rowtile(p, rt);
  const uint32_t v = lr->tile[rt];
  RowTile r;
  r.e = (int)(v & 511u);
  r.nrows = (int)((v >> 9) & 127u);
  r.r0 = (int)(v >> 16);
  return r;
}

// Per-launch sizes, all derived from T (the symbolic batch dimension).
struct Ctx {
  uint32_t* set;     // counter set of this launch (NULL for kernel-by-kernel)
  uint32_t* status;  // where error bits go
  int T, H, E, k, I;
  int bn1;  // G1 gate (and up) columns per tile, chosen per launch from T
  int bn2;  // G2 output columns per tile, chosen per launch from T
  int bm;   // grouped rows per row tile (kBigBM in the big-tile variant, else kBM)
  int nTT, nET, nR, nK, nC, nN1, nN2;
  uint64_t budget;  // watchdog of one wait, wall-clock ticks
};

__device__ __forceinline__ Ctx make_ctx(const MoeParams& p, uint32_t* set) {
  Ctx c;
  c.set = set;
  c.status = set ? set + W_STATUS : p.ctrl + C_REPORT;
  c.T = p.T; c.H = p.H; c.E = p.E; c.k = p.k; c.I = p.I;
  c.nTT = (p.T + kRouterT - 1) / kRouterT;
  c.nET = (p.E + router_experts(p.T) - 1) / router_experts(p.T);
  c.nR = c.nTT * c.nET;
  c.nK = c.nTT;
  c.nC = (p.T + kCombineT - 1) / kCombineT;
  // tile shapes of the variant a launch of T tokens runs (the host picks the
  // variant with the same rule)
  const bool big = big_variant(p.T, p.k, p.H, p.I);
  c.bn1 = big ? kBigBN1 : g1_cols(p.T, p.k, p.H);
  c.nN1 = p.I / c.bn1;
  c.bn2 = big ? kBigBN2 : g2_cols(p.T, p.k, p.I);
  c.nN2 = p.H / c.bn2;
  c.bm = big ? kBigBM : kBM;
  c.budget = p.budget;
  return c;
}

struct Shared {
  int pairs[2 * kCombineT * kMaxK];  // C: (weight, slot) pairs
  uint32_t claim[4];                 // ORDERED: claimed ordinals handed to every thread
};

__device__ __forceinline__ void dbg_task(const MoeParams& p, int type) {
  if (p.debug && threadIdx.x == 0) atomicAdd(p.debug + 2 * p.E + (type - 1), 1);
}

// Optional per-task trace (thread 0): wall-clock ticks before the wait,
// after it, after the task body, and after the notifies.
// Records of workgroup w fill slots [w*per_wg, (w+1)*per_wg) in task order;
// only thread 0 writes them, so the running count lives in LDS.
__shared__ uint32_t s_trace_n;

__device__ __forceinline__ void trace_init(const MoeParams& p) {
  if (threadIdx.x != 0) return;
  s_trace_n = 0;
  if (p.trace && blockIdx.x == 0) {
    p.trace[1] = p.trace_records / gridDim.x;
    p.trace[2] = gridDim.x;
  }
}

__device__ __forceinline__ void trace_task(const MoeParams& p, int type, int a, int b, uint64_t tw,
                                           uint64_t ts, uint64_t tb) {
  if (!p.trace || threadIdx.x != 0) return;
  const uint64_t te = now_ticks();
  const uint32_t per_wg = p.trace_records / gridDim.x;
  const uint32_t j = s_trace_n++;
  if (j >= per_wg) return;
  uint32_t* q = p.trace + 16 + 8 * ((size_t)blockIdx.x * per_wg + j);
  q[0] = blockIdx.x | ((uint32_t)type << 24);
  q[1] = (uint32_t)a;
  q[2] = (uint32_t)b;
  q[3] = (uint32_t)tw;
  q[4] = (uint32_t)(tw >> 32);
  q[5] = (uint32_t)ts;
  q[6] = (uint32_t)tb;
  q[7] = (uint32_t)te;
}

// ====================================================== event helpers ========
// Event elements live in the launch's counter set; see etc_rt.h for the
// counting and coherence rules.
// Each element sits on its own 128-byte line (kEvStride words apart): the
// atomics of producers that notify different elements at the same time then
// do not queue behind one another on a shared line.
__device__ __forceinline__ uint32_t* ev_logit(const MoeParams& p, const Ctx& c, int i) {
  return c.set + p.o_ev_logit + (int64_t)i * kEvStride;
}
__device__ __forceinline__ uint32_t* ev_exp(const MoeParams& p, const Ctx& c, int e) {
  return c.set + p.o_ev_exp + (int64_t)e * kEvStride;
}
__device__ __forceinline__ uint32_t* ev_h(const MoeParams& p, const Ctx& c, int rt) {
  return c.set + p.o_ev_h + (int64_t)rt * kEvStride;
}
__device__ __forceinline__ uint32_t* ev_y(const MoeParams& p, const Ctx& c, int rt) {
  return c.set + p.o_ev_y + (int64_t)rt * kEvStride;
}
__device__ __forceinline__ uint32_t* ev_c(const MoeParams& p, const Ctx& c, int ct) {
  return c.set + p.o_ev_c + (int64_t)ct * kEvStride;
}

// Notify one event element; returns true if this notify completed it.
__device__ __forceinline__ bool notify1(const Ctx& c, uint32_t* ev, uint32_t target) {
  const uint32_t old = add_relaxed(ev, 1u);
  if (old + 1u > target) or_relaxed(c.status, ST_OVER_NOTIFY | ST_ABORT);
  return old + 1u == target;
}

// n arrivals at once (a workgroup's batch of tasks); true when they complete
// the event.
__device__ __forceinline__ bool notify_n(const Ctx& c, uint32_t* ev, uint32_t n, uint32_t target) {
  const uint32_t old = add_relaxed(ev, n);
  if (old + n > target) or_relaxed(c.status, ST_OVER_NOTIFY | ST_ABORT);
  return old + n == target;
}

// Notify without checking for over-notification unless the debug buffer is
// set (then notify1 records any notify past the wait count).
__device__ __forceinline__ void notify_fast(const MoeParams& p, const Ctx& c, uint32_t* ev, uint32_t target) {
  if (p.debug) {
    asm volatile("" ::: "memory");  // keeps the two atomics from being merged into one returning atomic
    notify1(c, ev, target);
  } else {
    (void)__hip_atomic_fetch_add(ev, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ===================================================== task bodies ==========
// R: router logits L[t, e] = sum_h x[t, h] * wr[e, h] (+ b[e]) of kRouterT
// tokens x (4 * EPW) experts; wave w computes experts et * 4 * EPW + w * EPW
// + j, j < EPW.  Each logit is one wave's sum in a fixed order: lane l takes
// the 8-element chunks l, l + 64, ... of the hidden dimension with ascending
// fused multiply-adds, then a halving xor butterfly combines the 64 lane sums
// (its lane-0 result equals the tree acc[l] += acc[l + s], s = 32..1), then
// the bias.  This fixed order is what makes the top-k decision reproducible
// bit for bit.  A batch of four chunks per lane is loaded before its
// arithmetic.
// The big-tile router stream's logits, after the butterfly: every lane
// holds every sum (each xor step adds the same two values in either order,
// so all 64 lanes end with lane 0's bits).  Lane r stores token r's EPW
// logits as 16-byte stores of four consecutive experts, EPW / 4 of them,
// instead of lane 0 storing 4 * EPW values one by one (the token index stays
// a compile-time constant: a lane-indexed pick would put the sums in
// scratch memory).  Full tiles only: E a multiple of 4 * EPW.
template <int EPW>
__device__ __forceinline__ void router_store_tile(const MoeParams& p, const Ctx& c, int t0, int e0,
                                                  const float (&acc)[EPW][kRouterT]) {
  static_assert(EPW % 4 == 0, "four consecutive experts a store");
  const int lane = threadIdx.x & 63;
  const rsrc_t rl = r_logits(p);
#pragma unroll
  for (int r = 0; r < kRouterT; ++r) {
    if (lane != r) continue;
    float v[EPW];
#pragma unroll
    for (int j = 0; j < EPW; ++j) v[j] = p.has_bias ? acc[j][r] + p.br[e0 + j] : acc[j][r];
    const uint32_t off = (uint32_t)((t0 + r) * c.E + e0) * 4u;
#pragma unroll
    for (int q = 0; q < EPW / 4; ++q) {
      u32x4_t o;
      o.x = __float_as_uint(v[4 * q]);
      o.y = __float_as_uint(v[4 * q + 1]);
      o.z = __float_as_uint(v[4 * q + 2]);
      o.w = __float_as_uint(v[4 * q + 3]);
      co_st128(rl, off + 16u * q, o);
    }
  }
}

template <int EPW, int U>
__device__ __forceinline__ void router_body(const MoeParams& p, const Ctx& c, int tt, int et) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e0 = et * 4 * EPW + wv * EPW;
  if (e0 >= c.E) return;
  const int t0 = tt * kRouterT;
  const int ntok = min(kRouterT, c.T - t0);
  const int ne = min(EPW, c.E - e0);
  float acc[EPW][kRouterT];
#pragma unroll
  for (int j = 0; j < EPW; ++j)
#pragma unroll
    for (int r = 0; r < kRouterT; ++r) acc[j][r] = 0.0f;
  const int nchunk = c.H >> 3;
  const uint16_t* xrow = p.x + (size_t)t0 * c.H;
  const uint16_t* wrow = p.wr + (size_t)e0 * c.H;
  if (ntok == kRouterT && ne == EPW && nchunk % (64 * U) == 0) {
    // full tile: no per-load or per-product predicates.  Per logit the
    // products still go chunk by chunk in ascending order, 8 elements each.
    for (int c0 = lane; c0 < nchunk; c0 += 64 * U) {
      u32x4_t xv4[U][kRouterT], wv4[EPW][U];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < kRouterT; ++r) xv4[u][r] = ld4(xrow + (size_t)r * c.H + (c0 + 64 * u) * 8);
#pragma unroll
      for (int j = 0; j < EPW; ++j)
#pragma unroll
        for (int u = 0; u < U; ++u) wv4[j][u] = ld4(wrow + (size_t)j * c.H + (c0 + 64 * u) * 8);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float wf[EPW][8];
#pragma unroll
        for (int j = 0; j < EPW; ++j) unpack8(wv4[j][u], wf[j]);
#pragma unroll
        for (int r = 0; r < kRouterT; ++r) {
          float xf[8];
          unpack8(xv4[u][r], xf);
#pragma unroll
          for (int j = 0; j < EPW; ++j)
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[j][r] = __builtin_fmaf(xf[q], wf[j][q], acc[j][r]);
        }
      }
    }
  } else {
  for (int c0 = lane; c0 < nchunk; c0 += 64 * U) {
    // the batch's token chunks and every expert's weight chunks
    u32x4_t xv4[U][kRouterT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ch = c0 + 64 * u;
#pragma unroll
      for (int r = 0; r < kRouterT; ++r)
        if (ch < nchunk && r < ntok) xv4[u][r] = ld4(xrow + (size_t)r * c.H + ch * 8);
    }
    u32x4_t wv4[EPW][U];  // all weight chunks of the batch in flight together
#pragma unroll
    for (int j = 0; j < EPW; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ch = c0 + 64 * u;
        if (ch < nchunk && j < ne) wv4[j][u] = ld4(wrow + (size_t)j * c.H + ch * 8);
      }
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ch = c0 + 64 * u;
        if (ch < nchunk && j < ne) {
          float wf[8];
          unpack8(wv4[j][u], wf);
#pragma unroll
          for (int r = 0; r < kRouterT; ++r) {
            if (r < ntok) {
              float xf[8];
              unpack8(xv4[u][r], xf);
#pragma unroll
              for (int q = 0; q < 8; ++q) acc[j][r] = __builtin_fmaf(xf[q], wf[q], acc[j][r]);
            }
          }
        }
      }
    }
  }
  }
#pragma unroll
  for (int j = 0; j < EPW; ++j)
#pragma unroll
    for (int r = 0; r < kRouterT; ++r) {
#pragma unroll
      for (int s = 32; s >= 1; s >>= 1) acc[j][r] = acc[j][r] + __shfl_xor(acc[j][r], s);
    }
  if (lane == 0) {
    const rsrc_t rl = r_logits(p);
#pragma unroll
    for (int j = 0; j < EPW; ++j) {
#pragma unroll
      for (int r = 0; r < kRouterT; ++r) {
        if (j < ne && r < ntok) {
          float v = acc[j][r];
          if (p.has_bias) v = v + p.br[e0 + j];
          co_stf(rl, (uint32_t)((t0 + r) * c.E + e0 + j) * 4u, v);
        }
      }
    }
  }
}
template <bool XL = true>
__device__ __forceinline__ void task_router(const MoeParams& p, const Ctx& c, int tt, int et) {
  // The tile's experts follow the same rule as the task count (nET); the
  // eight-experts-a-wave tile exists only where XL is set, and the variant
  // without it counts its tasks for four experts a wave.  U: 8-element chunks
  // a lane loads per batch, halved for eight experts a wave to bound the
  // registers.
  const int re = router_experts(c.T);
  if (XL && re == kRouterEXL)
    router_body<kRouterEXL / 4, 2>(p, c, tt, et);
  else if (re >= kRouterEL)
    router_body<kRouterEL / 4, 4>(p, c, tt, et);
  else
    router_body<kRouterE / 4, 4>(p, c, tt, et);
}

// Big-tile variant, all of a workgroup's router tasks (i0, i0 + G, ...) as
// one stream: the next step's chunks load while the current step multiplies,
// across task boundaries (one wave a SIMD in this variant, so a wave hides
// its own load latency or nobody does), and the logits' stores are drained
// once, after the last task, before the notifies of every task of the
// stream.  Each logit is the same sequence of fused multiply-adds, butterfly
// and bias as in router_body.  Full tiles only (the caller checks T, E and
// H); EPW experts a wave, U chunks a lane a step, steps taken in pairs.
template <int EPW, int U>
__device__ __forceinline__ void router_stream(const MoeParams& p, const Ctx& c, int i0, int G) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int H = c.H, nit = (H >> 3) / (64 * U);  // steps a task (even)
  const bool tr = p.trace != nullptr;
  u32x4_t xa[U][kRouterT], wa[EPW][U], xb[U][kRouterT], wb[EPW][U];
  auto load = [&](int i, int it, u32x4_t (&xv)[U][kRouterT], u32x4_t (&wvv)[EPW][U]) {
    const uint16_t* xrow = p.x + (size_t)(i / c.nET) * kRouterT * H;
    const uint16_t* wrow = p.wr + (size_t)((i % c.nET) * 4 * EPW + wv * EPW) * H;
    const int c0 = lane + it * 64 * U;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < kRouterT; ++r) xv[u][r] = ld4(xrow + (size_t)r * H + (c0 + 64 * u) * 8);
#pragma unroll
    for (int j = 0; j < EPW; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) wvv[j][u] = ld4(wrow + (size_t)j * H + (c0 + 64 * u) * 8);
  };
  auto step = [&](const u32x4_t (&xv)[U][kRouterT], const u32x4_t (&wvv)[EPW][U], float (&acc)[EPW][kRouterT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float wf[EPW][8];
#pragma unroll
      for (int j = 0; j < EPW; ++j) unpack8(wvv[j][u], wf[j]);
#pragma unroll
      for (int r = 0; r < kRouterT; ++r) {
        float xf[8];
        unpack8(xv[u][r], xf);
#pragma unroll
        for (int j = 0; j < EPW; ++j)
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[j][r] = __builtin_fmaf(xf[q], wf[j][q], acc[j][r]);
      }
    }
  };
  load(i0, 0, xa, wa);
  for (int i = i0; i < c.nR; i += G) {
    uint64_t tw = 0;
    if (tr) tw = now_ticks();
    float acc[EPW][kRouterT];
#pragma unroll
    for (int j = 0; j < EPW; ++j)
#pragma unroll
      for (int r = 0; r < kRouterT; ++r) acc[j][r] = 0.0f;
    for (int it = 0; it < nit; it += 2) {
      load(i, it + 1, xb, wb);
      step(xa, wa, acc);
      if (it + 2 < nit)
        load(i, it + 2, xa, wa);
      else if (i + G < c.nR)
        load(i + G, 0, xa, wa);  // the next task's first step
      step(xb, wb, acc);
    }
#pragma unroll
    for (int j = 0; j < EPW; ++j)
#pragma unroll
      for (int r = 0; r < kRouterT; ++r) {
#pragma unroll
        for (int s2 = 32; s2 >= 1; s2 >>= 1) acc[j][r] = acc[j][r] + __shfl_xor(acc[j][r], s2);
      }
    router_store_tile<EPW>(p, c, (i / c.nET) * kRouterT, (i % c.nET) * 4 * EPW + wv * EPW, acc);
    dbg_task(p, TT_R);
    if (tr) {
      const uint64_t tb = now_ticks();
      trace_task(p, TT_R, i / c.nET, i % c.nET, tw, tw, tb);
    }
  }
}

// K: top-k per token (one wave per token): k rounds of a wave-wide arg-max
// on (logit descending, expert index ascending); weights exp(l_j - l_max)
// normalised over the chosen k (norm_topk) or over all E.
//
// Each round takes the wave maximum of the lanes' best remaining logits with
// six DPP steps (pair swap, quad swap, half-row and row mirror, then the two
// row broadcasts that carry a row's maximum into the next rows; lane 63 ends
// with the maximum of all 64 lanes), then picks the lowest expert index that
// holds that value from one ballot per 64-expert slice: expert e = lane +
// 64 j, so the first slice with a hit and its lowest set lane give the lowest
// index.  Ties therefore go to the lower expert, and equality is float
// equality (+0 and -0 tie), as in a (logit desc, index asc) ordering.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float x) {
  const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xf, false);
  return fmaxf(x, __int_as_float(y));
}
__device__ __forceinline__ float wave_max(float x) {
  x = dpp_max_step<0xB1, 0xf>(x);   // quad_perm [1,0,3,2]
  x = dpp_max_step<0x4E, 0xf>(x);   // quad_perm [2,3,0,1]
  x = dpp_max_step<0x141, 0xf>(x);  // row_half_mirror
  x = dpp_max_step<0x140, 0xf>(x);  // row_mirror
  x = dpp_max_step<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_max_step<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
// hist: when given (a workgroup's stream of top-k tasks), the expert-event
// arrivals are counted there, in LDS, and notified by the caller once for
// the whole stream (one atomic per expert instead of one per routed pair:
// with few experts, all T*k pairs would otherwise hit the same counters).
__device__ __forceinline__ void task_topk(const MoeParams& p, const Ctx& c, int tt, int* hist = nullptr) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = tt * kRouterT + wv;
  if (t >= c.T) return;
  const float NEG_INF = -__builtin_inff();
  const rsrc_t rl = r_logits(p);
  float v[4];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    float x = NEG_INF;
    if (e < c.E) {
      x = co_ldf(rl, (uint32_t)(t * c.E + e) * 4u);
      if (x != x) { bad = true; x = NEG_INF; }
    }
    v[j] = x;
  }
  if (__any(bad) && lane == 0) or_relaxed(c.status, ST_NONFINITE);
  uint32_t avail = 0;  // bit j: expert lane + 64 j exists and is not yet taken
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane + 64 * j < c.E) avail |= 1u << j;
  float my_v = 0.0f, v0 = 0.0f;
  int my_e = 0;
  for (int r = 0; r < c.k; ++r) {
    float lv = NEG_INF;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((avail >> j) & 1u) lv = fmaxf(lv, v[j]);
    const float m = wave_max(lv);
    int be = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned long long hit = __ballot(((avail >> j) & 1u) && v[j] == m);
      if (be < 0 && hit) be = 64 * j + (__ffsll(hit) - 1);
    }
    if ((be & 63) == lane) avail &= ~(1u << (be >> 6));
    if (lane == r) { my_v = m; my_e = be; }
    if (r == 0) v0 = m;
  }
  float part = 0.0f;
  if (p.norm_topk) {
    if (lane < c.k) part = expf(my_v - v0);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < c.E) part += expf(v[j] - v0);
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) part = part + __shfl_xor(part, s);
  if (lane < c.k) {
    const uint32_t off = (uint32_t)(t * c.k + lane) * 4u;
    co_st32(r_ids(p), off, (uint32_t)my_e);
    co_stf(r_topw(p), off, expf(my_v - v0) / part);
    // the routed (token, slot) joins its expert's event: ev_exp[e] counts
    // arrivals up to counts[e], a wait count known only once S has run
    // (data-dependent event update).  Nothing it guards is written here
    // (G1 reads x, an input, and S's tables, ordered by S's own event), so
    // the notify needs no drain.
    if (c.set) {
      if (hist)
        atomicAdd(hist + my_e, 1);
      else
        notify_fast(p, c, ev_exp(p, c, my_e), 0xffffffffu);
      if (p.debug) atomicAdd(p.debug + my_e, 1);
    }
  }
}

// K over up to NT of a workgroup's token tiles at once (k0, k0 + G, ...,
// n of them): wave w takes token tile * kRouterT + w of each, issues the
// logit loads of all of them together and runs their selections side by
// side, so the tiles cost about one memory latency instead of one each.
// Per token the arithmetic is task_topk's: the same maximum, tie rule,
// weights and stores.  The routed pairs join their experts' events through
// the LDS histogram `hist`.
template <int NT>
__device__ __forceinline__ void task_topk_n(const MoeParams& p, const Ctx& c, int k0, int G, int n, int* hist) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float NEG_INF = -__builtin_inff();
  const rsrc_t rl = r_logits(p);
  int t[NT];
  bool live[NT];
  float v[NT][4];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    t[i] = (k0 + i * G) * kRouterT + wv;
    live[i] = i < n && t[i] < c.T;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      float x = NEG_INF;
      if (live[i] && e < c.E) {
        x = co_ldf(rl, (uint32_t)(t[i] * c.E + e) * 4u);
        if (x != x) { bad = true; x = NEG_INF; }
      }
      v[i][j] = x;
    }
  }
  if (__any(bad) && lane == 0) or_relaxed(c.status, ST_NONFINITE);
  uint32_t avail[NT];
  float my_v[NT], v0[NT];
  int my_e[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    avail[i] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < c.E) avail[i] |= 1u << j;
    my_v[i] = 0.0f;
    v0[i] = 0.0f;
    my_e[i] = 0;
  }
  for (int r = 0; r < c.k; ++r) {
    float m[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      float lv = NEG_INF;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((avail[i] >> j) & 1u) lv = fmaxf(lv, v[i][j]);
      m[i] = wave_max(lv);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      int be = -1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned long long hit = __ballot(((avail[i] >> j) & 1u) && v[i][j] == m[i]);
        if (be < 0 && hit) be = 64 * j + (__ffsll(hit) - 1);
      }
      if ((be & 63) == lane) avail[i] &= ~(1u << (be >> 6));
      if (lane == r) { my_v[i] = m[i]; my_e[i] = be; }
      if (r == 0) v0[i] = m[i];
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float part = 0.0f;
    if (p.norm_topk) {
      if (lane < c.k) part = expf(my_v[i] - v0[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j < c.E) part += expf(v[i][j] - v0[i]);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) part = part + __shfl_xor(part, s);
    if (live[i] && lane < c.k) {
      const uint32_t off = (uint32_t)(t[i] * c.k + lane) * 4u;
      co_st32(r_ids(p), off, (uint32_t)my_e[i]);
      co_stf(r_topw(p), off, expf(my_v[i] - v0[i]) / part);
      atomicAdd(hist + my_e[i], 1);
      if (p.debug) atomicAdd(p.debug + my_e[i], 1);
    }
  }
}

// N exclusive scans at once over the workgroup (one pair of barriers for
// all of them); tmp holds 4 * N ints.
template <int N>
__device__ void block_excl_scan_n(const int (&v)[N], int (&ex)[N], int (&total)[N], int* tmp) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl[N];
#pragma unroll
  for (int q = 0; q < N; ++q) incl[q] = v[q];
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const int o = __shfl_up(incl[q], s);
      if (lane >= s) incl[q] += o;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < N; ++q) tmp[wv * N + q] = incl[q];
  }
  lds_barrier();
#pragma unroll
  for (int q = 0; q < N; ++q) {
    int off = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = tmp[i * N + q];
      if (i < wv) off += x;
      tot += x;
    }
    ex[q] = off + incl[q] - v[q];
    total[q] = tot;
  }
  lds_barrier();
}

// S: counts, exp_indptr (exclusive prefix sum of counts, ends at T*k), the
// stable permutation (rows of one expert keep ascending token order) and
// the row-tile table.  One workgroup.  Tokens are taken kScanChunkT at a
// time: a per-expert token bitmap of the chunk in LDS gives each routed pair
// its rank among the same expert's earlier tokens of the chunk, and a
// per-expert running count carries the ranks across chunks, so the LDS the
// scan needs does not grow with T.  The ids are read with 128-bit loads, a
// whole chunk's in flight at once.  The slot of each pair is stored in pair
// order; perm and row_rt are indexed by grouped row, so each chunk's pairs
// are first placed in LDS by grouped position and then stored in that
// order, as runs of consecutive rows (stored in pair order they would scatter
// one row per transaction).
//
// Row tiles are numbered heaviest first: tiles of four 16-row blocks (more
// than 32 rows), then of two, then of one, each class in expert order.  The
// lists deal G1 and G2 tasks in tile order, so the longest tasks start first
// and the short ones fill in at the end (longest processing time first).
// Returns the number of row tiles (uniform over the workgroup).
//
// LOCAL: the same computation for a small batch (one chunk) into `lr`, in
// the workgroup's own LDS, with no memory written.
// PART 0: the whole scan in one task.  Large batches split it into per-chunk
// tasks: PART 1 counts chunk pch's rows per expert (into ccnt[pch]); PART 3,
// once every chunk is counted, takes the totals and the earlier chunks'
// counts from ccnt, rebuilds the prefix sums and the tile numbering (the
// same arithmetic as PART 0, so the same results) and places chunk pch's
// rows; the placement of chunk 0 also writes counts, exp_indptr, the row-tile
// count and the tile table.
template <bool LOCAL = false, bool PREFETCH = true, int PART = 0>
__device__ __forceinline__ int task_scan(const MoeParams& p, const Ctx& c, uint8_t* smem, LocalRoute* lr = nullptr,
                                         int pch = 0) {
  static_assert(PART == 0 || (!LOCAL && !PREFETCH), "the per-chunk parts use the memory tables, no prefetch");
  const int tid = threadIdx.x;
  const int E = c.E, k = c.k, n = c.T * c.k;
  const int nch = (c.T + kScanChunkT - 1) / kScanChunkT;
  const int W = (min(c.T, kScanChunkT) + 31) >> 5;  // bitmap words per expert and chunk
  // LDS at fixed offsets (sized for kMaxE), so that no table address is
  // kept in a register
  int* cnt = reinterpret_cast<int*>(smem);
  int* iptr = cnt + 260;
  int* tmp = iptr + 260;         // 32 words for the block scans
  int* tfirst = tmp + 32;        // per expert: first four-block tile | (number of them << 16)
  int* ttail = tfirst + 260;     // per expert: the tile of its last rows when that tile is smaller
  int* base = ttail + 260;       // per expert: grouped row of the chunk's grouped position 0
  // [w][e] word-major, so that thread e walking its words touches one bank
  // per lane: the chunk's token bitmap and each word's first rank
  uint32_t* bits = reinterpret_cast<uint32_t*>(base + 260);
  int* pre = reinterpret_cast<int*>(bits + kMaxE * kScanW);
  uint32_t* eid4 = reinterpret_cast<uint32_t*>(pre + kMaxE * kScanW);  // the chunk's expert ids, a byte each
  const uint8_t* eid = reinterpret_cast<const uint8_t*>(eid4);
  uint16_t* lrow = reinterpret_cast<uint16_t*>(eid4 + kScanChunkT * kMaxK / 4);  // the chunk's pairs, grouped
  const rsrc_t rids = r_ids(p);
  auto tok = [&](int f) { return f / k; };  // the token of pair f
  // Ids [g0, g1) into registers with 128-bit loads (g0 a multiple of 4),
  // every load of the batch in flight at once: one latency per batch.
  constexpr int kLd = 4;
  constexpr int kBatch = 4 * kThreads * kLd;  // ids a batch covers (a whole chunk for k <= 8)
  auto load_ids = [&](int g0, int g1, u32x4_t (&v)[kLd]) {
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      const int f = g0 + 4 * (i * kThreads + tid);
      v[i] = (u32x4_t){0u, 0u, 0u, 0u};
      if (g0 + 4 * i * kThreads >= g1) continue;  // uniform
      if (f + 4 <= g1) {
        v[i] = co_ld128(rids, (uint32_t)f * 4u);
      } else if (f < g1) {  // the last one to three ids: no load reaches past g1
        v[i].x = co_ld32(rids, (uint32_t)f * 4u);
        if (f + 1 < g1) v[i].y = co_ld32(rids, (uint32_t)(f + 1) * 4u);
        if (f + 2 < g1) v[i].z = co_ld32(rids, (uint32_t)(f + 2) * 4u);
      }
    }
  };
  // fn(e, t, ok) for each id of the batch: pair f = t * k + slot routes to
  // expert e; ok is false past g1 (then e = t = 0 and fn must change
  // nothing).  Selects, not branches, so that no per-id lane masks are kept.
  auto each_id = [&](int g0, int g1, const u32x4_t (&v)[kLd], auto&& fn) {
#pragma unroll
    for (int i = 0; i < kLd; ++i) {
      if (g0 + 4 * i * kThreads >= g1) break;  // uniform: no thread has ids from load i on
      const int f = g0 + 4 * (i * kThreads + tid);
      const uint32_t ids[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = f + j < g1;
        fn(ok ? (int)ids[j] : 0, ok ? tok(f + j) : 0, ok);
      }
    }
  };
  auto chunk_end = [&](int ch) { return min(n, (ch + 1) * kScanChunkT * k); };
  // chunk `ch`: its ids into LDS and its bitmap (bit t - ch * kScanChunkT of
  // word (w, e) is set when token t routes to expert e); `v` holds the
  // chunk's first batch when `loaded`
  auto build_bits = [&](int ch, u32x4_t (&v)[kLd], bool loaded) {
    const int f0 = ch * kScanChunkT * k, f1 = chunk_end(ch);
    if (tid < E)
      for (int w = 0; w < W; ++w) bits[w * kMaxE + tid] = 0u;
    lds_barrier();  // the bitmap is clear before the ors
    for (int g0 = f0; g0 < f1; g0 += kBatch) {
      const int g1 = min(f1, g0 + kBatch);
      if (g0 != f0 || !loaded) load_ids(g0, g1, v);
#pragma unroll
      for (int i = 0; i < kLd; ++i) {
        const int f = g0 + 4 * (i * kThreads + tid);
        if (f < g1)  // f0 and g0 are multiples of 4: one word a load
          eid4[(f - f0) >> 2] = (v[i].x & 0xffu) | ((v[i].y & 0xffu) << 8) | ((v[i].z & 0xffu) << 16) | (v[i].w << 24);
      }
      each_id(g0, g1, v, [&](int e, int t, bool ok) {
        const int tl = ok ? t - ch * kScanChunkT : 0;
        atomicOr(&bits[(tl >> 5) * kMaxE + e], ok ? 1u << (tl & 31) : 0u);
      });
    }
    lds_barrier();
  };
  // PREFETCH: the next chunk's first batch of ids is loaded while the
  // current chunk is stored (sixteen more registers held across the chunk)
  u32x4_t v[kLd];
  if constexpr (PART == 1) {
    build_bits(pch, v, false);
    if (tid < E) {
      int run = 0;
      for (int w = 0; w < W; ++w) run += __popc(bits[w * kMaxE + tid]);
      co_st32(r_ccnt(p), (uint32_t)(pch * E + tid) * 4u, (uint32_t)run);
    }
    return 0;
  }
  int runch = 0;  // PART 3: thread e's rows in the chunks before pch
  const bool outputs = PART != 3 || pch == 0;  // this task writes the routing outputs
  if (PART == 3) {
    if (tid < E) {
      const rsrc_t rcc = r_ccnt(p);
      int tot = 0;
      for (int q0 = 0; q0 < nch; q0 += 8) {  // eight loads in flight at a time
        int cv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) cv[u] = q0 + u < nch ? (int)co_ld32(rcc, (uint32_t)((q0 + u) * E + tid) * 4u) : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          tot += cv[u];
          runch += q0 + u < pch ? cv[u] : 0;
        }
      }
      cnt[tid] = tot;
    }
  } else if (nch == 1) {  // one chunk: the counts come from its bitmap
    build_bits(0, v, false);
    if (tid < E) {
      int run = 0;
      for (int w = 0; w < W; ++w) run += __popc(bits[w * kMaxE + tid]);
      cnt[tid] = run;
    }
  } else if (c.set) {
    // several chunks with events on: S runs after every top-k task, whose
    // arrivals on expert e's event count exactly the pairs routed to e
    if (PREFETCH) load_ids(0, chunk_end(0), v);
    if (tid < E) cnt[tid] = (int)ld_relaxed(ev_exp(p, c, tid));
  } else {
    if (tid < E) cnt[tid] = 0;
    lds_barrier();
    for (int g0 = 0; g0 < n; g0 += kBatch) {
      const int g1 = min(n, g0 + kBatch);
      load_ids(g0, g1, v);
      each_id(g0, g1, v, [&](int e, int, bool ok) { atomicAdd(&cnt[e], ok ? 1 : 0); });
    }
    if (PREFETCH) load_ids(0, chunk_end(0), v);
  }
  lds_barrier();
  const int my = tid < E ? cnt[tid] : 0;
  // Row tiles of bm rows.  Tiles of up to kBM rows are numbered by size
  // class (tiles of 33 to 64 rows first, then 17 to 32, then 1 to 16, each
  // class by expert); big tiles are numbered by expert only.
  const int bm = c.bm;
  const bool big = bm != kBM;
  const int mytiles = (my + bm - 1) / bm;
  const int rem = my % bm;
  const int n4 = big ? mytiles : my / kBM + (rem > 32 ? 1 : 0), n2 = (!big && rem > 16 && rem <= 32) ? 1 : 0,
            n1 = (!big && rem > 0 && rem <= 16) ? 1 : 0;
  const int sv[5] = {my, mytiles, n4, n2, n1};
  int sx[5], st[5];
  block_excl_scan_n<5>(sv, sx, st, tmp);
  const int ex = sx[0], ex4 = sx[2], ex2 = sx[3], ex1 = sx[4];
  const int tot_rows = st[0], tot_tiles = st[1], tot4 = st[2], tot2 = st[3];
  const rsrc_t rc = r_counts(p), ri = r_indptr(p);
  if (tid < E) {
    iptr[tid] = ex;
    tfirst[tid] = ex4 | (n4 << 16);
    ttail[tid] = (big || rem > 32) ? -1 : (rem > 16 ? tot4 + ex2 : tot4 + tot2 + ex1);
    if (LOCAL) {
      lr->cnt[tid] = (uint16_t)my;
    } else if (outputs) {
      co_st32(rc, (uint32_t)tid * 4u, (uint32_t)my);
      co_st32(ri, (uint32_t)tid * 4u, (uint32_t)ex);
    }
  }
  if (!LOCAL && outputs && tid < E && c.set && p.debug) {
    // every routed pair has notified by now (S runs after all of K): the
    // expert event holds exactly counts[e] arrivals and fires once
    if (my > 0 && ld_relaxed(ev_exp(p, c, tid)) == (uint32_t)my) atomicAdd(p.debug + E + tid, 1);
  }
  if (tid == 0) {
    iptr[E] = tot_rows;
    if (!LOCAL && outputs) {
      co_st32(ri, (uint32_t)E * 4u, (uint32_t)tot_rows);
      st_relaxed(p.meta + M_NRT, (uint32_t)tot_tiles);
    }
  }
  lds_barrier();
  if constexpr (LOCAL) {
    // one chunk: grouped row of a pair = iptr[e] + rank among e's tokens
    if (tid < E) {
      int r = ex;
      for (int w = 0; w < W; ++w) {
        pre[w * kMaxE + tid] = r;
        r += __popc(bits[w * kMaxE + tid]);
      }
    }
    lds_barrier();
    for (int f = tid; f < n; f += kThreads) {
      const int e = eid[f];
      const int tl = tok(f);
      const int i = (tl >> 5) * kMaxE + e;
      lr->perm[pre[i] + __popc(bits[i] & ((1u << (tl & 31)) - 1u))] = (uint16_t)f;
    }
  } else {
    const rsrc_t rs = r_slot(p), rp = r_perm(p), rrt = r_rowrt(p);
    int run = runch;  // thread e: rows of expert e in earlier chunks
    const int ch_lo = PART == 3 ? pch : 0, ch_hi = PART == 3 ? pch + 1 : nch;
    for (int ch = ch_lo; ch < ch_hi; ++ch) {
      if (nch > 1) build_bits(ch, v, PREFETCH);
      const int f0 = ch * kScanChunkT * k, f1 = chunk_end(ch);
      if (PREFETCH && ch + 1 < nch) load_ids(f1, chunk_end(ch + 1), v);  // in flight while this chunk is stored
      // The chunk's pairs in grouped order (expert, then token) get positions
      // 0, 1, ...; thread e numbers its words from the chunk's earlier
      // experts on, and expert e's rows of this chunk follow its rows of the
      // earlier chunks.
      int ce = 0;
      if (tid < E) {
        for (int w = 0; w < W; ++w) {
          pre[w * kMaxE + tid] = ce;
          ce += __popc(bits[w * kMaxE + tid]);
        }
      }
      const int cv[1] = {ce};
      int cx[1], ct[1];
      block_excl_scan_n<1>(cv, cx, ct, tmp);
      if (tid < E) {
        for (int w = 0; w < W; ++w) pre[w * kMaxE + tid] += cx[0];
        base[tid] = ex + run - cx[0];
        run += ce;
      }
      lds_barrier();
      // pair order: the slot of each pair (a contiguous store) and the pair
      // at each grouped position, in LDS; four pairs a thread at a time so
      // that their LDS round trips overlap
      for (int fa = f0 + tid; fa < f1; fa += 4 * kThreads) {
        int e[4], tl[4], q[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int f = fa + u * kThreads;
          e[u] = f < f1 ? eid[f - f0] : 0;
          tl[u] = f < f1 ? tok(f) - ch * kScanChunkT : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = (tl[u] >> 5) * kMaxE + e[u];
          q[u] = pre[i] + __popc(bits[i] & ((1u << (tl[u] & 31)) - 1u));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int f = fa + u * kThreads;
          if (f < f1) {
            lrow[q[u]] = (uint16_t)(f - f0);
            co_st32(rs, (uint32_t)f * 4u, (uint32_t)(base[e[u]] + q[u]));
          }
        }
      }
      lds_barrier();
      // grouped order: perm and row_rt of consecutive rows go out as runs
      const int np = f1 - f0;
      for (int qa = tid; qa < np; qa += 4 * kThreads) {
        int fl[4], e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) fl[u] = qa + u * kThreads < np ? lrow[qa + u * kThreads] : 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = eid[fl[u]];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = qa + u * kThreads;
          if (q < np) {
            const int s = base[e[u]] + q;
            co_st32(rp, (uint32_t)s * 4u, (uint32_t)(f0 + fl[u]));
            const int mt = (s - iptr[e[u]]) / bm, tf = tfirst[e[u]];  // the row's tile, numbered as below
            co_st32(rrt, (uint32_t)s * 4u, (uint32_t)(mt < (tf >> 16) ? (tf & 0xffff) + mt : ttail[e[u]]));
          }
        }
      }
      lds_barrier();  // this chunk's LDS tables are read before the next chunk rebuilds them
    }
  }
  const rsrc_t rr = r_rtinfo(p);
  if (tid < E && outputs) {
    for (int mt = 0; mt * bm < my; ++mt) {
      const int rows = min(bm, my - mt * bm);
      const int rt = (big || rows > 32) ? ex4 + mt : (rows > 16 ? tot4 + ex2 : tot4 + tot2 + ex1);
      if (LOCAL) {
        lr->tile[rt] = (uint32_t)tid | ((uint32_t)rows << 9) | ((uint32_t)(ex + mt * bm) << 16);
        continue;
      }
      u32x4_t q;
      q.x = (uint32_t)tid;
      q.y = (uint32_t)(ex + mt * bm);
      q.z = (uint32_t)rows;
      q.w = 0u;
      co_st128(rr, (uint32_t)rt * 16u, q);
    }
  }
  if (LOCAL) lds_barrier();  // the tables are read by every thread next
  return tot_tiles;
}

// Grouped-GEMM tasks.  A row tile holds up to kBM = 64 grouped rows of one
// expert: NB = 1, 2 or 4 row blocks of 16 (three round up to four).  The 4
// waves always split K in quarters, and each wave multiplies every row block
// of the tile with the same weight fragment, so a weight byte is loaded once
// per task and feeds up to four MFMA row blocks (a decode tile has one block;
// a prefill tile of a hot expert has four).  The per-wave partial sums are
// reduced in LDS in wave order, block by block.
__device__ __forceinline__ int row_blocks(int nrows) { return nrows <= 16 ? 1 : (nrows <= 32 ? 2 : 4); }

// G1: one row tile of expert e times 16 gate and 16 up columns of W13,
// SwiGLU, Hmid = bf16(silu(g) * u).  bf16 MFMA 16x16x32 with fp32
// accumulation; the weight slab (2 x 16 rows x H) streams from HBM straight
// into registers; rows past the expert's count are zero-filled, never loaded.
// The A rows are gathered from x itself: grouped row r of the tile is token
// perm[r] / k (the dispatch is fused into this load), and x is never written
// during a launch, so ordinary cached loads serve.  `tok` holds, per lane,
// the token of row 16 b + (lane % 16) of each row block when the caller has
// loaded them ahead; otherwise they are loaded here.
__device__ __forceinline__ uint32_t row_perm(const MoeParams& p, const RowTile tile, int b,
                                             const LocalRoute* lr = nullptr) {
  const int r = b * 16 + (threadIdx.x & 15);
  if (r >= tile.nrows) return 0u;
  return lr ? (uint32_t)lr->perm[tile.r0 + r] : co_ld32(r_perm(p), (uint32_t)(tile.r0 + r) * 4u);
}
template <int NB, int U, int CB, bool PIPE = true>
__device__ __forceinline__ void g1_body(const MoeParams& p, const Ctx& c, const RowTile tile, int nt, float* red,
                                        const uint32_t* pre) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = lane & 15, kg = lane >> 4;
  const int H = c.H, I = c.I;
  const int kw = H >> 2;
  const int nsteps = kw >> 5;
  constexpr int BN = 16 * CB;  // gate (and up) columns of the tile
  bool valid[NB];
  const uint16_t* pa[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int r = b * 16 + m;
    valid[b] = r < tile.nrows;
    const uint32_t f = pre ? pre[b] : row_perm(p, tile, b);
    const int t = valid[b] ? (int)(f / (uint32_t)c.k) : 0;
    pa[b] = p.x + (size_t)t * H + wv * kw + kg * 8;
  }
  const uint16_t* pg = p.w13 + ((size_t)tile.e * 2 * I + (size_t)nt * BN + m) * H + wv * kw + kg * 8;
  const uint16_t* pu = pg + (size_t)I * H;
  const size_t cbs = (size_t)16 * H;  // next 16-column block of W13
  f32x4_t accg[NB][CB], accu[NB][CB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q = 0; q < CB; ++q) accg[b][q] = accu[b][q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  if (PIPE && nsteps % U == 0) {
    // Rolling pipeline over U register slots: the loads of step s + U go
    // into slot s % U as soon as step s has been multiplied, so each wave
    // keeps U - 1 to U steps of loads in flight the whole time rather than
    // draining a batch before issuing the next (workgroups that start their
    // tasks together then keep the memory system busy).  Rows past the count
    // load row 0 (a valid token row): MFMA output rows depend only on their
    // own A rows, and those output rows are never stored.
    u32x4_t a[U][NB], bg[U][CB], bu[U][CB];
    auto issue = [&](int u, int st) {
      const int k0 = st * 32;
#pragma unroll
      for (int b = 0; b < NB; ++b) a[u][b] = ld4(pa[b] + k0);
#pragma unroll
      for (int q = 0; q < CB; ++q) {
        bg[u][q] = ld4(pg + q * cbs + k0);
        bu[u][q] = ld4(pu + q * cbs + k0);
      }
    };
    auto mma = [&](int u) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < CB; ++q) {
          accg[b][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u][b]), as_bf(bg[u][q]), accg[b][q], 0, 0, 0);
          accu[b][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u][b]), as_bf(bu[u][q]), accu[b][q], 0, 0, 0);
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) issue(u, u);
    for (int s0 = U; s0 < nsteps; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        mma(u);
        issue(u, s0 + u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mma(u);
  } else
  // batches of U k-steps ((NB + 2 CB) * U loads of 16 bytes a lane in
  // flight); two workgroups per CU overlap each other's batch boundaries
  for (int s0 = 0; s0 < nsteps; s0 += U) {
    u32x4_t a[U][NB], bg[U][CB], bu[U][CB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < nsteps) {
        const int k0 = (s0 + u) * 32;
#pragma unroll
        for (int b = 0; b < NB; ++b) a[u][b] = valid[b] ? ld4(pa[b] + k0) : zero;
#pragma unroll
        for (int q = 0; q < CB; ++q) {
          bg[u][q] = ld4(pg + q * cbs + k0);
          bu[u][q] = ld4(pu + q * cbs + k0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < nsteps) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int q = 0; q < CB; ++q) {
            accg[b][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u][b]), as_bf(bg[u][q]), accg[b][q], 0, 0, 0);
            accu[b][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u][b]), as_bf(bu[u][q]), accu[b][q], 0, 0, 0);
          }
      }
    }
  }
  const int tid = threadIdx.x;
  // element (lane', i) of a 16x16 MFMA result: row 4*(lane'/16) + i, column lane' % 16
  const int ol = tid >> 2, oi = tid & 3;
  const int row = 4 * (ol >> 4) + oi, col = ol & 15;
  uint16_t* stage = reinterpret_cast<uint16_t*>(red + 4096);  // [64 rows][BN cols] bf16
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    // cross-wave reduction: red[w][q][0 = gate, 1 = up][lane * 4 + i]; the
    // first barrier keeps earlier readers of `red` ahead of these writes
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CB; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[((wv * CB + q) * 2 + 0) * 256 + lane * 4 + i] = accg[b][q][i];
        red[((wv * CB + q) * 2 + 1) * 256 + lane * 4 + i] = accu[b][q][i];
      }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CB; ++q) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        g += red[((w * CB + q) * 2 + 0) * 256 + tid];
        u += red[((w * CB + q) * 2 + 1) * 256 + tid];
      }
      stage[(b * 16 + row) * BN + q * 16 + col] = (uint16_t)f2bf(g / (1.0f + __expf(-g)) * u);
    }
  }
  __syncthreads();
  // wave 0 alone writes the tile (rows x 2 BN bytes, 16-byte chunks), so
  // only wave 0 has stores to drain before the notify
  if (tid < 64) {
    constexpr int cpr = BN / 8;
#pragma unroll
    for (int h = 0; h < cpr; ++h) {
      const int idx = tid + 64 * h;
      const int r = idx / cpr, q8 = idx % cpr;
      if (r < tile.nrows) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * BN + q8 * 8);
        co_st128(r_hh(p), (uint32_t)(((size_t)(tile.r0 + r) * I + nt * BN + q8 * 8) * 2), v);
      }
    }
  }
}

// G1 for large batches, 64-column tiles (c.bn1 = 64): the four waves split
// the columns instead of K.  Wave w owns gate columns nt * 64 + 16 w .. + 16
// and the same up columns over all of H, so it holds complete dot products
// (no cross-wave reduction).  The tile's A rows (up to 64 gathered x rows)
// are shared through LDS: they are staged 128 k at a time (wave b stages
// row block b, with the row's token from `pre`), double buffered, so each x
// row is read from memory once per 64 columns.  Rows are padded to 272
// bytes so that the 16 rows of an MFMA fragment read fall in distinct
// banks.  The next chunk's A rows and weights are loaded while the current
// chunk multiplies; the barrier that ends a chunk orders LDS only.
constexpr int kCsKC = 128;                  // k per staged chunk (4 MFMA k-steps)
constexpr int kCsRowB = kCsKC * 2 + 16;     // bytes per staged row
template <int NB>
__device__ __forceinline__ void g1_cs_body(const MoeParams& p, const Ctx& c, const RowTile tile, int nt, float* red,
                                           const uint32_t* pre) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = lane & 15, kg = lane >> 4;
  const int H = c.H, I = c.I;
  const int nch = H / kCsKC;
  uint8_t* lds = reinterpret_cast<uint8_t*>(red);  // two [64][kCsRowB] A buffers, then the output stage
  // A staging: wave b (< NB) loads row block b; lane (m, kg) loads 16-byte
  // column groups kg, kg + 4, kg + 8, kg + 12 of row 16 b + m
  const bool stager = wv < NB;
  const int srow = wv * 16 + m;
  // this wave's row block's entry of pre[], blended with masks (an indexed
  // pick would put the array on the stack)
  const uint32_t f = (pre[0] & (0u - (uint32_t)(wv == 0))) | (pre[1] & (0u - (uint32_t)(wv == 1))) |
                     (pre[2] & (0u - (uint32_t)(wv == 2))) | (pre[3] & (0u - (uint32_t)(wv == 3)));
  const int stok = (stager && srow < tile.nrows) ? (int)(f / (uint32_t)c.k) : 0;  // rows past the count: any row
  const uint16_t* sa = p.x + (size_t)stok * H + kg * 8;
  const uint16_t* pg = p.w13 + ((size_t)tile.e * 2 * I + (size_t)nt * 64 + wv * 16 + m) * H + kg * 8;
  const uint16_t* pu = pg + (size_t)I * H;
  f32x4_t accg[NB], accu[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) accg[b] = accu[b] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  u32x4_t ar[4], bc[4][2], bn[4][2];
  auto load_a = [&](int j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = ld4(sa + j * kCsKC + i * 32);
  };
  auto store_a = [&](int buf) {
    uint8_t* dst = lds + buf * 64 * kCsRowB + srow * kCsRowB + kg * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(dst + i * 64) = ar[i];
  };
  auto load_b = [&](int j, u32x4_t (&bb)[4][2]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bb[s][0] = ld4(pg + j * kCsKC + s * 32);
      bb[s][1] = ld4(pu + j * kCsKC + s * 32);
    }
  };
  if (stager) load_a(0);
  load_b(0, bc);
  if (stager) store_a(0);
  lds_barrier();
  for (int j = 0; j < nch; ++j) {
    const bool more = j + 1 < nch;
    if (more) {
      if (stager) load_a(j + 1);
      load_b(j + 1, bn);
    }
    const uint8_t* src = lds + (j & 1) * 64 * kCsRowB + m * kCsRowB + kg * 16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(src + b * 16 * kCsRowB + s * 64);
        accg[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a), as_bf(bc[s][0]), accg[b], 0, 0, 0);
        accu[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a), as_bf(bc[s][1]), accu[b], 0, 0, 0);
      }
    }
    if (more && stager) store_a((j + 1) & 1);
    lds_barrier();  // the next chunk is staged; this chunk's buffer is free again
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bc[s][0] = bn[s][0];
      bc[s][1] = bn[s][1];
    }
  }
  // SwiGLU into the output stage [64 rows][64 cols] bf16 (the A buffers are
  // free: every wave passed the last chunk's barrier)
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds);
  const int col = wv * 16 + (lane & 15);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = accg[b][i], u = accu[b][i];
      stage[(b * 16 + 4 * (lane >> 4) + i) * 64 + col] = (uint16_t)f2bf(g / (1.0f + __expf(-g)) * u);
    }
  __syncthreads();
  // wave 0 alone writes the tile (rows x 128 bytes, 16-byte chunks), so only
  // wave 0 has stores to drain before the notify
  if (threadIdx.x < 64) {
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const int idx = threadIdx.x + 64 * h;
      const int r = idx >> 3, q8 = idx & 7;
      if (r < tile.nrows) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * 64 + q8 * 8);
        co_st128(r_hh(p), (uint32_t)(((size_t)(tile.r0 + r) * I + nt * 64 + q8 * 8) * 2), v);
      }
    }
  }
}

#include "big_tiles.h"

// k-steps per load batch (U) by row blocks, measured on MI355X: short
// batches stream better in the persistent kernel (two workgroups per CU);
// the separate G kernels of the kernel-by-kernel launch keep longer batches
// for four-block tiles, where they are faster there.  Tiles twice as wide
// (c.bn1 = 32: large batches, where a four-block tile's gathered x rows
// outweigh its weights) read each tile's x rows once for 32 gate and 32 up
// columns instead of 16.
template <bool KBK = false, int WIDE = kVarWide>
__device__ __forceinline__ void task_g1(const MoeParams& p, const Ctx& c, const RowTile tile, int rt, int nt, float* red,
                        const uint32_t* pre = nullptr) {
  (void)rt;
  // the rolling load pipeline in the small-batch persistent variant (the
  // separate G kernels, three workgroups a CU, measured faster without it)
  constexpr bool PIPE = !KBK && WIDE == kVarSmall;
  if constexpr (WIDE == kVarBig) {
    big_body<true>(p, c, tile, nt, reinterpret_cast<uint8_t*>(red));
    return;
  }
  if (WIDE && c.bn1 == 4 * kBN1) {
    // column-split tiles need their row tokens per row block: load them
    // here when the caller has not
    uint32_t f[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) f[b] = pre ? pre[b] : row_perm(p, tile, b);
    switch (row_blocks(tile.nrows)) {
      case 1: g1_cs_body<1>(p, c, tile, nt, red, f); break;
      case 2: g1_cs_body<2>(p, c, tile, nt, red, f); break;
      default: g1_cs_body<4>(p, c, tile, nt, red, f); break;
    }
    return;
  }
  if (c.bn1 == 2 * kBN1) {  // mid-size batches: 32 gate + 32 up columns, K-split
    switch (row_blocks(tile.nrows)) {
      case 1: g1_body<1, 2, 2, PIPE>(p, c, tile, nt, red, pre); break;
      case 2: g1_body<2, 2, 2, PIPE>(p, c, tile, nt, red, pre); break;
      default: g1_body<4, 1, 2, PIPE>(p, c, tile, nt, red, pre); break;
    }
    return;
  }
  switch (row_blocks(tile.nrows)) {
    case 1: g1_body<1, 4, 1, PIPE>(p, c, tile, nt, red, pre); break;
    case 2: g1_body<2, 4, 1, PIPE>(p, c, tile, nt, red, pre); break;
    default: g1_body<4, KBK ? 4 : 2, 1, PIPE>(p, c, tile, nt, red, pre); break;
  }
}

// G2: one row tile times kBN2 output columns of Wd[e]: Y = bf16(Hmid Wd^T).
// K = I split in quarters over the waves; each wave keeps kBN2 / 16 column blocks
// for every row block.
template <int NB, int U, bool PIPE = true>
__device__ __forceinline__ void g2_body(const MoeParams& p, const Ctx& c, const RowTile tile, int nt2, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = lane & 15, kg = lane >> 4;
  const int H = c.H, I = c.I;
  const int kw = I >> 2;
  const int nsteps = kw >> 5;
  const rsrc_t rh = r_hh(p);
  bool valid[NB];
  uint32_t aoff[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int r = b * 16 + m;
    valid[b] = r < tile.nrows;
    aoff[b] = (uint32_t)(((size_t)(tile.r0 + (valid[b] ? r : 0)) * I + wv * kw + kg * 8) * 2);
  }
  const uint16_t* pb = p.w2 + ((size_t)tile.e * H + (size_t)nt2 * kBN2 + m) * I + wv * kw + kg * 8;
  const size_t cbs = (size_t)16 * I;  // next 16-column block of Wd
  f32x4_t acc[NB][kCB2];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q = 0; q < kCB2; ++q) acc[b][q] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  if (PIPE && nsteps % U == 0) {
    // rolling pipeline over U register slots, as in g1_body (rows past the
    // count load the tile's first row; their output rows are not stored)
    u32x4_t a[U][NB], bb[U][kCB2];
    auto issue = [&](int u, int st) {
      const int ks = st;
#pragma unroll
      for (int b = 0; b < NB; ++b) a[u][b] = co_ld128(rh, aoff[b] + (uint32_t)ks * 64u);
#pragma unroll
      for (int q = 0; q < kCB2; ++q) bb[u][q] = ld4(pb + q * cbs + ks * 32);
    };
    auto mma = [&](int u) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int q = 0; q < kCB2; ++q)
          acc[b][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u][b]), as_bf(bb[u][q]), acc[b][q], 0, 0, 0);
    };
#pragma unroll
    for (int u = 0; u < U; ++u) issue(u, u);
    for (int s0 = U; s0 < nsteps; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        mma(u);
        issue(u, s0 + u);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mma(u);
  } else
  for (int s0 = 0; s0 < nsteps; s0 += U) {
    u32x4_t a[U][NB], bb[U][kCB2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < nsteps) {
        const int ks = s0 + u;
#pragma unroll
        for (int b = 0; b < NB; ++b) a[u][b] = valid[b] ? co_ld128(rh, aoff[b] + (uint32_t)ks * 64u) : zero;
#pragma unroll
        for (int q = 0; q < kCB2; ++q) bb[u][q] = ld4(pb + q * cbs + ks * 32);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < nsteps) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int q = 0; q < kCB2; ++q)
            acc[b][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u][b]), as_bf(bb[u][q]), acc[b][q], 0, 0, 0);
      }
    }
  }
  const int tid = threadIdx.x;
  const int ol = tid >> 2, oi = tid & 3;
  const int row = 4 * (ol >> 4) + oi, col = ol & 15;
  uint16_t* stage = reinterpret_cast<uint16_t*>(red + 4 * kCB2 * 256);  // [64 rows][kBN2 cols] bf16
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCB2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wv * kCB2 + q) * 256 + lane * 4 + i] = acc[b][q][i];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kCB2; ++q) {
      float y = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) y += red[(w * kCB2 + q) * 256 + tid];
      stage[(b * 16 + row) * kBN2 + q * 16 + col] = (uint16_t)f2bf(y);
    }
  }
  __syncthreads();
  // wave 0 alone writes the tile (rows x kBN2 * 2 bytes, 16-byte chunks)
  if (tid < 64) {
    constexpr int cpr = kBN2 / 8;
    const int nchunks = tile.nrows * cpr;
    for (int idx = tid; idx < nchunks; idx += 64) {
      const int r = idx / cpr, q = idx % cpr;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * kBN2 + q * 8);
      co_st128(r_y(p), (uint32_t)(((size_t)(tile.r0 + r) * H + nt2 * kBN2 + q * 8) * 2), v);
    }
  }
}

// G2 for large batches, 128-column tiles (c.bn2 = 128): as g1_cs_body, the
// waves split the columns (wave w owns output columns nt2 * 128 + 32 w ..
// + 32, two MFMA column blocks, over all of I) and share the tile's Hmid
// rows through LDS, staged 128 k at a time with device-coherent loads (G1
// tasks of other workgroups wrote them), so each Hmid row is read once per
// 128 output columns instead of 64.
template <int NB>
__device__ __forceinline__ void g2_cs_body(const MoeParams& p, const Ctx& c, const RowTile tile, int nt2, float* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = lane & 15, kg = lane >> 4;
  const int H = c.H, I = c.I;
  const int nch = I / kCsKC;
  uint8_t* lds = reinterpret_cast<uint8_t*>(red);  // two [64][kCsRowB] A buffers, then the output stage
  const rsrc_t rh = r_hh(p);
  const bool stager = wv < NB;
  const int srow = wv * 16 + m;
  const int grow = tile.r0 + (srow < tile.nrows ? srow : 0);  // rows past the count: any row of the tile
  const uint32_t sa = (uint32_t)(((size_t)grow * I + kg * 8) * 2);
  const uint16_t* pb = p.w2 + ((size_t)tile.e * H + (size_t)nt2 * 128 + wv * 32 + m) * I + kg * 8;
  const size_t cbs = (size_t)16 * I;  // the wave's second 16-column block of Wd
  f32x4_t acc[NB][2];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b][0] = acc[b][1] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  u32x4_t ar[4], bc[4][2], bn[4][2];
  auto load_a = [&](int j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = co_ld128(rh, sa + (uint32_t)(j * kCsKC + i * 32) * 2u);
  };
  auto store_a = [&](int buf) {
    uint8_t* dst = lds + buf * 64 * kCsRowB + srow * kCsRowB + kg * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4_t*>(dst + i * 64) = ar[i];
  };
  auto load_b = [&](int j, u32x4_t (&bb)[4][2]) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      bb[s2][0] = ld4(pb + j * kCsKC + s2 * 32);
      bb[s2][1] = ld4(pb + cbs + j * kCsKC + s2 * 32);
    }
  };
  if (stager) load_a(0);
  load_b(0, bc);
  if (stager) store_a(0);
  lds_barrier();
  for (int j = 0; j < nch; ++j) {
    const bool more = j + 1 < nch;
    if (more) {
      if (stager) load_a(j + 1);
      load_b(j + 1, bn);
    }
    const uint8_t* src = lds + (j & 1) * 64 * kCsRowB + m * kCsRowB + kg * 16;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(src + b * 16 * kCsRowB + s2 * 64);
        acc[b][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a), as_bf(bc[s2][0]), acc[b][0], 0, 0, 0);
        acc[b][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a), as_bf(bc[s2][1]), acc[b][1], 0, 0, 0);
      }
    }
    if (more && stager) store_a((j + 1) & 1);
    lds_barrier();  // the next chunk is staged; this chunk's buffer is free again
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      bc[s2][0] = bn[s2][0];
      bc[s2][1] = bn[s2][1];
    }
  }
  // Y in bf16 into the output stage [64 rows][128 cols] (the A buffers are free)
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stage[(b * 16 + 4 * (lane >> 4) + i) * 128 + wv * 32 + q * 16 + (lane & 15)] = (uint16_t)f2bf(acc[b][q][i]);
  __syncthreads();
  // wave 0 alone writes the tile (rows x 256 bytes, 16-byte chunks)
  if (threadIdx.x < 64) {
    for (int idx = threadIdx.x; idx < tile.nrows * 16; idx += 64) {
      const int r = idx >> 4, q8 = idx & 15;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + r * 128 + q8 * 8);
      co_st128(r_y(p), (uint32_t)(((size_t)(tile.r0 + r) * H + nt2 * 128 + q8 * 8) * 2), v);
    }
  }
}

template <bool KBK = false, int WIDE = kVarWide>
__device__ __forceinline__ void task_g2(const MoeParams& p, const Ctx& c, const RowTile tile, int rt, int nt2, float* red) {
  constexpr bool PIPE = !KBK && WIDE == kVarSmall;  // as in task_g1
  if constexpr (WIDE == kVarBig) {
    big_body<false>(p, c, tile, nt2, reinterpret_cast<uint8_t*>(red));
    return;
  }
  (void)rt;
  if (WIDE && c.bn2 == 2 * kBN2) {
    switch (row_blocks(tile.nrows)) {
      case 1: g2_cs_body<1>(p, c, tile, nt2, red); break;
      case 2: g2_cs_body<2>(p, c, tile, nt2, red); break;
      default: g2_cs_body<4>(p, c, tile, nt2, red); break;
    }
    return;
  }
  switch (row_blocks(tile.nrows)) {
    case 1: g2_body<1, 2, PIPE>(p, c, tile, nt2, red); break;
    case 2: g2_body<2, 2, PIPE>(p, c, tile, nt2, red); break;
    default: g2_body<4, KBK ? 2 : 1, PIPE>(p, c, tile, nt2, red); break;
  }
}

// C: out[t, :] = bf16(sum_j w[t, j] * Y[slot[t*k+j], :]), fp32 in j order.
// The task's (weight, slot) pairs are staged in LDS first; then each thread
// issues the loads of all k expert rows of its chunk before the arithmetic.
// The weighted sums of a list of ntok tokens: tok(n) gives list entry n's
// token (or -1 past the end), s_pair[2 (n k + j)] and [2 (n k + j) + 1]
// the weight and grouped row of its j-th routed row.  IB items (entry,
// 8-column chunk) a thread at a time, JB of each item's k rows requested
// together: IB * JB = 8 row loads in flight (one item of 8 rows for k >= 8,
// eight items of one row for k = 1; combine_items picks by k).  Each item
// sums its rows in ascending slot order.
template <int IB, int JB, class Tok>
__device__ __forceinline__ void combine_items_t(const MoeParams& p, const Ctx& c, int ntok, Tok tok, const int* s_pair) {
  const int cpr = c.H >> 3;
  const int k = c.k;
  const rsrc_t ry = r_y(p);
  const int nit = ntok * cpr;
  for (int i0 = threadIdx.x; i0 < nit; i0 += IB * kThreads) {
    int r[IB], ch[IB], t[IB];
    bool ok[IB];
    float acc[IB][8];
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      const int idx = i0 + b * kThreads;
      const int ii = idx < nit ? idx : i0;
      r[b] = ii / cpr;
      ch[b] = ii - r[b] * cpr;
      t[b] = tok(r[b]);
      ok[b] = idx < nit && t[b] >= 0;
      if (!ok[b]) {  // a valid row and chunk to read (nothing is stored)
        r[b] = 0;
        ch[b] = 0;
        t[b] = tok(0);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[b][q] = 0.f;
    }
    // Every lane loads (items past the end read entry 0's rows, whose pairs
    // are valid), so that only the uniform row-count test guards the
    // loads: a per-lane test there costs a branch and a wait per load.
    u32x4_t rvv[IB];
    if (p.resid) {
      // decoder layer: the residual stream's rows go out with the first loads
      const rsrc_t rr = make_rsrc(p.resid, p.resid_bytes);
#pragma unroll
      for (int b = 0; b < IB; ++b) rvv[b] = co_ld128(rr, (uint32_t)(((size_t)t[b] * c.H + ch[b] * 8) * 2));
    }
    for (int j0 = 0; j0 < k; j0 += JB) {
      u32x4_t yv[IB][JB];
#pragma unroll
      for (int b = 0; b < IB; ++b)
#pragma unroll
        for (int u = 0; u < JB; ++u)
          if (j0 + u < k)
            yv[b][u] = co_ld128(ry, (uint32_t)(((size_t)s_pair[2 * (r[b] * k + j0 + u) + 1] * c.H + ch[b] * 8) * 2));
#pragma unroll
      for (int b = 0; b < IB; ++b)
#pragma unroll
        for (int u = 0; u < JB; ++u) {
          if (j0 + u < k) {
            const float wj = __int_as_float(s_pair[2 * (r[b] * k + j0 + u)]);
            float yf[8];
            unpack8(yv[b][u], yf);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[b][q] = __builtin_fmaf(wj, yf[q], acc[b][q]);
          }
        }
    }
#pragma unroll
    for (int b = 0; b < IB; ++b) {
      if (!ok[b]) continue;
      if (p.resid) {
        // decoder layer: out = bf16(x2 + bf16(MoE sum)), x2 the residual stream
        float rv[8];
        unpack8(rvv[b], rv);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[b][q] = rv[q] + __uint_as_float(f2bf(acc[b][q]) << 16);
      }
      u32x4_t o;
      o.x = f2bf(acc[b][0]) | (f2bf(acc[b][1]) << 16);
      o.y = f2bf(acc[b][2]) | (f2bf(acc[b][3]) << 16);
      o.z = f2bf(acc[b][4]) | (f2bf(acc[b][5]) << 16);
      o.w = f2bf(acc[b][6]) | (f2bf(acc[b][7]) << 16);
      st4(p.out + (size_t)t[b] * c.H + ch[b] * 8, o);
    }
  }
}
template <class Tok>
__device__ __forceinline__ void combine_items(const MoeParams& p, const Ctx& c, int ntok, Tok tok, const int* s_pair) {
  if (c.k >= 8)
    combine_items_t<2, 8>(p, c, ntok, tok, s_pair);
  else if (c.k >= 4)
    combine_items_t<2, 4>(p, c, ntok, tok, s_pair);
  else if (c.k >= 2)
    combine_items_t<4, 2>(p, c, ntok, tok, s_pair);
  else
    combine_items_t<8, 1>(p, c, ntok, tok, s_pair);
}

// C(ct): tokens ct * kCombineT .. + kCombineT - 1.  Their (weight, slot)
// pairs go to s_pair first, unless the caller has staged them.
__device__ __forceinline__ void task_combine(const MoeParams& p, const Ctx& c, int ct, int* s_pair, bool staged = false) {
  const int t0 = ct * kCombineT;
  const int ntok = min(kCombineT, c.T - t0);
  const int k = c.k;
  if (!staged && threadIdx.x < ntok * k) {
    const uint32_t fo = (uint32_t)(t0 * k + threadIdx.x) * 4u;
    s_pair[2 * threadIdx.x] = (int)co_ld32(r_topw(p), fo);
    s_pair[2 * threadIdx.x + 1] = (int)co_ld32(r_slot(p), fo);
  }
  __syncthreads();
  combine_items(p, c, ntok, [&](int n) { return t0 + n; }, s_pair);
}

#include "decoder_tasks.h"

// =================================================== event plumbing ========
// STATIC and ORDERED: the notifies after the router, top-k and scan tasks
// (the G runners notify inline).  The dynamic schedule's notifies and
// pushes live in dyn_sched.h.
template <int MODE>
__device__ __forceinline__ void after_router(const MoeParams& p, const Ctx& c, int tt) {
  if (MODE == MODE_STATIC || MODE == MODE_ORDERED) {
    wg_publish();
    if (threadIdx.x == 0) notify1(c, ev_logit(p, c, tt), (uint32_t)c.nET);
  }
}

template <int MODE>
__device__ __forceinline__ void after_topk(const MoeParams& p, const Ctx& c) {
  if (MODE == MODE_STATIC || MODE == MODE_ORDERED) {
    wg_publish();
    if (threadIdx.x == 0) notify1(c, c.set + W_EV_ROUTE, (uint32_t)c.nK);
  }
}

template <int MODE>
__device__ __forceinline__ void after_scan(const MoeParams& p, const Ctx& c, int nrt) {
  if (MODE == MODE_STATIC || MODE == MODE_ORDERED) {
    wg_publish();
    // the scan event is complete at any value >= 1; S stores nrt + 1, so
    // that a waiter learns the row-tile count from the poll that frees it
    if (threadIdx.x == 0) xchg_relaxed(c.set + W_EV_SCAN, (uint32_t)nrt + 1u);
  }
}

// ==================================================== schedules ==========
// Grid-wide barrier (BARRIER comparator only).  Two words that only grow
// (the counter set is zeroed before every launch): the arrival count, and
// the release word, on its own line so that the waiters' polls do not slow
// the arrivals' atomics.  Barrier b completes at the sum of the party counts
// of barriers 1..b, which every workgroup reaching barrier b holds in
// `target` (all of them passed the same earlier barriers); the arrival that
// brings the count there stores that sum into the release word, which the
// others poll.  Barrier b + 1 cannot complete before barrier b's release, so
// the release word only grows.  No reset, no generation: no arrival can be
// lost to a late reset.  Bounded by the same watchdog as every other wait.
__device__ __forceinline__ bool grid_barrier(const Ctx& c, int parties, uint32_t& target) {
  wg_publish();
  target += (uint32_t)parties;
  int fail = 0;
  if (threadIdx.x == 0) {
    if (add_relaxed(c.set + W_BAR_COUNT, 1u) + 1u == target)
      (void)xchg_relaxed(c.set + W_BAR_RELEASE, target);
    else
      fail = spin_until_geq(c.set + W_BAR_RELEASE, target, c.status, c.budget) ? 0 : 1;
  }
  fail = __syncthreads_or(fail);
  return fail == 0;
}

// Static G1 / G2 lists with the waits taken off the critical path: the row
// tile of the task after next and the event state (arrivals, wait_count) of
// the next task are loaded before the current task's weights, so by the time
// a task starts its event is usually known to be released and thread 0 skips
// polling.  Only wave 0 writes a task's outputs, so only wave 0 drains its
// stores before the notify; the notify needs no workgroup barrier.  With the
// debug buffer the notify also checks for over-notification.

__device__ bool wait_known(const uint32_t* ctr, uint32_t target, uint32_t known, const Ctx& c) {
  int fail = 0;
  if (threadIdx.x == 0 && known < target) fail = spin_until_geq(ctr, target, c.status, c.budget) ? 0 : 1;
  fail = __syncthreads_or(fail);
  return fail == 0;
}

// C(ct) may run once every row tile holding one of its tokens' k rows has
// finished all of its G2 column tiles: wave 0 polls those ev_y elements, one
// row a lane (at most kCombineT * k <= 32 rows), under the watchdog.
// It also stages the task's (weight, slot) pairs in `s_pair` for task_combine,
// so that the combine, on the critical path's tail, starts with its Y loads.
__device__ __forceinline__ bool wait_rows_done(const MoeParams& p, const Ctx& c, int ct, int* s_pair) {
  int fail = 0;
  if (threadIdx.x < 64) {
    const int t0 = ct * kCombineT, nrow = min(kCombineT, c.T - t0) * c.k;
    const bool mine = (int)threadIdx.x < nrow;
    uint32_t* ctr = ev_y(p, c, 0);
    if (mine) {
      const uint32_t fo = (uint32_t)(t0 * c.k + (int)threadIdx.x) * 4u;
      const uint32_t s = co_ld32(r_slot(p), fo);
      s_pair[2 * threadIdx.x] = (int)co_ld32(r_topw(p), fo);
      s_pair[2 * threadIdx.x + 1] = (int)s;
      const uint32_t rt = co_ld32(r_rowrt(p), s * 4u);
      ctr = ev_y(p, c, (int)rt);
      if (p.debug) {  // count the rows whose mapped tile really holds them
        const u32x4_t q = co_ld128(r_rtinfo(p), rt * 16u);
        if (s >= q.y && s < q.y + q.z) atomicAdd(p.debug + 2 * c.E + 7, 1);
      }
    }
    const uint32_t tgt = (uint32_t)c.nN2;
    const uint64_t t_start = now_ticks();
    for (uint32_t spins = 1;; ++spins) {
      const bool ok = !mine || ld_relaxed(ctr) >= tgt;
      if (__all(ok)) break;
      if ((spins & 7u) == 0u) {
        if (ld_relaxed(c.status) & ST_ABORT) { fail = 1; break; }
        if (now_ticks() - t_start > c.budget) {
          if (threadIdx.x == 0) or_relaxed(c.status, ST_TIMEOUT | ST_ABORT);
          fail = 1;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  fail = __syncthreads_or(fail);
  return fail == 0;
}

// Large batches: a workgroup's combine tasks c0, c0 + G, ..., c0 + (n-1) G
// as one stream (n kCombineT k <= kThreads routed rows).  Thread q takes
// routed row q (task q / (kCombineT k), then its token and slot), stages
// its (weight, slot) pair in s_pair[2 q .. 2 q + 1] and polls its row
// tile's ev_y, all threads at once; then one item loop covers every token
// of the stream.  Returns false when a wait gave up (uniform).
__device__ __forceinline__ bool combine_stream(const MoeParams& p, const Ctx& c, int c0, int G, int n, int* s_pair) {
  const int k = c.k, per = kCombineT * k;
  int fail = 0;
  {
    const int q = threadIdx.x;
    const int m = q / per, loc = q - m * per;
    const int t = (c0 + m * G) * kCombineT + loc / k;
    const bool mine = q < n * per && t < c.T;
    uint32_t* ctr = ev_y(p, c, 0);
    if (mine) {
      const uint32_t fo = (uint32_t)(t * k + loc % k) * 4u;
      const uint32_t sl = co_ld32(r_slot(p), fo);
      s_pair[2 * q] = (int)co_ld32(r_topw(p), fo);
      s_pair[2 * q + 1] = (int)sl;
      ctr = ev_y(p, c, (int)co_ld32(r_rowrt(p), sl * 4u));
    } else if (q < n * per) {  // a token past T: a valid row that is never stored
      s_pair[2 * q] = 0;
      s_pair[2 * q + 1] = 0;
    }
    const uint32_t tgt = (uint32_t)c.nN2;
    const uint64_t t_start = now_ticks();
    for (uint32_t spins = 1;; ++spins) {
      const bool ok = !mine || ld_relaxed(ctr) >= tgt;
      if (__all(ok)) break;
      if ((spins & 7u) == 0u) {
        if (ld_relaxed(c.status) & ST_ABORT) { fail = 1; break; }
        if (now_ticks() - t_start > c.budget) {
          if ((threadIdx.x & 63) == 0) or_relaxed(c.status, ST_TIMEOUT | ST_ABORT);
          fail = 1;
          break;
        }
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  if (__syncthreads_or(fail)) return false;
  combine_items(p, c, n * kCombineT, [&](int e) {
    const int t = (c0 + (e / kCombineT) * G) * kCombineT + e % kCombineT;
    return t < c.T ? t : -1;
  }, s_pair);
  return true;
}

// Row tile and column tile of G task i (of nrt row tiles x nn column tiles):
// row-major, except in the big-tile variant, whose tasks follow big_task's
// L2-friendly order (in the large-batch variant that order measured the
// same at the Zipf prefill, 187.2 vs 187.6 us, and cost registers).
template <int WG>
__device__ __forceinline__ TileRC g_tile(int i, int nrt, int nn) {
  if constexpr (WG == kVarBig) {
    return big_task(i, nrt, nn);
  } else {
    TileRC t;
    t.rt = i / nn;
    t.nt = i % nn;
    return t;
  }
}

template <int WG>
__device__ __forceinline__ void run_g1_static(const MoeParams& p, const Ctx& c, float* red, int i0, int n, int G,
                              const LocalRoute* lr) {
  if (i0 >= n) return;
  const bool tr = p.trace != nullptr;
  uint64_t tw = 0, ts = 0, tb = 0;
  const rsrc_t rcnt = r_counts(p);
  const int nrt = n / c.nN1;
  RowTile cur = get_tile(p, lr, g_tile<WG>(i0, nrt, c.nN1).rt);
  RowTile nxt = cur;
  if (i0 + G < n) nxt = get_tile(p, lr, g_tile<WG>(i0 + G, nrt, c.nN1).rt);
  uint32_t cur_tgt = 0, cur_arr = 0;
  if (threadIdx.x == 0) {
    cur_tgt = (lr ? (uint32_t)lr->cnt[cur.e] : co_ld32(rcnt, (uint32_t)cur.e * 4u));
    // with the LDS tables every expert event is known released: the tables
    // were built after the route event, which each top-k task notifies only
    // once its expert notifies have completed
    cur_arr = lr ? cur_tgt : ld_relaxed(ev_exp(p, c, cur.e));
  }
  // grouped-row permutation entries of the tile's rows (A gather), one task ahead
  uint32_t cur_f[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) cur_f[b] = row_perm(p, cur, b, lr);
  // Enter the loop with nothing in flight: otherwise the compiler, merging
  // the entry path (prefetch loads pending) with the back edge (only the
  // notify pending), waits for all memory operations at the top of every
  // task, the previous notify's round trip included.
  __builtin_amdgcn_s_waitcnt(0);
  for (int i = i0; i < n; i += G) {
    const TileRC tt = g_tile<WG>(i, nrt, c.nN1);
    const int rt = tt.rt, nt = tt.nt;
    if (tr) tw = now_ticks();
    if (!wait_known(ev_exp(p, c, cur.e), cur_tgt, cur_arr, c)) return;
    if (tr) ts = now_ticks();
    RowTile nn = nxt;
    if (i + 2 * G < n) nn = get_tile(p, lr, g_tile<WG>(i + 2 * G, nrt, c.nN1).rt);
    uint32_t nxt_tgt = 0, nxt_arr = 0;
    if (threadIdx.x == 0 && i + G < n) {
      nxt_tgt = (lr ? (uint32_t)lr->cnt[nxt.e] : co_ld32(rcnt, (uint32_t)nxt.e * 4u));
      nxt_arr = ld_relaxed(ev_exp(p, c, nxt.e));
    }
    uint32_t nxt_f[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) nxt_f[b] = i + G < n ? row_perm(p, nxt, b, lr) : 0u;
    task_g1<false, WG>(p, c, cur, rt, nt, red, cur_f);
    // wave 0 wrote the tile: drain its stores, then notify.  The drain is
    // outside the notify branch so that, after the branch, only the notify
    // is in flight and the prefetched registers need no further wait.
    __builtin_amdgcn_s_waitcnt(0);
    if (threadIdx.x == 0) notify_fast(p, c, ev_h(p, c, rt), (uint32_t)c.nN1);
    if (tr) tb = now_ticks();
    dbg_task(p, TT_G1);
    trace_task(p, TT_G1, rt, nt, tw, ts, tb);
    cur = nxt;
    nxt = nn;
    cur_tgt = nxt_tgt;
    cur_arr = nxt_arr;
#pragma unroll
    for (int b = 0; b < 4; ++b) cur_f[b] = nxt_f[b];
  }
}

template <int WG>
__device__ __forceinline__ void run_g2_static(const MoeParams& p, const Ctx& c, float* red, int i0, int n, int G,
                              const LocalRoute* lr) {
  if (i0 >= n) return;
  const bool tr = p.trace != nullptr;
  uint64_t tw = 0, ts = 0, tb = 0;
  const uint32_t tgt = (uint32_t)c.nN1;
  const int nrt = n / c.nN2;
  RowTile cur = get_tile(p, lr, g_tile<WG>(i0, nrt, c.nN2).rt);
  RowTile nxt = cur;
  if (i0 + G < n) nxt = get_tile(p, lr, g_tile<WG>(i0 + G, nrt, c.nN2).rt);
  uint32_t cur_arr = 0;
  if (threadIdx.x == 0) cur_arr = ld_relaxed(ev_h(p, c, g_tile<WG>(i0, nrt, c.nN2).rt));
  __builtin_amdgcn_s_waitcnt(0);  // loop entry with nothing in flight (see run_g1_static)
  for (int i = i0; i < n; i += G) {
    const TileRC tt = g_tile<WG>(i, nrt, c.nN2);
    const int rt = tt.rt, nt = tt.nt;
    if (tr) tw = now_ticks();
    if (!wait_known(ev_h(p, c, rt), tgt, cur_arr, c)) return;
    if (tr) ts = now_ticks();
    RowTile nn = nxt;
    if (i + 2 * G < n) nn = get_tile(p, lr, g_tile<WG>(i + 2 * G, nrt, c.nN2).rt);
    uint32_t nxt_arr = 0;
    if (threadIdx.x == 0 && i + G < n) nxt_arr = ld_relaxed(ev_h(p, c, g_tile<WG>(i + G, nrt, c.nN2).rt));
    // combine tile of each row's token (wave 0, one row a lane)
    task_g2<false, WG>(p, c, cur, rt, nt, red);
    __builtin_amdgcn_s_waitcnt(0);  // wave 0 wrote the rows: drain, then notify (as in G1)
    if (threadIdx.x == 0) notify_fast(p, c, ev_y(p, c, rt), (uint32_t)c.nN2);
    if (tr) tb = now_ticks();
    dbg_task(p, TT_G2);
    trace_task(p, TT_G2, rt, nt, tw, ts, tb);
    cur = nxt;
    nxt = nn;
    cur_arr = nxt_arr;
  }
}

// ORDERED: the G tiles are claimed in index order, all G1 tiles before any
// G2 tile, from one counter per group of workgroups (group = workgroup index
// mod 8; the dispatcher deals consecutive workgroups over the 8 XCDs, so a
// group is one XCD's workgroups).  Ordinal k of group g is tile k * ngrp + g.
// A workgroup that streams faster (the first of the two on a CU, a CU whose
// tiles are cheaper) claims more tiles, so the phases end together, while
// every tile still waits on its event as in STATIC.  Deadlock freedom: G1
// waits only on K, which is complete before S, so every claimed G1 tile
// completes; a workgroup holds a G2 ordinal only once its group has handed
// out all of its G1 tiles, so every G1 tile is claimed and every G2 wait is
// met; C waits only on G2.  Claims from one thread to one counter are
// ordered (same-location coherence), so a workgroup's ordinals increase and
// the first one past the end ends its stream.  The first three claims are
// separate claims, so that with few tiles the first claims of all
// workgroups interleave and spread the tiles.  The runner keeps three
// ordinals ahead of the running tile: the claim round trip, the next
// row-tile descriptor and the next event state arrive while earlier tiles
// stream, as in the STATIC runners.
struct ClaimQ {
  uint32_t* ctr;
  int grp, ngrp, n;
  int base;  // tile of ordinal 0 (tiles below it are dealt, not claimed)
};
__device__ __forceinline__ int claimed_task(const ClaimQ& q, uint32_t k) {
  const int64_t i = q.base + (int64_t)k * q.ngrp + q.grp;
  return i < q.n ? (int)i : q.n;
}

// The G tiles of one stream: index i < nG1 is G1 tile (i / nN1, i % nN1),
// otherwise G2 tile j = i - nG1 is (j / nN2, j % nN2).
struct GTask {
  int g2, rt, nt;
};
template <int WG>
__device__ __forceinline__ GTask gtask(const Ctx& c, int i, int nG1) {
  GTask t;
  t.g2 = i >= nG1;
  const int j = t.g2 ? i - nG1 : i, nn = t.g2 ? c.nN2 : c.nN1;
  const TileRC r = g_tile<WG>(j, nG1 / c.nN1, nn);
  t.rt = r.rt;
  t.nt = r.nt;
  return t;
}

// ORDERED: one claim stream per group over the G1 tiles and then the G2
// tiles, so the pipeline runs on across the G1 -> G2 boundary.  The event a
// tile waits on is ev_exp[e] (target counts[e]) for G1 and ev_h[rt] (target
// I/16) for G2; its state is fetched one tile ahead, the row-tile descriptor
// two ahead and the claim three ahead.  Returns false when a wait gave up
// (the launch is aborting).
template <int WG>
__device__ __forceinline__ bool run_g_ordered(const MoeParams& p, const Ctx& c, float* red, const ClaimQ& q, int nG1, uint32_t* sk,
                              const LocalRoute* lr) {
  const int n = q.n;
  const bool tr = p.trace != nullptr;
  uint64_t tw = 0, ts = 0, tb = 0;
  const rsrc_t rcnt = r_counts(p);
  // sk[0..2] hold the first three claims, taken by the caller before S ended
  int cur = claimed_task(q, sk[0]), nxt = claimed_task(q, sk[1]);
  if (cur >= n) return true;
  // event element and target of a tile; thread 0 loads the arrival count
  auto ev_of = [&](const GTask& t, const RowTile& r) -> uint32_t* {
    return t.g2 ? ev_h(p, c, t.rt) : ev_exp(p, c, r.e);
  };
  auto tgt_of = [&](const GTask& t, const RowTile& r) -> uint32_t {
    if (t.g2) return (uint32_t)c.nN1;
    return lr ? (uint32_t)lr->cnt[r.e] : co_ld32(rcnt, (uint32_t)r.e * 4u);
  };
  GTask tc = gtask<WG>(c, cur, nG1), tn = tc;
  RowTile rc = get_tile(p, lr, tc.rt);
  RowTile rn = rc;
  if (nxt < n) {
    tn = gtask<WG>(c, nxt, nG1);
    rn = get_tile(p, lr, tn.rt);
  }
  uint32_t cur_tgt = 0, cur_arr = 0;
  if (threadIdx.x == 0) {
    cur_tgt = tgt_of(tc, rc);
    cur_arr = ld_relaxed(ev_of(tc, rc));
  }
  uint32_t cur_f[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) cur_f[b] = tc.g2 ? 0u : row_perm(p, rc, b, lr);
  __builtin_amdgcn_s_waitcnt(0);  // loop entry with nothing in flight (see run_g1_static)
  int par = 2;  // claim slot that holds the ordinal after nxt
  for (;;) {
    if (tr) tw = now_ticks();
    if (!wait_known(ev_of(tc, rc), cur_tgt, cur_arr, c)) return false;
    if (tr) ts = now_ticks();
    const int aft = claimed_task(q, sk[par]);
    uint32_t knew = 0xffffffffu;
    if (threadIdx.x == 0 && aft < n) knew = add_relaxed(q.ctr, 1u);
    GTask ta = tn;
    RowTile ra = rn;
    if (aft < n) {
      ta = gtask<WG>(c, aft, nG1);
      ra = get_tile(p, lr, ta.rt);
    }
    uint32_t nxt_tgt = 0, nxt_arr = 0;
    if (threadIdx.x == 0 && nxt < n) {
      nxt_tgt = tgt_of(tn, rn);
      nxt_arr = ld_relaxed(ev_of(tn, rn));
    }
    uint32_t nxt_f[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) nxt_f[b] = (nxt < n && !tn.g2) ? row_perm(p, rn, b, lr) : 0u;
    if (!tc.g2) {
      task_g1<false, WG>(p, c, rc, tc.rt, tc.nt, red, cur_f);
    } else {
      task_g2<false, WG>(p, c, rc, tc.rt, tc.nt, red);
    }
    __builtin_amdgcn_s_waitcnt(0);  // wave 0 wrote the tile: drain, then notify (see run_g1_static)
    if (threadIdx.x == 0) {
      if (!tc.g2)
        notify_fast(p, c, ev_h(p, c, tc.rt), (uint32_t)c.nN1);
      else
        notify_fast(p, c, ev_y(p, c, tc.rt), (uint32_t)c.nN2);
      sk[par ^ 1] = knew;
    }
    if (tr) tb = now_ticks();
    dbg_task(p, tc.g2 ? TT_G2 : TT_G1);
    trace_task(p, tc.g2 ? TT_G2 : TT_G1, tc.rt, tc.nt, tw, ts, tb);
    cur = nxt;
    nxt = aft;
    tc = tn;
    tn = ta;
    rc = rn;
    rn = ra;
    cur_tgt = nxt_tgt;
    cur_arr = nxt_arr;
#pragma unroll
    for (int b = 0; b < 4; ++b) cur_f[b] = nxt_f[b];
    par ^= 1;
    if (cur >= n) break;
  }
  return true;
}

// ORDERED with the routing tables in LDS (small batches): the same stream
// with fewer claimed tiles held ahead.  Descriptors, row indices and wait
// counts come from LDS, so the next tile's state needs no second stage of
// lookahead: at the start of a tile the next one is known and the claim
// for the one after it is in flight.  Once the held tile is among the
// stream's last 2G, a workgroup claims only when it holds none (the claim
// in flight is then the next tile), so fewer tiles wait behind a running
// one while other workgroups have run out: with one tile held to the end,
// a third of the grid started its last tile after the first workgroup had
// gone idle (decode 169.3 us; 168.8 with this endgame).
// One counter serves the whole grid, so the XCDs, which stream at somewhat
// different rates, end together (with one counter per XCD group the groups
// ended up to 6 us apart at decode).  A workgroup's first two tiles are
// dealt (d and G + d), so that the grid's first claims do not all meet on
// that counter at once (claimed, they held the first G1 tile back by
// 6 us); ordinal o of the counter is tile 2G + o.  d = w, except that the
// workgroup that ran S and workgroup G - 1 swap: the one still busy with S
// and its tables is dealt the last tile of each round, not an early G1
// tile that later G2 tiles wait for (every workgroup's tiles still ascend,
// and the dealt set is the same).  Thread 0 hands a
// claim's result to the other threads through sk[0] and an LDS barrier.
// Deadlock freedom as in run_g_ordered: a workgroup's tiles come in
// ascending index order, every G1 tile below every G2 tile.
template <int WG>
__device__ __forceinline__ bool run_g_ordered_local(const MoeParams& p, const Ctx& c, float* red, const ClaimQ& q,
                                                    int nG1, uint32_t* sk, const LocalRoute* lr, int d) {
  const int n = q.n;
  const bool tr = p.trace != nullptr;
  uint64_t tw = 0, ts = 0, tb = 0;
  const int G = gridDim.x;
  int cur = d < n ? d : n;
  if (cur >= n) return true;
  int nxt = G + d < n ? G + d : n;  // the tile held after the running one (n: none)
  bool more = true;                 // the counter may still hand out tiles
  auto ev_of = [&](const GTask& t, const RowTile& r) -> uint32_t* {
    return t.g2 ? ev_h(p, c, t.rt) : ev_exp(p, c, r.e);
  };
  auto tgt_of = [&](const GTask& t, const RowTile& r) -> uint32_t {
    return t.g2 ? (uint32_t)c.nN1 : (uint32_t)lr->cnt[r.e];
  };
  GTask tc = gtask<WG>(c, cur, nG1);
  RowTile rc = get_tile(p, lr, tc.rt);
  uint32_t cur_tgt = 0, cur_arr = 0;
  if (threadIdx.x == 0) {
    cur_tgt = tgt_of(tc, rc);
    // a G1 tile's expert event is known released (the tables were built
    // after the route event; see run_g1_static), so the first tile starts
    // without a load round trip
    cur_arr = tc.g2 ? ld_relaxed(ev_of(tc, rc)) : cur_tgt;
  }
  uint32_t cur_f[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) cur_f[b] = tc.g2 ? 0u : row_perm(p, rc, b, lr);
  __builtin_amdgcn_s_waitcnt(0);  // loop entry with nothing in flight (see run_g1_static)
  for (;;) {
    if (tr) tw = now_ticks();
    if (!wait_known(ev_of(tc, rc), cur_tgt, cur_arr, c)) return false;
    if (tr) ts = now_ticks();
    // claim the tile after the held one while the stream is long; near its
    // end (held tile within the last 2G) claim only with none held
    const bool claim = more && (nxt < n ? nxt < n - 2 * G : true);
    uint32_t knew = 0xffffffffu;
    if (threadIdx.x == 0 && claim) knew = add_relaxed(q.ctr, 1u);
    GTask tn = tc;
    RowTile rn = rc;
    uint32_t nxt_tgt = 0, nxt_arr = 0;
    uint32_t nxt_f[4] = {0u, 0u, 0u, 0u};
    if (nxt < n) {
      tn = gtask<WG>(c, nxt, nG1);
      rn = get_tile(p, lr, tn.rt);
      if (threadIdx.x == 0) {
        nxt_tgt = tgt_of(tn, rn);
        nxt_arr = ld_relaxed(ev_of(tn, rn));
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) nxt_f[b] = tn.g2 ? 0u : row_perm(p, rn, b, lr);
    }
    if (!tc.g2) {
      task_g1<false, WG>(p, c, rc, tc.rt, tc.nt, red, cur_f);
    } else {
      task_g2<false, WG>(p, c, rc, tc.rt, tc.nt, red);
    }
    __builtin_amdgcn_s_waitcnt(0);  // wave 0 wrote the tile: drain, then notify (see run_g1_static)
    if (threadIdx.x == 0) {
      if (!tc.g2)
        notify_fast(p, c, ev_h(p, c, tc.rt), (uint32_t)c.nN1);
      else
        notify_fast(p, c, ev_y(p, c, tc.rt), (uint32_t)c.nN2);
      if (claim) sk[0] = knew;
    }
    if (tr) tb = now_ticks();
    dbg_task(p, tc.g2 ? TT_G2 : TT_G1);
    trace_task(p, tc.g2 ? TT_G2 : TT_G1, tc.rt, tc.nt, tw, ts, tb);
    int got = n;  // the claimed tile, handed to every thread (sk[0] is next
                  // written only after this task's and the next task's barriers)
    if (claim) {
      lds_barrier();
      got = claimed_task(q, sk[0]);
      if (got >= n) more = false;
    }
    if (nxt < n) {
      tc = tn;
      rc = rn;
      cur_tgt = nxt_tgt;
      cur_arr = nxt_arr;
#pragma unroll
      for (int b = 0; b < 4; ++b) cur_f[b] = nxt_f[b];
      nxt = got;
    } else if (got < n) {
      // none was held: the tile claimed during this one runs next; its
      // event state is polled by the wait (a G1 tile's is known released)
      tc = gtask<WG>(c, got, nG1);
      rc = get_tile(p, lr, tc.rt);
      if (threadIdx.x == 0) {
        cur_tgt = tgt_of(tc, rc);
        cur_arr = tc.g2 ? 0u : cur_tgt;
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) cur_f[b] = tc.g2 ? 0u : row_perm(p, rc, b, lr);
    } else {
      break;
    }
  }
  return true;
}

// STATIC / BARRIER: each phase's tasks are dealt round-robin over the
// workgroups, continuing from where the previous phase stopped, and every
// workgroup runs its list in phase order.  In STATIC a task waits only on
// events produced by earlier phases, so with every workgroup resident no
// wait can be circular and the schedule cannot deadlock.  Task counts of the
// phases after S are read from S's output (data-dependent instantiation).
template <int MODE, int WG>
__device__ __forceinline__ void run_lists(const MoeParams& p, const Ctx& c, uint8_t* smem, Shared& sh,
                                          int64_t off0 = 0) {
  const int G = gridDim.x, w = blockIdx.x;
  float* red = reinterpret_cast<float*>(smem);
  constexpr bool EV = (MODE == MODE_STATIC || MODE == MODE_ORDERED);
  uint32_t bar = 0;  // BARRIER: arrivals that complete the next grid barrier
  const bool tr = p.trace != nullptr;
  uint64_t tw = 0, ts = 0, tb = 0;
  int64_t off = off0;
  // decoder layer: the router reads the attention block's output (h2),
  // complete once every N2 task has notified
  if (p.dec && first_of(w, off, G) < c.nR &&
      !wg_wait(c.set + W_DEC_N2, (uint32_t)((c.T + kDecNormT - 1) / kDecNormT), c.status, c.budget))
    return;
  // big-tile variant, full router tiles: the workgroup's tasks as one
  // pipelined stream, one drain, then the notifies of all of them
  bool streamed = false;
  if constexpr (WG == kVarBig) {
    const int rx = router_experts(c.T);
    if (EV && rx >= kRouterEL && c.T % kRouterT == 0 && c.E % rx == 0 && (c.H >> 3) % (2 * 64) == 0) {
      const int i0 = first_of(w, off, G);
      if (i0 < c.nR) {
        // one chunk a lane a step: two steps' operands and the unpacked
        // weights stay within the 256 VGPRs (two-chunk steps spilled into
        // the accumulation registers)
        if (rx == kRouterEXL)
          router_stream<kRouterEXL / 4, 1>(p, c, i0, G);
        else
          router_stream<kRouterEL / 4, 1>(p, c, i0, G);
        wg_publish();
        // one thread a task: the arrivals leave together, not one round trip
        // after another
        for (int i = i0 + (int)threadIdx.x * G; i < c.nR; i += G * kThreads)
          notify1(c, ev_logit(p, c, i / c.nET), (uint32_t)c.nET);
      }
      streamed = true;
    }
  }
  for (int i = first_of(w, off, G); !streamed && i < c.nR; i += G) {
    if (tr) tw = ts = now_ticks();
    task_router<(WG != kVarSmall)>(p, c, i / c.nET, i % c.nET);
    if (tr) tb = now_ticks();
    dbg_task(p, TT_R);
    after_router<MODE>(p, c, i / c.nET);
    trace_task(p, TT_R, i / c.nET, i % c.nET, tw, ts, tb);
  }
  off += c.nR;
  if (!EV && !grid_barrier(c, G, bar)) return;
  // Large batches: a workgroup's top-k tasks as one stream.  Wave 0 polls
  // all of their logit events at once (a lane each), the tasks run back to
  // back, and one drain and one notify of the whole count follow (top-k
  // tasks notify nothing else that waits on their stores).
  const int k0 = first_of(w, off, G);
  const int nmine = k0 < c.nK ? (c.nK - k0 + G - 1) / G : 0;
  if (EV && WG != kVarSmall && nmine > 1 && nmine <= 64) {
    if (tr) tw = now_ticks();
    int fail = 0;
    if (threadIdx.x < 64) {
      const bool mine = (int)threadIdx.x < nmine;
      const uint32_t* ctr = ev_logit(p, c, mine ? k0 + (int)threadIdx.x * G : k0);
      const uint64_t t0 = now_ticks();
      for (uint32_t spins = 1;; ++spins) {
        const bool ok = !mine || ld_relaxed(ctr) >= (uint32_t)c.nET;
        if (__all(ok)) break;
        if ((spins & 7u) == 0u) {
          if (ld_relaxed(c.status) & ST_ABORT) { fail = 1; break; }
          if (now_ticks() - t0 > c.budget) {
            if (threadIdx.x == 0) or_relaxed(c.status, ST_TIMEOUT | ST_ABORT);
            fail = 1;
            break;
          }
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __shared__ int khist[kMaxE];
    for (int e = threadIdx.x; e < c.E; e += kThreads) khist[e] = 0;
    if (__syncthreads_or(fail)) return;
    if (tr) ts = now_ticks();
    // four token tiles at a time, their loads and selections side by side
    for (int q = 0; q < nmine; q += 4) task_topk_n<4>(p, c, k0 + q * G, G, min(4, nmine - q), khist);
    for (int i = k0; i < c.nK; i += G) dbg_task(p, TT_K);
    if (tr) tb = now_ticks();
    __syncthreads();  // every task's LDS counts are in
    for (int e = threadIdx.x; e < c.E; e += kThreads)
      if (khist[e]) (void)add_relaxed(ev_exp(p, c, e), (uint32_t)khist[e]);
    wg_publish();
    if (threadIdx.x == 0) notify_n(c, c.set + W_EV_ROUTE, (uint32_t)nmine, (uint32_t)c.nK);
    trace_task(p, TT_K, k0, nmine, tw, ts, tb);
  } else {
    for (int i = k0; i < c.nK; i += G) {
      if (tr) tw = now_ticks();
      if (EV && !wg_wait(ev_logit(p, c, i), (uint32_t)c.nET, c.status, c.budget)) return;
      if (tr) ts = now_ticks();
      task_topk(p, c, i);
      if (tr) tb = now_ticks();
      dbg_task(p, TT_K);
      after_topk<MODE>(p, c);
      trace_task(p, TT_K, i, 0, tw, ts, tb);
    }
  }
  off += c.nK;
  if (!EV && !grid_barrier(c, G, bar)) return;
  // Large batches with events: the scan as per-chunk tasks (count every
  // chunk, then place every chunk), so that no workgroup walks all T*k
  // pairs alone; the last placement to finish releases the scan event.
  const int nsch = (c.T + kScanChunkT - 1) / kScanChunkT;
  if (EV && WG != kVarSmall && nsch > 1) {
    for (int i = first_of(w, off, G); i < nsch; i += G) {
      if (tr) tw = now_ticks();
      if (!wg_wait(c.set + W_EV_ROUTE, (uint32_t)c.nK, c.status, c.budget)) return;
      if (tr) ts = now_ticks();
      task_scan<false, false, 1>(p, c, smem, nullptr, i);
      if (tr) tb = now_ticks();
      wg_publish();
      if (threadIdx.x == 0) (void)add_relaxed(c.set + W_SCAN_S1, 1u);
      trace_task(p, TT_S, i, 1, tw, ts, tb);
    }
    off += nsch;
    for (int i = first_of(w, off, G); i < nsch; i += G) {
      if (tr) tw = now_ticks();
      if (!wg_wait(c.set + W_SCAN_S1, (uint32_t)nsch, c.status, c.budget)) return;
      if (tr) ts = now_ticks();
      const int nrt_s = task_scan<false, false, 3>(p, c, smem, nullptr, i);
      if (tr) tb = now_ticks();
      dbg_task(p, TT_S);
      wg_publish();  // this chunk's rows (and, for chunk 0, the tables) are out
      // the scan event is complete at any value >= 1; the last placement
      // stores nrt + 1 (every other placement drained before its arrival)
      if (threadIdx.x == 0 && add_relaxed(c.set + W_SCAN_S3, 1u) == (uint32_t)nsch - 1u)
        xchg_relaxed(c.set + W_EV_SCAN, (uint32_t)nrt_s + 1u);
      trace_task(p, TT_S, i, 3, tw, ts, tb);
    }
    off += nsch;
  } else {
    if (first_of(w, off, G) == 0) {
      if (tr) tw = now_ticks();
      if (EV && !wg_wait(c.set + W_EV_ROUTE, (uint32_t)c.nK, c.status, c.budget)) return;
      if (tr) ts = now_ticks();
      const int nrt_s = task_scan(p, c, smem);
      if (tr) tb = now_ticks();
      dbg_task(p, TT_S);
      after_scan<MODE>(p, c, nrt_s);
      trace_task(p, TT_S, 0, 0, tw, ts, tb);
    }
    off += 1;
  }
  // Small batch: each workgroup rebuilds the routing tables in its own LDS
  // as soon as every top-k task is done, so G1 does not wait for S (S still
  // writes the routing outputs, which C reads).
  const bool local = WG != kVarBig && EV && c.T <= kScanChunkT && c.T * c.k <= kLocalRows;
  // ORDERED claim counters: one per XCD group for large batches, where the
  // first three claims are taken while S still runs (an ordinal does not
  // depend on S's result); one for the whole grid with the LDS tables,
  // whose runner deals its first two tiles instead of claiming them.
  const int ngrp = (G % 8 == 0 && !local) ? 8 : 1, grp = w % ngrp;
  if (MODE == MODE_ORDERED && !local && threadIdx.x == 0) {
    uint32_t* ctr = c.set + W_CLAIM_G1 + grp * 32;
    sh.claim[0] = add_relaxed(ctr, 1u);
    sh.claim[1] = add_relaxed(ctr, 1u);
    sh.claim[2] = add_relaxed(ctr, 1u);
  }
  int nrt;
  __shared__ LocalRoute lroute;
  const LocalRoute* lr = nullptr;
  if (local) {
    if (tr) tw = now_ticks();
    if (!wg_wait(c.set + W_EV_ROUTE, (uint32_t)c.nK, c.status, c.budget)) return;
    if (tr) ts = now_ticks();
    nrt = task_scan<true>(p, c, smem, &lroute);
    lr = &lroute;
    if (tr) tb = now_ticks();
    trace_task(p, TT_L, nrt, 0, tw, ts, tb);
  } else if (EV) {
    if (threadIdx.x == 0) {
      uint32_t v = 0;
      sh.claim[3] = spin_value_geq(c.set + W_EV_SCAN, 1u, c.status, c.budget, &v) ? v : 0u;
    }
    __syncthreads();
    if (sh.claim[3] == 0u) return;  // aborting
    nrt = (int)sh.claim[3] - 1;
  } else {
    if (!grid_barrier(c, G, bar)) return;
    nrt = (int)ld_relaxed(p.meta + M_NRT);
  }
  const int nG1 = nrt * c.nN1, nG2 = nrt * c.nN2;
  // Few GEMM tasks (at most three a CU): deal G1, G2 and C over only the
  // first workgroup of each CU, so that no two weight streams share a CU's
  // load path; the other workgroups are done (and BARRIER's later barriers
  // count only the ones left).  Workgroups are placed one a CU before any
  // CU takes a second, so the first solo_wgs workgroups sit on distinct CUs.
  const int Gt = (MODE != MODE_ORDERED && p.solo_wgs > 0 && nG1 <= 3 * p.solo_wgs) ? p.solo_wgs : G;
  if (w >= Gt) return;
  if (MODE == MODE_ORDERED) {
    const ClaimQ q{c.set + W_CLAIM_G1 + grp * 32, grp, ngrp, nG1 + nG2, local ? 2 * G : 0};
    const int s_wg = (int)((off - 1) % G);  // the workgroup that ran S (one task, the local tables' case)
    const int d = w == s_wg ? G - 1 : (w == G - 1 ? s_wg : w);
    if (lr ? !run_g_ordered_local<WG>(p, c, red, q, nG1, sh.claim, lr, d)
           : !run_g_ordered<WG>(p, c, red, q, nG1, sh.claim, lr))
      return;
    off += nG1 + nG2;
  } else {
  if (EV) {
    run_g1_static<WG>(p, c, red, first_of(w, off, Gt), nG1, Gt, lr);
  } else {
    // no wait separates this loop's tasks: a barrier keeps the next task's
    // LDS writes (A staging, partial sums) behind the previous task's last
    // LDS reads (wave 0 reads the output stage while it stores the tile)
    for (int i = first_of(w, off, Gt); i < nG1; i += Gt) {
      const TileRC tt = g_tile<WG>(i, nrt, c.nN1);
      const int rt = tt.rt;
      if (i >= Gt) lds_barrier();
      if (tr) tw = ts = now_ticks();
      task_g1<false, WG>(p, c, load_rowtile(p, rt), rt, tt.nt, red);
      if (tr) tb = now_ticks();
      dbg_task(p, TT_G1);
      trace_task(p, TT_G1, rt, tt.nt, tw, ts, tb);
    }
  }
  off += nG1;
  if (!EV && !grid_barrier(c, Gt, bar)) return;
  if (EV) {
    run_g2_static<WG>(p, c, red, first_of(w, off, Gt), nG2, Gt, lr);
  } else {
    for (int i = first_of(w, off, Gt); i < nG2; i += Gt) {
      const TileRC tt = g_tile<WG>(i, nrt, c.nN2);
      const int rt = tt.rt;
      if (i >= Gt) lds_barrier();  // as in the G1 loop
      if (tr) tw = ts = now_ticks();
      task_g2<false, WG>(p, c, load_rowtile(p, rt), rt, tt.nt, red);
      if (tr) tb = now_ticks();
      dbg_task(p, TT_G2);
      trace_task(p, TT_G2, rt, tt.nt, tw, ts, tb);
    }
  }
  off += nG2;
  if (!EV && !grid_barrier(c, Gt, bar)) return;
  }
  // C reads S's routing outputs (slot, row -> tile map)
  if (local && first_of(w, off, Gt) < c.nC && !wg_wait(c.set + W_EV_SCAN, 1u, c.status, c.budget)) return;
  {
    const int c0 = first_of(w, off, Gt);
    const int nmine = c0 < c.nC ? (c.nC - c0 + Gt - 1) / Gt : 0;
    if (EV && WG != kVarSmall && nmine > 1 && nmine * kCombineT * c.k <= kThreads) {
      __shared__ int s_cpairs[2 * kThreads];
      if (tr) tw = now_ticks();
      if (!combine_stream(p, c, c0, Gt, nmine, s_cpairs)) return;
      if (tr) ts = tb = now_ticks();
      for (int i = c0; i < c.nC; i += Gt) dbg_task(p, TT_C);
      trace_task(p, TT_C, c0, nmine, tw, tw, ts);
      return;
    }
  }
  for (int i = first_of(w, off, Gt); i < c.nC; i += Gt) {
    // wave 0 fills sh.pairs for this task (in the wait, or in the combine)
    // while the other waves may still read the previous task's pairs
    if (i >= Gt) lds_barrier();
    if (tr) tw = now_ticks();
    if (EV && !wait_rows_done(p, c, i, sh.pairs)) return;
    if (tr) ts = now_ticks();
    task_combine(p, c, i, sh.pairs, EV);
    if (tr) tb = now_ticks();
    dbg_task(p, TT_C);
    trace_task(p, TT_C, i, 0, tw, ts, tb);
  }
}

// DYNAMIC (Event Tensor pages, Figs. 8 and 9; podcast cue 11): the control
// logic (queue, pushes on completed events, the exit rule) is dyn::run_moe
// in dyn_sched.h, shared with a host harness that drives it with threads.
// DynTasks gives it this kernel's task bodies, event elements and trace.
template <int WG>
struct DynTasks {
  const MoeParams& p;
  const Ctx& c;
  uint8_t* smem;
  Shared& ksh;
  RowTile tile;  // the row tile of the last G2 task (its rows arrive at their combine events)
  uint64_t tw, tb;
  __device__ __forceinline__ void router(int tt, int et) { task_router<(WG != kVarSmall)>(p, c, tt, et); }
  __device__ __forceinline__ void topk(int tt) { task_topk(p, c, tt); }
  __device__ __forceinline__ int scan() { return task_scan<false, false>(p, c, smem); }
  __device__ __forceinline__ void g1(int rt, int nt) {
    task_g1<false, WG>(p, c, load_rowtile(p, rt), rt, nt, reinterpret_cast<float*>(smem));
  }
  __device__ __forceinline__ void g2(int rt, int nt) {
    tile = load_rowtile(p, rt);
    task_g2<false, WG>(p, c, tile, rt, nt, reinterpret_cast<float*>(smem));
  }
  __device__ __forceinline__ void combine(int ct) { task_combine(p, c, ct, ksh.pairs); }
  __device__ __forceinline__ uint32_t* ev_logit(int tt) { return etc::ev_logit(p, c, tt); }
  __device__ __forceinline__ uint32_t* ev_route() { return c.set + W_EV_ROUTE; }
  __device__ __forceinline__ uint32_t* ev_h(int rt) { return etc::ev_h(p, c, rt); }
  __device__ __forceinline__ uint32_t* ev_y(int rt) { return etc::ev_y(p, c, rt); }
  __device__ __forceinline__ uint32_t* ev_c(int ct) { return etc::ev_c(p, c, ct); }
  __device__ __forceinline__ int tile_rows(int) { return tile.nrows; }
  __device__ __forceinline__ int row_ctile(int, int r) {
    const int f = (int)co_ld32(r_perm(p), (uint32_t)(tile.r0 + r) * 4u);
    return (f / c.k) / kCombineT;
  }
  __device__ __forceinline__ void trace_start() {
    if (p.trace) tw = now_ticks();
  }
  __device__ __forceinline__ void trace_body() {
    if (p.trace) tb = now_ticks();
  }
  __device__ __forceinline__ void trace_end(int type, int a, int b) {
    dbg_task(p, type);
    trace_task(p, type, a, b, tw, tw, tb);
  }
};

// The persistent megakernel.  Counter sets are double buffered by the
// parity of a device-side epoch: this launch works in set[epoch & 1] (zeroed
// by the previous launch) and zeroes set[1 - (epoch & 1)] for the next one;
// the last workgroup to finish advances the epoch.  No host memset, no host
// state: the workspace is self-resetting, also after an aborted launch.
// WG: the kernel variant (kVarSmall, kVarWide, kVarBig), picked per launch
// from T * k: the large-batch variant holds the wide G1 tiles, the small one
// the narrow tiles only, so that small batches run code that carries none
// of the wide tiles' register pressure, and the big-tile variant (its own
// kernel, moe_persistent_big) the 256-row tiles.  All come from the one
// code object; T stays a kernel argument.
// DEC: the decoder layer: the attention block's tasks run first, in the same
// kernel, and the MoE block's router waits on their last event.
template <int MODE, int WG, bool DEC>
__device__ __forceinline__ void persistent_body(const MoeParams& p) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ Shared sh;
  __shared__ uint32_t s_epoch;
  __shared__ uint64_t s_wgt[2];  // trace: entry, counter set known (kept out of the registers)
  if (p.trace && threadIdx.x == 0) s_wgt[0] = now_ticks();
  if (threadIdx.x == 0) s_epoch = ld_relaxed(p.ctrl + C_EPOCH);
  trace_init(p);
  __syncthreads();
  const uint32_t epoch = s_epoch;
  uint32_t* set = (epoch & 1u) ? p.set1 : p.set0;
  uint32_t* other = (epoch & 1u) ? p.set0 : p.set1;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < p.set_words;
       i += (int64_t)gridDim.x * kThreads)
    other[i] = 0u;
  Ctx c = make_ctx(p, set);
  if (p.trace && threadIdx.x == 0) s_wgt[1] = now_ticks();
  {
    // task counts and tile widths of the variant this launch runs (the
    // small-batch variant holds neither the eight-experts-a-wave router tile
    // nor the column-split G tiles)
    const dyn::MoeGraph g = dyn::launch_graph(p.T, p.E, p.k, p.H, p.I, WG);
    c.nET = g.nET;
    c.nR = g.nR;
    c.nN1 = g.nN1;
    c.bn1 = p.I / g.nN1;
    c.nN2 = g.nN2;
    c.bn2 = p.H / g.nN2;
    c.bm = WG == kVarBig ? kBigBM : kBM;
    if (MODE == MODE_DYNAMIC) {
      dyn::Queue q;
      q.head = set + W_HEAD;
      q.tail = set + W_TAIL;
      q.total = set + W_TOTAL;
      q.status = c.status;
      q.slot = set + p.o_queue;
      q.cap = p.q_cap;
      q.prefix = (uint32_t)g.nR;
      q.known_total = 0u;
      q.budget = p.budget;
      __shared__ dyn::Shared dsh;
      DynTasks<WG> tk{p, c, smem, sh, RowTile{0, 0, 0}, 0, 0};
      dyn::run_moe<DevPlat>(tk, q, g, dsh);
    }
  }
  if (DEC) {
    int64_t off = 0;
    if (run_decoder_front(p, c, smem, off)) run_lists<MODE, WG>(p, c, smem, sh, off);
  } else if (MODE != MODE_DYNAMIC) {
    run_lists<MODE, WG>(p, c, smem, sh);
  }
  const uint64_t t_out = p.trace ? now_ticks() : 0;  // end of the task lists
  wg_publish();
  if (threadIdx.x == 0) {
    const uint32_t st = ld_relaxed(c.status) & ~ST_ABORT;
    if (st) or_relaxed(p.ctrl + C_REPORT, st);
    const uint32_t old = add_relaxed(set + W_DONE, 1u);
    if (old == gridDim.x - 1u) xchg_relaxed(p.ctrl + C_EPOCH, epoch + 1u);
  }
  if (p.trace) trace_task(p, TT_WG, 0, 0, s_wgt[0], s_wgt[1], t_out);
}
template <int MODE, int WG, bool DEC = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
moe_persistent(MoeParams p) {
  persistent_body<MODE, WG, DEC>(p);
}
// The small- and large-batch kernels are instantiated here, ahead of the
// big-tile kernels, so that their place in the code object does not move
// when a big-tile kernel changes size (the same instructions, moved, were
// measured up to 1.5 us a decode layer apart).
template __global__ void moe_persistent<MODE_ORDERED, kVarSmall, false>(MoeParams);
template __global__ void moe_persistent<MODE_STATIC, kVarSmall, false>(MoeParams);
template __global__ void moe_persistent<MODE_BARRIER, kVarSmall, false>(MoeParams);
template __global__ void moe_persistent<MODE_DYNAMIC, kVarSmall, false>(MoeParams);
template __global__ void moe_persistent<MODE_ORDERED, kVarWide, false>(MoeParams);
template __global__ void moe_persistent<MODE_STATIC, kVarWide, false>(MoeParams);
template __global__ void moe_persistent<MODE_BARRIER, kVarWide, false>(MoeParams);
template __global__ void moe_persistent<MODE_DYNAMIC, kVarWide, false>(MoeParams);
// The big-tile variant: one workgroup a CU (its G tiles take 128 KB of LDS
// and the full register file), so its G bodies may keep 256 accumulators.
template <int MODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
moe_persistent_big(MoeParams p) {
  persistent_body<MODE, kVarBig, false>(p);
}

// ------------------------------------------- kernel-by-kernel comparator --
__global__ void __launch_bounds__(kThreads) kbk_router(MoeParams p) {
  const Ctx c = make_ctx(p, nullptr);
  task_router(p, c, blockIdx.x / c.nET, blockIdx.x % c.nET);
}
__global__ void __launch_bounds__(kThreads) kbk_topk(MoeParams p) {
  const Ctx c = make_ctx(p, nullptr);
  task_topk(p, c, blockIdx.x);
}
__global__ void __launch_bounds__(kThreads) kbk_scan(MoeParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Ctx c = make_ctx(p, nullptr);
  task_scan(p, c, smem);
}
// large batches: the scan as per-chunk tasks, one chunk a workgroup
__global__ void __launch_bounds__(kThreads) kbk_scan_count(MoeParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Ctx c = make_ctx(p, nullptr);
  task_scan<false, false, 1>(p, c, smem, nullptr, blockIdx.x);
}
__global__ void __launch_bounds__(kThreads) kbk_scan_place(MoeParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Ctx c = make_ctx(p, nullptr);
  task_scan<false, false, 3>(p, c, smem, nullptr, blockIdx.x);
}
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) kbk_g1(MoeParams p) {
  // the larger of the K-split bodies' reduction and stage and the
  // column-split body's two staged A buffers
  __shared__ float red[(2 * 64 * kCsRowB) / 4 > 4 * kCB2 * 256 + kBM * kBN2 / 2 ? (2 * 64 * kCsRowB) / 4
                                                                                 : 4 * kCB2 * 256 + kBM * kBN2 / 2];
  const Ctx c = make_ctx(p, nullptr);
  const int nrt = (int)ld_relaxed(p.meta + M_NRT);
  if ((int)blockIdx.x >= nrt * c.nN1) return;
  const int rt = blockIdx.x / c.nN1;
  task_g1<true>(p, c, load_rowtile(p, rt), rt, blockIdx.x % c.nN1, red);
}
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) kbk_g2(MoeParams p) {
  __shared__ float red[(2 * 64 * kCsRowB) / 4 > 4 * kCB2 * 256 + kBM * kBN2 / 2 ? (2 * 64 * kCsRowB) / 4
                                                                                 : 4 * kCB2 * 256 + kBM * kBN2 / 2];
  const Ctx c = make_ctx(p, nullptr);
  const int nrt = (int)ld_relaxed(p.meta + M_NRT);
  if ((int)blockIdx.x >= nrt * c.nN2) return;
  const int rt = blockIdx.x / c.nN2;
  task_g2<true>(p, c, load_rowtile(p, rt), rt, blockIdx.x % c.nN2, red);
}
// big-tile G tasks, one a workgroup (kBigLdsBytes of dynamic LDS each)
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1))) kbk_g1_big(MoeParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Ctx c = make_ctx(p, nullptr);
  const int nrt = (int)ld_relaxed(p.meta + M_NRT);
  if ((int)blockIdx.x >= nrt * c.nN1) return;
  const TileRC t = big_task(blockIdx.x, nrt, c.nN1);
  task_g1<true, kVarBig>(p, c, load_rowtile(p, t.rt), t.rt, t.nt, reinterpret_cast<float*>(smem));
}
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1))) kbk_g2_big(MoeParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Ctx c = make_ctx(p, nullptr);
  const int nrt = (int)ld_relaxed(p.meta + M_NRT);
  if ((int)blockIdx.x >= nrt * c.nN2) return;
  const TileRC t = big_task(blockIdx.x, nrt, c.nN2);
  task_g2<true, kVarBig>(p, c, load_rowtile(p, t.rt), t.rt, t.nt, reinterpret_cast<float*>(smem));
}
__global__ void __launch_bounds__(kThreads) kbk_combine(MoeParams p) {
  __shared__ int pairs[2 * kCombineT * kMaxK];
  const Ctx c = make_ctx(p, nullptr);
  task_combine(p, c, blockIdx.x, pairs);
}

// ------------------------------------- decoder layer, kernel by kernel --
__global__ void __launch_bounds__(kThreads) kd_norm1(MoeParams p) {
  const Ctx c = make_ctx(p, nullptr);
  task_norm1(p, c, blockIdx.x);
}
__global__ void __launch_bounds__(kThreads) kd_qkv(MoeParams p) {
  __shared__ float red[1024 + 256 + 128];
  const Ctx c = make_ctx(p, nullptr);
  task_qkv(p, c, blockIdx.x, red);
}
__global__ void __launch_bounds__(kThreads) kd_attn(MoeParams p) {
  __shared__ float lds[kAttnLdsFloats];
  const Ctx c = make_ctx(p, nullptr);
  const int i = blockIdx.x;
  task_attn(p, c, i / (p.nkv * p.nchunk), (i / p.nchunk) % p.nkv, i % p.nchunk, lds);
}
__global__ void __launch_bounds__(kThreads) kd_attn_merge(MoeParams p) {
  const Ctx c = make_ctx(p, nullptr);
  task_attn_merge(p, c, blockIdx.x / p.nkv, blockIdx.x % p.nkv);
}
__global__ void __launch_bounds__(kThreads) kd_oproj(MoeParams p) {
  __shared__ float red[1024 + 256];
  const Ctx c = make_ctx(p, nullptr);
  task_oproj(p, c, blockIdx.x / kDecOSplit, blockIdx.x % kDecOSplit, red);
}
__global__ void __launch_bounds__(kThreads) kd_norm2(MoeParams p) {
  const Ctx c = make_ctx(p, nullptr);
  task_norm2(p, c, blockIdx.x);
}

// ------------------------------------------------------- host launchers --
// The variant a launch of T tokens runs: the wide G1 tiles from T * k on.
template <int MODE>
static void launch_variant(const MoeParams& p, int var, int grid, int lds_bytes, hipStream_t s) {
  if (var == kVarBig)
    hipLaunchKernelGGL((moe_persistent_big<MODE>), dim3(grid), dim3(kThreads), lds_bytes, s, p);
  else if (var == kVarWide)
    hipLaunchKernelGGL((moe_persistent<MODE, kVarWide>), dim3(grid), dim3(kThreads), lds_bytes, s, p);
  else
    hipLaunchKernelGGL((moe_persistent<MODE, kVarSmall>), dim3(grid), dim3(kThreads), lds_bytes, s, p);
}

int launch_moe_persistent(const MoeParams& p, int sched, int grid, int lds_bytes, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int wide = launch_variant_of(p.T, p.k, p.H, p.I);
  if (p.dec) {  // decoder layer: at most 16 tokens, the small-batch variant
    if (sched == ETC_SCHED_STATIC)
      hipLaunchKernelGGL((moe_persistent<MODE_STATIC, kVarSmall, true>), dim3(grid), dim3(kThreads), lds_bytes, s, p);
    else if (sched == ETC_SCHED_ORDERED)
      hipLaunchKernelGGL((moe_persistent<MODE_ORDERED, kVarSmall, true>), dim3(grid), dim3(kThreads), lds_bytes, s, p);
    else
      return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
  }
  switch (sched) {
    case ETC_SCHED_STATIC:
      launch_variant<MODE_STATIC>(p, wide, grid, lds_bytes, s);
      break;
    case ETC_SCHED_DYNAMIC:
      launch_variant<MODE_DYNAMIC>(p, wide, grid, lds_bytes, s);
      break;
    case ETC_SCHED_BARRIER:
      launch_variant<MODE_BARRIER>(p, wide, grid, lds_bytes, s);
      break;
    case ETC_SCHED_ORDERED:
      launch_variant<MODE_ORDERED>(p, wide, grid, lds_bytes, s);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Workgroups per CU that stay resident: the smaller of the small- and
// large-batch variants' (the grid must be resident whichever of the two a
// launch runs); the big-tile variant has its own grid (kBigSchedBase).
template <int MODE>
static hipError_t occupancy_both(int* blocks_per_cu, int lds_bytes) {
  int a = 0, b = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&a, moe_persistent<MODE, kVarSmall>, kThreads, lds_bytes);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, moe_persistent<MODE, kVarWide>, kThreads, lds_bytes);
  *blocks_per_cu = a < b ? a : b;
  return e;
}
template <int MODE>
static hipError_t occupancy_big(int* blocks_per_cu, int lds_bytes) {
  // the dynamic LDS above 64 KB must be allowed before the query and launch
  hipError_t e = hipFuncSetAttribute((const void*)moe_persistent_big<MODE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, moe_persistent_big<MODE>, kThreads, lds_bytes);
}

int moe_persistent_occupancy(int sched, int lds_bytes, int* blocks_per_cu) {
  hipError_t e;
  switch (sched) {
    case kDecSchedBase + ETC_SCHED_STATIC:
      return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, moe_persistent<MODE_STATIC, kVarSmall, true>,
                                                               kThreads, lds_bytes);
    case kDecSchedBase + ETC_SCHED_ORDERED:
      return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, moe_persistent<MODE_ORDERED, kVarSmall, true>,
                                                               kThreads, lds_bytes);
    case kBigSchedBase + ETC_SCHED_STATIC:
      return (int)occupancy_big<MODE_STATIC>(blocks_per_cu, lds_bytes);
    case kBigSchedBase + ETC_SCHED_ORDERED:
      return (int)occupancy_big<MODE_ORDERED>(blocks_per_cu, lds_bytes);
    case kBigSchedBase + ETC_SCHED_BARRIER:
      return (int)occupancy_big<MODE_BARRIER>(blocks_per_cu, lds_bytes);
    case kBigSchedBase + ETC_SCHED_DYNAMIC:
      return (int)occupancy_big<MODE_DYNAMIC>(blocks_per_cu, lds_bytes);
    case ETC_SCHED_STATIC:
      e = occupancy_both<MODE_STATIC>(blocks_per_cu, lds_bytes);
      break;
    case ETC_SCHED_DYNAMIC:
      e = occupancy_both<MODE_DYNAMIC>(blocks_per_cu, lds_bytes);
      break;
    case ETC_SCHED_BARRIER:
      e = occupancy_both<MODE_BARRIER>(blocks_per_cu, lds_bytes);
      break;
    case ETC_SCHED_ORDERED:
      e = occupancy_both<MODE_ORDERED>(blocks_per_cu, lds_bytes);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)e;
}

int launch_decoder_kbk(const MoeParams& p, int lds_bytes, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nN = (p.T + kDecNormT - 1) / kDecNormT;
  hipLaunchKernelGGL(kd_norm1, dim3(nN), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(kd_qkv, dim3((p.nq + 2 * p.nkv) * (kDecHd / 16)), dim3(kThreads), 0, s, p);
  if (p.nchunk > 0) hipLaunchKernelGGL(kd_attn, dim3(p.T * p.nkv * p.nchunk), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(kd_attn_merge, dim3(p.T * p.nkv), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(kd_oproj, dim3((p.H / 16) * kDecOSplit), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(kd_norm2, dim3(nN), dim3(kThreads), 0, s, p);
  const int e = (int)hipGetLastError();
  if (e != (int)hipSuccess) return e;
  return launch_moe_kbk(p, lds_bytes, stream);
}

int launch_moe_kbk(const MoeParams& p, int lds_bytes, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nTT = (p.T + kRouterT - 1) / kRouterT;
  const int nET = (p.E + router_experts(p.T) - 1) / router_experts(p.T);
  const int nC = (p.T + kCombineT - 1) / kCombineT;
  const int64_t rows = (int64_t)p.T * p.k;
  const bool big = big_variant(p.T, p.k, p.H, p.I);
  const int bm = big ? kBigBM : kBM;
  const int64_t max_rt = (rows + bm - 1) / bm + (rows < p.E ? rows : p.E);
  const int nN1 = p.I / (big ? kBigBN1 : g1_cols(p.T, p.k, p.H)), nN2 = p.H / (big ? kBigBN2 : g2_cols(p.T, p.k, p.I));
  hipLaunchKernelGGL(kbk_router, dim3(nTT * nET), dim3(kThreads), 0, s, p);
  hipLaunchKernelGGL(kbk_topk, dim3(nTT), dim3(kThreads), 0, s, p);
  const int nsch = (p.T + kScanChunkT - 1) / kScanChunkT;
  if (nsch > 1 && wide_variant(p.T, p.k, p.H, p.I)) {  // the persistent kernels' rule
    hipLaunchKernelGGL(kbk_scan_count, dim3(nsch), dim3(kThreads), lds_bytes, s, p);
    hipLaunchKernelGGL(kbk_scan_place, dim3(nsch), dim3(kThreads), lds_bytes, s, p);
  } else {
    hipLaunchKernelGGL(kbk_scan, dim3(1), dim3(kThreads), lds_bytes, s, p);
  }
  if (big) {
    hipError_t e = hipFuncSetAttribute((const void*)kbk_g1_big, hipFuncAttributeMaxDynamicSharedMemorySize, kBigLdsBytes);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)kbk_g2_big, hipFuncAttributeMaxDynamicSharedMemorySize, kBigLdsBytes);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(kbk_g1_big, dim3((unsigned)(max_rt * nN1)), dim3(kThreads), kBigLdsBytes, s, p);
    hipLaunchKernelGGL(kbk_g2_big, dim3((unsigned)(max_rt * nN2)), dim3(kThreads), kBigLdsBytes, s, p);
  } else {
    hipLaunchKernelGGL(kbk_g1, dim3((unsigned)(max_rt * nN1)), dim3(kThreads), 0, s, p);
    hipLaunchKernelGGL(kbk_g2, dim3((unsigned)(max_rt * nN2)), dim3(kThreads), 0, s, p);
  }
  hipLaunchKernelGGL(kbk_combine, dim3(nC), dim3(kThreads), 0, s, p);
  return (int)hipGetLastError();
}

// ------------------------------------------- static scratch (no-alloc) --
// The workspace of moe_layer_launch_noalloc, for callers that cannot
// allocate device memory.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress,
// once per device with that device current, and only that address is handed
// to kernels and to the fill kernel below.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

static std::mutex g_scratch_mu;
static std::vector<void*> g_scratch_ptr;  // per device

int moe_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return (int)hipSuccess;
}

__global__ void __launch_bounds__(256) fill_zero_u32(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

int moe_scratch_clear(void* ptr, size_t bytes, void* stream) {
  const size_t n = bytes / 4;
  const unsigned blocks = (unsigned)(n / 256 + 1 < 1024 ? n / 256 + 1 : 1024);
  hipLaunchKernelGGL(fill_zero_u32, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(ptr), n);
  return (int)hipGetLastError();
}

// ------------------------------------------- coherence self-test --
// Message passing between workgroups on different XCDs with exactly the
// protocol every notify and wait of the kernels relies on (no fences):
// the producer writes a 4 KB message with device-coherent stores, every
// wave waits for its stores, a workgroup barrier, then thread 0's relaxed
// device-scope atomic add; the consumer's thread 0 polls the counter with
// relaxed device-scope loads, a workgroup barrier, then device-coherent
// loads of the message, every word checked.  The consumer acknowledges
// each round the same way before the producer writes the next.  Workgroup
// 2 i produces for workgroup 2 i + 1 (consecutive workgroups are dealt to
// different XCDs).  Every wait has the watchdog, so the grid always drains.
// Words: ws[0] mismatched words, ws[1] timed-out waits; then per pair a
// ready and an ack counter on lines of their own, then the messages.
constexpr int kSelftestWords = kThreads * 4;  // message words a pair
__global__ void __launch_bounds__(kThreads) coherence_selftest(uint32_t* ws, int rounds, uint32_t msg_off,
                                                               uint64_t budget) {
  const int pair = blockIdx.x >> 1, role = blockIdx.x & 1, tid = threadIdx.x;
  uint32_t* ready = ws + kEvStride * (1 + 2 * pair);
  uint32_t* ack = ready + kEvStride;
  const rsrc_t rm = make_rsrc(ws + msg_off + (size_t)pair * kSelftestWords, kSelftestWords * 4u);
  uint32_t* status = ws + 1;  // a timeout sets it; every wait then gives up
  uint32_t bad = 0;
  for (int r = 1; r <= rounds; ++r) {
    if (role == 0) {
      if (r > 1 && !wg_wait(ack, (uint32_t)(r - 1), status, budget)) break;
      const u32x4_t v = {(uint32_t)r, (uint32_t)r ^ (uint32_t)tid, (uint32_t)r * 7u + (uint32_t)tid, ~(uint32_t)r};
      co_st128(rm, (uint32_t)tid * 16u, v);
      wg_publish();
      if (tid == 0) (void)add_relaxed(ready, 1u);
    } else {
      if (!wg_wait(ready, (uint32_t)r, status, budget)) break;
      const u32x4_t v = co_ld128(rm, (uint32_t)tid * 16u);
      bad += (v.x != (uint32_t)r) + (v.y != ((uint32_t)r ^ (uint32_t)tid)) +
             (v.z != (uint32_t)r * 7u + (uint32_t)tid) + (v.w != ~(uint32_t)r);
      __syncthreads();  // every thread has its message words before the ack
      if (tid == 0) (void)add_relaxed(ack, 1u);
    }
  }
  if (bad) atomicAdd(ws, bad);
}

int launch_coherence_selftest(uint32_t* ws, int pairs, int rounds, uint64_t budget, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t words = (size_t)kEvStride * (1 + 2 * pairs) + (size_t)pairs * kSelftestWords;
  hipLaunchKernelGGL(fill_zero_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, ws, words);
  hipLaunchKernelGGL(coherence_selftest, dim3(2 * pairs), dim3(kThreads), 0, s, ws, rounds,
                     (uint32_t)(kEvStride * (1 + 2 * pairs)), budget);
  return (int)hipGetLastError();
}
int coherence_selftest_occupancy(int* blocks_per_cu) {
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, coherence_selftest, kThreads, 0);
}
size_t coherence_selftest_words(int pairs) {
  return (size_t)kEvStride * (1 + 2 * pairs) + (size_t)pairs * kSelftestWords;
}


}  // namespace etc
