// Device-side event-tensor runtime for gfx950 (CDNA4): counters in HBM,
// notify = device-scope atomic add, wait = polling with s_sleep back-off and
// a wall-clock watchdog.
//
// An event tensor element is a 32-bit arrival counter that starts at zero;
// it is released once `wait_count` notifies have arrived.  The pages count
// down from the wait_count to zero (Event Tensor, arXiv 2604.13327, Fig. 7;
// podcast cue 11); counting arrivals up to the wait_count is the same state
// machine (remaining = wait_count - arrivals) and lets a counter that the
// kernel has just zeroed serve any wait_count, including one written later by
// the task that computes it (data-dependent update, Fig. 5b; podcast cue 7).
//
// Coherence across the 8 XCDs (each with its own write-back L2).  Release and
// acquire fences at agent scope are implemented on this chip as an L2-wide
// write-back and an L2-wide invalidate; issued per task by hundreds of
// workgroups they cost more than the tasks themselves.  The kernels therefore
// never use them.  Instead every datum that crosses workgroups is written and
// read with device-coherent accesses (the sc1 cache policy: buffer loads and
// stores below, and device-scope atomics for counters), and a producer's
// waves each wait until their own stores have completed (s_waitcnt) before
// the workgroup barrier that precedes the notifying atomic.  A consumer that
// has observed the counter then reads the data with device-coherent loads.
// Ordinary (cached) accesses are used only for data no workgroup writes during
// the launch (weights, activations) and for the final output.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "etc_internal.h"

namespace etc {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// ---- counters: device-scope atomics, relaxed (ordering comes from the
// store-completion wait and barrier described above) -----------------------
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t xchg_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- device-coherent data accesses through buffer resources --------------
// A buffer resource also bounds every access: offsets past `bytes` read 0
// and drop the store.
constexpr int kCoherent = 16;  // cache policy bit sc1: device scope
typedef unsigned int gcc_u32x4 __attribute__((__vector_size__(16)));
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t co_ld128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent));
}
__device__ __forceinline__ void co_st128(rsrc_t r, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(gcc_u32x4, v), r, (int)off, 0, kCoherent);
}
__device__ __forceinline__ uint32_t co_ld32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCoherent);
}
__device__ __forceinline__ void co_st32(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kCoherent);
}
__device__ __forceinline__ float co_ldf(rsrc_t r, uint32_t off) { return __uint_as_float(co_ld32(r, off)); }
__device__ __forceinline__ void co_stf(rsrc_t r, uint32_t off, float v) { co_st32(r, off, __float_as_uint(v)); }

// ---- watchdog ---------------------------------------------------------------
// Every in-kernel wait gives up once `budget` ticks of the constant-rate
// wall clock have passed since it began (the host converts microseconds to
// ticks with the device's wall-clock rate), so a wait ends in bounded time
// however contended the polled line is.
__device__ __forceinline__ uint64_t now_ticks() { return wall_clock64(); }

// Spin (one thread) until *ctr >= target.  Returns false if the launch is
// aborting or the watchdog expired (then ST_TIMEOUT | ST_ABORT is set so
// every other workgroup leaves its own waits too and the grid drains).
__device__ __forceinline__ bool spin_until_geq(const uint32_t* ctr, uint32_t target, uint32_t* status,
                                               uint64_t budget) {
  if (ld_relaxed(ctr) >= target) return true;
  const uint64_t t0 = now_ticks();
  for (uint32_t spins = 1;; ++spins) {
    if (ld_relaxed(ctr) >= target) return true;
    if ((spins & 7u) == 0u) {
      if (ld_relaxed(status) & ST_ABORT) return false;
      if (now_ticks() - t0 > budget) {
        or_relaxed(status, ST_TIMEOUT | ST_ABORT);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// As spin_until_geq, and hands back the value that satisfied the wait.
__device__ __forceinline__ bool spin_value_geq(const uint32_t* ctr, uint32_t target, uint32_t* status,
                                               uint64_t budget, uint32_t* seen) {
  const uint64_t t0 = now_ticks();
  for (uint32_t spins = 1;; ++spins) {
    const uint32_t v = ld_relaxed(ctr);
    if (v >= target) {
      *seen = v;
      return true;
    }
    if ((spins & 7u) == 0u) {
      if (ld_relaxed(status) & ST_ABORT) return false;
      if (now_ticks() - t0 > budget) {
        or_relaxed(status, ST_TIMEOUT | ST_ABORT);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Whole-workgroup wait on one event element: thread 0 polls, the barrier
// releases the others.  Data produced before the notifies is then read with
// device-coherent loads.  Returns false on abort (uniform in the workgroup).
__device__ __forceinline__ bool wg_wait(const uint32_t* ctr, uint32_t target, uint32_t* status,
                                        uint64_t budget) {
  int fail = 0;
  if (threadIdx.x == 0) fail = spin_until_geq(ctr, target, status, budget) ? 0 : 1;
  fail = __syncthreads_or(fail);
  return fail == 0;
}

// Before a notify: each wave waits until its own (device-coherent) stores
// have completed, then the barrier orders all of them before the notifying
// thread's atomic.
// Workgroup barrier that orders LDS accesses only: global stores issued
// before it keep draining across it (__syncthreads also waits for their
// acknowledgements).  For phases that hand each other LDS tables while
// their results go out to memory; a wg_publish still precedes any notify.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void wg_publish() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// The device side of the dynamic schedule's platform interface (dyn_sched.h):
// relaxed device-scope atomics, the coherent polling load, s_sleep, the
// wall clock and the workgroup barriers above.
struct DevPlat {
  static constexpr int kThreads = etc::kThreads;
  __device__ __forceinline__ static int tid() { return (int)threadIdx.x; }
  __device__ __forceinline__ static uint32_t add(uint32_t* p, uint32_t v) { return add_relaxed(p, v); }
  __device__ __forceinline__ static uint32_t load(const uint32_t* p) { return ld_relaxed(p); }
  // descriptors and the total are published with a swap (a read-modify-write
  // is performed where every XCD's coherent loads see it)
  __device__ __forceinline__ static void put(uint32_t* p, uint32_t v) { (void)xchg_relaxed(p, v); }
  __device__ __forceinline__ static void orr(uint32_t* p, uint32_t v) { or_relaxed(p, v); }
  __device__ __forceinline__ static uint64_t now() { return now_ticks(); }
  __device__ __forceinline__ static void pause() { __builtin_amdgcn_s_sleep(2); }
  __device__ __forceinline__ static void barrier() { __syncthreads(); }
  __device__ __forceinline__ static void publish() { wg_publish(); }
  __device__ __forceinline__ static int lds_add(int* p, int v) { return atomicAdd(p, v); }
};

}  // namespace etc
