// Device-side event-tensor runtime for gfx950 (CDNA4): counters in HBM,
// notify = agent-scope atomic add after a release fence, wait = relaxed
// polling with s_sleep back-off and a spin budget, then an acquire fence.
//
// An event tensor element is a 32-bit arrival counter that starts at zero;
// it is released once `wait_count` notifies have arrived.  The pages count
// down from the wait_count to zero (Event Tensor, arXiv 2604.13327, Fig. 7;
// podcast cue 11); counting arrivals up to the wait_count is the same state
// machine (remaining = wait_count - arrivals) and lets a counter that the
// kernel has just zeroed serve any wait_count, including one written later
// by the task that computes it (data-dependent update, Fig. 5b; podcast
// cue 7).
//
// Coherence across the 8 XCDs (each with its own L2) relies on the AMDGPU
// memory model at agent scope: a release fence makes this wave's prior global
// stores visible device-wide before the counter update; an acquire fence
// after observing the counter makes the producer's data visible to the
// following loads.  Counters themselves are only touched with agent-scope
// atomics.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "etc_internal.h"

namespace etc {

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_relaxed64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Signals that another workgroup polls are always written with an atomic
// read-modify-write (swap), never with a plain or atomic store.  A release
// store writes the L2 back *before* the signal, so the signal word itself can
// stay dirty in the writer's XCD-local L2 while pollers on other XCDs read
// past it; read-modify-writes are performed where every XCD sees them (the
// event counters rely on exactly that).
__device__ __forceinline__ void sig_put(uint32_t* p, uint32_t v) {
  (void)__hip_atomic_exchange(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void sig_put64(uint64_t* p, uint64_t v) {
  (void)__hip_atomic_exchange(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
// Plain relaxed store: only for words read after a kernel boundary.
__device__ __forceinline__ void st_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_acqrel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_relaxed(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void or_relaxed(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }

// Wall-clock watchdog: every in-kernel wait gives up once `budget` ticks of
// the constant-rate real-time counter have passed since the wait began (the
// host converts microseconds to ticks with the device's wall-clock rate), so
// a wait ends in bounded time however contended the polled line is.
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

// Whole-workgroup wait on one event element.  Thread 0 polls; the others
// wait at the barrier; everyone then takes an acquire fence.  Returns false
// on abort (uniform across the workgroup).
__device__ __forceinline__ bool wg_wait(const uint32_t* ctr, uint32_t target, uint32_t* status,
                                        uint64_t budget) {
  int fail = 0;
  if (threadIdx.x == 0) fail = spin_until_geq(ctr, target, status, budget) ? 0 : 1;
  fail = __syncthreads_or(fail);
  fence_acquire();
  return fail == 0;
}

// Publish the workgroup's global writes before a notify: every thread
// releases its own stores at agent scope, then the barrier orders them
// before the notifying thread's atomic.
__device__ __forceinline__ void wg_publish() {
  fence_release();
  __syncthreads();
}

}  // namespace etc
