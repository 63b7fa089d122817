// The split-K row-sum example through the device event runtime (Event
// Tensor, arXiv 2604.13327, Fig. 3; podcast cue 3):
//   partial_sum(i, j): B[i, j] = sum of A[i, j*bk .. (j+1)*bk), then notify
//                      the event element of its out-edge     (the pages: "ij->i")
//   final_sum(i)     : wait on the element of its in-edge      (the pages: "i->i")
//                      until wait_count notifies, then C[i] = sum_j B[i, j]
// The edges arrive compiled (etc_edge_compile): an element index is
// sum_d coord[src[d]] * stride[d] of the task's coordinate.  Row i's final
// sum starts as soon as its own partial sums land, whatever the other rows
// are doing.
//
// Counters: final_sum(i) is the only waiter of its element, so after its
// wait it returns the counter to zero; the control words (queue head / tail, done
// count) are returned to zero by the last workgroup to finish; each queue
// slot is cleared by the workgroup that pops it.  The next launch therefore
// finds everything at rest without a host-side memset.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "etc_internal.h"
#include "etc_rt.h"

namespace etc {

struct SkParams {
  const int32_t* A;
  int32_t* B;
  int32_t* C;
  uint32_t* ev;
  etc_edge ne, we;      // out-edge of partial_sum (grid [n, nsplit]), in-edge of final_sum (grid [n])
  uint32_t wait_count;  // notifies that complete an element (the out-edge's fan-in)
  uint32_t* ctl;
  uint32_t* queue;
  int64_t q_cap;
  int n, nsplit, bk;
  uint64_t budget;
};

__device__ int block_sum_i32(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  if (lane == 0) tmp[wv] = v;
  __syncthreads();
  const int r = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return r;
}

// B crosses workgroups: written and read with device-coherent accesses
__device__ __forceinline__ rsrc_t r_B(const SkParams& p) {
  return make_rsrc(p.B, (uint32_t)((int64_t)p.n * p.nsplit * 4));
}

__device__ void sk_partial(const SkParams& p, int i, int j, int* tmp) {
  const int32_t* row = p.A + ((size_t)i * p.nsplit + j) * p.bk;
  int v = 0;
  for (int c = threadIdx.x; c < p.bk; c += kThreads) v += row[c];
  v = block_sum_i32(v, tmp);
  if (threadIdx.x == 0) co_st32(r_B(p), (uint32_t)(i * p.nsplit + j) * 4u, (uint32_t)v);
}

__device__ void sk_final(const SkParams& p, int i, int* tmp) {
  const rsrc_t rb = r_B(p);
  int v = 0;
  for (int j = threadIdx.x; j < p.nsplit; j += kThreads) v += (int)co_ld32(rb, (uint32_t)(i * p.nsplit + j) * 4u);
  v = block_sum_i32(v, tmp);
  if (threadIdx.x == 0) p.C[i] = v;
}

// the element an edge maps a task coordinate to
__device__ __forceinline__ uint32_t edge_elem(const etc_edge& e, int c0, int c1) {
  int64_t f = 0;
  for (int d = 0; d < e.event_ndim; ++d) f += (int64_t)(e.src[d] == 0 ? c0 : c1) * e.stride[d];
  return (uint32_t)f;
}
// notify element e; true if this notify released it
__device__ __forceinline__ bool sk_notify(const SkParams& p, uint32_t e) {
  const uint32_t old = add_relaxed(p.ev + e, 1u);
  if (old + 1u > p.wait_count) or_relaxed(p.ctl + SK_STATUS, ST_OVER_NOTIFY | ST_ABORT);
  return old + 1u == p.wait_count;
}

struct SkTasks {
  const SkParams& p;
  int* tmp;
  __device__ __forceinline__ uint32_t notify_elem(uint32_t i, uint32_t j) { return edge_elem(p.ne, (int)i, (int)j); }
  // the in-edge pairs every element with one final sum (the host checked):
  // a 1-d grid onto a 1-d tensor, element e is waited on by final_sum(e)
  __device__ __forceinline__ uint32_t waiter(uint32_t e) { return e; }
  __device__ __forceinline__ void partial(uint32_t i, uint32_t j) { sk_partial(p, (int)i, (int)j, tmp); }
  __device__ __forceinline__ void final_sum(uint32_t i) {
    if (threadIdx.x == 0) xchg_relaxed(p.ev + edge_elem(p.we, (int)i, 0), 0u);  // sole waiter: back to rest
    sk_final(p, (int)i, tmp);
  }
};

template <int MODE>
__global__ void __launch_bounds__(kThreads) splitk_persistent(SkParams p) {
  __shared__ int tmp[8];
  const int G = gridDim.x, w = blockIdx.x;
  const int nP = p.n * p.nsplit;
  uint32_t* status = p.ctl + SK_STATUS;
  dyn::Queue q;
  q.head = p.ctl + SK_HEAD;
  q.tail = p.ctl + SK_TAIL;
  q.total = nullptr;
  q.status = status;
  q.slot = p.queue;
  q.cap = p.q_cap;
  q.prefix = (uint32_t)nP;
  q.known_total = (uint32_t)(nP + p.n);
  q.budget = p.budget;
  if (MODE == ETC_SCHED_STATIC) {
    // phase-ordered lists: all partial sums, then all final sums
    for (int t = w; t < nP; t += G) {
      const int i = t / p.nsplit, j = t % p.nsplit;
      sk_partial(p, i, j, tmp);
      wg_publish();
      if (threadIdx.x == 0) sk_notify(p, edge_elem(p.ne, i, j));
    }
    for (int i = (w - nP % G + G) % G; i < p.n; i += G) {
      const uint32_t e = edge_elem(p.we, i, 0);
      if (!wg_wait(p.ev + e, p.wait_count, status, p.budget)) break;
      if (threadIdx.x == 0) xchg_relaxed(p.ev + e, 0u);  // sole waiter: back to rest
      sk_final(p, i, tmp);
    }
  } else {
    // push / pop (dyn_sched.h): the partial sums are the ready prefix; the
    // notify that completes event i pushes final_sum(i) at once
    __shared__ dyn::Shared dsh;
    SkTasks tk{p, tmp};
    dyn::run_splitk<DevPlat>(tk, q, (uint32_t)p.nsplit, p.wait_count, p.ev, dsh);
  }
  wg_publish();
  if (threadIdx.x == 0) {
    const uint32_t old = add_relaxed(p.ctl + SK_DONE, 1u);
    if (old == (uint32_t)G - 1u) {
      const uint32_t st = ld_relaxed(status) & ~ST_ABORT;
      if (st) or_relaxed(p.ctl + SK_REPORT, st);
      dyn::splitk_reset<DevPlat>(q);
      xchg_relaxed(p.ctl + SK_DONE, 0u);
    }
  }
}

int launch_splitk(int n, int nsplit, int bk, const int32_t* A, int32_t* B, int32_t* C, int32_t* ev,
                  const etc_edge& notify_edge, const etc_edge& wait_edge, int32_t wait_count, uint32_t* ctl,
                  uint32_t* queue, int64_t q_cap, int sched, int grid, uint64_t budget, void* stream) {
  SkParams p;
  p.A = A; p.B = B; p.C = C;
  p.ev = reinterpret_cast<uint32_t*>(ev);
  p.ne = notify_edge;
  p.we = wait_edge;
  p.wait_count = (uint32_t)wait_count;
  p.ctl = ctl;
  p.queue = queue;
  p.q_cap = q_cap;
  p.n = n; p.nsplit = nsplit; p.bk = bk;
  p.budget = budget;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (sched == ETC_SCHED_STATIC)
    hipLaunchKernelGGL((splitk_persistent<ETC_SCHED_STATIC>), dim3(grid), dim3(kThreads), 0, s, p);
  else if (sched == ETC_SCHED_DYNAMIC)
    hipLaunchKernelGGL((splitk_persistent<ETC_SCHED_DYNAMIC>), dim3(grid), dim3(kThreads), 0, s, p);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

int splitk_occupancy(int sched, int* blocks_per_cu) {
  if (sched == ETC_SCHED_STATIC)
    return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(
        blocks_per_cu, splitk_persistent<ETC_SCHED_STATIC>, kThreads, 0);
  return (int)hipOccupancyMaxActiveBlocksPerMultiprocessor(
      blocks_per_cu, splitk_persistent<ETC_SCHED_DYNAMIC>, kThreads, 0);
}

}  // namespace etc
