// Host side of the C ABI declared in include/etc.h: argument validation,
// event-tensor handles, workspace layout, grid sizing from the occupancy
// query, launch, and the status report read back by etc_sync.  Allocates
// nothing on the MoE launch path.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "etc_internal.h"

using namespace etc;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(ETC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Launches since the last etc_sync on each stream: where their status
// report word lives.
struct Pending {
  void* stream;
  uint32_t* report;
};
std::mutex g_mu;
std::vector<Pending> g_pending;

void add_pending(void* stream, uint32_t* report) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (const Pending& p : g_pending)
    if (p.stream == stream && p.report == report) return;
  g_pending.push_back({stream, report});
}

int status_to_code(uint32_t st) {
  if (st & ST_TIMEOUT) return fail(ETC_ERR_TIMEOUT, "an in-kernel wait outlived its watchdog (status 0x%x)", st);
  if (st & (ST_OVER_NOTIFY | ST_QUEUE_OVERFLOW))
    return fail(ETC_ERR_INVARIANT, "event over-notified or queue overflow (status 0x%x)", st);
  if (st & ST_NONFINITE) return fail(ETC_ERR_NONFINITE, "NaN router logit (status 0x%x)", st);
  return ETC_OK;
}

// Per-device facts for grid sizing and the watchdog.
struct OccEntry {
  int sched, lds, blocks_per_cu;
};
struct DeviceFacts {
  int cus = 0;
  int wall_khz = 0;  // rate of the constant wall clock the kernels read
  std::vector<OccEntry> occ;  // persistent kernels' occupancy, queried once per (schedule, LDS bytes)
};
std::mutex g_dev_mu;
std::vector<DeviceFacts> g_dev;

int device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  if (g_dev[dev].cus == 0) {
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
    g_dev[dev].cus = v;
  }
  *cus = g_dev[dev].cus;
  return ETC_OK;
}

// Microseconds of wall time (0 = default) to ticks of the device wall clock.
int watchdog_ticks(uint32_t us, uint64_t* ticks) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int khz = 0;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
    if (g_dev[dev].wall_khz == 0) {
      int v = 0;
      e = hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev);
      if (e != hipSuccess || v <= 0) v = 100000;  // 100 MHz, the CDNA real-time counter
      g_dev[dev].wall_khz = v;
    }
    khz = g_dev[dev].wall_khz;
  }
  const uint64_t u = us ? us : kDefaultWatchdogUs;
  *ticks = u * (uint64_t)khz / 1000u;
  if (*ticks == 0) *ticks = 1;
  return ETC_OK;
}

int wg_per_cu_cap() {
  const char* s = std::getenv("ETC_WG_PER_CU");
  if (s && *s) {
    int v = std::atoi(s);
    if (v >= 1 && v <= 16) return v;
  }
  return 2;
}

int desc_check(const etc_moe_desc* d) {
  if (!d) return fail(ETC_ERR_INVALID, "descriptor is NULL");
  if (d->T_max < 1 || d->T_max > kMaxTmax) return fail(ETC_ERR_INVALID, "T_max %d outside [1, %d]", d->T_max, kMaxTmax);
  if (d->H < 128 || d->H % 128 || d->H > kMaxHI) return fail(ETC_ERR_INVALID, "H %d must be a positive multiple of 128, <= %d", d->H, kMaxHI);
  if (d->I < 128 || d->I % 128 || d->I > kMaxHI) return fail(ETC_ERR_INVALID, "I %d must be a positive multiple of 128, <= %d", d->I, kMaxHI);
  if (d->E < 1 || d->E > kMaxE) return fail(ETC_ERR_INVALID, "E %d outside [1, %d]", d->E, kMaxE);
  if (d->k < 1 || d->k > kMaxK || d->k > d->E) return fail(ETC_ERR_INVALID, "k %d outside [1, min(E, %d)]", d->k, kMaxK);
  if ((int64_t)d->T_max * d->k * (d->H > d->I ? d->H : d->I) * 2 >= (int64_t)1 << 31)
    return fail(ETC_ERR_INVALID, "T_max * k * max(H, I) * 2 bytes must stay below 2 GiB");
  if (d->norm_topk != 0 && d->norm_topk != 1) return fail(ETC_ERR_INVALID, "norm_topk must be 0 or 1");
  if (d->has_bias != 0 && d->has_bias != 1) return fail(ETC_ERR_INVALID, "has_bias must be 0 or 1");
  return ETC_OK;
}

int64_t lds_bytes_for(const etc_moe_desc* d) {
  int64_t s = scan_lds_bytes(d->E, d->T_max);
  return s > kGemmLdsBytes ? s : kGemmLdsBytes;
}
// the big-tile variant's dynamic LDS: its G stages, or the scan's if larger
int64_t big_lds_bytes(const etc_moe_desc* d) {
  const int64_t s = lds_bytes_for(d);
  return s > kBigLdsBytes ? s : kBigLdsBytes;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Persistent grid: as many workgroups as stay resident together (capped per
// CU).  `solo` is the CU count when the grid holds several workgroups a CU
// (the first `solo` workgroups are then placed on distinct CUs), else 0.
int persistent_grid(int sched, int lds, int* grid, int* solo = nullptr) {
  int cus = 0;
  int rc = device_cus(&cus);
  if (rc) return rc;
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  int nb = -1;
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    for (const OccEntry& o : g_dev[dev].occ)
      if (o.sched == sched && o.lds == lds) nb = o.blocks_per_cu;
  }
  if (nb < 0) {  // first launch of this schedule and LDS size on this device
    int e = moe_persistent_occupancy(sched, lds, &nb);
    if (e != hipSuccess) return hip_fail((hipError_t)e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
    std::lock_guard<std::mutex> lk(g_dev_mu);
    g_dev[dev].occ.push_back({sched, lds, nb});
  }
  if (nb < 1) return fail(ETC_ERR_UNSUPPORTED, "persistent kernel does not fit on a CU (lds %d)", lds);
  const int cap = wg_per_cu_cap();
  if (nb > cap) nb = cap;
  *grid = nb * cus;
  if (solo) *solo = nb >= 2 ? cus : 0;
  return ETC_OK;
}

// library-owned control block for the split-K example (one per device)
struct SplitkCtl {
  uint32_t* ctl = nullptr;
  uint32_t* queue = nullptr;
  int64_t q_cap = 0;
};
std::vector<SplitkCtl> g_sk;

}  // namespace

// ======================================================== event tensors ==
struct etc_etensor {
  int ndim;
  int64_t shape[ETC_MAX_DIMS];  // declared (may hold ETC_DIM_SYMBOLIC)
  int64_t bound[ETC_MAX_DIMS];  // current instantiation
  int instantiated;
  int32_t wait_count;
  int32_t* counters;
  int owns;
  int64_t capacity;  // counters available
  int needs_zero;
};

extern "C" int etensor_create(etc_etensor** out, int ndim, const int64_t* shape, int32_t wait_count,
                              int32_t* dev_counters) {
  if (!out || !shape) return fail(ETC_ERR_INVALID, "NULL argument");
  *out = nullptr;
  if (ndim < 1 || ndim > ETC_MAX_DIMS) return fail(ETC_ERR_INVALID, "ndim %d outside [1, %d]", ndim, ETC_MAX_DIMS);
  if (wait_count < 0 && wait_count != ETC_WAIT_DATA_DEPENDENT) return fail(ETC_ERR_INVALID, "wait_count %d", wait_count);
  for (int i = 0; i < ndim; ++i)
    if (shape[i] < 1 && shape[i] != ETC_DIM_SYMBOLIC) return fail(ETC_ERR_INVALID, "shape[%d] = %lld", i, (long long)shape[i]);
  etc_etensor* et = new (std::nothrow) etc_etensor();
  if (!et) return fail(ETC_ERR_INVALID, "out of host memory");
  et->ndim = ndim;
  bool symbolic = false;
  for (int i = 0; i < ETC_MAX_DIMS; ++i) {
    et->shape[i] = i < ndim ? shape[i] : 1;
    et->bound[i] = et->shape[i];
    if (i < ndim && shape[i] == ETC_DIM_SYMBOLIC) symbolic = true;
  }
  et->instantiated = symbolic ? 0 : 1;
  et->wait_count = wait_count;
  et->counters = dev_counters;
  et->owns = 0;
  et->capacity = dev_counters ? INT64_MAX : 0;
  et->needs_zero = 0;
  *out = et;
  return ETC_OK;
}

extern "C" int etensor_instantiate(etc_etensor* et, const int64_t* concrete) {
  if (!et || !concrete) return fail(ETC_ERR_INVALID, "NULL argument");
  for (int i = 0; i < et->ndim; ++i) {
    if (concrete[i] < 1) return fail(ETC_ERR_INVALID, "concrete_shape[%d] = %lld", i, (long long)concrete[i]);
    if (et->shape[i] != ETC_DIM_SYMBOLIC && et->shape[i] != concrete[i])
      return fail(ETC_ERR_INVALID, "dimension %d is fixed at %lld, got %lld", i, (long long)et->shape[i],
                  (long long)concrete[i]);
  }
  for (int i = 0; i < et->ndim; ++i) et->bound[i] = concrete[i];
  et->instantiated = 1;
  return ETC_OK;
}

extern "C" int etensor_shape(const etc_etensor* et, int64_t* shape_out, int* ndim_out, int64_t* numel_out) {
  if (!et) return fail(ETC_ERR_INVALID, "NULL event tensor");
  int64_t numel = 1;
  for (int i = 0; i < et->ndim; ++i) {
    const int64_t d = et->instantiated ? et->bound[i] : et->shape[i];
    if (shape_out) shape_out[i] = d;
    numel *= d;
  }
  if (shape_out)
    for (int i = et->ndim; i < ETC_MAX_DIMS; ++i) shape_out[i] = 0;
  if (ndim_out) *ndim_out = et->ndim;
  if (numel_out) *numel_out = et->instantiated ? numel : 0;
  return ETC_OK;
}

extern "C" int etensor_destroy(etc_etensor* et) {
  if (!et) return ETC_OK;
  if (et->owns && et->counters) (void)hipFree(et->counters);
  delete et;
  return ETC_OK;
}

static int etensor_numel(const etc_etensor* et) {
  int64_t n = 0;
  etensor_shape(et, nullptr, nullptr, &n);
  return (int)n;
}

// Counters for a launch: caller-owned, or allocated here once (a set-up
// cost, never on the MoE path) and zeroed.
static int etensor_device_counters(etc_etensor* et, int64_t numel, void* stream) {
  if (et->counters && et->capacity >= numel && !et->needs_zero) return ETC_OK;
  if (!et->counters || et->capacity < numel) {
    if (et->counters && !et->owns)
      return fail(ETC_ERR_INVALID, "caller-owned counters are smaller than the instantiation");
    if (et->counters) (void)hipFree(et->counters);
    et->counters = nullptr;
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&et->counters), (size_t)numel * 4);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(event counters)");
    et->owns = 1;
    et->capacity = numel;
    et->needs_zero = 1;
  }
  if (et->needs_zero) {
    hipError_t e = hipMemsetAsync(et->counters, 0, (size_t)et->capacity * 4, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync(event counters)");
    et->needs_zero = 0;
  }
  return ETC_OK;
}

// ================================================================= edges ==
extern "C" int etc_edge_compile(const etc_etensor* et, const char* spec, const int64_t* task_shape, int task_ndim,
                                etc_edge* out) {
  if (!et || !spec || !task_shape || !out) return fail(ETC_ERR_INVALID, "NULL argument");
  if (!et->instantiated) return fail(ETC_ERR_INVALID, "event tensor is not instantiated");
  if (task_ndim < 1 || task_ndim > ETC_MAX_DIMS)
    return fail(ETC_ERR_INVALID, "task_ndim %d outside [1, %d]", task_ndim, ETC_MAX_DIMS);
  const char* arrow = std::strstr(spec, "->");
  if (!arrow || std::strstr(arrow + 2, "->")) return fail(ETC_ERR_INVALID, "edge \"%s\": expected one \"->\"", spec);
  std::string L, R;
  for (const char* c = spec; *c; ++c) {
    if (c == arrow || c == arrow + 1) continue;
    if (*c == ' ') continue;
    if (*c < 'a' || *c > 'z') return fail(ETC_ERR_INVALID, "edge \"%s\": '%c' is not a lowercase letter", spec, *c);
    (c < arrow ? L : R).push_back(*c);
  }
  if ((int)L.size() != task_ndim)
    return fail(ETC_ERR_INVALID, "edge \"%s\" names %zu task dimensions, the grid has %d", spec, L.size(), task_ndim);
  if ((int)R.size() != et->ndim)
    return fail(ETC_ERR_INVALID, "edge \"%s\" names %zu event dimensions, the tensor has %d", spec, R.size(),
                et->ndim);
  for (size_t a = 0; a < L.size(); ++a)
    for (size_t b = a + 1; b < L.size(); ++b)
      if (L[a] == L[b]) return fail(ETC_ERR_INVALID, "edge \"%s\": task letter '%c' repeats", spec, L[a]);
  for (size_t a = 0; a < R.size(); ++a)
    for (size_t b = a + 1; b < R.size(); ++b)
      if (R[a] == R[b]) return fail(ETC_ERR_INVALID, "edge \"%s\": event letter '%c' repeats", spec, R[a]);
  for (int i = 0; i < task_ndim; ++i)
    if (task_shape[i] < 1) return fail(ETC_ERR_INVALID, "task_shape[%d] = %lld", i, (long long)task_shape[i]);
  etc_edge e{};
  e.task_ndim = task_ndim;
  e.event_ndim = et->ndim;
  for (int i = 0; i < task_ndim; ++i) e.task_shape[i] = task_shape[i];
  int64_t stride = 1;
  for (int d = et->ndim - 1; d >= 0; --d) {
    const size_t pos = L.find(R[d]);
    if (pos == std::string::npos)
      return fail(ETC_ERR_INVALID, "edge \"%s\": event letter '%c' is not a task letter", spec, R[d]);
    if (task_shape[pos] != et->bound[d])
      return fail(ETC_ERR_INVALID, "edge \"%s\": task dimension '%c' has %lld, event dimension %d has %lld", spec,
                  R[d], (long long)task_shape[pos], d, (long long)et->bound[d]);
    e.src[d] = (int32_t)pos;
    e.stride[d] = stride;
    stride *= et->bound[d];
  }
  e.event_numel = stride;
  e.fan_in = 1;
  for (int i = 0; i < task_ndim; ++i)
    if (R.find(L[i]) == std::string::npos) e.fan_in *= task_shape[i];
  *out = e;
  return ETC_OK;
}

extern "C" int64_t etc_edge_index(const etc_edge* edge, const int64_t* task_coord) {
  if (!edge || !task_coord) return -1;
  int64_t f = 0;
  for (int d = 0; d < edge->event_ndim; ++d) f += task_coord[edge->src[d]] * edge->stride[d];
  return f;
}

extern "C" int etc_splitk_launch(etc_etensor* ev, int32_t n, int32_t nsplit, int32_t bk, const int32_t* A,
                                 int32_t* B, int32_t* C, const etc_edge* notify_edge, const etc_edge* wait_edge,
                                 int sched, void* stream) {
  if (!ev || !A || !B || !C || !notify_edge || !wait_edge) return fail(ETC_ERR_INVALID, "NULL argument");
  if (sched != ETC_SCHED_STATIC && sched != ETC_SCHED_DYNAMIC)
    return fail(ETC_ERR_UNSUPPORTED, "split-K runs under STATIC or DYNAMIC only");
  if (sched == ETC_SCHED_DYNAMIC)
    return fail(ETC_ERR_UNSUPPORTED,
                "the dynamic (push/pop) schedule is switched off: it shares the queue protocol of the MoE "
                "dynamic schedule, whose launch did not complete on the GPU");
  if (n < 1 || nsplit < 1 || bk < 1 || (int64_t)n * nsplit > (1 << 28))
    return fail(ETC_ERR_INVALID, "bad sizes n=%d nsplit=%d bk=%d", n, nsplit, bk);
  if (!ev->instantiated) return fail(ETC_ERR_INVALID, "event tensor is not instantiated");
  const int64_t numel = etensor_numel(ev);
  const etc_edge& ne = *notify_edge;
  const etc_edge& we = *wait_edge;
  if (ne.task_ndim != 2 || ne.task_shape[0] != n || ne.task_shape[1] != nsplit)
    return fail(ETC_ERR_INVALID, "notify edge must be compiled for the partial-sum grid [n=%d, nsplit=%d]", n, nsplit);
  if (we.task_ndim != 1 || we.task_shape[0] != n)
    return fail(ETC_ERR_INVALID, "wait edge must be compiled for the final-sum grid [n=%d]", n);
  if (ne.event_ndim != ev->ndim || we.event_ndim != ev->ndim || ne.event_numel != numel || we.event_numel != numel)
    return fail(ETC_ERR_INVALID, "edges were compiled for another instantiation of the event tensor");
  if (ev->wait_count != ne.fan_in)
    return fail(ETC_ERR_INVALID, "event wait_count %d != the notify edge's fan-in %lld", ev->wait_count,
                (long long)ne.fan_in);
  // every element is waited on by exactly one final sum (it returns the
  // counter to rest after its wait, and the dynamic schedule pushes it)
  if (we.fan_in != 1 || numel != n)
    return fail(ETC_ERR_INVALID, "wait edge must pair each event element with one final sum");
  int rc = etensor_device_counters(ev, numel, stream);
  if (rc) return rc;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_sk.size() <= dev) g_sk.resize(dev + 1);
  }
  SplitkCtl& sk = g_sk[dev];
  if (sk.q_cap < n) {
    if (sk.ctl) (void)hipFree(sk.ctl);
    const int64_t cap = n > 4096 ? n : 4096;
    const size_t bytes = kSkCtlBytes + (size_t)cap * 4;
    void* mem = nullptr;
    e = hipMalloc(&mem, bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(split-K control)");
    e = hipMemsetAsync(mem, 0, bytes, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync(split-K control)");
    sk.ctl = static_cast<uint32_t*>(mem);
    sk.queue = reinterpret_cast<uint32_t*>(static_cast<char*>(mem) + kSkCtlBytes);
    sk.q_cap = cap;
  }
  int cus = 0;
  rc = device_cus(&cus);
  if (rc) return rc;
  int nb = 0;
  e = (hipError_t)splitk_occupancy(sched, &nb);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  if (nb < 1) nb = 1;
  if (nb > 2) nb = 2;
  uint64_t ticks = 0;
  rc = watchdog_ticks(0, &ticks);
  if (rc) return rc;
  e = (hipError_t)launch_splitk(n, nsplit, bk, A, B, C, ev->counters, ne, we, ev->wait_count, sk.ctl, sk.queue,
                                sk.q_cap, sched, nb * cus, ticks, stream);
  if (e != hipSuccess) return hip_fail(e, "split-K launch");
  add_pending(stream, sk.ctl + SK_REPORT);
  return ETC_OK;
}

// ============================================================ MoE layer ==
extern "C" size_t moe_layer_workspace_size(const etc_moe_desc* d) {
  if (desc_check(d) != ETC_OK) return 0;
  return (size_t)moe_layout(*d).total_bytes;
}

extern "C" int moe_layer_info(const etc_moe_desc* d, etc_moe_info* info) {
  int rc = desc_check(d);
  if (rc) return rc;
  if (!info) return fail(ETC_ERR_INVALID, "info is NULL");
  std::memset(info, 0, sizeof *info);
  info->bm = kBM;
  info->bn1 = kBN1;
  info->bn1_large = g1_cols(kWideG1Rows, 1, d->H);
  info->bn1_large_from_rows = kWideG1Rows;
  info->bn2_large = g2_cols(kWideG1Rows, 1, d->I);
  info->bn1_mid = g1_cols(kMidG1Rows, 1, d->H);
  info->bn1_mid_from_rows = kMidG1Rows;
  info->bn2 = kBN2;
  info->router_tokens = kRouterT;
  info->router_experts = kRouterE;
  info->router_experts_large = kRouterEL;
  info->router_experts_xl = kRouterEXL;
  info->router_xl_from = kRouterXLT;
  info->router_large_from = kRouterLargeT;
  info->dispatch_tokens = 0;  // no dispatch tasks: G1 gathers its rows from x
  info->combine_tokens = kCombineT;
  info->threads = kThreads;
  info->lds_bytes = (int32_t)lds_bytes_for(d);
  int grid = 0;
  rc = persistent_grid(ETC_SCHED_STATIC, info->lds_bytes, &grid);
  if (rc) return rc;
  info->grid = grid;
  if (big_variant(kBigRows, 1, d->H, d->I)) {
    info->big_from_rows = kBigRows;
    info->bm_big = kBigBM;
    info->bn1_big = kBigBN1;
    info->bn2_big = kBigBN2;
    info->lds_bytes_big = (int32_t)big_lds_bytes(d);
    rc = persistent_grid(kBigSchedBase + ETC_SCHED_STATIC, info->lds_bytes_big, &grid);
    if (rc) return rc;
    info->grid_big = grid;
  }
  uint64_t per_ms = 0;
  rc = watchdog_ticks(1000, &per_ms);
  if (rc) return rc;
  info->wall_clock_khz = (int32_t)per_ms;
  return ETC_OK;
}

extern "C" int moe_workspace_init(const etc_moe_desc* d, void* ws, size_t bytes, void* stream) {
  int rc = desc_check(d);
  if (rc) return rc;
  const MoeLayout L = moe_layout(*d);
  if (!ws || !aligned16(ws)) return fail(ETC_ERR_INVALID, "workspace NULL or not 16-byte aligned");
  if (bytes < (size_t)L.total_bytes) return fail(ETC_ERR_INVALID, "workspace has %zu bytes, needs %lld", bytes, (long long)L.total_bytes);
  hipError_t e = hipMemsetAsync(ws, 0, (size_t)L.b_meta, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync(workspace control)");
  return ETC_OK;
}

// One launch on the workspace `ws` (the caller's, or the static scratch of
// moe_layer_launch_noalloc): validation of everything but the workspace
// pointer, the kernel parameters, the grid and the launch.
static int layer_launch(const etc_moe_desc* d, int32_t T, const etc_moe_args* a, int sched, void* stream,
                        uint8_t* ws, size_t ws_bytes, const etc_decoder_desc* dd = nullptr, int32_t pos = 0,
                        const etc_decoder_args* da = nullptr) {
  int rc = desc_check(d);
  if (rc) return rc;
  if (!a) return fail(ETC_ERR_INVALID, "args is NULL");
  if (T < 1 || T > d->T_max) return fail(ETC_ERR_INVALID, "T %d outside [1, T_max=%d]", T, d->T_max);
  if (sched != ETC_SCHED_STATIC && sched != ETC_SCHED_DYNAMIC && sched != ETC_SCHED_KBK && sched != ETC_SCHED_BARRIER &&
      sched != ETC_SCHED_ORDERED)
    return fail(ETC_ERR_INVALID, "unknown schedule %d", sched);
  if (sched == ETC_SCHED_DYNAMIC)
    return fail(ETC_ERR_UNSUPPORTED,
                "the dynamic (push/pop) schedule is switched off: its launch did not complete on the GPU "
                "and the cause is not yet found");
  const void* bf[] = {dd ? da->x : a->x, a->w_router, a->w13, a->w2, a->out, ws};
  const char* bfn[] = {"x", "w_router", "w13", "w2", "out", "workspace"};
  for (int i = 0; i < 6; ++i)
    if (!bf[i] || !aligned16(bf[i])) return fail(ETC_ERR_INVALID, "%s is NULL or not 16-byte aligned", bfn[i]);
  const void* iv[] = {a->topk_ids, a->topk_w, a->counts, a->exp_indptr, a->perm, a->slot};
  const char* ivn[] = {"topk_ids", "topk_w", "counts", "exp_indptr", "perm", "slot"};
  for (int i = 0; i < 6; ++i)
    if (!iv[i] || !aligned4(iv[i])) return fail(ETC_ERR_INVALID, "%s is NULL or not 4-byte aligned", ivn[i]);
  if (d->has_bias && (!a->b_router || !aligned4(a->b_router))) return fail(ETC_ERR_INVALID, "b_router is NULL or misaligned");
  if (a->debug && !aligned4(a->debug)) return fail(ETC_ERR_INVALID, "debug misaligned");
  if (a->trace && (!aligned4(a->trace) || a->trace_records == 0))
    return fail(ETC_ERR_INVALID, "trace misaligned or trace_records is 0");
  const MoeLayout L = moe_layout(*d, dd ? (int64_t)d->T_max * dd->n_kv : 0);
  const DecLayout D = dd ? decoder_layout(*dd, L.total_bytes) : DecLayout{};
  const int64_t need = dd ? D.total_bytes : L.total_bytes;
  if (ws_bytes < (size_t)need)
    return fail(ETC_ERR_INVALID, "workspace has %zu bytes, needs %lld", ws_bytes, (long long)need);

  MoeParams p{};
  p.x = static_cast<const uint16_t*>(a->x);
  p.wr = static_cast<const uint16_t*>(a->w_router);
  p.br = d->has_bias ? a->b_router : nullptr;
  p.w13 = static_cast<const uint16_t*>(a->w13);
  p.w2 = static_cast<const uint16_t*>(a->w2);
  p.out = static_cast<uint16_t*>(a->out);
  p.ids = a->topk_ids;
  p.topw = a->topk_w;
  p.counts = a->counts;
  p.indptr = a->exp_indptr;
  p.perm = a->perm;
  p.slot = a->slot;
  p.debug = a->debug;
  p.ctrl = reinterpret_cast<uint32_t*>(ws + L.b_ctrl);
  p.set0 = reinterpret_cast<uint32_t*>(ws + L.b_set0);
  p.set1 = reinterpret_cast<uint32_t*>(ws + L.b_set1);
  p.meta = reinterpret_cast<uint32_t*>(ws + L.b_meta);
  p.rt_info = reinterpret_cast<int32_t*>(ws + L.b_rt_info);
  p.row_rt = reinterpret_cast<int32_t*>(ws + L.b_row_rt);
  p.logits = reinterpret_cast<float*>(ws + L.b_logits);
  p.hh = reinterpret_cast<uint16_t*>(ws + L.b_hh);
  p.y = reinterpret_cast<uint16_t*>(ws + L.b_y);
  p.ccnt = reinterpret_cast<int32_t*>(ws + L.b_ccnt);
  p.set_words = L.set_words;
  p.o_ev_logit = L.o_ev_logit;
  p.o_ev_exp = L.o_ev_exp;
  p.o_ev_h = L.o_ev_h;
  p.o_ev_y = L.o_ev_y;
  p.o_ev_c = L.o_ev_c;
  p.o_ev_att = L.o_ev_att;
  p.o_queue = L.o_queue;
  p.q_cap = L.q_cap;
  p.T = T;
  p.H = d->H;
  p.E = d->E;
  p.k = d->k;
  p.I = d->I;
  p.norm_topk = d->norm_topk;
  p.has_bias = d->has_bias;
  p.max_rt = L.max_rt;
  p.T_max = d->T_max;
  {
    const int64_t rows = (int64_t)d->T_max * d->k;
    p.hh_bytes = (uint32_t)(rows * d->I * 2);
    p.y_bytes = (uint32_t)(rows * d->H * 2);
    p.logits_bytes = (uint32_t)((int64_t)d->T_max * d->E * 4);
    p.rows_bytes = (uint32_t)(rows * 4);
    p.ccnt_bytes = (uint32_t)(cdiv(d->T_max, kScanChunkT) * d->E * 4);
  }
  p.trace = a->trace;
  p.trace_records = a->trace ? a->trace_records : 0;
  rc = watchdog_ticks(a->watchdog_us, &p.budget);
  if (rc) return rc;
  if (dd) {
    const int64_t Tm = d->T_max, H = d->H, hd = dd->head_dim;
    p.dec = 1;
    p.dx = static_cast<const uint16_t*>(da->x);
    p.g1 = static_cast<const uint16_t*>(da->g1);
    p.g2 = static_cast<const uint16_t*>(da->g2);
    p.wqkv = static_cast<const uint16_t*>(da->w_qkv);
    p.wo = static_cast<const uint16_t*>(da->w_o);
    p.kc = static_cast<uint16_t*>(da->k_cache);
    p.vc = static_cast<uint16_t*>(da->v_cache);
    p.h1 = reinterpret_cast<uint16_t*>(ws + D.b_h1);
    p.qb = reinterpret_cast<uint16_t*>(ws + D.b_q);
    p.part = reinterpret_cast<float*>(ws + D.b_part);
    p.ob = reinterpret_cast<uint16_t*>(ws + D.b_o);
    p.apart = reinterpret_cast<float*>(ws + D.b_apart);
    p.resid = reinterpret_cast<uint16_t*>(ws + D.b_x2);
    p.x = reinterpret_cast<const uint16_t*>(ws + D.b_h2);  // the MoE block's input: RMSNorm(x2) * g2
    p.nq = dd->n_q;
    p.nkv = dd->n_kv;
    p.Lcap = dd->L_cap;
    p.pos = pos;
    p.nchunk = (int32_t)cdiv(pos, kDecChunk);  // cache entries 0 .. pos-1 in chunks
    p.nchunk_max = D.nchunk_max;
    p.part_floats = D.part_floats;
    p.theta = dd->rope_theta;
    p.eps = dd->rms_eps;
    p.cache_bytes = (uint32_t)((int64_t)T * dd->n_kv * dd->L_cap * hd * 2);
    p.h1_bytes = (uint32_t)(Tm * H * 2);
    p.q_bytes = (uint32_t)(Tm * dd->n_q * hd * 2);
    p.part_bytes = (uint32_t)(Tm * dd->n_kv * D.nchunk_max * D.part_floats * 4);
    p.apart_bytes = (uint32_t)(kDecOSplit * Tm * H * 4);
    p.resid_bytes = (uint32_t)(Tm * H * 2);
  }

  // the kernel variant of this T (the decoder layer's T <= 16 never runs
  // the big tiles); the big-tile variant has its own LDS size and grid
  const bool big = !dd && big_variant(T, d->k, d->H, d->I);
  const int lds = (int)(big ? big_lds_bytes(d) : lds_bytes_for(d));
  int e;
  if (sched == ETC_SCHED_KBK) {
    e = dd ? launch_decoder_kbk(p, (int)scan_lds_bytes(d->E, d->T_max), stream)
           : launch_moe_kbk(p, (int)scan_lds_bytes(d->E, d->T_max), stream);
  } else {
    int grid = 0, solo = 0;
    rc = persistent_grid(dd ? kDecSchedBase + sched : (big ? kBigSchedBase + sched : sched), lds, &grid, &solo);
    if (rc) return rc;
    p.solo_wgs = solo;
    e = launch_moe_persistent(p, sched, grid, lds, stream);
  }
  if (e != hipSuccess) return hip_fail((hipError_t)e, "MoE launch");
  add_pending(stream, p.ctrl + C_REPORT);
  return ETC_OK;
}

extern "C" int moe_layer_launch(const etc_moe_desc* d, int32_t T, const etc_moe_args* a, int sched, void* stream) {
  if (!a) return fail(ETC_ERR_INVALID, "args is NULL");
  return layer_launch(d, T, a, sched, stream, static_cast<uint8_t*>(a->workspace), a->workspace_bytes);
}

// ------------------------------------------------- no-allocation variant --
// The workspace of the last no-allocation launch on each device: its layout
// follows the descriptor, so a launch with another descriptor starts from a
// cleared control block and counter sets.
namespace {
struct ScratchState {
  bool init = false;
  etc_moe_desc last{};
};
std::mutex g_scr_mu;
std::vector<ScratchState> g_scr;
}  // namespace

extern "C" int moe_layer_launch_noalloc(const etc_moe_desc* d, int32_t T, const etc_moe_args* a, int sched,
                                        void* stream) {
  int rc = desc_check(d);
  if (rc) return rc;
  if (!a) return fail(ETC_ERR_INVALID, "args is NULL");
  if (a->workspace || a->workspace_bytes)
    return fail(ETC_ERR_INVALID, "the no-allocation launch takes no workspace (workspace must be NULL, 0 bytes)");
  const MoeLayout L = moe_layout(*d);
  if ((uint64_t)L.total_bytes > (uint64_t)kNoallocScratchBytes)
    return fail(ETC_ERR_INVALID, "this descriptor needs %lld bytes of workspace; the static scratch holds %llu",
                (long long)L.total_bytes, (unsigned long long)kNoallocScratchBytes);
  void* scr = nullptr;
  int e = moe_scratch(&scr);
  if (e != hipSuccess) return hip_fail((hipError_t)e, "hipGetSymbolAddress(scratch)");
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(he, "hipGetDevice");
  {
    std::lock_guard<std::mutex> lk(g_scr_mu);
    if ((int)g_scr.size() <= dev) g_scr.resize(dev + 1);
    ScratchState& st = g_scr[dev];
    if (!st.init || std::memcmp(&st.last, d, sizeof *d) != 0) {
      // control block and both counter sets to zero, with a fill kernel
      e = moe_scratch_clear(scr, (size_t)L.b_meta, stream);
      if (e != hipSuccess) return hip_fail((hipError_t)e, "scratch clear");
      st.init = true;
      st.last = *d;
    }
  }
  return layer_launch(d, T, a, sched, stream, static_cast<uint8_t*>(scr), kNoallocScratchBytes);
}

// ========================================================= decoder layer ==
static int decoder_check(const etc_decoder_desc* dd) {
  if (!dd) return fail(ETC_ERR_INVALID, "descriptor is NULL");
  int rc = desc_check(&dd->moe);
  if (rc) return rc;
  if (dd->moe.T_max > kDecMaxT) return fail(ETC_ERR_INVALID, "decoder T_max %d > %d", dd->moe.T_max, kDecMaxT);
  if (dd->moe.has_bias) return fail(ETC_ERR_INVALID, "the decoder layer's router has no bias");
  if (dd->head_dim != kDecHd) return fail(ETC_ERR_INVALID, "head_dim %d != %d", dd->head_dim, kDecHd);
  if (dd->n_kv < 1 || dd->n_q < 1 || dd->n_q % dd->n_kv)
    return fail(ETC_ERR_INVALID, "n_q %d must be a positive multiple of n_kv %d", dd->n_q, dd->n_kv);
  const int gq = dd->n_q / dd->n_kv;
  if (gq > kDecMaxGroup || (gq & (gq - 1)))
    return fail(ETC_ERR_INVALID, "n_q / n_kv = %d must be 1, 2, 4 or 8", gq);
  if ((dd->n_q * dd->head_dim) % (128 * kDecOSplit))
    return fail(ETC_ERR_INVALID, "n_q * head_dim must be a multiple of %d", 128 * kDecOSplit);
  if (dd->L_cap < 1 || (int64_t)kDecMaxT * dd->n_kv * dd->L_cap * dd->head_dim * 2 >= ((int64_t)1 << 31))
    return fail(ETC_ERR_INVALID, "L_cap %d out of range", dd->L_cap);
  if (!(dd->rope_theta > 0.f) || !(dd->rms_eps >= 0.f)) return fail(ETC_ERR_INVALID, "rope_theta / rms_eps");
  return ETC_OK;
}

extern "C" size_t decoder_layer_workspace_size(const etc_decoder_desc* dd) {
  if (decoder_check(dd) != ETC_OK) return 0;
  const MoeLayout L = moe_layout(dd->moe, (int64_t)dd->moe.T_max * dd->n_kv);
  return (size_t)decoder_layout(*dd, L.total_bytes).total_bytes;
}

extern "C" int decoder_workspace_init(const etc_decoder_desc* dd, void* ws, size_t bytes, void* stream) {
  int rc = decoder_check(dd);
  if (rc) return rc;
  const MoeLayout L = moe_layout(dd->moe, (int64_t)dd->moe.T_max * dd->n_kv);
  const DecLayout D = decoder_layout(*dd, L.total_bytes);
  if (!ws || !aligned16(ws)) return fail(ETC_ERR_INVALID, "workspace NULL or not 16-byte aligned");
  if (bytes < (size_t)D.total_bytes)
    return fail(ETC_ERR_INVALID, "workspace has %zu bytes, needs %lld", bytes, (long long)D.total_bytes);
  hipError_t e = hipMemsetAsync(ws, 0, (size_t)L.b_meta, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync(workspace control)");
  return ETC_OK;
}

extern "C" int decoder_layer_launch(const etc_decoder_desc* dd, int32_t T, int32_t pos, const etc_decoder_args* da,
                                    int sched, void* stream) {
  int rc = decoder_check(dd);
  if (rc) return rc;
  if (!da) return fail(ETC_ERR_INVALID, "args is NULL");
  if (sched != ETC_SCHED_STATIC && sched != ETC_SCHED_ORDERED && sched != ETC_SCHED_KBK)
    return fail(ETC_ERR_UNSUPPORTED, "the decoder layer runs under STATIC, ORDERED or KBK");
  if (pos < 0 || pos >= dd->L_cap) return fail(ETC_ERR_INVALID, "pos %d outside [0, L_cap=%d)", pos, dd->L_cap);
  const void* bf[] = {da->x, da->g1, da->w_qkv, da->w_o, da->g2, da->k_cache, da->v_cache};
  const char* bfn[] = {"x", "g1", "w_qkv", "w_o", "g2", "k_cache", "v_cache"};
  for (int i = 0; i < 7; ++i)
    if (!bf[i] || !aligned16(bf[i])) return fail(ETC_ERR_INVALID, "%s is NULL or not 16-byte aligned", bfn[i]);
  return layer_launch(&dd->moe, T, &da->moe, sched, stream, static_cast<uint8_t*>(da->moe.workspace),
                      da->moe.workspace_bytes, dd, pos, da);
}

// ==================================================== coherence self-test ==
extern "C" size_t etc_coherence_selftest_bytes(int32_t pairs) {
  if (pairs < 1 || pairs > kSelftestMaxPairs) return 0;
  return coherence_selftest_words(pairs) * 4;
}

extern "C" int etc_coherence_selftest(int32_t pairs, int32_t rounds, void* workspace, size_t workspace_bytes,
                                      uint32_t* result, void* stream) {
  if (pairs < 1 || pairs > kSelftestMaxPairs) return fail(ETC_ERR_INVALID, "pairs %d outside [1, %d]", pairs, kSelftestMaxPairs);
  if (rounds < 1 || rounds > (1 << 20)) return fail(ETC_ERR_INVALID, "rounds %d outside [1, 2^20]", rounds);
  if (!workspace || !aligned16(workspace)) return fail(ETC_ERR_INVALID, "workspace NULL or not 16-byte aligned");
  if (workspace_bytes < coherence_selftest_words(pairs) * 4)
    return fail(ETC_ERR_INVALID, "workspace %zu bytes, need %zu", workspace_bytes, coherence_selftest_words(pairs) * 4);
  if (!result) return fail(ETC_ERR_INVALID, "result is NULL");
  // every pair's two workgroups must be resident together
  int cus = 0, nb = 0;
  int rc = device_cus(&cus);
  if (rc) return rc;
  hipError_t e = (hipError_t)coherence_selftest_occupancy(&nb);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  if ((int64_t)2 * pairs > (int64_t)nb * cus)
    return fail(ETC_ERR_INVALID, "%d pairs do not fit at once (%d workgroups a CU, %d CUs)", pairs, nb, cus);
  uint64_t ticks = 0;
  rc = watchdog_ticks(0, &ticks);
  if (rc) return rc;
  e = (hipError_t)launch_coherence_selftest(static_cast<uint32_t*>(workspace), pairs, rounds, ticks, stream);
  if (e != hipSuccess) return hip_fail(e, "coherence self-test launch");
  e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  e = hipMemcpy(result, workspace, 2 * sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  return ETC_OK;
}

extern "C" int etc_sync(void* stream) {
  hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  std::vector<uint32_t*> reports;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (size_t i = 0; i < g_pending.size();) {
      if (g_pending[i].stream == stream) {
        reports.push_back(g_pending[i].report);
        g_pending[i] = g_pending.back();
        g_pending.pop_back();
      } else {
        ++i;
      }
    }
  }
  int result = ETC_OK;
  for (uint32_t* r : reports) {
    uint32_t st = 0;
    e = hipMemcpy(&st, r, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(status report)");
    if (st) {
      const uint32_t zero = 0;
      e = hipMemcpy(r, &zero, 4, hipMemcpyHostToDevice);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpy(clear status report)");
      const int code = status_to_code(st);
      if (result == ETC_OK) result = code;
    }
  }
  if (result == ETC_OK) g_err.clear();
  return result;
}

extern "C" const char* etc_last_error(void) { return g_err.c_str(); }
