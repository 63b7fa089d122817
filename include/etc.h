/*
 * etc.h -- C ABI of the MI355X event-tensor MoE megakernel library (libetc.so).
 *
 * One Mixture-of-Experts layer runs as ONE persistent HIP kernel that executes
 * a graph of tiled tasks coordinated through event tensors in HBM:
 *
 *   R(t-tile, e-tile) router logits  --ev_logit-->  K(t-tile) top-k + weights,
 *   one ev_exp[e] arrival per routed (token, slot)  --ev_route--> S scan:
 *   counts (the wait counts of ev_exp), exp_indptr, permutation, row tiles
 *   --ev_scan, ev_exp[e]--> G1(row tile, n-tile) gate/up + SwiGLU on rows
 *   gathered from x --ev_h[row tile]--> G2(row tile, n-tile) down projection
 *   --ev_c[t-tile]--> C(t-tile) combine.
 *
 * Sources (page title, then figure / table / transcript cue):
 *   "Event Tensor: A Unified Abstraction for Compiling Dynamic Megakernel"
 *   (arXiv 2604.13327): Fig. 2 (event tensor, runtime topk / exp_indptr),
 *   Fig. 3 (split-K example), Fig. 4 (symbolic shapes instantiated at run
 *   time), Fig. 5b (data-dependent MoE graph), Figs. 6-7 (static schedule,
 *   notify/wait), Figs. 8-9 (dynamic schedule, push/pop), Fig. 10 (no task
 *   graph materialised at run time), Table 2 (static vs dynamic on the MoE
 *   layer).  The podcast episode on the paper, cues 3, 5, 7, 9, 11 and 13,
 *   restates those mechanisms in prose.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are caller-owned DEVICE pointers (HBM), except
 *     where a parameter says "host".  The library keeps no reference to them
 *     after the call returns (launches are asynchronous: the memory must stay
 *     valid until the stream reaches the launch).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Return value: ETC_OK (0) or a negative ETC_ERR_* code.  Nothing throws
 *     across the ABI.  etc_last_error() gives a thread-local message.
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns, row-major, 16-byte
 *     aligned base pointers.
 */
#ifndef ETC_H
#define ETC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- codes -- */
enum {
  ETC_OK = 0,
  ETC_ERR_INVALID = -1,     /* bad size, pointer, alignment, enum or state   */
  ETC_ERR_UNSUPPORTED = -2, /* valid request this build does not implement   */
  ETC_ERR_HIP = -3,         /* a HIP runtime call failed                     */
  ETC_ERR_TIMEOUT = -4,     /* a bounded in-kernel wait ran out (watchdog)   */
  ETC_ERR_INVARIANT = -5,   /* an event was notified beyond its wait_count,
                               or a queue overflowed                          */
  ETC_ERR_NONFINITE = -6    /* a router logit was NaN                        */
};

/* Scheduling of the persistent kernel.
 *   STATIC : per-workgroup task lists fixed in closed form before any task
 *            runs (phase ordered), every dependency a notify / wait on an
 *            event counter [Figs. 6-7; podcast cue 11].
 *   DYNAMIC: a notify that completes an event pushes the released tasks at
 *            once onto one HBM queue; idle workgroups pop [Figs. 8-9].
 *   KBK    : comparator, one kernel launch per task type (kernel-by-kernel
 *            model of Fig. 1), same device task code.
 *   BARRIER: comparator, the persistent kernel with a grid-wide barrier
 *            between task types instead of fine-grained events (the
 *            "unfused megakernel" reading of Table 2).
 *   ORDERED: STATIC's events and routing front, but the G1 and then the G2
 *            tiles are claimed in index order from a counter per group of
 *            workgroups instead of being dealt in fixed lists: a workgroup
 *            that streams faster takes more tiles.  Each claimed tile still
 *            waits on its event before it runs.                              */
enum { ETC_SCHED_STATIC = 0, ETC_SCHED_DYNAMIC = 1, ETC_SCHED_KBK = 2, ETC_SCHED_BARRIER = 3,
       ETC_SCHED_ORDERED = 4 };

/* ------------------------------------------------------- event tensors -- */
/* An event tensor [Fig. 2; podcast cue 3]: a tensor of dependency counters,
 * one per element, each released after `wait_count` notifies.  A dimension
 * may be symbolic (ETC_DIM_SYMBOLIC): the tensor is then a template bound to
 * a concrete shape at run time by etensor_instantiate, with nothing
 * recompiled and nothing captured [Fig. 4; podcast cue 5].  The wait count
 * may be data dependent (ETC_WAIT_DATA_DEPENDENT): it is then written at run
 * time by the task that computes it [Fig. 5b; podcast cue 7].               */
#define ETC_DIM_SYMBOLIC (-1)
#define ETC_WAIT_DATA_DEPENDENT (-1)
#define ETC_MAX_DIMS 8

typedef struct etc_etensor etc_etensor;

/* Declare an event tensor.  ndim in [1, ETC_MAX_DIMS]; shape (host array)
 * holds positive sizes or ETC_DIM_SYMBOLIC; wait_count >= 0 or
 * ETC_WAIT_DATA_DEPENDENT.  dev_counters: caller-owned device array of
 * int32 counters with room for every instantiation the caller will use (it
 * must start zeroed), or NULL to let the library allocate on first launch.
 * The handle is library-owned until etensor_destroy.  Makes no HIP call.
 * Errors: ETC_ERR_INVALID for a bad ndim, size or wait_count.               */
int etensor_create(etc_etensor** out, int ndim, const int64_t* shape, int32_t wait_count,
                   int32_t* dev_counters);

/* Bind every dimension: concrete_shape (host, ndim entries) must match the
 * fixed dimensions and give a positive size for each symbolic one.  May be
 * called again with another shape (a new instantiation of the same
 * template).  Makes no HIP call.  Errors: ETC_ERR_INVALID.                  */
int etensor_instantiate(etc_etensor* et, const int64_t* concrete_shape);

/* Current shape (host out-array of ETC_MAX_DIMS; symbolic dimensions read
 * ETC_DIM_SYMBOLIC before instantiation), ndim and element count (0 when not
 * instantiated).  Errors: ETC_ERR_INVALID for NULL arguments.               */
int etensor_shape(const etc_etensor* et, int64_t* shape_out, int* ndim_out, int64_t* numel_out);

/* Release the handle and any counters the library allocated for it.        */
int etensor_destroy(etc_etensor* et);

/* --------------------------------------------------------------- edges -- */
/* An edge wires a grid of tasks to an event tensor [Fig. 3; podcast cue 3].
 * It is written "<task letters>-><event letters>": one distinct lowercase
 * letter per dimension of the task grid on the left, and on the right one
 * letter per dimension of the event tensor, each naming the task dimension
 * whose coordinate indexes that event dimension.  Task (c_0, c_1, ...) then
 * touches the event element whose d-th coordinate is c[src[d]].  As an
 * out-edge every task notifies the element it touches, so an element
 * receives one notify per task that maps to it: fan_in, the product of the
 * task-grid sizes of the letters missing on the right.  As an in-edge the
 * task waits on the element it touches.  "ij->i": task (i, j) notifies event
 * i; "i->i": task i waits on event i.                                       */
typedef struct {
  int32_t task_ndim;                /* letters left of "->"                    */
  int32_t event_ndim;               /* letters right of "->" (the tensor's ndim) */
  int32_t src[ETC_MAX_DIMS];        /* event dimension d is task coordinate src[d] */
  int64_t stride[ETC_MAX_DIMS];     /* row-major element stride of event dimension d */
  int64_t task_shape[ETC_MAX_DIMS]; /* the task grid the edge was compiled for */
  int64_t event_numel;              /* elements of the instantiated tensor     */
  int64_t fan_in;                   /* tasks that touch one event element      */
} etc_edge;

/* Compile `spec` (host string) against the instantiated event tensor `et`
 * and a task grid of shape task_shape[task_ndim] (host array).  The task
 * grid's size along each letter on the right must equal the event tensor's
 * size along that dimension.  Host only: makes no HIP call.
 * Errors: ETC_ERR_INVALID (syntax; a repeated, unknown or non-lowercase
 * letter; rank or size mismatch; `et` not instantiated; NULL argument).      */
int etc_edge_compile(const etc_etensor* et, const char* spec, const int64_t* task_shape, int task_ndim,
                     etc_edge* out);

/* The flat event element a task at task_coord (host array of task_ndim
 * entries) touches through `edge`: sum_d task_coord[src[d]] * stride[d], the
 * index the kernels compute.  Returns -1 for a NULL argument.               */
int64_t etc_edge_index(const etc_edge* edge, const int64_t* task_coord);

/* The split-K row-sum example of Fig. 3 (podcast cue 3), run through the
 * same device runtime as the MoE layer, its event wiring given by compiled
 * edges: partial_sum(i, j) writes B[i, j] = sum of A[i, j*bk .. (j+1)*bk)
 * and notifies the element `notify_edge` maps (i, j) to (the pages' wiring:
 * "ij->i" over a task grid [n, nsplit]); final_sum(i) waits on the element
 * `wait_edge` maps i to ("i->i" over a task grid [n]) and writes
 * C[i] = sum_j B[i, j].  `ev` must be instantiated, with wait_count equal to
 * notify_edge's fan_in; under DYNAMIC the wait edge must pair every element
 * with exactly one final_sum (then the notify that completes an element
 * pushes that task).  A is [n, nsplit*bk] int32, B [n, nsplit], C [n]
 * (device); the edges are host structs.  sched: ETC_SCHED_STATIC or
 * ETC_SCHED_DYNAMIC.  Asynchronous; errors found in the kernel are reported
 * by etc_sync.
 * Errors: ETC_ERR_INVALID (edges that do not fit the task grids or the
 * tensor, wait_count != fan_in, bad sizes), ETC_ERR_UNSUPPORTED (sched),
 * ETC_ERR_HIP.                                                              */
int etc_splitk_launch(etc_etensor* ev, int32_t n, int32_t nsplit, int32_t bk, const int32_t* A,
                      int32_t* B, int32_t* C, const etc_edge* notify_edge, const etc_edge* wait_edge,
                      int sched, void* stream);

/* ------------------------------------------------------------ MoE layer -- */
/* Layer shape.  Router: logits = x @ w_router^T (+ b_router), top-k over E,
 * weights = softmax renormalised over the chosen k (norm_topk = 1) or the
 * plain softmax value (norm_topk = 0).  Experts: SwiGLU,
 * y = (silu(x Wg^T) * (x Wu^T)) Wd^T with Wg = w13[e, 0:I, :],
 * Wu = w13[e, I:2I, :], Wd = w2[e].  Output: sum_j topk_w[t, j] * y_j.
 * Limits: H and I multiples of 128 and <= 40960; 1 <= E <= 256;
 * 1 <= k <= min(E, 16); 1 <= T_max <= 16384 and T_max * k * max(H, I) * 2
 * bytes below 2 GiB.                                                        */
typedef struct {
  int32_t T_max;     /* largest token count any launch will use            */
  int32_t H;         /* hidden size                                        */
  int32_t E;         /* number of experts                                  */
  int32_t k;         /* experts per token                                  */
  int32_t I;         /* expert intermediate size                           */
  int32_t norm_topk; /* 1: renormalise the k weights to sum to 1           */
  int32_t has_bias;  /* 1: b_router is read and added to the logits        */
} etc_moe_desc;

/* Device pointers of one launch.  Layouts (row-major):
 *   x        [T, H]      bf16   input tokens
 *   w_router [E, H]      bf16
 *   b_router [E]         fp32   (read only when has_bias)
 *   w13      [E, 2I, H]  bf16   rows 0..I-1 gate, rows I..2I-1 up
 *   w2       [E, H, I]   bf16   down projection
 *   out      [T, H]      bf16   layer output (written)
 *   topk_ids [T, k] int32, topk_w [T, k] fp32: routing, by descending logit,
 *            ties to the lower expert index (written)
 *   counts   [E] int32: tokens routed to each expert (written)
 *   exp_indptr [E+1] int32: exclusive prefix sum of counts, ends at T*k
 *   perm     [T*k] int32: perm[s] = flat index t*k+j held by grouped row s;
 *            rows of one expert keep ascending t (stable)      (written)
 *   slot     [T*k] int32: inverse of perm                      (written)
 *   workspace: moe_layer_workspace_size(desc) bytes, prepared once by
 *            moe_workspace_init; one workspace serves one launch at a time
 *            (launches that overlap on one workspace race).
 *   debug    NULL, or ETC_DEBUG_WORDS(E) int32 zeroed by the caller; the
 *            kernel adds per-event notify and fire counts (layout below).
 *   watchdog_us: 0 = default (2 s); else the wall time, in microseconds,
 *            after which any single in-kernel wait gives up: the launch then
 *            drains (every workgroup leaves its waits) and etc_sync reports
 *            ETC_ERR_TIMEOUT.                                               */
typedef struct {
  const void* x;
  const void* w_router;
  const float* b_router;
  const void* w13;
  const void* w2;
  void* out;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* counts;
  int32_t* exp_indptr;
  int32_t* perm;
  int32_t* slot;
  void* workspace;
  size_t workspace_bytes;
  int32_t* debug;
  uint32_t watchdog_us;
  uint32_t trace_records; /* capacity of `trace` in records (0 = no trace)  */
  uint32_t* trace;        /* NULL, or ETC_TRACE_WORDS(trace_records) uint32,
                             zeroed by the caller (see below)               */
} etc_moe_args;

/* Per-task trace, when etc_moe_args.trace is non-NULL (persistent schedules).
 * Each workgroup owns per_wg = trace_records / grid consecutive records and
 * fills them in task order with plain stores (no atomics, so tracing barely
 * perturbs the timing); records past per_wg are dropped, unused ones stay
 * zero.  Words 1 and 2 receive per_wg and the grid size.  Record r occupies
 * words [16 + 8r, 16 + 8r + 8), workgroup w's records start at r = w*per_wg:
 *   workgroup | task type << 24 (type 1..7 = R, K, S, D, G1, G2, C; type 8 =
 *   the routing tables a workgroup rebuilds in its LDS for a small batch,
 *   waiting on the route event; 9..14 = the decoder layer's N1, QKV,
 *   attention, merge, output projection, N2; type 15 = the workgroup
 *   itself, its last record: entry, counter set known, end of its task
 *   lists, after its exit arrival), task
 *   index a, b, then wall-clock ticks: before the task's wait (low, high 32
 *   bits), and the low 32 bits after the wait, after the task body, and after
 *   its notifies.  Ticks are those of the device's constant wall clock
 *   (etc_moe_info.wall_clock_khz).                                          */
#define ETC_TRACE_WORDS(records) (16 + 8 * (size_t)(records))

/* Debug counters (int32), when etc_moe_args.debug is non-NULL:
 *   [0, E)        notifies received by ev_exp[e]   (expected: counts[e])
 *   [E, 2E)       times ev_exp[e] was completed    (expected: 1 if counts[e] > 0)
 *   [2E + i]      tasks executed of type i, i = 0..6 in the order
 *                 R, K, S, D, G1, G2, C; D stays 0 (the dispatch is fused
 *                 into G1's row gather)
 *   [2E + 7]      STATIC / ORDERED: rows whose row tile, as looked up by
 *                 their C task, holds them              (expected: T*k)     */
#define ETC_DEBUG_WORDS(E) (2 * (E) + 8)

/* Tile geometry and task counts of this build, for tests and benchmarks.   */
typedef struct {
  int32_t bm;          /* rows per grouped-GEMM row tile                    */
  int32_t bn1;         /* gate (and up) columns per G1 tile                 */
  int32_t bn2;         /* output columns per G2 tile                        */
  int32_t router_tokens, router_experts; /* R tile                          */
  int32_t dispatch_tokens; /* tokens per dispatch task; 0: there are none, the
                              gate/up tiles gather their rows from x      */
  int32_t combine_tokens;
  int32_t grid;        /* persistent workgroups (0 before the first query)  */
  int32_t threads;     /* threads per workgroup                             */
  int32_t lds_bytes;   /* dynamic LDS per workgroup                         */
  int32_t wall_clock_khz; /* rate of the clock the watchdog and trace read  */
  int32_t router_experts_large; /* R tile's experts when T > router_large_from */
  int32_t router_large_from;    /* (router_experts applies up to that T)       */
  int32_t bn1_large;   /* gate (and up) columns per G1 tile when T*k >=
                          bn1_large_from_rows (bn1 applies below)          */
  int32_t bn1_large_from_rows;
  int32_t bn2_large;   /* output columns per G2 tile from the same T*k on   */
  int32_t bn1_mid;     /* gate (and up) columns per G1 tile when
                          bn1_mid_from_rows <= T*k < bn1_large_from_rows  */
  int32_t bn1_mid_from_rows;
  int32_t router_experts_xl; /* R tile's experts when T >= router_xl_from      */
  int32_t router_xl_from;    /* (below it, router_experts / _large apply)       */
  int32_t big_from_rows;     /* T*k from which launches run the big-tile
                                variant (0: this descriptor's H, I never do) */
  int32_t bm_big, bn1_big, bn2_big; /* its row tile, G1 and G2 widths        */
  int32_t grid_big;          /* its persistent workgroups (one a CU)          */
  int32_t lds_bytes_big;     /* its dynamic LDS per workgroup                 */
} etc_moe_info;

/* Fill `info` for `desc` (host struct).  Queries the device for the grid.
 * Errors: ETC_ERR_INVALID (desc), ETC_ERR_HIP.                               */
int moe_layer_info(const etc_moe_desc* desc, etc_moe_info* info);

/* Bytes of workspace a launch with this descriptor needs (0 if the
 * descriptor is invalid).  Makes no HIP call.                               */
size_t moe_layer_workspace_size(const etc_moe_desc* desc);

/* Zero the workspace's control block (once after allocation, and after an
 * ETC_ERR_TIMEOUT if the caller wants a clean slate).  Asynchronous on
 * `stream`.  Errors: ETC_ERR_INVALID, ETC_ERR_HIP.                           */
int moe_workspace_init(const etc_moe_desc* desc, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Asynchronous launch of one MoE layer for T tokens, 1 <= T <= desc->T_max.
 * T is a kernel argument: every event-tensor shape and task count is derived
 * from it inside the kernel, so one compiled kernel serves every batch size
 * with no recompile and no graph capture [Fig. 4].  Per-expert event counters
 * are set from the routed counts at run time and release each expert's
 * grouped-GEMM tiles over [exp_indptr[e], exp_indptr[e+1]) [Fig. 5b; podcast
 * cues 7 and 9].  Allocates nothing, compiles nothing.
 * Errors (returned before any launch): ETC_ERR_INVALID (descriptor limits, T
 * range, NULL or misaligned pointer, small workspace, bad sched),
 * ETC_ERR_HIP.  Errors inside the kernel are reported by etc_sync.           */
int moe_layer_launch(const etc_moe_desc* desc, int32_t T, const etc_moe_args* args, int sched,
                     void* stream);

/* -------------------------------------------------------- decoder layer -- */
/* One decoder layer around the MoE layer, as ONE persistent kernel: the
 * attention block, then the MoE block, each with its residual add [the
 * pages evaluate the MoE layer inside end-to-end serving, Fig. 14; the
 * layer's steps are the textbook pre-norm block]:
 *   h1 = RMSNorm(x) * g1                       N1 tasks (one token each)
 *   q, k, v = h1 Wqkv^T; RoPE on q and k at position pos; k, v written into
 *            the caches at index pos           QKV tasks (16 columns each)
 *   o = softmax(q k^T / sqrt(d)) v over cache entries 0..pos, query head h
 *       reading key/value head h / (n_q / n_kv)   attention tasks (256 cache
 *            entries of one token and one kv head each), then merge tasks
 *   x2 = x + o Wo^T                            projection tasks, N2 tasks
 *                                              (one token each)
 *   out = x2 + MoE(RMSNorm(x2) * g2)           the MoE layer's tasks, its
 *            router waiting on the N2 tasks' event
 * Every activation is stored bf16, sums are fp32.  Each phase notifies an
 * event that the next phase's tasks wait on, as in the MoE graph.         */
typedef struct {
  int32_t n_q;         /* query heads                                          */
  int32_t n_kv;        /* key / value heads; n_q / n_kv in {1, 2, 4, 8}        */
  int32_t head_dim;    /* 128                                                   */
  int32_t L_cap;       /* cache entries per sequence and kv head (pos < L_cap)  */
  float rope_theta;    /* rotary base (1e6 for Qwen3)                           */
  float rms_eps;       /* RMSNorm epsilon (1e-6)                                */
  etc_moe_desc moe;    /* the MoE block; moe.T_max <= 16 is the largest batch,
                          moe.has_bias must be 0                               */
} etc_decoder_desc;

/* Device pointers of one decoder-layer launch (row-major, bf16 unless said):
 *   x       [T, H]  residual input;   g1, g2 [H] RMSNorm weights
 *   w_qkv   [(n_q + 2 n_kv) head_dim, H]: rows of the query heads, then of
 *           the key heads, then of the value heads
 *   w_o     [H, n_q head_dim]
 *   k_cache, v_cache [T, n_kv, L_cap, head_dim]: entries 0..pos-1 are read,
 *           entry pos is written (the new token's key after RoPE, its value)
 *   moe     the MoE block's arguments: w_router, w13, w2, out (the layer
 *           output [T, H]), the routing outputs, workspace
 *           (decoder_layer_workspace_size bytes, prepared once by
 *           decoder_workspace_init), debug, watchdog_us, trace; moe.x is
 *           ignored (the MoE block reads RMSNorm(x2) from the workspace).  */
typedef struct {
  const void* x;
  const void* g1;
  const void* w_qkv;
  const void* w_o;
  const void* g2;
  void* k_cache;
  void* v_cache;
  etc_moe_args moe;
} etc_decoder_args;

/* Workspace bytes of a decoder-layer launch (0 if the descriptor is
 * invalid).  Makes no HIP call.                                             */
size_t decoder_layer_workspace_size(const etc_decoder_desc* desc);

/* Zero the workspace's control block (once after allocation).  Asynchronous
 * on `stream`.  Errors: ETC_ERR_INVALID, ETC_ERR_HIP.                        */
int decoder_workspace_init(const etc_decoder_desc* desc, void* workspace, size_t workspace_bytes, void* stream);

/* Asynchronous launch of one decoder layer for T tokens (1 <= T <=
 * moe.T_max), every token decoding at position pos (0 <= pos < L_cap).
 * sched: ETC_SCHED_STATIC or ETC_SCHED_ORDERED (the MoE block's G tiles
 * dealt or claimed, the attention block's tasks dealt), or ETC_SCHED_KBK
 * (one kernel launch per task type).  Allocates nothing, compiles nothing.
 * Errors: ETC_ERR_INVALID (limits, NULL or misaligned pointers, small
 * workspace), ETC_ERR_UNSUPPORTED (sched), ETC_ERR_HIP; in-kernel errors are
 * reported by etc_sync.                                                     */
int decoder_layer_launch(const etc_decoder_desc* desc, int32_t T, int32_t pos, const etc_decoder_args* args,
                         int sched, void* stream);

/* moe_layer_launch without a caller workspace, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array
 * of the library, 8 MiB on each GPU it runs on, held until the process ends:
 * descriptors whose moe_layer_workspace_size exceeds 8 MiB are rejected
 * (at the Qwen3-30B-A3B MoE shape that admits T_max up to 178).
 * args->workspace must be NULL and args->workspace_bytes 0; everything else
 * is as for moe_layer_launch.  Calls no hipMalloc, hipFree or allocating
 * routine: the array's device address is looked up once per device, and
 * when the descriptor differs from the previous call's on the device, the
 * array's control block and counter sets are zeroed by a small fill kernel
 * on `stream` first.  Every call on one GPU shares its array, so calls that
 * overlap on one GPU (on different streams, or with another process-wide
 * user of the array) race.
 * Errors: as moe_layer_launch; ETC_ERR_INVALID also for a non-NULL
 * workspace or a descriptor too large for the array (checked before any HIP
 * call).                                                                    */
int moe_layer_launch_noalloc(const etc_moe_desc* desc, int32_t T, const etc_moe_args* args, int sched,
                             void* stream);

/* ------------------------------------------------- coherence self-test -- */
/* Every notify and wait of the kernels moves data between workgroups with
 * the same protocol and no fences (an event is released by arrivals on its
 * counter [Event Tensor pages, Fig. 7]; the data it guards must be visible
 * to the waiter): the producer writes with device-coherent stores, waits for
 * its stores, passes a workgroup barrier, then one thread adds to the
 * counter with a relaxed device-scope atomic; the consumer polls the counter
 * with relaxed device-scope loads, passes a barrier, then reads with
 * device-coherent loads.  This self-test runs that protocol between `pairs`
 * producer/consumer workgroup pairs placed on different XCDs, `rounds`
 * messages of 4 KB each way with an acknowledgement per round, and checks
 * every word the consumers read.
 *   etc_coherence_selftest_bytes: device workspace the test needs (0 if
 *            pairs is outside [1, 1024]).
 *   workspace: caller-owned device memory of at least that size, 16-byte
 *            aligned; zeroed by the call on `stream`.
 *   result:  host pointer to 2 words: [0] message words read wrong, [1]
 *            non-zero if a wait gave up (the watchdog); both 0 on success.
 * Blocks until the test has run.  Errors: ETC_ERR_INVALID (ranges, NULL or
 * misaligned pointers, a workspace too small, more pairs than fit on the
 * GPU at once), ETC_ERR_HIP.                                               */
size_t etc_coherence_selftest_bytes(int32_t pairs);
int etc_coherence_selftest(int32_t pairs, int32_t rounds, void* workspace, size_t workspace_bytes,
                           uint32_t* result, void* stream);

/* Wait for `stream`, then report the first in-kernel error of every launch
 * made on it since the previous etc_sync (and clear it): ETC_OK,
 * ETC_ERR_TIMEOUT, ETC_ERR_INVARIANT, ETC_ERR_NONFINITE or ETC_ERR_HIP.
 * (Named etc_sync rather than sync so as not to shadow POSIX sync(2).)      */
int etc_sync(void* stream);

/* Thread-local description of the last error on this thread ("" if none).
 * The string is library-owned and valid until the next call on the thread.  */
const char* etc_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* ETC_H */
