// Internal shared definitions of libetc: tile constants, the workspace
// layout (computed on the host, passed to the kernels) and the kernel
// parameter block.  Not part of the public C ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/etc.h"

#ifndef ETC_HD
#define ETC_HD __host__ __device__ inline __attribute__((always_inline))
#endif
#include "etc_tiles.h"
#include "dyn_sched.h"

namespace etc {

// status bits (word 0 of a counter set, OR-ed into the report word)
enum : uint32_t {
  ST_TIMEOUT = 1u,
  ST_OVER_NOTIFY = 2u,
  ST_NONFINITE = 4u,
  ST_QUEUE_OVERFLOW = 8u,
  ST_ABORT = 0x80000000u,
};
static_assert(ST_TIMEOUT == dyn::kStTimeout && ST_OVER_NOTIFY == dyn::kStOverNotify &&
                  ST_QUEUE_OVERFLOW == dyn::kStOverflow && ST_ABORT == dyn::kStAbort,
              "one status word, one set of bits");

constexpr int kEvStride = 32;   // words between event elements (one 128-byte line each)
constexpr int kSelftestMaxPairs = 1024;  // coherence self-test: producer/consumer pairs at most
constexpr int kMaxK = 16;
constexpr int kMaxE = 256;
constexpr int kMaxTmax = 16384;
constexpr int kMaxHI = 40960;  // covers the dense MLPs of the pages' appendix table (I up to 36864)
constexpr int kScanChunkT = 512;       // S: tokens per bitmap pass
constexpr int kScanW = kScanChunkT / 32;  // S: bitmap words per expert and pass
// Small batches (T <= kScanChunkT and T*k <= kLocalRows): every persistent
// workgroup rebuilds the routing tables in its own LDS
constexpr int kLocalRows = 4096;
constexpr int kLocalTiles = kLocalRows / 64 + 256 + 16;
// watchdog of one in-kernel wait, in microseconds of wall time; a healthy
// wait lasts microseconds
constexpr uint32_t kDefaultWatchdogUs = 2000000u;

// task types (the dynamic schedule's queue descriptors carry them in their
// top three bits, dyn_sched.h; 0 = empty slot)
enum TaskType : int { TT_R = 1, TT_K = 2, TT_S = 3, TT_D = 4, TT_G1 = 5, TT_G2 = 6, TT_C = 7,
                      TT_L = 8 /* trace only: a workgroup's LDS routing tables */,
                      // trace only: the decoder layer's attention-block tasks
                      TT_DN1 = 9, TT_DQKV = 10, TT_DATT = 11, TT_DATTC = 12, TT_DO = 13, TT_DN2 = 14,
                      // trace only: one record a workgroup of the persistent kernel, stamped
                      // at entry, once its counter set is known, after its task lists and
                      // after its exit arrival
                      TT_WG = 15 };
static_assert(dyn::T_R == TT_R && dyn::T_K == TT_K && dyn::T_S == TT_S && dyn::T_G1 == TT_G1 &&
                  dyn::T_G2 == TT_G2 && dyn::T_C == TT_C,
              "the dynamic runner's task types are the kernels' task types");

// ---- counter set (u32 words) ------------------------------------------------
// Words that many workgroups poll or update each sit on their own 128-byte
// line, so the status poll, the queue head and the queue tail do not queue
// up behind one another.
enum : int {
  W_STATUS = 0,
  W_DONE = 32,
  W_HEAD = 64,
  W_TAIL = 96,
  W_TOTAL = 128,
  W_BAR_COUNT = 160,
  W_BAR_RELEASE = 192,
  W_EV_ROUTE = 224,
  W_EV_SCAN = 256,
  W_CLAIM_G1 = 288,  // ORDERED: 8 claim counters for the G tiles, 32 words apart
  // decoder layer: one event per phase of the attention block
  W_DEC_N1 = 544,    // RMSNorm tasks done
  W_DEC_QKV = 576,   // QKV projection tiles done
  W_DEC_ATTC = 608,  // attention merges done
  W_DEC_O = 640,     // output projection tiles done
  W_DEC_N2 = 672,    // residual + RMSNorm tasks done
  W_SCAN_S1 = 704,   // large batches: per-chunk count tasks of the scan done
  W_SCAN_S3 = 736,   // large batches: per-chunk placement tasks of the scan done
  W_FIXED = 768,     // start of the variable-size event tensors
};
// split-K example: control words (u32) of its library-owned block, each on
// its own 128-byte line, followed by the queue
enum : int { SK_STATUS = 0, SK_HEAD = 32, SK_TAIL = 64, SK_DONE = 96, SK_REPORT = 128 };
constexpr int kSkCtlBytes = 1024;

// control block (u32 words)
enum : int { C_EPOCH = 0, C_REPORT = 1, C_WORDS = 64 };

struct MoeLayout {
  // sizes derived from the descriptor's T_max
  int32_t ntt_max, max_rt, nct_max;
  int64_t q_cap;
  // word offsets inside a counter set
  int64_t o_ev_logit, o_ev_exp, o_ev_h, o_ev_y, o_ev_c, o_ev_att, o_queue;  // word offsets
  int64_t set_words;
  // byte offsets inside the workspace
  int64_t b_ctrl, b_set0, b_set1, b_meta, b_rt_info, b_row_rt, b_logits, b_hh, b_y, b_ccnt;
  int64_t total_bytes;
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// meta words (outside the double-buffered sets): written by the scan task
enum : int { M_NRT = 0, M_WORDS = 16 };

// Decoder layer around the MoE layer (the attention block before it):
// geometry of its tasks.
constexpr int kDecMaxT = 16;     // tokens a launch takes (one 16-row MFMA block)
constexpr int kDecHd = 128;      // head size
constexpr int kDecChunk = 256;   // cache entries per attention task
constexpr int kDecOSplit = 4;    // K split of the output projection
constexpr int kDecNormT = 1;     // tokens per RMSNorm task (the four waves split H)
constexpr int kDecMaxGroup = 8;  // query heads per key/value head

// Decoder buffers, appended to the MoE workspace.
struct DecLayout {
  int32_t nchunk_max;   // attention tasks per (token, kv head) at the largest position
  int32_t part_floats;  // floats of one attention partial: gq x d values, then gq maxima, gq sums
  int64_t b_h1, b_q, b_part, b_o, b_apart, b_x2, b_h2, total_bytes;
};

inline MoeLayout moe_layout(const etc_moe_desc& d, int64_t att_events = 0) {
  MoeLayout L{};
  const int64_t Tm = d.T_max;
  L.ntt_max = (int32_t)cdiv(Tm, kRouterT);
  L.nct_max = (int32_t)cdiv(Tm, kCombineT);
  const int64_t rows = Tm * d.k;
  L.max_rt = (int32_t)(cdiv(rows, kBM) + (rows < d.E ? rows : d.E));
  // every task except the router prefix goes through the queue
  L.q_cap = dyn::moe_queue_capacity(Tm, L.max_rt, d.I, d.H, kBN1, kBN2, kRouterT, kCombineT);
  int64_t w = W_FIXED;
  L.o_ev_logit = w; w += (int64_t)L.ntt_max * kEvStride;
  L.o_ev_exp = w;   w += (int64_t)d.E * kEvStride;
  L.o_ev_h = w;     w += (int64_t)L.max_rt * kEvStride;
  L.o_ev_y = w;     w += (int64_t)L.max_rt * kEvStride;
  L.o_ev_c = w;     w += (int64_t)L.nct_max * kEvStride;
  L.o_ev_att = w;   w += att_events * kEvStride;  // decoder layer: per (token, kv head)
  L.o_queue = w;    w += L.q_cap;  // 32-bit descriptors
  L.set_words = align_up(w, 64);
  int64_t b = 0;
  L.b_ctrl = b;          b += C_WORDS * 4;
  L.b_set0 = b;          b += L.set_words * 4;
  L.b_set1 = b;          b += L.set_words * 4;
  L.b_meta = b;          b += M_WORDS * 4;
  L.b_rt_info = b;       b += align_up((int64_t)L.max_rt * 16, 256);
  L.b_row_rt = b;        b += align_up(rows * 4, 256);
  L.b_logits = b;        b += align_up(Tm * d.E * 4, 256);
  L.b_hh = b;            b += align_up(rows * d.I * 2, 256);
  L.b_y = b;             b += align_up(rows * d.H * 2, 256);
  L.b_ccnt = b;          b += align_up(cdiv(Tm, kScanChunkT) * d.E * 4, 256);  // rows per (scan chunk, expert)
  L.total_bytes = b;
  return L;
}

inline DecLayout decoder_layout(const etc_decoder_desc& dd, int64_t base) {
  DecLayout D{};
  const int64_t Tm = dd.moe.T_max, H = dd.moe.H, d = dd.head_dim;
  const int64_t gq = dd.n_q / dd.n_kv;
  D.nchunk_max = (int32_t)cdiv(dd.L_cap, kDecChunk);
  D.part_floats = (int32_t)(gq * d + 2 * gq);
  int64_t b = base;
  D.b_h1 = b;    b += align_up(Tm * H * 2, 256);
  D.b_q = b;     b += align_up(Tm * dd.n_q * d * 2, 256);
  D.b_part = b;  b += align_up(Tm * dd.n_kv * D.nchunk_max * D.part_floats * 4, 256);
  D.b_o = b;     b += align_up(Tm * dd.n_q * d * 2, 256);
  D.b_apart = b; b += align_up(kDecOSplit * Tm * H * 4, 256);
  D.b_x2 = b;    b += align_up(Tm * H * 2, 256);
  D.b_h2 = b;    b += align_up(Tm * H * 2, 256);
  D.total_bytes = b;
  return D;
}

// LDS bytes the scan task needs: five per-expert tables (counts,
// exp_indptr, tile numbering, the chunk's grouped base), the scan's partial
// sums, one chunk's presence bitmap and per-word prefixes, and the chunk's
// expert ids (a byte each) and grouped pair order (two bytes each).  Sized
// for kMaxE so every table sits at a fixed offset; independent of T_max
// (the scan walks the tokens in chunks).
inline int64_t scan_lds_bytes(int E, int T_max) {
  (void)E;
  (void)T_max;
  return 5 * 260 * 4 + 128 + (int64_t)kMaxE * kScanW * 4 * 2 + kScanChunkT * kMaxK * 3;
}
// G2: cross-wave reduction buffer (4 waves x 4 blocks x 256 fp32) plus the
// bf16 staging of the kBM x 64 output tile
// G tasks' LDS: the K-split bodies' reduction and output stage, or the
// column-split G1 body's two staged A chunks (64 rows of 128 k, padded)
constexpr int64_t kGemmLdsBytes = (4 * kCB2 * 256 * 4 + kBM * kBN2 * 2) > 2 * 64 * (128 * 2 + 16)
                                      ? (4 * kCB2 * 256 * 4 + kBM * kBN2 * 2)
                                      : 2 * 64 * (128 * 2 + 16);

struct MoeParams {
  const uint16_t* x;
  const uint16_t* wr;
  const float* br;
  const uint16_t* w13;
  const uint16_t* w2;
  uint16_t* out;
  int32_t* ids;
  float* topw;
  int32_t* counts;
  int32_t* indptr;
  int32_t* perm;
  int32_t* slot;
  int32_t* debug;
  uint32_t* ctrl;
  uint32_t* set0;
  uint32_t* set1;
  uint32_t* meta;
  int32_t* rt_info;  // [max_rt][4]: expert, first grouped row, rows, 0
  int32_t* row_rt;   // [T_max*k]: row tile of each grouped row
  float* logits;
  uint16_t* hh;
  uint16_t* y;
  int32_t* ccnt;  // [ceil(T_max / kScanChunkT)][E]: rows of each expert in each scan chunk
  int64_t set_words;
  int64_t o_ev_logit, o_ev_exp, o_ev_h, o_ev_y, o_ev_c, o_ev_att, o_queue, q_cap;
  int32_t T, H, E, k, I, norm_topk, has_bias;
  int32_t max_rt;
  int32_t T_max;
  int32_t solo_wgs;  // persistent grids: workgroups that each have a CU to themselves (0: no such split)
  // byte sizes of the device-coherent buffers (bounds of their resources)
  uint32_t hh_bytes, y_bytes, logits_bytes, rows_bytes, ccnt_bytes;
  uint64_t budget;  // watchdog, in wall-clock ticks
  uint32_t* trace;
  uint32_t trace_records;
  // Decoder layer (dec = 1): the attention block runs first and writes the
  // MoE block's input (x above: RMSNorm of the residual stream) and the
  // residual the combine adds (resid); otherwise all of these are unused.
  int32_t dec;
  const uint16_t* dx;    // residual input [T, H]
  const uint16_t* g1;    // RMSNorm weights [H]
  const uint16_t* g2;
  const uint16_t* wqkv;  // [(nq + 2 nkv) d, H]
  const uint16_t* wo;    // [H, nq d]
  uint16_t* kc;          // key / value caches [T, nkv, Lcap, d], written at `pos`
  uint16_t* vc;
  uint16_t* h1;          // RMSNorm(dx) [T_max, H]
  uint16_t* qb;          // queries after RoPE [T_max, nq d]
  float* part;           // attention partials [T_max, nkv, nchunk_max, part_floats]
  uint16_t* ob;          // attention output [T_max, nq d]
  float* apart;          // output projection partial sums [kDecOSplit, T_max, H]
  uint16_t* resid;       // x2 = dx + attention block [T_max, H]; the combine adds it
  int32_t nq, nkv, Lcap, pos, nchunk, nchunk_max, part_floats;
  float theta, eps;
  uint32_t cache_bytes, h1_bytes, q_bytes, part_bytes, apart_bytes, resid_bytes;
};

// Static device scratch of moe_layer_launch_noalloc (moe_kernels.hip): one
// per GPU the library runs on, held until the process ends.
constexpr size_t kNoallocScratchBytes = (size_t)8 << 20;
// Its device address on the current device (hipGetSymbolAddress, taken once
// per device), and a fill kernel that zeroes its first `bytes`.
int moe_scratch(void** ptr);
int moe_scratch_clear(void* ptr, size_t bytes, void* stream);

// Host-side launchers (moe_kernels.hip).  Return a hipError_t value.
int launch_moe_persistent(const MoeParams& p, int sched, int grid, int lds_bytes, void* stream);
int launch_moe_kbk(const MoeParams& p, int lds_bytes, void* stream);
int launch_decoder_kbk(const MoeParams& p, int lds_bytes, void* stream);
// The coherence self-test (moe_kernels.hip): its workspace words for
// `pairs` producer/consumer pairs, and the launch (a fill kernel zeroes the
// workspace first).
size_t coherence_selftest_words(int pairs);
int launch_coherence_selftest(uint32_t* ws, int pairs, int rounds, uint64_t budget, void* stream);
int coherence_selftest_occupancy(int* blocks_per_cu);
// occupancy queries of the decoder-layer variants: kDecSchedBase + sched
constexpr int kDecSchedBase = 16;
// occupancy queries of the big-tile variant: kBigSchedBase + sched
constexpr int kBigSchedBase = 32;
// the big-tile variant's G tasks: two LDS stages of 512 rows x 64 k (bf16)
constexpr int kBigLdsBytes = 2 * 512 * 64 * 2;
int moe_persistent_occupancy(int sched, int lds_bytes, int* blocks_per_cu);
int launch_splitk(int n, int nsplit, int bk, const int32_t* A, int32_t* B, int32_t* C, int32_t* ev,
                  const etc_edge& notify_edge, const etc_edge& wait_edge, int32_t wait_count, uint32_t* ctl,
                  uint32_t* queue, int64_t q_cap, int sched, int grid,
                  uint64_t budget, void* stream);
int splitk_occupancy(int sched, int* blocks_per_cu);

}  // namespace etc
