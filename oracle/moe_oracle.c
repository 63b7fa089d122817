/*
 * Plain CPU oracle for one Mixture-of-Experts layer run as a graph of tiled
 * tasks, and for the split-K row-sum example.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  It shares no code,
 * header, table or constant with the HIP path: every helper below (bf16
 * conversion included) is written here on its own, straight from the
 * definitions, in loops meant to be checked by eye.
 *
 * Sources (cited by page title and figure/table/cue, as printed on the pages):
 *   [ET-fig N]      "Event Tensor: A Unified Abstraction for Compiling Dynamic
 *                   Megakernel" (arXiv 2604.13327), caption of Figure N.
 *   [ET-table N]    same paper, Table N.
 *   [ET-cast cue N] podcast episode on the same paper ("prompt-boundary-aware
 *                   scheduling with event tensors for dynamic kernels"),
 *                   transcript cue N.
 *
 * What the pages fix: the router's top-k drives per-expert token counts and
 * the exp_indptr prefix sum [ET-fig 2, ET-fig 5b, ET-cast cue 7, cue 9]; each
 * expert's tile range is [exp_indptr[e], exp_indptr[e+1]) [ET-cast cue 9];
 * the split-K example sums row i of A through an event of shape n with
 * wait_count 4 [ET-fig 3, ET-cast cue 3].  Everything else (summation order
 * of the router, tie-break, rounding points, SwiGLU, weighted combine) is a
 * stated reading; each function says which.
 *
 * The per-row loops of oracle_moe and oracle_moe_tokens carry an OpenMP
 * pragma: rows are independent and each is computed in the same order on
 * any thread, so the thread count changes the time, never a value.
 *
 * Floating point: fp64 everywhere except where a float decides an integer
 * (the router logits feeding top-k), which follows the fixed fp32 order
 * documented at oracle_router_logits, so both sides take the top-k decision
 * on identical values.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_INVALID (-1)
#define ORACLE_ERR_NONFINITE (-2)

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32, written from the format definition: bf16 is the upper 16
 * bits of an IEEE binary32.  Rounding is round-to-nearest, ties-to-even.   */

static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint16_t float_to_bf16_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u) {
    /* NaN: keep it a quiet NaN with the same sign */
    return (uint16_t)((u >> 16) | 0x0040u);
  }
  uint32_t lower = u & 0xffffu;      /* the 16 bits that are dropped   */
  uint32_t upper = u >> 16;          /* the kept part                   */
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

uint16_t oracle_f32_to_bf16(float f) { return float_to_bf16_bits(f); }

/* Threads for the per-row loops below (OpenMP; each routed row and each
 * token is computed on its own, in the same order, so the results do not
 * depend on the thread count).  n <= 0 leaves the OpenMP default.          */
void oracle_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
int oracle_max_threads(void) { return omp_get_max_threads(); }
float oracle_bf16_to_f32(uint16_t b) { return bf16_bits_to_float(b); }

/* ------------------------------------------------------------------------ */
/* Router logits, fixed-order fp32 (reading; the pages give no order).
 *
 * L[t,e] = sum_h X[t,h] * Wr[e,h]  (+ bias[e]).
 *
 * The order is a contract, so that the top-k decision is taken on the same
 * fp32 values on both sides:
 *   - the hidden dimension is cut into 8-element chunks c = 0 .. H/8-1;
 *     chunk c belongs to virtual lane l = c mod 64;
 *   - each lane starts from +0.0f and, over its chunks in ascending c and
 *     the 8 elements of a chunk in ascending h, does acc = fmaf(x, w, acc);
 *   - the 64 lane sums are combined by a halving tree: for s = 32,16,...,1
 *     and every l < s, acc[l] = acc[l] + acc[l + s];
 *   - the logit is acc[0], then + bias[e] (one fp32 add) if a bias is given.
 * H must be a multiple of 8; lanes that own no chunk keep +0.0f.           */
int oracle_router_logits(int T, int H, int E, const uint16_t *X,
                         const uint16_t *Wr, const float *bias, float *L) {
  if (T < 0 || H <= 0 || E <= 0 || (H % 8) != 0) return ORACLE_ERR_INVALID;
  const int nchunk = H / 8;
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      float lane[64];
      for (int l = 0; l < 64; ++l) lane[l] = 0.0f;
      for (int c = 0; c < nchunk; ++c) {
        int l = c % 64;
        for (int q = 0; q < 8; ++q) {
          int h = 8 * c + q;
          float x = bf16_bits_to_float(X[(size_t)t * H + h]);
          float w = bf16_bits_to_float(Wr[(size_t)e * H + h]);
          lane[l] = fmaf(x, w, lane[l]);
        }
      }
      for (int s = 32; s >= 1; s /= 2)
        for (int l = 0; l < s; ++l) lane[l] = lane[l] + lane[l + s];
      float v = lane[0];
      if (bias) v = v + bias[e];
      L[(size_t)t * E + e] = v;
    }
  }
  return ORACLE_OK;
}

/* Naive fp64 dot product of the same logits, for the sanity bound only.   */
int oracle_router_logits_f64(int T, int H, int E, const uint16_t *X,
                             const uint16_t *Wr, const float *bias, double *L) {
  if (T < 0 || H <= 0 || E <= 0) return ORACLE_ERR_INVALID;
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += (double)bf16_bits_to_float(X[(size_t)t * H + h]) *
               (double)bf16_bits_to_float(Wr[(size_t)e * H + h]);
      if (bias) acc += (double)bias[e];
      L[(size_t)t * E + e] = acc;
    }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Top-k and routing weights [ET-fig 2: the runtime tensor "topk"].
 *
 * Reading: per token the k largest logits, listed by descending logit; on
 * equal logits the lower expert index ranks first.  Weights (fp64, stored
 * fp32): with norm_topk, softmax over E renormalised over the chosen k,
 * i.e. exp(l_j - l_max) / sum_{i in topk} exp(l_i - l_max); without it,
 * the plain softmax over all E logits.  NaN logits are rejected.          */
static int ranks_before(float a, int ia, float b, int ib) {
  /* does (a, ia) rank strictly before (b, ib)? */
  if (a > b) return 1;
  if (a < b) return 0;
  return ia < ib;
}

int oracle_topk(int T, int E, int k, const float *L, int norm_topk,
                int32_t *ids, float *w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return ORACLE_ERR_INVALID;
  int *order = (int *)malloc(sizeof(int) * (size_t)E);
  if (!order) return ORACLE_ERR_INVALID;
  for (int t = 0; t < T; ++t) {
    const float *row = L + (size_t)t * E;
    for (int e = 0; e < E; ++e) {
      if (isnan(row[e])) { free(order); return ORACLE_ERR_NONFINITE; }
      order[e] = e;
    }
    /* selection: position j receives the best of the remaining entries */
    for (int j = 0; j < k; ++j) {
      int best = j;
      for (int m = j + 1; m < E; ++m)
        if (ranks_before(row[order[m]], order[m], row[order[best]], order[best]))
          best = m;
      int tmp = order[j]; order[j] = order[best]; order[best] = tmp;
    }
    double lmax = (double)row[order[0]];
    double denom = 0.0;
    if (norm_topk) {
      for (int j = 0; j < k; ++j) denom += exp((double)row[order[j]] - lmax);
    } else {
      for (int e = 0; e < E; ++e) denom += exp((double)row[e] - lmax);
    }
    for (int j = 0; j < k; ++j) {
      ids[(size_t)t * k + j] = order[j];
      w[(size_t)t * k + j] = (float)(exp((double)row[order[j]] - lmax) / denom);
    }
  }
  free(order);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Counts, exp_indptr and the token permutation [ET-cast cue 7, cue 9;
 * ET-fig 5b].  counts[e] is the number of (t,j) routed to e; exp_indptr is
 * the exclusive prefix sum (length E+1, ends at T*k).  Reading: the
 * permutation is the stable one, i.e. within expert e the routed pairs keep
 * ascending flat index t*k+j.  perm[s] = flat index held by slot s;
 * slot[f] = the slot of flat index f.                                       */
int oracle_route_scan(int T, int E, int k, const int32_t *ids, int32_t *counts,
                      int32_t *exp_indptr, int32_t *perm, int32_t *slot) {
  if (T < 0 || E <= 0 || k <= 0) return ORACLE_ERR_INVALID;
  const int n = T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int f = 0; f < n; ++f) {
    int e = ids[f];
    if (e < 0 || e >= E) return ORACLE_ERR_INVALID;
    counts[e] += 1;
  }
  exp_indptr[0] = 0;
  for (int e = 0; e < E; ++e) exp_indptr[e + 1] = exp_indptr[e] + counts[e];
  int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  if (!fill) return ORACLE_ERR_INVALID;
  for (int f = 0; f < n; ++f) {
    int e = ids[f];
    int s = exp_indptr[e] + fill[e];
    fill[e] += 1;
    perm[s] = f;
    slot[f] = s;
  }
  free(fill);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Expert computation for one routed row (reading: SwiGLU experts, with the
 * stored intermediates rounded to bf16 because activations are bf16).
 *   gate_i = sum_h x[h] * W13[e, i, h],   up_i = sum_h x[h] * W13[e, I+i, h]
 *   hmid_i = bf16( float( silu(gate_i) * up_i ) ),  silu(z) = z / (1 + e^-z)
 *   y_n    = bf16( float( sum_i hmid_i * Wd[e, n, i] ) )
 * Sums in fp64.                                                             */
static void expert_row(int H, int I, const uint16_t *x, const uint16_t *W13e,
                       const uint16_t *Wde, uint16_t *hmid, uint16_t *y) {
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    const uint16_t *wg = W13e + (size_t)i * H;
    const uint16_t *wu = W13e + (size_t)(I + i) * H;
    for (int h = 0; h < H; ++h) {
      double xv = (double)bf16_bits_to_float(x[h]);
      g += xv * (double)bf16_bits_to_float(wg[h]);
      u += xv * (double)bf16_bits_to_float(wu[h]);
    }
    double silu = g / (1.0 + exp(-g));
    hmid[i] = float_to_bf16_bits((float)(silu * u));
  }
  for (int n = 0; n < H; ++n) {
    double acc = 0.0;
    const uint16_t *wd = Wde + (size_t)n * I;
    for (int i = 0; i < I; ++i)
      acc += (double)bf16_bits_to_float(hmid[i]) * (double)bf16_bits_to_float(wd[i]);
    y[n] = float_to_bf16_bits((float)acc);
  }
}

/* Weighted combine (reading of "followed by a weighted combine"):
 *   out[t, n] = bf16( float( sum_{j<k} w[t,j] * Y[slot[t*k+j], n] ) ), fp64. */

/* Full layer.  Inputs: X [T,H], Wr [E,H], bias [E] or NULL, W13 [E,2I,H],
 * Wd [E,H,I] (bf16 bits).  Outputs: routing tensors and out [T,H] (bf16),
 * plus the grouped intermediates Xp [T*k,H], Hmid [T*k,I], Y [T*k,H] when
 * those pointers are non-NULL.                                              */
int oracle_moe(int T, int H, int E, int k, int I, int norm_topk,
               const uint16_t *X, const uint16_t *Wr, const float *bias,
               const uint16_t *W13, const uint16_t *Wd, float *logits,
               int32_t *ids, float *w, int32_t *counts, int32_t *exp_indptr,
               int32_t *perm, int32_t *slot, uint16_t *Xp, uint16_t *Hmid,
               uint16_t *Y, uint16_t *out) {
  if (T < 0 || H <= 0 || E <= 0 || k <= 0 || k > E || I <= 0)
    return ORACLE_ERR_INVALID;
  int rc = oracle_router_logits(T, H, E, X, Wr, bias, logits);
  if (rc) return rc;
  rc = oracle_topk(T, E, k, logits, norm_topk, ids, w);
  if (rc) return rc;
  rc = oracle_route_scan(T, E, k, ids, counts, exp_indptr, perm, slot);
  if (rc) return rc;
  const int n = T * k;
  uint16_t *yall = Y ? Y : (uint16_t *)malloc(sizeof(uint16_t) * (size_t)n * H);
  if (!yall) return ORACLE_ERR_INVALID;
  /* every grouped row s belongs to the expert e with exp_indptr[e] <= s <
   * exp_indptr[e+1]; rows are independent, so they are spread over threads */
  int fail = 0;
#pragma omp parallel
  {
    uint16_t *hrow = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
    if (!hrow) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int s = 0; s < n; ++s) {
      if (!hrow) continue;
      int e = 0;
      while (exp_indptr[e + 1] <= s) ++e;
      int t = perm[s] / k;
      const uint16_t *x = X + (size_t)t * H;
      if (Xp) memcpy(Xp + (size_t)s * H, x, sizeof(uint16_t) * (size_t)H);
      expert_row(H, I, x, W13 + (size_t)e * 2 * I * H, Wd + (size_t)e * H * I,
                 hrow, yall + (size_t)s * H);
      if (Hmid) memcpy(Hmid + (size_t)s * I, hrow, sizeof(uint16_t) * (size_t)I);
    }
    free(hrow);
  }
  if (fail) { if (!Y) free(yall); return ORACLE_ERR_INVALID; }
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) {
        int s = slot[(size_t)t * k + j];
        acc += (double)w[(size_t)t * k + j] *
               (double)bf16_bits_to_float(yall[(size_t)s * H + h]);
      }
      out[(size_t)t * H + h] = float_to_bf16_bits((float)acc);
    }
  if (!Y) free(yall);
  return ORACLE_OK;
}

/* Output rows for a subset of tokens, given routing already computed by
 * oracle_moe's first three steps (ids, w).  Lets large workloads be checked
 * token by token: out_rows[r, :] is the layer output of token tok[r].      */
int oracle_moe_tokens(int H, int k, int I, int ntok, const int32_t *tok,
                      const uint16_t *X, const uint16_t *W13, const uint16_t *Wd,
                      const int32_t *ids, const float *w, uint16_t *out_rows) {
  if (H <= 0 || k <= 0 || I <= 0 || ntok < 0) return ORACLE_ERR_INVALID;
  int fail = 0;
  /* tokens are independent: spread over threads */
#pragma omp parallel
  {
    uint16_t *hrow = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)I);
    uint16_t *y = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)k * H);
    if (!hrow || !y) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int r = 0; r < ntok; ++r) {
      if (!hrow || !y) continue;
      int t = tok[r];
      for (int j = 0; j < k; ++j) {
        int e = ids[(size_t)t * k + j];
        expert_row(H, I, X + (size_t)t * H, W13 + (size_t)e * 2 * I * H,
                   Wd + (size_t)e * H * I, hrow, y + (size_t)j * H);
      }
      for (int h = 0; h < H; ++h) {
        double acc = 0.0;
        for (int j = 0; j < k; ++j)
          acc += (double)w[(size_t)t * k + j] *
                 (double)bf16_bits_to_float(y[(size_t)j * H + h]);
        out_rows[(size_t)r * H + h] = float_to_bf16_bits((float)acc);
      }
    }
    free(hrow);
    free(y);
  }
  return fail ? ORACLE_ERR_INVALID : ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Split-K row sum [ET-fig 3, ET-cast cue 3].  A is [n, nsplit*bk] int32.
 * partial_sum(i, j): B[i, j] = sum of A[i, c] over tile j's columns
 * c in [j*bk, (j+1)*bk), then notify event i (edge "ij->i").  final_sum(i)
 * waits on event i (edge "i->i"), whose wait_count is nsplit, and writes
 * C[i] = sum_j B[i, j].  Integer sums, so the order of completion is
 * irrelevant.  Also returns the number of notifies each event receives.    */
int oracle_splitk(int n, int nsplit, int bk, const int32_t *A, int32_t *B,
                  int32_t *C, int32_t *notifies) {
  if (n < 0 || nsplit <= 0 || bk <= 0) return ORACLE_ERR_INVALID;
  for (int i = 0; i < n; ++i) notifies[i] = 0;
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < nsplit; ++j) {
      int32_t acc = 0;
      for (int c = j * bk; c < (j + 1) * bk; ++c)
        acc += A[(size_t)i * nsplit * bk + c];
      B[(size_t)i * nsplit + j] = acc;
      notifies[i] += 1; /* edge "ij->i": tile (i, j) notifies event i */
    }
  for (int i = 0; i < n; ++i) {
    int32_t acc = 0;
    for (int j = 0; j < nsplit; ++j) acc += B[(size_t)i * nsplit + j];
    C[i] = acc;
  }
  return ORACLE_OK;
}

/* ======================================================================== */
/* One decoder layer around the MoE layer (a Qwen3-30B-A3B-shaped layer at  */
/* decode: the fifth workload of the build).  The pages evaluate the MoE    */
/* layer inside end-to-end serving [ET-fig 14] but print no decoder layer;  */
/* every step below is the textbook definition, with these readings:        */
/*   - pre-norm residual block: x2 = x + Attn(RMSNorm(x)),                  */
/*     out = x2 + MoE(RMSNorm(x2));                                         */
/*   - RMSNorm(v) = v / sqrt(mean(v^2) + eps) * g, eps = 1e-6;              */
/*   - grouped-query attention: query head h reads key/value head           */
/*     h / (nq / nkv); scores scaled by 1/sqrt(d); no QK norm;              */
/*   - rotary embedding on q and k, rotate-half pairs (i, i + d/2) with     */
/*     angle pos * theta^(-2i/d), theta = 1e6;                              */
/*   - the new token sits at position `pos`: its key and value are written  */
/*     into the cache at index pos, and it attends to cache entries 0..pos; */
/*   - every stored activation (norm outputs, q/k/v after RoPE, attention   */
/*     output, projection output, residual sums, layer output) is bf16;     */
/*     sums are fp64.                                                       */

/* y[t, :] = bf16( x[t, :] / sqrt(mean_h x[t, h]^2 + eps) * g ), fp64.      */
int oracle_rmsnorm(int T, int H, const uint16_t *x, const uint16_t *g, double eps, uint16_t *y) {
  if (T < 0 || H <= 0 || eps < 0.0) return ORACLE_ERR_INVALID;
  for (int t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int h = 0; h < H; ++h) {
      double v = (double)bf16_bits_to_float(x[(size_t)t * H + h]);
      ss += v * v;
    }
    double r = 1.0 / sqrt(ss / (double)H + eps);
    for (int h = 0; h < H; ++h)
      y[(size_t)t * H + h] = float_to_bf16_bits(
          (float)((double)bf16_bits_to_float(x[(size_t)t * H + h]) * r *
                  (double)bf16_bits_to_float(g[h])));
  }
  return ORACLE_OK;
}

/* y[t, n] = bf16( sum_k x[t, k] * W[n, k] ), fp64 (W row-major [N, K]).    */
int oracle_linear(int T, int K, int N, const uint16_t *x, const uint16_t *W, uint16_t *y) {
  if (T < 0 || K <= 0 || N <= 0) return ORACLE_ERR_INVALID;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k)
        acc += (double)bf16_bits_to_float(x[(size_t)t * K + k]) *
               (double)bf16_bits_to_float(W[(size_t)n * K + k]);
      y[(size_t)t * N + n] = float_to_bf16_bits((float)acc);
    }
  return ORACLE_OK;
}

/* Rotary embedding, in place on nvec vectors of d bf16 values (d even):
 * for i < d/2, a = pos * theta^(-2i/d):
 *   v'[i]       = v[i] cos a - v[i + d/2] sin a
 *   v'[i + d/2] = v[i + d/2] cos a + v[i] sin a      (fp64, stored bf16)  */
int oracle_rope(int nvec, int d, uint16_t *v, double pos, double theta) {
  if (nvec < 0 || d <= 0 || d % 2 || theta <= 0.0) return ORACLE_ERR_INVALID;
  const int half = d / 2;
  for (int r = 0; r < nvec; ++r) {
    uint16_t *u = v + (size_t)r * d;
    for (int i = 0; i < half; ++i) {
      double a = pos * pow(theta, -2.0 * (double)i / (double)d);
      double x0 = (double)bf16_bits_to_float(u[i]);
      double x1 = (double)bf16_bits_to_float(u[i + half]);
      u[i] = float_to_bf16_bits((float)(x0 * cos(a) - x1 * sin(a)));
      u[i + half] = float_to_bf16_bits((float)(x1 * cos(a) + x0 * sin(a)));
    }
  }
  return ORACLE_OK;
}

/* Decode attention of one token.  q [nq, d]; the token's key and value
 * caches Kc, Vc [nkv, Lcap, d] (row-major), of which entries 0..L-1 are
 * read; query head h uses key/value head h / (nq / nkv).
 *   o[h, :] = bf16( sum_j p_j V[g, j, :] ),  p = softmax_j( q_h . K[g, j] / sqrt(d) )
 * in fp64 (the maximum is subtracted before exp).                          */
int oracle_attention(int nq, int nkv, int d, int L, int Lcap, const uint16_t *q, const uint16_t *Kc,
                     const uint16_t *Vc, uint16_t *o) {
  if (nq <= 0 || nkv <= 0 || nq % nkv || d <= 0 || L <= 0 || L > Lcap) return ORACLE_ERR_INVALID;
  double *s = (double *)malloc(sizeof(double) * (size_t)L);
  if (!s) return ORACLE_ERR_INVALID;
  const double scale = 1.0 / sqrt((double)d);
  for (int h = 0; h < nq; ++h) {
    const int g = h / (nq / nkv);
    const uint16_t *K = Kc + (size_t)g * Lcap * d;
    const uint16_t *V = Vc + (size_t)g * Lcap * d;
    double m = -INFINITY;
    for (int j = 0; j < L; ++j) {
      double acc = 0.0;
      for (int c = 0; c < d; ++c)
        acc += (double)bf16_bits_to_float(q[(size_t)h * d + c]) *
               (double)bf16_bits_to_float(K[(size_t)j * d + c]);
      s[j] = acc * scale;
      if (s[j] > m) m = s[j];
    }
    double den = 0.0;
    for (int j = 0; j < L; ++j) {
      s[j] = exp(s[j] - m);
      den += s[j];
    }
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < L; ++j) acc += s[j] * (double)bf16_bits_to_float(V[(size_t)j * d + c]);
      o[(size_t)h * d + c] = float_to_bf16_bits((float)(acc / den));
    }
  }
  free(s);
  return ORACLE_OK;
}

/* The decoder layer for T tokens, token t decoding at position pos with its
 * own caches kcache/vcache [T, nkv, Lcap, d] (updated in place at index pos).
 * Wqkv [(nq + 2 nkv) d, H]: rows of the query heads, then of the key heads,
 * then of the value heads.  Wo [H, nq d].  The MoE arguments are those of
 * oracle_moe; its routing outputs are returned.  Intermediates (any may be
 * NULL): h1 [T, H], qkv [T, (nq + 2 nkv) d] after RoPE, att [T, nq d],
 * a [T, H], x2 [T, H], h2 [T, H], moe_out [T, H].                           */
int oracle_decoder(int T, int H, int nq, int nkv, int d, int pos, int Lcap, double theta, double eps,
                   const uint16_t *x, const uint16_t *g1, const uint16_t *Wqkv, uint16_t *kcache,
                   uint16_t *vcache, const uint16_t *Wo, const uint16_t *g2,
                   int E, int k, int I, int norm_topk, const uint16_t *Wr, const uint16_t *W13,
                   const uint16_t *Wd, float *logits, int32_t *ids, float *w, int32_t *counts,
                   int32_t *exp_indptr, int32_t *perm, int32_t *slot, uint16_t *out,
                   uint16_t *h1, uint16_t *qkv, uint16_t *att, uint16_t *a, uint16_t *x2, uint16_t *h2,
                   uint16_t *moe_out) {
  if (T <= 0 || H <= 0 || nq <= 0 || nkv <= 0 || nq % nkv || d <= 0 || d % 2 || pos < 0 || pos >= Lcap)
    return ORACLE_ERR_INVALID;
  const int nqkv = (nq + 2 * nkv) * d;
  uint16_t *b_h1 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * H);
  uint16_t *b_qkv = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * nqkv);
  uint16_t *b_att = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * nq * d);
  uint16_t *b_a = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * H);
  uint16_t *b_x2 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * H);
  uint16_t *b_h2 = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * H);
  uint16_t *b_moe = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)T * H);
  int rc = ORACLE_ERR_INVALID;
  if (!b_h1 || !b_qkv || !b_att || !b_a || !b_x2 || !b_h2 || !b_moe) goto done;
  /* attention block */
  rc = oracle_rmsnorm(T, H, x, g1, eps, b_h1);
  if (rc) goto done;
  rc = oracle_linear(T, H, nqkv, b_h1, Wqkv, b_qkv);
  if (rc) goto done;
  for (int t = 0; t < T; ++t) {
    uint16_t *row = b_qkv + (size_t)t * nqkv;
    rc = oracle_rope(nq + nkv, d, row, (double)pos, theta); /* the query heads, then the key heads */
    if (rc) goto done;
    for (int g = 0; g < nkv; ++g) {
      size_t at = (((size_t)t * nkv + g) * Lcap + pos) * d;
      memcpy(kcache + at, row + (size_t)(nq + g) * d, sizeof(uint16_t) * (size_t)d);
      memcpy(vcache + at, row + (size_t)(nq + nkv + g) * d, sizeof(uint16_t) * (size_t)d);
    }
    rc = oracle_attention(nq, nkv, d, pos + 1, Lcap, row, kcache + (size_t)t * nkv * Lcap * d,
                          vcache + (size_t)t * nkv * Lcap * d, b_att + (size_t)t * nq * d);
    if (rc) goto done;
  }
  rc = oracle_linear(T, nq * d, H, b_att, Wo, b_a);
  if (rc) goto done;
  for (size_t i = 0; i < (size_t)T * H; ++i)
    b_x2[i] = float_to_bf16_bits((float)((double)bf16_bits_to_float(x[i]) + (double)bf16_bits_to_float(b_a[i])));
  /* MoE block */
  rc = oracle_rmsnorm(T, H, b_x2, g2, eps, b_h2);
  if (rc) goto done;
  rc = oracle_moe(T, H, E, k, I, norm_topk, b_h2, Wr, NULL, W13, Wd, logits, ids, w, counts, exp_indptr, perm,
                  slot, NULL, NULL, NULL, b_moe);
  if (rc) goto done;
  for (size_t i = 0; i < (size_t)T * H; ++i)
    out[i] = float_to_bf16_bits((float)((double)bf16_bits_to_float(b_x2[i]) + (double)bf16_bits_to_float(b_moe[i])));
  if (h1) memcpy(h1, b_h1, sizeof(uint16_t) * (size_t)T * H);
  if (qkv) memcpy(qkv, b_qkv, sizeof(uint16_t) * (size_t)T * nqkv);
  if (att) memcpy(att, b_att, sizeof(uint16_t) * (size_t)T * nq * d);
  if (a) memcpy(a, b_a, sizeof(uint16_t) * (size_t)T * H);
  if (x2) memcpy(x2, b_x2, sizeof(uint16_t) * (size_t)T * H);
  if (h2) memcpy(h2, b_h2, sizeof(uint16_t) * (size_t)T * H);
  if (moe_out) memcpy(moe_out, b_moe, sizeof(uint16_t) * (size_t)T * H);
  rc = ORACLE_OK;
done:
  free(b_h1); free(b_qkv); free(b_att); free(b_a); free(b_x2); free(b_h2); free(b_moe);
  return rc;
}
