// Task bodies of the attention block that runs before the MoE block in the
// decoder-layer launch.  Included by moe_kernels.hip, inside its namespace,
// after the MoE task bodies, whose helpers (bf16 conversion, coherent
// accesses, Ctx, events) it uses.
//
//   N1(t)       h1 = RMSNorm(x) * g1 for token t (the four waves split H)
//   QKV(c)      16 columns of h1 Wqkv^T; for query and key heads the 16
//               columns are 8 rotary pairs (i, i + d/2), rotated at `pos`;
//               queries go to qb, keys and values into the caches at `pos`
//   ATT(t,g,ch) 256 cache entries of token t, kv head g: scores for the
//               group's query heads (bf16 MFMA), their maximum, the
//               exponentials and the weighted value sum (fp32), stored as a
//               partial (sum, maximum, normaliser)
//   ATTC(t,g)   merges the partials with the new entry's own score and
//               value into the attention output of the group's heads
//   O(c,ks)     16 columns of o Wo^T over one quarter of the inner dimension
//               (fp32 partial sums)
//   N2(t)       a = bf16(sum of the quarters), x2 = bf16(x + a),
//               h2 = RMSNorm(x2) * g2: h2 is the MoE block's input, x2 the
//               residual its combine adds
// Data one task writes and another reads moves through device-coherent
// accesses (qb, the caches' entry `pos`, partials, o, the projection sums,
// x2, h2); inputs (x, weights, cache entries below `pos`) through the caches.
#pragma once
// (included inside namespace etc)

__device__ __forceinline__ rsrc_t r_h1(const MoeParams& p) { return make_rsrc(p.h1, p.h1_bytes); }
__device__ __forceinline__ rsrc_t r_qb(const MoeParams& p) { return make_rsrc(p.qb, p.q_bytes); }
__device__ __forceinline__ rsrc_t r_ob(const MoeParams& p) { return make_rsrc(p.ob, p.q_bytes); }
__device__ __forceinline__ rsrc_t r_part(const MoeParams& p) { return make_rsrc(p.part, p.part_bytes); }
__device__ __forceinline__ rsrc_t r_apart(const MoeParams& p) { return make_rsrc(p.apart, p.apart_bytes); }
__device__ __forceinline__ rsrc_t r_resid(const MoeParams& p) { return make_rsrc(p.resid, p.resid_bytes); }
__device__ __forceinline__ rsrc_t r_h2(const MoeParams& p) { return make_rsrc(p.x, p.resid_bytes); }
__device__ __forceinline__ rsrc_t r_kc(const MoeParams& p) { return make_rsrc(p.kc, p.cache_bytes); }
__device__ __forceinline__ rsrc_t r_vc(const MoeParams& p) { return make_rsrc(p.vc, p.cache_bytes); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}
__device__ __forceinline__ float bf_round(float f) { return __uint_as_float(f2bf(f) << 16); }

// Decoder task counts of a launch
struct DecCounts {
  int nN, nQKV, nATT, nATTC, nO;
};
__device__ __forceinline__ DecCounts dec_counts(const MoeParams& p, const Ctx& c) {
  DecCounts n;
  n.nN = (c.T + kDecNormT - 1) / kDecNormT;
  n.nQKV = (p.nq + 2 * p.nkv) * (kDecHd / 16);
  n.nATT = c.T * p.nkv * p.nchunk;
  n.nATTC = c.T * p.nkv;
  n.nO = (c.H / 16) * kDecOSplit;
  return n;
}

// Sum of one value per thread over the workgroup: a shuffle tree inside
// each wave, then the four wave sums through LDS.
__device__ __forceinline__ float block_sum(float v, float* s4) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) s4[threadIdx.x >> 6] = v;
  __syncthreads();
  return (s4[0] + s4[1]) + (s4[2] + s4[3]);
}
// The RMSNorm tasks keep up to kNormPer 8-element chunks a thread in
// registers between the sum of squares and the scaling (H <= 8192); chunks
// beyond are read again.
constexpr int kNormPer = 4;

// N1: h1 = bf16(x * r * g1), r = 1 / sqrt(mean(x^2) + eps), fp32.  Every
// chunk of the token's row and of g1 is requested at once.
__device__ __forceinline__ void task_norm1(const MoeParams& p, const Ctx& c, int t) {
  __shared__ float s4[4];
  const int tid = threadIdx.x;
  const int H = c.H, nch = H >> 3;
  const uint16_t* xr = p.dx + (size_t)t * H;
  u32x4_t xv[kNormPer], gv[kNormPer];
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int ch = tid + j * kThreads;
    if (ch < nch) {
      xv[j] = ld4(xr + ch * 8);
      gv[j] = ld4(p.g1 + ch * 8);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    if (tid + j * kThreads < nch) {
      float f[8];
      unpack8(xv[j], f);
#pragma unroll
      for (int q = 0; q < 8; ++q) ss = __builtin_fmaf(f[q], f[q], ss);
    }
  }
  for (int ch = tid + kNormPer * kThreads; ch < nch; ch += kThreads) {
    float f[8];
    unpack8(ld4(xr + ch * 8), f);
#pragma unroll
    for (int q = 0; q < 8; ++q) ss = __builtin_fmaf(f[q], f[q], ss);
  }
  ss = block_sum(ss, s4);
  const float r = 1.0f / sqrtf(ss / (float)H + p.eps);
  const rsrc_t rh = r_h1(p);
  auto out = [&](int ch, const float* f, const float* g) {
    u32x4_t o;
    o.x = f2bf(f[0] * r * g[0]) | (f2bf(f[1] * r * g[1]) << 16);
    o.y = f2bf(f[2] * r * g[2]) | (f2bf(f[3] * r * g[3]) << 16);
    o.z = f2bf(f[4] * r * g[4]) | (f2bf(f[5] * r * g[5]) << 16);
    o.w = f2bf(f[6] * r * g[6]) | (f2bf(f[7] * r * g[7]) << 16);
    co_st128(rh, (uint32_t)(((size_t)t * H + ch * 8) * 2), o);
  };
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int ch = tid + j * kThreads;
    if (ch < nch) {
      float f[8], g[8];
      unpack8(xv[j], f);
      unpack8(gv[j], g);
      out(ch, f, g);
    }
  }
  for (int ch = tid + kNormPer * kThreads; ch < nch; ch += kThreads) {
    float f[8], g[8];
    unpack8(ld4(xr + ch * 8), f);
    unpack8(ld4(p.g1 + ch * 8), g);
    out(ch, f, g);
  }
}

// One 16-column tile of rows [0, T) of A times W^T over K = kend - kbeg:
// A (bf16, rows of `astride` elements) through a coherent resource, W's
// rows `wrow(n)` through the caches; the four waves split K, reduce in
// `red` (4 x 256 fp32) and leave the tile in `stage` [16 rows][16 cols].
template <class WRow>
__device__ __forceinline__ void tile16(rsrc_t ra, uint32_t astride, const uint16_t* W, uint32_t wstride, int T, int kbeg,
                                       int kend, WRow wrow, float* red, float* stage) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int m = lane & 15, kg = lane >> 4;
  const int kw = (kend - kbeg) >> 2, nsteps = kw >> 5;
  const bool valid = m < T;
  const uint32_t aoff = (uint32_t)(((size_t)(valid ? m : 0) * astride + kbeg + wv * kw + kg * 8) * 2);
  const uint16_t* pb = W + (size_t)wrow(m) * wstride + kbeg + wv * kw + kg * 8;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  constexpr int U = 8;
  if (nsteps % U == 0) {
    // rolling pipeline over U register slots (as the MoE block's small G
    // tiles): U - 1 to U steps of loads in flight, so a task of one tile is
    // about one memory latency plus its stream.  Rows past T load row 0;
    // their output rows are never stored.
    u32x4_t a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = co_ld128(ra, aoff + (uint32_t)u * 64u);
      b[u] = ld4(pb + u * 32);
    }
    for (int s0 = U; s0 < nsteps; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u]), as_bf(b[u]), acc, 0, 0, 0);
        a[u] = co_ld128(ra, aoff + (uint32_t)(s0 + u) * 64u);
        b[u] = ld4(pb + (s0 + u) * 32);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u]), as_bf(b[u]), acc, 0, 0, 0);
  } else
  for (int s0 = 0; s0 < nsteps; s0 += 4) {
    u32x4_t a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0 + u < nsteps) {
        a[u] = valid ? co_ld128(ra, aoff + (uint32_t)(s0 + u) * 64u) : zero;
        b[u] = ld4(pb + (s0 + u) * 32);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + u < nsteps) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(a[u]), as_bf(b[u]), acc, 0, 0, 0);
  }
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wv * 256 + lane * 4 + i] = acc[i];
  __syncthreads();
  {
    // element (lane', i) of a 16x16 MFMA result: row 4 (lane' / 16) + i, column lane' % 16
    const int ol = tid >> 2, oi = tid & 3;
    const float v = red[tid] + red[256 + tid] + red[512 + tid] + red[768 + tid];
    stage[(4 * (ol >> 4) + oi) * 16 + (ol & 15)] = v;
  }
  __syncthreads();
}

// QKV tile ct.  Head tiles (query and key heads, 8 a head) hold columns
// i0 .. i0+7 and i0+d/2 .. i0+d/2+7 of one head: the MFMA's columns 0..7 and
// 8..15, so that each rotary pair is in one tile.  Value tiles hold 16
// consecutive columns.  The projection is rounded to bf16, then rotated.
__device__ __forceinline__ void task_qkv(const MoeParams& p, const Ctx& c, int ct, float* red) {
  const int d = kDecHd, half = kDecHd / 2, tph = kDecHd / 16;
  const int nhead_tiles = (p.nq + p.nkv) * tph;
  const bool rope = ct < nhead_tiles;
  const int hh = rope ? ct / tph : 0, i0 = rope ? (ct % tph) * 8 : 0;
  const int vcol0 = rope ? 0 : (ct - nhead_tiles) * 16;  // column inside the value block
  float* stage = red + 1024;
  uint16_t* ostage = reinterpret_cast<uint16_t*>(red + 1024 + 256);  // [16 rows][16 cols] bf16
  auto wrow = [&](int n) {
    return rope ? hh * d + (n < 8 ? i0 + n : half + i0 + n - 8) : (p.nq + p.nkv) * d + vcol0 + n;
  };
  tile16(r_h1(p), (uint32_t)c.H, p.wqkv, (uint32_t)c.H, c.T, 0, c.H, wrow, red, stage);
  const int tid = threadIdx.x;
  if (rope) {
    if (tid < 128) {
      const int row = tid >> 3, j = tid & 7, i = i0 + j;
      const float x0 = bf_round(stage[row * 16 + j]), x1 = bf_round(stage[row * 16 + 8 + j]);
      const double a = (double)p.pos * pow((double)p.theta, -2.0 * (double)i / (double)d);
      double sa, ca;
      sincos(a, &sa, &ca);
      const float cf = (float)ca, sf = (float)sa;
      ostage[row * 16 + j] = (uint16_t)f2bf(x0 * cf - x1 * sf);
      ostage[row * 16 + 8 + j] = (uint16_t)f2bf(x1 * cf + x0 * sf);
    }
  } else {
    const int row = tid >> 4, col = tid & 15;
    ostage[row * 16 + col] = (uint16_t)f2bf(stage[row * 16 + col]);
  }
  __syncthreads();
  // rows x two 16-byte halves (one rotary half each, or 8 + 8 value columns)
  if (tid < 2 * c.T) {
    const int row = tid >> 1, hf = tid & 1;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(ostage + row * 16 + hf * 8);
    if (rope && hh < p.nq) {
      co_st128(r_qb(p), (uint32_t)(((size_t)row * p.nq * d + hh * d + hf * half + i0) * 2), v);
    } else {
      const int g = rope ? hh - p.nq : vcol0 / d;
      const int col = rope ? hf * half + i0 : vcol0 % d + hf * 8;
      const uint32_t off = (uint32_t)(((((size_t)row * p.nkv + g) * p.Lcap + p.pos) * d + col) * 2);
      co_st128(rope ? r_kc(p) : r_vc(p), off, v);
    }
  }
}

// LDS of one attention task: the scores P [16 rows][kDecChunk], whose space
// then holds the four waves' value sums [4][group heads][head size], then
// 64 + 32 floats of maxima and sums
constexpr int kAttnPFloats =
    16 * kDecChunk > 4 * kDecMaxGroup * kDecHd ? 16 * kDecChunk : 4 * kDecMaxGroup * kDecHd;
constexpr int kAttnLdsFloats = kAttnPFloats + 64 + 32;
static_assert(kAttnLdsFloats * 4 <= kGemmLdsBytes, "the persistent kernels' LDS holds an attention task");
// ATT: cache entries k0 .. k0 + nk - 1 (k0 = ch * kDecChunk, all below pos)
// of token t and kv head g, for the group's gq query heads.  Scores by bf16
// MFMA (A = the heads' queries, 16 rows with gq used; B = 16 entries a
// column block, wave w covering entries w*64 .. w*64+63); softmax maximum
// and sums across the waves in LDS; the weighted value sum on the VALU.
// Chunks of 256 entries give the grid one task a workgroup at the decoder
// workload (8 tokens x 4 kv heads x 16 chunks), and each task issues all of
// its key loads, then all of its value loads, at once: the task is a few
// memory latencies long instead of one per batch.  (Every schedule uses
// the same chunks, so all of them sum in the same order.)
// The partial holds, per head, the unnormalised sum over the chunk, the
// chunk's maximum score and the sum of exp(score - maximum).
__device__ __forceinline__ void task_attn(const MoeParams& p, const Ctx& c, int t, int g, int ch, float* lds) {
  (void)c;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, tid = threadIdx.x;
  const int m = lane & 15, kg = lane >> 4;
  const int d = kDecHd, gq = p.nq / p.nkv;
  const int k0 = ch * kDecChunk, nk = min(kDecChunk, p.pos - k0);
  float* P = lds;                          // [16 rows][kDecChunk], later the waves' value sums
  float* wred = lds + kAttnPFloats;        // [4 waves][16 rows]
  float* mrow = wred + 64;                 // [16] row maxima, then [16] sums
  const float scale = 1.0f / sqrtf((float)d);
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t qa[4];
  const rsrc_t rq = r_qb(p);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qa[s] = m < gq ? co_ld128(rq, (uint32_t)((((size_t)t * p.nq + g * gq + m) * d + s * 32 + kg * 8) * 2)) : zero;
  const size_t cbase = (((size_t)t * p.nkv + g) * p.Lcap + k0) * d;
  const uint16_t* kb = p.kc + cbase;
  // every key block of the wave in flight at once: one memory latency
  constexpr int NBW = kDecChunk / 64;  // 16-entry column blocks a wave
  constexpr int EPW = kDecChunk / 4;   // entries a wave
  f32x4_t sc[NBW];
  u32x4_t b[NBW][4];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int e = wv * EPW + nb * 16 + m;
#pragma unroll
    for (int s = 0; s < 4; ++s) b[nb][s] = e < nk ? ld4(kb + (size_t)e * d + s * 32 + kg * 8) : zero;
  }
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(qa[s]), as_bf(b[nb][s]), acc, 0, 0, 0);
    sc[nb] = acc;
  }
  // lane holds rows 4 kg + i (heads), entry wv*EPW + nb*16 + m of every block
  const float NEG_INF = -__builtin_inff();
  float mx[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const bool ok = wv * EPW + nb * 16 + m < nk;
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = ok ? fmaxf(mx[i], sc[nb][i] * scale) : mx[i];
  }
#pragma unroll
  for (int s = 1; s < 16; s <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], s));
  if (m == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) wred[wv * 16 + 4 * kg + i] = mx[i];
  lds_barrier();
  if (tid < 16) mrow[tid] = fmaxf(fmaxf(wred[tid], wred[16 + tid]), fmaxf(wred[32 + tid], wred[48 + tid]));
  lds_barrier();
  float rm[4], sm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) rm[i] = mrow[4 * kg + i];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int e = wv * EPW + nb * 16 + m;
    const bool ok = e < nk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = ok ? __expf(sc[nb][i] * scale - rm[i]) : 0.f;
      P[(4 * kg + i) * kDecChunk + e] = pv;
      sm[i] += pv;
    }
  }
#pragma unroll
  for (int s = 1; s < 16; s <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm[i] += __shfl_xor(sm[i], s);
  if (m == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) wred[wv * 16 + 4 * kg + i] = sm[i];
  lds_barrier();
  if (tid < 16) mrow[16 + tid] = wred[tid] + wred[16 + tid] + wred[32 + tid] + wred[48 + tid];
  // Weighted value sum on the VALU.  Wave wv, lane (kq = lane / 32,
  // cg = lane % 32) takes entries e = 2 wv + kq + 8 i and dims 4 cg ..
  // 4 cg + 3, for every head of the group; all of its values load at once
  // (one memory latency).  The 8 (wave, kq) partial sums are then added:
  // across kq by a shuffle, across the waves in LDS (over P, which is no
  // longer read by then).
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const int kq = lane >> 5, cg = lane & 31;
  const int e0 = 2 * wv + kq;
  const uint16_t* vb = p.vc + cbase + 4 * cg;
  float acc[kDecMaxGroup][4];
#pragma unroll
  for (int h = 0; h < kDecMaxGroup; ++h)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[h][q] = 0.f;
  const u32x2_t zero2 = {0u, 0u};
  constexpr int NV = kDecChunk / 8;  // entries a thread takes
  u32x2_t vv[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = e0 + 8 * u;
    vv[u] = e < nk ? *reinterpret_cast<const u32x2_t*>(vb + (size_t)e * d) : zero2;
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int e = e0 + 8 * u;
    if (e < nk) {
      const float v[4] = {bf_lo(vv[u].x), bf_hi(vv[u].x), bf_lo(vv[u].y), bf_hi(vv[u].y)};
#pragma unroll
      for (int h = 0; h < kDecMaxGroup; ++h) {
        if (h < gq) {
          const float pw = P[h * kDecChunk + e];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[h][q] = __builtin_fmaf(pw, v[q], acc[h][q]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < kDecMaxGroup; ++h)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[h][q] += __shfl_xor(acc[h][q], 32);
  lds_barrier();  // every wave is done with P: its space holds the waves' sums
  float* osum = P;  // [4 waves][gq heads][d]
  if (kq == 0) {
#pragma unroll
    for (int h = 0; h < kDecMaxGroup; ++h)
      if (h < gq)
#pragma unroll
        for (int q = 0; q < 4; ++q) osum[(wv * gq + h) * d + 4 * cg + q] = acc[h][q];
  }
  lds_barrier();
  const rsrc_t rp = r_part(p);
  const uint32_t pbase = (uint32_t)((((size_t)t * p.nkv + g) * p.nchunk_max + ch) * p.part_floats * 4);
  for (int i = tid; i < gq * d; i += kThreads) {
    const float v = osum[i] + osum[gq * d + i] + osum[2 * gq * d + i] + osum[3 * gq * d + i];
    co_stf(rp, pbase + (uint32_t)(i * 4), v);
  }
  if (tid < gq) {
    co_stf(rp, pbase + (uint32_t)((gq * d + tid) * 4), mrow[tid]);
    co_stf(rp, pbase + (uint32_t)((gq * d + gq + tid) * 4), mrow[16 + tid]);
  }
}

// ATTC: the attention output of token t's heads g*gq .. g*gq+gq-1.  Thread
// (h = tid / 32, lane l = tid % 32) owns dims 4l .. 4l+3 of head h.  The new
// entry (index pos, written by the QKV tasks) joins as one more score.
__device__ __forceinline__ void task_attn_merge(const MoeParams& p, const Ctx& c, int t, int g) {
  (void)c;
  const int tid = threadIdx.x, h = tid >> 5, l = tid & 31;
  const int d = kDecHd, gq = p.nq / p.nkv;
  const float scale = 1.0f / sqrtf((float)d);
  const size_t at = ((((size_t)t * p.nkv + g) * p.Lcap + p.pos) * d + 4 * l) * 2;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};
  (void)zero4;
  // q_h . k_new over this thread's 4 dims, summed over the 32 threads of the head
  const rsrc_t rq = r_qb(p);
  const uint32_t qo = (uint32_t)((((size_t)t * p.nq + g * gq + (h < gq ? h : 0)) * d + 4 * l) * 2);
  const uint32_t q01 = co_ld32(rq, qo), q23 = co_ld32(rq, qo + 4);
  const uint32_t k01 = co_ld32(r_kc(p), (uint32_t)at), k23 = co_ld32(r_kc(p), (uint32_t)at + 4);
  const uint32_t v01 = co_ld32(r_vc(p), (uint32_t)at), v23 = co_ld32(r_vc(p), (uint32_t)at + 4);
  float s = bf_lo(q01) * bf_lo(k01) + bf_hi(q01) * bf_hi(k01) + bf_lo(q23) * bf_lo(k23) + bf_hi(q23) * bf_hi(k23);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) s += __shfl_xor(s, o);
  s *= scale;
  if (h >= gq) return;
  const rsrc_t rp = r_part(p);
  const uint32_t pb0 = (uint32_t)((((size_t)t * p.nkv + g) * p.nchunk_max) * p.part_floats * 4);
  const uint32_t pstep = (uint32_t)(p.part_floats * 4);
  float M = s, L = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  // eight chunks a batch, every load of the batch in flight together; the
  // running maximum rescales what is summed so far (online softmax merge)
  for (int c0 = 0; c0 < p.nchunk; c0 += 8) {
    float mc[8], lc[8];
    u32x4_t ov[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t pb = pb0 + (uint32_t)(c0 + u) * pstep;
      const bool ok = c0 + u < p.nchunk;
      mc[u] = ok ? co_ldf(rp, pb + (uint32_t)((gq * d + h) * 4)) : -__builtin_inff();
      lc[u] = ok ? co_ldf(rp, pb + (uint32_t)((gq * d + gq + h) * 4)) : 0.f;
      ov[u] = ok ? co_ld128(rp, pb + (uint32_t)((h * d + 4 * l) * 4)) : (u32x4_t){0u, 0u, 0u, 0u};
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < 8; ++u) Mn = fmaxf(Mn, mc[u]);
    const float r = __expf(M - Mn);
    L *= r;
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] *= r;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = c0 + u < p.nchunk ? __expf(mc[u] - Mn) : 0.f;
      L = __builtin_fmaf(lc[u], f, L);
      acc[0] = __builtin_fmaf(f, __uint_as_float(ov[u].x), acc[0]);
      acc[1] = __builtin_fmaf(f, __uint_as_float(ov[u].y), acc[1]);
      acc[2] = __builtin_fmaf(f, __uint_as_float(ov[u].z), acc[2]);
      acc[3] = __builtin_fmaf(f, __uint_as_float(ov[u].w), acc[3]);
    }
    M = Mn;
  }
  // the new entry's own score and value
  const float fs = __expf(s - M);
  L += fs;
  acc[0] = __builtin_fmaf(fs, bf_lo(v01), acc[0]);
  acc[1] = __builtin_fmaf(fs, bf_hi(v01), acc[1]);
  acc[2] = __builtin_fmaf(fs, bf_lo(v23), acc[2]);
  acc[3] = __builtin_fmaf(fs, bf_hi(v23), acc[3]);
  const float inv = 1.0f / L;
  const uint32_t lo = f2bf(acc[0] * inv) | (f2bf(acc[1] * inv) << 16);
  const uint32_t hi = f2bf(acc[2] * inv) | (f2bf(acc[3] * inv) << 16);
  const rsrc_t ro = r_ob(p);
  co_st32(ro, qo, lo);
  co_st32(ro, qo + 4, hi);
}

// O(ct, ks): columns ct*16 .. ct*16+15 of o Wo^T over the inner quarter ks.
__device__ __forceinline__ void task_oproj(const MoeParams& p, const Ctx& c, int ct, int ks, float* red) {
  const int K = p.nq * kDecHd, Kq = K / kDecOSplit;
  float* stage = red + 1024;
  tile16(r_ob(p), (uint32_t)K, p.wo, (uint32_t)K, c.T, ks * Kq, (ks + 1) * Kq, [&](int n) { return ct * 16 + n; }, red,
         stage);
  const int tid = threadIdx.x, row = tid >> 4, col = tid & 15;
  if (row < c.T)
    co_stf(r_apart(p), (uint32_t)((((size_t)ks * p.T_max + row) * c.H + ct * 16 + col) * 4), stage[row * 16 + col]);
}

// N2: x2 = bf16(x + bf16(a)), a the sum of the projection's quarters;
// h2 = bf16(x2 * r * g2), r = 1 / sqrt(mean(x2^2) + eps).  x2 goes to the
// residual buffer (the combine adds it), h2 to the MoE block's input.
__device__ __forceinline__ void norm2_chunk(const MoeParams& p, int t, int ch, float* x2) {
  const rsrc_t ra = r_apart(p);
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kDecOSplit; ++ks) {
    const uint32_t o = (uint32_t)((((size_t)ks * p.T_max + t) * p.H + ch * 8) * 4);
    const u32x4_t u0 = co_ld128(ra, o), u1 = co_ld128(ra, o + 16);
    a[0] += __uint_as_float(u0.x); a[1] += __uint_as_float(u0.y);
    a[2] += __uint_as_float(u0.z); a[3] += __uint_as_float(u0.w);
    a[4] += __uint_as_float(u1.x); a[5] += __uint_as_float(u1.y);
    a[6] += __uint_as_float(u1.z); a[7] += __uint_as_float(u1.w);
  }
  float f[8];
  unpack8(ld4(p.dx + (size_t)t * p.H + ch * 8), f);
#pragma unroll
  for (int q = 0; q < 8; ++q) x2[q] = bf_round(f[q] + bf_round(a[q]));
}
__device__ __forceinline__ void task_norm2(const MoeParams& p, const Ctx& c, int t) {
  __shared__ float s4[4];
  const int tid = threadIdx.x;
  const int H = c.H, nch = H >> 3;
  const rsrc_t rr = r_resid(p), rh = r_h2(p);
  auto put = [&](rsrc_t rs, int ch, const float* v) {
    u32x4_t o;
    o.x = f2bf(v[0]) | (f2bf(v[1]) << 16);
    o.y = f2bf(v[2]) | (f2bf(v[3]) << 16);
    o.z = f2bf(v[4]) | (f2bf(v[5]) << 16);
    o.w = f2bf(v[6]) | (f2bf(v[7]) << 16);
    co_st128(rs, (uint32_t)(((size_t)t * H + ch * 8) * 2), o);
  };
  float x2[kNormPer][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int ch = tid + j * kThreads;
    if (ch < nch) {
      norm2_chunk(p, t, ch, x2[j]);
#pragma unroll
      for (int q = 0; q < 8; ++q) ss = __builtin_fmaf(x2[j][q], x2[j][q], ss);
      put(rr, ch, x2[j]);
    }
  }
  for (int ch = tid + kNormPer * kThreads; ch < nch; ch += kThreads) {
    float v[8];
    norm2_chunk(p, t, ch, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) ss = __builtin_fmaf(v[q], v[q], ss);
    put(rr, ch, v);
  }
  ss = block_sum(ss, s4);
  const float r = 1.0f / sqrtf(ss / (float)H + p.eps);
  auto scaled = [&](int ch, const float* v) {
    float g[8], h[8];
    unpack8(ld4(p.g2 + ch * 8), g);
#pragma unroll
    for (int q = 0; q < 8; ++q) h[q] = v[q] * r * g[q];
    put(rh, ch, h);
  };
#pragma unroll
  for (int j = 0; j < kNormPer; ++j) {
    const int ch = tid + j * kThreads;
    if (ch < nch) scaled(ch, x2[j]);
  }
  for (int ch = tid + kNormPer * kThreads; ch < nch; ch += kThreads) {
    float v[8];
    norm2_chunk(p, t, ch, v);
    scaled(ch, v);
  }
}

// The attention block under the persistent schedules: every phase's tasks
// dealt round-robin over the workgroups (continuing from the previous
// phase), each task waiting on the previous phase's event and notifying its
// own.  A phase waits only on earlier phases, so with every workgroup
// resident no wait is circular.  Returns false when a wait gave up.
__device__ __forceinline__ bool run_decoder_front(const MoeParams& p, const Ctx& c, uint8_t* smem, int64_t& off) {
  const int G = gridDim.x, w = blockIdx.x;
  float* red = reinterpret_cast<float*>(smem);
  const DecCounts n = dec_counts(p, c);
  auto first = [&]() { return first_of(w, off, G); };
  // per-task trace (when asked for): before the wait, after it, after the
  // body; the record itself is written after the notify
  const bool tr = p.trace != nullptr;
  uint64_t tw = 0, ts = 0, tb = 0;
  auto t_wait = [&]() { if (tr) tw = now_ticks(); };
  auto t_start = [&]() { if (tr) ts = now_ticks(); };
  auto done = [&](uint32_t* ev, uint32_t target, int type, int i) {
    if (tr) tb = now_ticks();
    wg_publish();
    if (threadIdx.x == 0) notify1(c, ev, target);
    trace_task(p, type, i, 0, tw, ts, tb);
  };
  for (int i = first(); i < n.nN; i += G) {
    t_wait();
    t_start();
    task_norm1(p, c, i);
    done(c.set + W_DEC_N1, (uint32_t)n.nN, TT_DN1, i);
  }
  off += n.nN;
  for (int i = first(); i < n.nQKV; i += G) {
    t_wait();
    if (!wg_wait(c.set + W_DEC_N1, (uint32_t)n.nN, c.status, c.budget)) return false;
    t_start();
    task_qkv(p, c, i, red);
    done(c.set + W_DEC_QKV, (uint32_t)n.nQKV, TT_DQKV, i);
  }
  off += n.nQKV;
  for (int i = first(); i < n.nATT; i += G) {
    t_wait();
    const int t = i / (p.nkv * p.nchunk), g = (i / p.nchunk) % p.nkv, ch = i % p.nchunk;
    if (!wg_wait(c.set + W_DEC_QKV, (uint32_t)n.nQKV, c.status, c.budget)) return false;
    t_start();
    task_attn(p, c, t, g, ch, red);
    done(c.set + p.o_ev_att + (int64_t)(t * p.nkv + g) * kEvStride, (uint32_t)p.nchunk, TT_DATT, i);
  }
  off += n.nATT;
  for (int i = first(); i < n.nATTC; i += G) {
    t_wait();
    if (!wg_wait(c.set + W_DEC_QKV, (uint32_t)n.nQKV, c.status, c.budget)) return false;
    if (p.nchunk > 0 && !wg_wait(c.set + p.o_ev_att + (int64_t)i * kEvStride, (uint32_t)p.nchunk, c.status, c.budget))
      return false;
    t_start();
    task_attn_merge(p, c, i / p.nkv, i % p.nkv);
    done(c.set + W_DEC_ATTC, (uint32_t)n.nATTC, TT_DATTC, i);
  }
  off += n.nATTC;
  for (int i = first(); i < n.nO; i += G) {
    t_wait();
    if (!wg_wait(c.set + W_DEC_ATTC, (uint32_t)n.nATTC, c.status, c.budget)) return false;
    t_start();
    task_oproj(p, c, i / kDecOSplit, i % kDecOSplit, red);
    done(c.set + W_DEC_O, (uint32_t)n.nO, TT_DO, i);
  }
  off += n.nO;
  for (int i = first(); i < n.nN; i += G) {
    t_wait();
    if (!wg_wait(c.set + W_DEC_O, (uint32_t)n.nO, c.status, c.budget)) return false;
    t_start();
    task_norm2(p, c, i);
    done(c.set + W_DEC_N2, (uint32_t)n.nN, TT_DN2, i);
  }
  off += n.nN;
  return true;
}
