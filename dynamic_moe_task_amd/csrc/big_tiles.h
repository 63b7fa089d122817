// Big-tile grouped-GEMM task bodies (the big-tile kernel variant, for the
// largest batches).  Included by moe_kernels.hip, inside its namespace,
// after the other G bodies, whose helpers (bf16 conversion, coherent
// accesses, RowTile, Ctx) it uses.
//
// A task multiplies one row tile of up to 256 grouped rows of expert e by
// 256 weight rows (G1: 128 gate and the 128 matching up rows of W13[e];
// G2: 256 rows of Wd[e]) over the whole inner dimension K (G1: H, G2: I):
//
//   G1(rt, nt)  Hmid[rows, 128 nt .. +127] = bf16(silu(g) * u),
//               g = Xg Wg^T, u = Xg Wu^T, Xg the tile's token rows of x
//   G2(rt, nt)  Y[rows, 256 nt .. +255] = bf16(Hmid[rows] Wd^T)
//
// The workgroup is four waves in a 2 x 2 arrangement, each owning 128 rows
// x 128 weight rows of the output as 4 x 4 blocks of 32 x 32 (bf16 MFMA
// 32x32x16, fp32 accumulation in the accumulation registers).  K is staged
// 64 at a time in LDS, two stages, each 256 A rows then 256 B rows of 128
// bytes whose 16-byte chunks are XOR-swizzled by row, so that the 32 rows of
// an MFMA operand read fall in distinct banks.  The stages are filled by
// direct-to-LDS loads (no register round trip): a wave's load instruction
// writes 1 KB of LDS, eight rows, and each lane fetches the chunk that the
// swizzle puts at its position.  Stage kc + 2 is requested as soon as stage
// kc has been read, and the operand registers of the next k16 step are read
// while the current step's MFMAs run.  Weight rows and A rows are read once
// per task.  Rows past the tile's count are neither read from LDS nor
// multiplied (the K loop is specialised on each wave's count of live 32-row
// blocks) nor stored; their loads repeat row 0.
#pragma once
// (included inside namespace etc)

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kBigBK = 64;                 // k per LDS stage
constexpr int kBigRowB = kBigBK * 2;       // bytes per staged row
constexpr int kBigStage = 512 * kBigRowB;  // 256 A rows + 256 B rows
constexpr int kBigLoads = 16;              // direct-to-LDS loads per wave per stage
static_assert(2 * kBigStage == kBigLdsBytes, "two stages fill the big variant's LDS");

__device__ __forceinline__ int big_sw(int row, int chunk) { return (chunk ^ ((row >> 1) & 7)) << 4; }
template <int N>
struct IntC {
  static constexpr int value = N;
};

template <bool G1>
__device__ __forceinline__ void big_body(const MoeParams& p, const Ctx& c, const RowTile tile, int nt, uint8_t* lds) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so its tests are scalar branches
  const int l32 = lane & 31, kh = lane >> 5;
  const int wr = wv >> 1, wc = wv & 1;
  const int H = c.H, I = c.I, K = G1 ? H : I;
  const int nrows = tile.nrows;
  // every wave is done with the LDS of the previous task (its output stage)
  __syncthreads();
  // This lane's source of each load of a stage: load j of wave w writes LDS
  // rows 8 (16 w + j) .. + 7; waves 0 and 1 fetch the 256 A rows, waves 2
  // and 3 the 256 weight rows.  A wave's sources share one base (x, Hmid, or
  // the expert's weights); each lane keeps 32-bit byte offsets from it (all
  // below 2 GiB, as the descriptor limits require).  Rows past the count
  // read row 0 (any valid row).
  const bool wave_a = wv < 2;
  const uint16_t* base_a = G1 ? p.x : p.hh;
  const uint16_t* base_b = G1 ? p.w13 + (size_t)tile.e * 2 * I * H : p.w2 + (size_t)tile.e * H * I;
  const uint16_t* gbase = wave_a ? base_a : base_b;
  uint32_t off[kBigLoads];
  const rsrc_t rp = r_perm(p);
#pragma unroll
  for (int j = 0; j < kBigLoads; ++j) {
    const int row = (wv * kBigLoads + j) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    uint32_t elem;
    if (wave_a) {
      const int r = row < nrows ? row : 0;
      if (G1) {
        const int t = (int)co_ld32(rp, (uint32_t)(tile.r0 + r) * 4u) / c.k;
        elem = (uint32_t)t * (uint32_t)H;
      } else {
        elem = (uint32_t)(tile.r0 + r) * (uint32_t)I;
      }
    } else {
      const int br = row - 256;
      const int wrow = G1 ? (br < 128 ? nt * 128 + br : I + nt * 128 + (br - 128)) : nt * 256 + br;
      elem = (uint32_t)wrow * (uint32_t)K;
    }
    off[j] = (elem + (uint32_t)chunk * 8u) * 2u;
  }
  const int nk = K / kBigBK;
  // Every wave issues all its loads (rows past the count repeat row 0), so
  // that the loop holds no branch: a branch around loads or MFMAs ends the
  // compiler's overlap of the LDS reads with the MFMAs.
  auto issue = [&](int kc) {
    uint8_t* base = lds + (kc & 1) * kBigStage + wv * kBigLoads * 1024;
    const uint8_t* g = reinterpret_cast<const uint8_t*>(gbase) + (size_t)kc * (kBigBK * 2);
    if (!G1 && wave_a) {
      // Hmid rows (G2's A) are written during the launch: device-coherent
      // loads; x and the weights are not
#pragma unroll
      for (int j = 0; j < kBigLoads; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(g + off[j]), (lds_ptr_t)(base + j * 1024), 16, 0, kCoherent);
    } else {
#pragma unroll
      for (int j = 0; j < kBigLoads; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(g + off[j]), (lds_ptr_t)(base + j * 1024), 16, 0, 0);
    }
  };
  // operand rows in the stage: A blocks of this wave's 128 rows; B blocks of
  // its 128 weight rows (G1: 64 gate rows, then the 64 matching up rows)
  int arow[4], brow[4];
  bool live[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    arow[b] = 128 * wr + 32 * b + l32;
    live[b] = 128 * wr + 32 * b < nrows;  // uniform per wave
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = G1 ? (n < 2 ? wc * 64 + 32 * n : 128 + wc * 64 + 32 * (n - 2)) : wc * 128 + 32 * n;
    brow[n] = 256 + r + l32;
  }
  f32x16_t acc[4][4];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[b][n][q] = 0.f;
  // The K loop, specialised on the wave's live 32-row blocks (NL: 4 to 0),
  // so that no per-block test sits in it; dead blocks are neither read nor
  // multiplied.
  auto kloop = [&](auto nl_tag) {
    constexpr int NL = decltype(nl_tag)::value;
    u32x4_t fa[2][4], fb[2][4];
    auto read = [&](int kc, int s, u32x4_t (&a)[4], u32x4_t (&b4)[4]) {
      const uint8_t* base = lds + (kc & 1) * kBigStage;
#pragma unroll
      for (int b = 0; b < NL; ++b)
        a[b] = *reinterpret_cast<const u32x4_t*>(base + arow[b] * kBigRowB + big_sw(arow[b], 2 * s + kh));
#pragma unroll
      for (int n = 0; n < 4; ++n)
        b4[n] = *reinterpret_cast<const u32x4_t*>(base + brow[n] * kBigRowB + big_sw(brow[n], 2 * s + kh));
    };
    auto mma = [&](const u32x4_t (&a)[4], const u32x4_t (&b4)[4]) {
#pragma unroll
      for (int b = 0; b < NL; ++b)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[b][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf(a[b]), as_bf(b4[n]), acc[b][n], 0, 0, 0);
    };
    issue(0);
    if (nk > 1) issue(1);
    __builtin_amdgcn_s_waitcnt(0);  // stage 0 (and 1) landed, as have the row lookups
    __syncthreads();
    if (NL > 0) read(0, 0, fa[0], fb[0]);
    for (int kc = 0; kc < nk; ++kc) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 3) {
          if (NL > 0) read(kc, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
        } else if (kc + 1 < nk) {
          // stage kc + 1 is the only one in flight: wait for it, then every
          // wave has read stage kc (the barrier waits for LDS reads), so its
          // buffer takes stage kc + 2
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
          __syncthreads();
          if (kc + 2 < nk) issue(kc + 2);
          if (NL > 0) read(kc + 1, 0, fa[0], fb[0]);
        }
        if (NL > 0) mma(fa[s & 1], fb[s & 1]);
      }
    }
  };
  const int nlive = min(4, max(0, (nrows - 128 * wr + 31) / 32));  // uniform per wave
  switch (nlive) {
    case 4: kloop(IntC<4>{}); break;
    case 3: kloop(IntC<3>{}); break;
    case 2: kloop(IntC<2>{}); break;
    case 1: kloop(IntC<1>{}); break;
    default: kloop(IntC<0>{}); break;
  }
  __syncthreads();  // the stages are free for the output
  // output through LDS, one half of the rows (the waves of one row) at a
  // time, then 16-byte device-coherent stores of the rows below the count
  uint16_t* st = reinterpret_cast<uint16_t*>(lds);
  constexpr int OC = G1 ? kBigBN1 : kBigBN2;  // output columns
  constexpr int SW = OC + 8;                  // staged row (elements), padded
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wr == half) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (!live[b]) continue;
        if (G1) {
#pragma unroll
          for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float g = acc[b][n][v], u = acc[b][n + 2][v];
              const int row = 32 * b + 8 * (v >> 2) + 4 * kh + (v & 3), col = wc * 64 + 32 * n + l32;
              st[row * SW + col] = (uint16_t)f2bf_int(g / (1.0f + __expf(-g)) * u);
            }
        } else {
#pragma unroll
          for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int row = 32 * b + 8 * (v >> 2) + 4 * kh + (v & 3), col = wc * 128 + 32 * n + l32;
              st[row * SW + col] = (uint16_t)f2bf_int(acc[b][n][v]);
            }
        }
      }
    }
    __syncthreads();
    constexpr int CPR = OC / 8;  // 16-byte chunks per row
    const int hrows = min(128, nrows - 128 * half);
    for (int idx = tid; idx < hrows * CPR; idx += kThreads) {
      const int r = idx / CPR, q = idx % CPR;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(st + r * SW + q * 8);
      const size_t grow = (size_t)tile.r0 + 128 * half + r;
      if (G1)
        co_st128(r_hh(p), (uint32_t)((grow * I + nt * OC + q * 8) * 2), v);
      else
        co_st128(r_y(p), (uint32_t)((grow * H + nt * OC + q * 8) * 2), v);
    }
    __syncthreads();  // the stage is read before the next half overwrites it
  }
  // every wave's stores have completed before the caller's notify
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}
