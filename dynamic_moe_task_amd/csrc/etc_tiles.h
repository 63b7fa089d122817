// Task geometry of the MoE layer graph: tile shapes and the rules that
// pick them from the batch size T.  Plain constants and inline functions, so
// that the kernels, the host library and a host-only test harness (g++) all
// read the same rules; a file compiled by hipcc defines ETC_HD as
// __host__ __device__ before including it.
#pragma once

#ifndef ETC_HD
#define ETC_HD inline
#endif

namespace etc {

constexpr int kThreads = 256;      // 4 wave64 per workgroup
// R task: kRouterT tokens x router_experts(T) experts.  One expert a wave up
// to T = kRouterLargeT; four a wave above it (fewer, longer tasks); eight a
// wave from T = kRouterXLT on, where even those fill the grid several times
// over (that tile exists only in the large-batch kernel variant).
constexpr int kRouterT = 4;
constexpr int kRouterE = 4;
constexpr int kRouterLargeT = 64;
constexpr int kRouterEL = 16;
constexpr int kRouterEXL = 32;
constexpr int kRouterXLT = 2048;
ETC_HD int router_experts(int T) {
  return T >= kRouterXLT ? kRouterEXL : (T > kRouterLargeT ? kRouterEL : kRouterE);
}
constexpr int kBM = 64;         // grouped-GEMM row tile (up to four 16-row MFMA blocks)
constexpr int kBN1 = 16;        // G1: gate columns (and as many up columns) per tile ...
constexpr int kMidG1Rows = 512;    // ... twice that from T * k routed rows on ...
constexpr int kWideG1Rows = 2048;  // ... and four times that from these on
// (column-split tiles; H a multiple of 128, as the ABI requires)
ETC_HD int g1_cols(int T, int k, int H) {
  return (T * k >= kWideG1Rows && H % 128 == 0) ? 4 * kBN1 : (T * k >= kMidG1Rows ? 2 * kBN1 : kBN1);
}
constexpr int kBN2 = 64;        // G2: output columns per tile
constexpr int kCB2 = kBN2 / 16;  // G2: 16-column MFMA blocks per tile
// G2 output columns per tile: twice kBN2 (column-split tiles) from the same
// batch on when I is a multiple of 128
ETC_HD int g2_cols(int T, int k, int I) {
  return (T * k >= kWideG1Rows && I % 128 == 0) ? 2 * kBN2 : kBN2;
}
constexpr int kCombineT = 2;    // C task: tokens per task
// Large batches run the big-tile kernel variant: row tiles of up to
// kBigBM grouped rows, G1 tiles of kBigBN1 gate and as many up columns, G2
// tiles of kBigBN2 output columns, K staged 64 at a time.  Each weight
// element streamed from memory then feeds up to 256 rows (the row tiles of
// the other variants hold at most 64), which is what lets the grouped GEMM
// approach the matrix cores' rate once experts hold hundreds of rows.
constexpr int kBigBM = 256;
constexpr int kBigBN1 = 128;
constexpr int kBigBN2 = 256;
constexpr int kBigRows = 8192;  // T * k from which the big tiles run
ETC_HD bool big_variant(int T, int k, int H, int I) {
  return T * k >= kBigRows && H % kBigBN2 == 0 && I % kBigBN1 == 0;
}
// kernel variants: small batches, large batches (column-split tiles), big tiles
enum : int { kVarSmall = 0, kVarWide = 1, kVarBig = 2 };

// Order of the big-tile variant's G tasks.  Task i of the R x C tiles of G1
// (or of G2) is taken by workgroup group i % 8
// (the grid deals consecutive workgroups, and claims, over the 8 XCDs, each
// with its own L2).  Two steps make the tiles an XCD runs at once share
// operands in its L2:
//  - dealing in chunks: the k-th task of group g is the (k % W)-th of chunk
//    (k / W) * 8 + g, so an XCD's W concurrent tasks (W = its workgroups)
//    are W consecutive entries of the order below (positions past the last
//    full round of 8 chunks keep their own index);
//  - grouped order: tiles come in groups of kBigGR row tiles, column-major
//    within a group, so consecutive entries share a weight slice across
//    kBigGR row tiles (an expert's tiles are numbered consecutively) and W
//    consecutive entries span W / kBigGR column tiles (their A rows).
// A bijection of [0, R * C) onto the tiles.
constexpr int kBigGR = 4;   // row tiles per group
constexpr int kBigW = 32;   // tasks an XCD runs at once, one workgroup a CU
struct TileRC {
  int rt, nt;
};
ETC_HD TileRC grouped_task(int i, int R, int C, int W) {
  const int n = R * C;
  const int full = (n / (8 * W)) * (8 * W);
  int t = i;
  if (i < full) {
    const int k = i >> 3, g = i & 7;
    t = ((k / W) * 8 + g) * W + k % W;
  }
  const int grp = t / (kBigGR * C), w = t % (kBigGR * C);
  const int gsz = R - grp * kBigGR < kBigGR ? R - grp * kBigGR : kBigGR;
  TileRC r;
  r.rt = grp * kBigGR + w % gsz;
  r.nt = w / gsz;
  return r;
}
ETC_HD TileRC big_task(int i, int R, int C) { return grouped_task(i, R, C, kBigW); }

}  // namespace etc
