// internal.h -- host-side plan shared by the C-ABI and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kSortBlock = 256;  // tokens per sort workgroup
constexpr int kFrontMaxT = 16;   // largest T routed/sorted/quantised by one fused launch
constexpr int kMTile = 16;       // rows per MFMA m-tile
// Head of the sync region (zeroed by the routing launch of every call): [0]
// set when a fused-launch wait gave up (a guard; never expected), [1, 9) the
// tiled GEMM1's per-XCD item counters, [9, 17) GEMM2's; then the fused
// launch's GEMM1 completion count per m-tile.
constexpr int kQueueBase = 1;
constexpr int kSyncHead = kQueueBase + 16;
constexpr int kUnit = 32;        // h columns per GEMM1 work unit (one requant block)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Prepacked weight layout of one matrix of R rows and K columns (R % 64 == 0,
// K % 128 == 0), in quads of four 16-row tiles (tile t = 4*u + q): codes
// [R/64 quads u][K/128 steps][4 tiles q][64 lanes][16 B], scales [R/64][K/128
// steps][64 lanes][4 B].  Lane l = 16*g + c of tile t holds row 16*t + c,
// columns [128*step + 32*g, +32) (the gfx950 scaled-MFMA B operand of one
// 16x16x128 step), so one K step of a quad is 4 KiB contiguous and a quad's
// steps follow each other; byte q of lane l's scale dword is the E8M0 scale
// of that lane's block in tile q (the MFMA picks the byte with its scale
// op_sel, so one dword serves the four tiles a wave owns).
struct PackDims {
  int R, K, steps;
  size_t code_bytes_per_tile() const { return (size_t)steps * 1024; }
  size_t scale_bytes_per_quad() const { return (size_t)steps * 256; }
  size_t code_bytes() const { return (size_t)(R / 16) * code_bytes_per_tile(); }
  size_t scale_bytes() const { return (size_t)(R / 64) * scale_bytes_per_quad(); }
};
inline PackDims pack_dims(int R, int K) { return PackDims{R, K, K / 128}; }

struct WsLayout {
  size_t off[MOE_WS_NUM];
  size_t hist;    // [nb][E] int32 per-sort-block histograms, then bases within the expert
  size_t mtoff;   // [E+1] int32 prefix sum of m-blocks per expert
  size_t mbexp;   // [N/16 + E] int32 expert of each m-block
  size_t mbrows;  // [N/16 + E] int32 pairs: first sorted row and row count of each m-block
  size_t wsorted; // [N] fp32 routing weight of sorted row p (assignment perm[p])
  size_t sync;    // [kSyncHead + N/16 + E + 1] int32: item counters, fused-launch sync (zeroed per call)
  size_t total;
  int nb;
};

inline WsLayout ws_layout(int T, int top_k, int E, int H, int I, int act) {
  WsLayout L{};
  const size_t N = (size_t)T * top_k;
  const size_t a1row = act == MOE_ACT_MXFP8_E4M3 ? (size_t)H : (size_t)H / 2;
  const size_t a2row = act == MOE_ACT_MXFP8_E4M3 ? (size_t)I : (size_t)I / 2;
  L.nb = ceil_div(T, kSortBlock);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes, 256); return r; };
  L.off[MOE_WS_IDS] = take(N * 4);
  L.off[MOE_WS_WEIGHTS] = take(N * 4);
  L.off[MOE_WS_COUNTS] = take((size_t)E * 4);
  L.off[MOE_WS_OFFSETS] = take((size_t)(E + 1) * 4);
  L.mtoff = take((size_t)(E + 1) * 4);
  L.mbexp = take((N / kMTile + E + 1) * 4);
  L.mbrows = take((N / kMTile + E + 1) * 8);
  L.hist = take((size_t)L.nb * E * 4);
  L.wsorted = take(N * 4);
  L.sync = take((kSyncHead + N / kMTile + E + 1) * 4);
  L.off[MOE_WS_PERM] = take(N * 4);
  L.off[MOE_WS_A1_CODES] = take((size_t)T * a1row);
  L.off[MOE_WS_A1_SCALES] = take((size_t)T * (H / 32));
  L.off[MOE_WS_A2_CODES] = take(N * a2row);
  L.off[MOE_WS_A2_SCALES] = take(N * (size_t)(I / 32));
  L.off[MOE_WS_ROWS] = take(N * (size_t)H * 4);
  L.off[MOE_WS_SLOT] = take(N * 4);
  L.total = o;
  return L;
}

// Sort-only workspace (moe_sort): histograms, m-block prefix and table,
// inverse permutation.
struct SortWs {
  size_t mtoff, hist, mbexp, inv, total;
};
inline SortWs sort_ws_layout(int T, int E, int top_k) {
  SortWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o = align_up(o + bytes, 256); return r; };
  const size_t N = (size_t)T * top_k;
  w.mtoff = take((size_t)(E + 1) * 4);
  w.hist = take((size_t)ceil_div(T, kSortBlock) * E * 4);
  w.mbexp = take((N / kMTile + E + 1) * 4);
  w.inv = take(N * 4);
  w.total = o;
  return w;
}

// ---- launchers (kernels.hip) -----------------------------------------------
hipError_t launch_route(const float *logits, int T, int E, int top_k, int32_t *ids, float *w,
                        hipStream_t s);
hipError_t launch_sort_hist(const int32_t *ids, int T, int E, int top_k, int32_t *hist, int nb,
                            hipStream_t s);
// mbrows may be null (no m-block row table)
hipError_t launch_sort_scan(int32_t *hist, int nb, int E, int32_t *counts, int32_t *offsets,
                            int32_t *mtoff, int32_t *mbexp, int32_t *mbrows, int bm,
                            int32_t *sync, int nsync, hipStream_t s);
hipError_t launch_sort_scatter(const int32_t *ids, int T, int E, int top_k, const int32_t *hist,
                               const int32_t *offsets, int32_t *perm, int32_t *inv,
                               const float *w, float *wsorted, hipStream_t s);
// Fused route + sort + quant for T <= kSortBlock (same outputs as the
// separate kernels; hist is not used).
struct FrontArgs {
  int32_t *sync;  // [nsync] zeroed (the fused GEMM launch's counters), or nsync 0
  int nsync;
  const float *logits;
  const uint16_t *x;  // null: no quantisation (the caller's codes feed GEMM1)
  int T, E, top_k, H, act, bm;
  int32_t *ids;
  float *wts;
  int32_t *counts, *offsets, *mtoff, *mbexp, *mbrows, *perm, *inv;
  float *wsorted;
  uint8_t *codes, *scales;
};
hipError_t launch_front(const FrontArgs &a, hipStream_t s);
hipError_t launch_quant(const uint16_t *x, long rows, int K, int act, uint8_t *codes,
                        uint8_t *scales, hipStream_t s);
hipError_t launch_prepack(const uint8_t *codes, const uint8_t *scales, int E, int R, int K,
                          bool interleave_gate_up, uint8_t *pcodes, uint8_t *pscales,
                          hipStream_t s);
// GEMM variant of one forward call (chosen on the host from the token count).
//   stream: 16-row m-tiles, the four waves of a workgroup split K, weights
//           go straight from HBM to VGPRs (decode: few rows per expert)
//   tiled:  bm = 16*MT rows per work item staged in LDS and shared by the
//           waves, two MFMA waves per 64 weight rows (prefill)
// Form of the tiled kernels (the only one built): MFMA waves that copy only
// their own weights, producer waves that copy the activations.
constexpr int kTiledSplit = 2;

struct GemmPlan {
  bool tiled;
  int mt;   // 16-row MFMA tiles per work item (1 for stream)
  int split;  // tiled kernel form (kTiledSplit)
  bool fused = false;  // stream only: GEMM1 and GEMM2 items in one persistent launch
  bool tm = false;     // stream only: token-major GEMM2 with the top-k combine folded in
  int bm() const { return 16 * mt; }
};
GemmPlan choose_plan(int T, int top_k, int E, int act);
// tiled m-tiles per item built (both activation formats)
inline bool tiled_mt_built(int act, int mt) {
  (void)act;
  return mt == 2 || mt == 4 || mt == 6 || mt == 8 || mt == 10 || mt == 12;
}

struct GemmArgs {
  int T, top_k, E, H, I, act;
  GemmPlan plan;
  long max_mtiles;  // host upper bound of m-blocks (ceil(N/bm) + min(N, E))
  int num_cus;
  const uint8_t *a1c, *a1s;
  uint8_t *a2c, *a2s;
  const int32_t *perm, *offsets, *mtoff, *mbexp;
  const int32_t *mbrows;  // [m-block][2]: first sorted row, rows (stream and fused plans)
  const float *wts;  // [N] routing weight of sorted row p
  const uint8_t *w13p, *w13sp, *w2p, *w2sp;
  float *rows;  // [N][H] weighted GEMM2 rows (layout by combine)
  int combine;  // moe_combine transport of the rows
  int32_t *sync;  // fused launch: work counter, wait flag, per-m-tile counts (zeroed)
  // token-major GEMM2 (plan.tm): routing by assignment and the output
  const int32_t *ids, *inv;  // [N] expert and sorted row of assignment a
  const float *wts_a;        // [N] routing weight of assignment a
  uint16_t *y;               // [T][H] bf16 output
};
// Whether launch_gemm2 writes y itself (token-major GEMM2 with the combine
// folded in; the FP32 transport only), so that no combine launch follows.
inline bool gemm2_writes_y(const GemmArgs &a) { return a.plan.tm && a.combine == MOE_COMBINE_FP32; }
hipError_t launch_gemm1(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemm2(const GemmArgs &a, hipStream_t s);
hipError_t launch_combine(const void *rows, const int32_t *inv, int T, int H, int top_k,
                          int combine, uint16_t *y, hipStream_t s);

// Device address, on the current device, of the library's static forward
// workspace of MOE_NOALLOC_SCRATCH_BYTES (noalloc.hip); looked up once per
// device.
hipError_t noalloc_scratch(void **ptr);

}  // namespace moe
