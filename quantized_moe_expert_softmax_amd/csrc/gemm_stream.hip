// gemm_stream.hip -- stream (decode) variant of the expert GEMMs, the per-call
// choice between it and the tiled variant, and the GEMM launchers.
// Conventions and operand layouts: gemm_common.h.
#include "gemm_common.h"

namespace moe {

// A operand for lane group g from a row's codes of one K step (128 E4M3
// bytes or 64 packed E2M1 bytes at `step`).
template <int FMT>
__device__ __forceinline__ v8i load_a(const uint8_t *__restrict__ step, int g) {
  v8i a;
  if (FMT == 0) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(step + 16 * g);
    const uint4 hi = *reinterpret_cast<const uint4 *>(step + 64 + 16 * g);
    a[0] = (int)lo.x; a[1] = (int)lo.y; a[2] = (int)lo.z; a[3] = (int)lo.w;
    a[4] = (int)hi.x; a[5] = (int)hi.y; a[6] = (int)hi.z; a[7] = (int)hi.w;
  } else {
    const uint4 lo = *reinterpret_cast<const uint4 *>(step + 16 * g);
    a[0] = (int)lo.x; a[1] = (int)lo.y; a[2] = (int)lo.z; a[3] = (int)lo.w;
    a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
  }
  return a;
}

// acc[q] += A(rows of this lane's m-tile) x B(prepacked tile q of one quad)
// over K steps [s, s + G): every load of the G steps (A operand, its scale
// byte, the weight scale dword, four weight fragments per step) is issued
// before the first MFMA, so a wave keeps 7G loads in flight.  (With a
// conditional per step the compiler issued each step's weight fragments one
// or two at a time behind the previous MFMA, and how many it overlapped
// changed with unrelated edits: the K-step-major A2 layout moved GEMM2 at
// T = 64 from two to one and cost 17%.)  arow / asrow: the lane's row's
// codes and scale dword of K step 0; K step s is cstep / sstep bytes further
// (a row-major A1 row: the step's code bytes and 4; A2: N times those).
template <int FMT, int G>
__device__ __forceinline__ void mma_group(v4f acc[4], const uint8_t *__restrict__ arow,
                                          const uint8_t *__restrict__ asrow, size_t cstep,
                                          size_t sstep, const uint8_t *__restrict__ wt,
                                          const uint32_t *__restrict__ wsq, int s, int lane) {
  const int g = lane >> 4;
  v8i a[G];
  int sa[G], sb[G];
  u32x4 b[G][4];
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const size_t st = (size_t)(s + u);
    a[u] = load_a<FMT>(arow + cstep * st, g);
    sa[u] = asrow[sstep * st + g];
    sb[u] = load_weight_scales(wsq + st * 64 + lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) b[u][q] = load_weights16(wt + st * 4096 + q * 1024 + lane * 16);
  }
  // keep the scheduler from sinking loads between the MFMAs
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < G; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v8i bq;
      bq[0] = (int)b[u][q][0]; bq[1] = (int)b[u][q][1]; bq[2] = (int)b[u][q][2]; bq[3] = (int)b[u][q][3];
      bq[4] = 0; bq[5] = 0; bq[6] = 0; bq[7] = 0;
      acc[q] = mfma_q<FMT>(q, a[u], bq, acc[q], sa[u], sb[u]);
    }
}

// The K steps [s0, s1) in groups of G, then one group of the remaining
// 1 .. G - 1 steps (G is 1, 2 or 4).
template <int FMT, int G>
__device__ __forceinline__ void mma_4tiles(v4f acc[4], const uint8_t *__restrict__ arow,
                                           const uint8_t *__restrict__ asrow, size_t cstep,
                                           size_t sstep, const uint8_t *__restrict__ wt,
                                           const uint32_t *__restrict__ wsq, int s0, int s1,
                                           int lane) {
  static_assert(G == 1 || G == 2 || G == 4, "group size");
  int s = s0;
  for (; s + G <= s1; s += G) mma_group<FMT, G>(acc, arow, asrow, cstep, sstep, wt, wsq, s, lane);
  const int r = s1 - s;
  if (G == 4 && r == 3) mma_group<FMT, 3>(acc, arow, asrow, cstep, sstep, wt, wsq, s, lane);
  if (G == 4 && r == 2) mma_group<FMT, 2>(acc, arow, asrow, cstep, sstep, wt, wsq, s, lane);
  if (G > 1 && r == 1) mma_group<FMT, 1>(acc, arow, asrow, cstep, sstep, wt, wsq, s, lane);
}

// Steps per load group (mma_group) of the stream GEMMs.  Per call on the
// decode sizes against the per-step loop with a conditional (eager us, one
// box, two rounds): 5120 x 640 E = 384 T = 64 250 -> 229, E = 128 T = 8
// 42.5 -> 38.0 and T = 64 114 -> 103, 5120 x 1152 T = 32 259 -> 240, 7168 x
// 3072 T = 8 267 -> 257 and T = 64 equal.  Larger groups (GEMM1 2, GEMM2 4)
// lowered occupancy for less: a GEMM1 of four-step groups held one 8-wave
// workgroup per CU and was 17% slower on the 5120 x 640 shard at T = 64.
constexpr int kStreamGroup1 = 1, kStreamGroup2 = 2;

template <int FMT, int NW>
__global__ __launch_bounds__(64 * NW) void gemm1_kernel(KArgs p) {
  using F = typename ActFmt<FMT>::F;
  __shared__ float red[NW][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NU = p.I / 32;
  const int n_mt = uniform(p.mtoff[p.E]);
  const long total = (long)n_mt * NU;
  const int S = p.H / 128;
  const int s0 = wave * S / NW, s1 = (wave + 1) * S / NW;
  const size_t a1row = FMT == 0 ? (size_t)p.H : (size_t)p.H / 2;
  const size_t N = (size_t)p.T * p.top_k;
  const size_t nquads = (size_t)(2 * p.I) / 64;
  // items m-tile major: consecutive workgroups stream consecutive quads of one
  // expert's weights (measured 2-3% faster at T = 8..64 than unit-major,
  // where they read the same quad of different experts)
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    const int mt = (int)(w / NU), j = (int)(w % NU);
    const int e = uniform(p.mbexp[mt]);
    const int2 mr = p.mbrows[mt];  // loaded beside e, not after it
    const int row0 = uniform(mr.x), nrows = uniform(mr.y);
    const int pr = row0 + min(lane & 15, nrows - 1);
    const int tok = p.perm[pr] / p.top_k;
    const uint8_t *arow = p.a1c + (size_t)tok * a1row;
    const uint8_t *asrow = p.a1s + (size_t)tok * (p.H / 32);
    const uint8_t *wt = p.wp + ((size_t)e * nquads + j) * (size_t)S * 4096;
    const uint32_t *wsq = p.wsp + ((size_t)e * nquads + j) * (size_t)S * 64;
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    mma_4tiles<FMT, kStreamGroup1>(acc, arow, asrow, FMT == 0 ? 128 : 64, 4, wt, wsq, s0, s1,
                                   lane);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][4 * q + r][lane] = acc[q][r];
    __syncthreads();
    if (wave == 0) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        v[i] = red[0][i][lane];
#pragma unroll
        for (int u = 1; u < NW; ++u) v[i] += red[u][i][lane];
      }
      const int c = lane & 15;
      // tiles: 0 = gate cols [32j, +16), 1 = gate [32j+16, +16), 2/3 = up
      float g0[4], g1[4], u0[4], u1[4];
      size_t prow[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (lane >> 4) + r;
        prow[r] = (size_t)(row0 + min(m, nrows - 1));
        g0[r] = v[0 * 4 + r]; g1[r] = v[1 * 4 + r]; u0[r] = v[2 * 4 + r]; u1[r] = v[3 * 4 + r];
      }
      swiglu_requant_n<F, FMT, 4>(g0, g1, u0, u1, p.a2c, p.a2s, prow, N, j, c);
    }
    __syncthreads();
  }
}

template <int FMT, int NW>
__global__ __launch_bounds__(64 * NW) void gemm2_kernel(KArgs p) {
  __shared__ float red[NW][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NB = p.H / 64;
  const int n_mt = uniform(p.mtoff[p.E]);
  const long total = (long)n_mt * NB;
  const int S = p.I / 128;
  const int s0 = wave * S / NW, s1 = (wave + 1) * S / NW;
  const size_t N = (size_t)p.T * p.top_k;
  const size_t nquads = (size_t)p.H / 64;
  for (long w = blockIdx.x; w < total; w += gridDim.x) {  // m-tile major, as in GEMM1
    const int mt = (int)(w / NB), nb = (int)(w % NB);
    const int e = uniform(p.mbexp[mt]);
    const int2 mr = p.mbrows[mt];  // loaded beside e, not after it
    const int row0 = uniform(mr.x), nrows = uniform(mr.y);
    const size_t pr = (size_t)(row0 + min(lane & 15, nrows - 1));
    const uint8_t *arow = p.a2c + a2c_at<FMT>(pr, 0, N);
    const uint8_t *asrow = p.a2s + a2s_at(pr, 0, N);
    const uint8_t *wt = p.wp + ((size_t)e * nquads + nb) * (size_t)S * 4096;
    const uint32_t *wsq = p.wsp + ((size_t)e * nquads + nb) * (size_t)S * 64;
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    mma_4tiles<FMT, kStreamGroup2>(acc, arow, asrow, a2c_at<FMT>(0, 1, N), a2s_at(0, 1, N), wt,
                                   wsq, s0, s1, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][4 * q + r][lane] = acc[q][r];
    __syncthreads();
    if (wave == 0) {
      const int c = lane & 15;
      size_t prow[4];
      float t[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // a padded row recomputes the last valid row and stores the same values
        const int m = min(4 * (lane >> 4) + r, nrows - 1);
        const float wt_a = p.wts[row0 + m];
        prow[r] = (size_t)(row0 + m);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 4 * q + r;
          float o = red[0][i][lane];
#pragma unroll
          for (int u = 1; u < NW; ++u) o += red[u][i][lane];
          t[r][q] = wt_a * o;
        }
      }
      stage_store_n<4>(p, prow, 64 * nb, c, t);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Token-major GEMM2 with the top-k combine folded in (decode batches, plan
// MOE_PLAN_DECODE; "feat(moe): FlyDSL MegaMoE fused EP-MoE integration",
// summary: one fused operation in place of the separate GEMM2 and combine).
// A work item is (token t, 16 TPI output columns).  The pairs (slot j, K step) of
// the token's top_k slots, top_k * I/128 of them, are split into contiguous
// ranges over the NW waves; a wave loads the weight fragments and A2 operands
// of four pairs at a time (they may span two slots) and accumulates per slot
// (all 16 rows of the MFMA tile carry the token's A2 row; row 0 is kept).  The
// token's per-slot expert, sorted row and routing weight are loaded once per
// item into lanes 0 .. top_k - 1 and read with readlane, so the operand loads
// of a group never wait on another load (loaded per pair, they cost 21.2 ->
// 18.4 us per GEMM2 at T = 1 and 33.4 -> 30.4 at T = 2 on the 7168 x 3072
// layer).  The per-(wave, slot) partial sums meet in LDS; wave j < top_k adds
// slot j's, scales them by its routing weight and stores the row to the
// assignment's staging row (the layout the combine kernel reads); wave 0 then
// writes y[t] = bf16 of the FP32 sum of the weighted rows in slot order: the
// combine kernel's result, without its launch or its reads of the staging.
// With eight waves per item it measured on the 7168 x 3072, 384 x 6 layer
// (us per call, eager, one box) T = 1: 58.5 against 55.0 for the stream plan
// (224 items for 256 CUs read six experts each: fewer, longer items than the
// stream GEMM2's 672); T = 2: 94.7 against 99.6; T = 3 .. 8: 3-5% slower
// (experts two tokens share are read twice).  With sixteen waves when there
// is at most one item per CU (one token) it is faster at T = 1 too, and the
// built-in choice for T <= 2 (choose_plan); 16-column items measured 5-20%
// slower than 32-column ones.
// ---------------------------------------------------------------------------
// Operands of four (slot, K step) pairs of one token's token-major GEMM2 item.
template <int TPI>
struct TmGroup {
  v8i a[4];
  u32x4 b[4][TPI];
  int sa[4], sb[4];
};

template <int FMT, int NW, int TPI>
__global__ __launch_bounds__(64 * NW) void gemm2_tm_kernel(KArgs p) {
  __shared__ float part[NW][8][TPI][16];  // [wave][slot][tile][column]: row 0 of each tile
  __shared__ float wrow[8][TPI][16];      // [slot][tile][column]: weighted rows
  static_assert(NW >= 8, "one wave per slot in the epilogue (top_k <= 8)");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4;
  const int NB = p.H / (16 * TPI), k = p.top_k, S = p.I / 128, P = k * S;
  const int i0 = wave * P / NW, i1 = (wave + 1) * P / NW;
  const size_t N = (size_t)p.T * k;
  const size_t ntiles = (size_t)p.H / 16;
  const long total = (long)p.T * NB;
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    const int t = (int)(w / NB), nb = (int)(w % NB);
    // the first tile of the item: tile u of quad qd is tile 4 qd + u
    const size_t tile0 = (size_t)nb * TPI;
    // lane j < top_k holds slot j's expert, sorted row and routing weight:
    // one load each per item, so no load below waits on another
    int slot_e = 0, slot_r = 0, slot_w = 0;
    if (lane < k) {
      slot_e = p.ids[t * k + lane];
      slot_r = p.inv[t * k + lane];
      slot_w = __builtin_bit_cast(int, p.wts_a[t * k + lane]);
    }
    // slots this wave's range does not reach keep zero partial sums
    for (int x = lane; x < 8 * TPI * 16; x += 64) (&part[wave][0][0][0])[x] = 0.0f;
    v4f acc[TPI];
#pragma unroll
    for (int q = 0; q < TPI; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    int cj = i0 / S;  // slot of the accumulation in progress
    // four pairs at a time: the weight fragments and A2 operands of all four
    // are loaded before their MFMAs (software-pipelining two such groups, with
    // the next group's loads issued before the current group's MFMAs,
    // measured slower: 70 against 61 us per call at T = 1)
    for (int i4 = i0; i4 < i1; i4 += 4) {
      TmGroup<TPI> G;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i4 + u;
        if (i < i1) {
          const int j = i / S, st = i - j * S;
          const size_t e = (size_t)__builtin_amdgcn_readlane(slot_e, j);
          const size_t pr = (size_t)__builtin_amdgcn_readlane(slot_r, j);
          G.a[u] = load_a<FMT>(p.a2c + a2c_at<FMT>(pr, st, N), g);
          G.sa[u] = p.a2s[a2s_at(pr, st, N) + g];
          const size_t qb = e * (ntiles / 4) + tile0 / 4;  // the item's tiles share a quad
#pragma unroll
          for (int q = 0; q < TPI; ++q)
            G.b[u][q] = load_weights16(p.wp + (qb * S + st) * 4096 + ((tile0 + q) % 4) * 1024 +
                                       lane * 16);
          G.sb[u] = load_weight_scales(p.wsp + (qb * S + st) * 64 + lane);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i4 + u;
        if (i < i1) {
          const int j = i / S;
          if (j != cj) {  // the range moves on to the next slot: park the finished one
            if (lane < 16)
#pragma unroll
              for (int q = 0; q < TPI; ++q) part[wave][cj][q][lane] = acc[q][0];
#pragma unroll
            for (int q = 0; q < TPI; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
            cj = j;
          }
#pragma unroll
          for (int q = 0; q < TPI; ++q) {
            v8i bq;
            bq[0] = (int)G.b[u][q][0]; bq[1] = (int)G.b[u][q][1];
            bq[2] = (int)G.b[u][q][2]; bq[3] = (int)G.b[u][q][3];
            bq[4] = 0; bq[5] = 0; bq[6] = 0; bq[7] = 0;
            // byte (tile0 + q) % 4 of the quad's scale dword is this tile's
            acc[q] = mfma_q<FMT>((int)((tile0 + q) % 4), G.a[u], bq, acc[q], G.sa[u], G.sb[u]);
          }
        }
      }
    }
    if (i0 < i1 && lane < 16)
#pragma unroll
      for (int q = 0; q < TPI; ++q) part[wave][cj][q][lane] = acc[q][0];
    __syncthreads();
    {
      // each weighted row is rounded on its own before it joins the sum (no
      // fused multiply-add), so y is exactly the slot-order sum of the rows
      // stored for the combine.  Wave j < top_k adds the waves' partial sums
      // of slot j (lane 16 q + c: tile q, column c) and stores the weighted
      // row; then wave 0 adds each column over the slots in slot order.
#pragma clang fp contract(off)
      if (wave < k && lane < 16 * TPI) {
        const int q = lane / 16, c = lane % 16;
        const float wj =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(slot_w, wave));
        const int rj = __builtin_amdgcn_readlane(slot_r, wave);
        float o = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) o += part[v][wave][q][c];
        const float tj = wj * o;
        p.rows[(size_t)rj * p.H + 16 * tile0 + lane] = tj;
        wrow[wave][q][c] = tj;
      }
      __syncthreads();
      if (wave == 0 && lane < 16 * TPI) {
        float sum = 0.f;
        for (int j = 0; j < k; ++j) sum += wrow[j][lane / 16][lane % 16];
        p.y[(size_t)t * p.H + 16 * tile0 + lane] = f32_to_bf16(sum);
      }
    }
    __syncthreads();  // part is free again
  }
}

// ---------------------------------------------------------------------------
// Fused stream launch (MegaMoE's single launch of Stage1 and Stage2, "add
// A4W4 and FP8 P2P transport support to MegaMoE"): the GEMM1 items (gate/up
// unit, m-tile) and then the GEMM2 items (64 output columns, m-tile) of one
// call form one list, which a persistent grid walks: workgroup b takes items
// b, b + G, b + 2G, ...  A GEMM1 item publishes its SwiGLU rows with device-
// coherent stores (they write through to the memory side all XCDs share),
// waits for their completion, then increments its m-tile's count; a GEMM2
// item waits until the count of its m-tile reaches I/32, then reads the
// activations with device-coherent loads (which miss any stale copy in the
// CU's and the XCD's caches), so no cache-wide writeback or invalidate is
// needed.  A workgroup takes all its GEMM1 items before any GEMM2 item, and G
// never exceeds the workgroups the device holds at once, so on an otherwise
// idle device every GEMM1 item a wait depends on is held by a running
// workgroup that never waits itself.  The wait is bounded all the same (a
// guard against a bug, or against other work holding CUs for seconds): past
// the limit it sets the flag word and goes on.
// ---------------------------------------------------------------------------
constexpr int kWaitLimit = 1 << 22;
constexpr int kBufferFlags = 0x00020000;  // buffer resource word 3 (raw byte addressing)
constexpr int kCoherent = 16;             // buffer load cache policy: sc1

template <int FMT, int NW>
__global__ __launch_bounds__(64 * NW) void fused_kernel(KArgs p) {
  using F = typename ActFmt<FMT>::F;
  __shared__ float red[NW][16][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4;
  const int NU = p.I / 32, NB2 = p.H / 64;
  const int n_mt = uniform(p.mtoff[p.E]);
  const long n1 = (long)n_mt * NU, total = n1 + (long)n_mt * NB2;
  const int S1 = p.H / 128, S2 = p.I / 128;
  const size_t a1row = FMT == 0 ? (size_t)p.H : (size_t)p.H / 2;
  const size_t N = (size_t)p.T * p.top_k;
  constexpr int A2B = FMT == 0 ? 128 : 64;  // A2 code bytes of a row per K step
  const size_t nq1 = (size_t)(2 * p.I) / 64, nq2 = (size_t)p.H / 64;
  int *const flag = p.sync, *const done = p.sync + kSyncHead;

  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    if (w < n1) {
      // GEMM1 item, m-tile minor as in the stream kernel
      const int j = (int)(w / n_mt), mt = (int)(w % n_mt);
      const int s0 = wave * S1 / NW, s1 = (wave + 1) * S1 / NW;
      const int e = uniform(p.mbexp[mt]);
      const int2 mr = p.mbrows[mt];  // loaded beside e, not after it
      const int row0 = uniform(mr.x), nrows = uniform(mr.y);
      const int tok = p.perm[row0 + min(lane & 15, nrows - 1)] / p.top_k;
      const uint8_t *wt = p.wp + ((size_t)e * nq1 + j) * (size_t)S1 * 4096;
      const uint32_t *wsq = p.wsp + ((size_t)e * nq1 + j) * (size_t)S1 * 64;
      v4f acc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
      mma_4tiles<FMT, kStreamGroup1>(acc, p.a1c + (size_t)tok * a1row,
                                     p.a1s + (size_t)tok * (p.H / 32), FMT == 0 ? 128 : 64, 4, wt,
                                     wsq, s0, s1, lane);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][4 * q + r][lane] = acc[q][r];
      __syncthreads();
      if (wave == 0) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[i] = red[0][i][lane];
#pragma unroll
          for (int u = 1; u < NW; ++u) v[i] += red[u][i][lane];
        }
        float g0[4], g1[4], u0[4], u1[4];
        size_t prow[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          prow[r] = (size_t)(row0 + min(4 * g + r, nrows - 1));
          g0[r] = v[r]; g1[r] = v[4 + r]; u0[r] = v[8 + r]; u1[r] = v[12 + r];
        }
        swiglu_requant_n<F, FMT, 4, true>(g0, g1, u0, u1, p.a2c, p.a2s, prow, N, j, lane & 15);
        // publish: the coherent stores above have completed before the count
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0)
          __hip_atomic_fetch_add(done + mt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      // GEMM2 item, m-tile minor
      const long w2 = w - n1;
      const int nb = (int)(w2 / n_mt), mt = (int)(w2 % n_mt);
      const int s0 = wave * S2 / NW, s1 = (wave + 1) * S2 / NW;
      const int e = uniform(p.mbexp[mt]);
      const int2 mr = p.mbrows[mt];  // loaded beside e, not after it
      const int row0 = uniform(mr.x), nrows = uniform(mr.y);
      const uint8_t *wt = p.w2p + ((size_t)e * nq2 + nb) * (size_t)S2 * 4096;
      const uint32_t *wsq = p.w2sp + ((size_t)e * nq2 + nb) * (size_t)S2 * 64;
      if (tid == 0) {
        int spins = 0;
        while (__hip_atomic_load(done + mt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < NU) {
          if (++spins > kWaitLimit) {
            atomicOr(flag, 1);
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
      }
      __syncthreads();
      // the m-tile's activation rows through device-coherent buffer loads
      // (cache policy sc1), from workgroup-uniform resources at its first row
      // in each K step
      const int r = min(lane & 15, nrows - 1);
      const int aoff = r * A2B + 16 * g, soff = r * 4 + g;
      v4f acc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
      // four K steps per unrolled group, as in mma_4tiles
      for (int s4 = s0; s4 < s1; s4 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int st = s4 + u;
          if (st < s1) {
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                p.a2c + a2c_at<FMT>(row0, st, N), (short)0, kMTile * A2B, kBufferFlags);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                p.a2s + a2s_at(row0, st, N), (short)0, kMTile * 4, kBufferFlags);
            v8i a;
            const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff, 0, kCoherent);
            a[0] = (int)lo[0]; a[1] = (int)lo[1]; a[2] = (int)lo[2]; a[3] = (int)lo[3];
            if (FMT == 0) {
              const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(ra, aoff + 64, 0, kCoherent);
              a[4] = (int)hi[0]; a[5] = (int)hi[1]; a[6] = (int)hi[2]; a[7] = (int)hi[3];
            } else {
              a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
            }
            const int sa = (int)__builtin_amdgcn_raw_buffer_load_b8(rs, soff, 0, kCoherent);
            const int sb = load_weight_scales(wsq + (size_t)st * 64 + lane);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4 bq = load_weights16(wt + (size_t)st * 4096 + q * 1024 + lane * 16);
              v8i b;
              b[0] = (int)bq[0]; b[1] = (int)bq[1]; b[2] = (int)bq[2]; b[3] = (int)bq[3];
              b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
              acc[q] = mfma_q<FMT>(q, a, b, acc[q], sa, sb);
            }
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) red[wave][4 * q + rr][lane] = acc[q][rr];
      __syncthreads();
      if (wave == 0) {
        size_t prow[4];
        float t[4][4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int m = min(4 * g + rr, nrows - 1);
          const float wt_a = p.wts[row0 + m];
          prow[rr] = (size_t)(row0 + m);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = 4 * q + rr;
            float o = red[0][i][lane];
#pragma unroll
            for (int u = 1; u < NW; ++u) o += red[u][i][lane];
            t[rr][q] = wt_a * o;
          }
        }
        stage_store_n<4>(p, prow, 64 * nb, lane & 15, t);
      }
    }
    __syncthreads();  // red is free again
  }
}

GemmPlan choose_plan(int T, int top_k, int E, int act) {
  // The average rows per expert decides between weight streaming (at most 4
  // rows) and the pipelined tiled kernel, whose BM covers the mean plus 1.5
  // standard deviations of a binomial expert load (under uniform routing
  // most experts are then one m-block and their weights are read once).  An
  // activation tile fills whole 1 KiB copies and splits over two MFMA waves
  // per quad (MT even), and MT <= 12 keeps the accumulators in registers;
  // both activation formats take the same rule (MXFP4 had only 64 and 128
  // rows before, so at a mean load of 128 rows half its experts read their
  // weights twice).  Both thresholds follow the plan tuner's measurements on the
  // 7168 x 3072 (E = 384, top_k = 6) and 5120 x {640, 1152} (E = 384 x 6 and
  // 128 x 3) layers: its pick matches this rule wherever the two differ by
  // more than ~2%.
  const long N = (long)T * top_k;
  const double avg = (double)N / E;
  // T <= 2: the token-major GEMM2 with the combine folded in (one launch
  // fewer), sixteen waves per item at one token; measured faster than two
  // launches on every measured layer at T = 1 and 2 (7168 x 3072: 53.6 ->
  // 52.9 and 92.9 -> 90.5 us per call; the 5120 x {640, 1152} shards 3-12%)
  // and 3-5% slower from T = 3 (experts two tokens share are read twice)
  // Up to 4 rows per expert on average the stream GEMMs (a step's loads
  // issued together) beat the tiled ones under uniform routing: per call,
  // 7168 x 3072 T = 128 1805 against 2039 us (tiled 32) and T = 192 1998
  // against 2206; 5120 x 640 E = 384 T = 128 321 / 377 and T = 256 370 / 410;
  // E = 128 T = 128 129 / 160; 5120 x 1152 E = 384 T = 128 527 / 592.  They
  // still win at 6 to 8 rows (7168 x 3072 T = 512: 2275 / 2463), but an
  // expert with more rows than its share re-reads its weights for every 16
  // rows, and under skewed routing (half the experts empty) the stream plan
  // is already 15% slower at a mean of 2 rows (T = 128: 670 against 572), so
  // the boundary stays where skewed calls of 512 tokens and more keep the
  // tiled plan.
  if (avg <= 4.0) return T <= 2 ? GemmPlan{false, 1, 1, false, true} : GemmPlan{false, 1, 1};
  const double want = avg + 1.5 * sqrt(avg);
  {
    int mt = (int)ceil(want / 16.0);
    mt = mt + (mt & 1);
    if (mt > 10) {
      // Experts span several m-blocks at any tile height: of BM = 128, 160
      // and 192 take the one with the fewest expected padded rows,
      // E[ceil(M / BM)] * BM for a load M ~ N(avg, avg); within 1% of the
      // fewest, the largest BM (fewer m-blocks, fewer weight re-reads).  On
      // the 5120 x {640, 1152} shards at T = 16384 and 32768 this picks what
      // the tuner measured fastest: 128 at a mean load of 384 rows, 192 at
      // 512 (4-6% ahead of 128 and 160), 160 at 256 and 768.
      auto padded = [&](double bm) {
        double blocks = 0.0;
        for (int j = 0; j < 64; ++j)  // P(M > j bm), summed: E[ceil(M / bm)]
          blocks += 0.5 * erfc((j * bm - avg) / sqrt(2.0 * avg));
        return blocks * bm;
      };
      const double p8 = padded(128.0), p10 = padded(160.0), p12 = padded(192.0);
      const double best = fmin(p8, fmin(p10, p12));
      mt = p12 <= 1.01 * best ? 12 : (p10 <= 1.01 * best ? 10 : 8);
    }
    // at least 64 rows: under uniform loads 64 costs 0.2-0.4% against 32 where
    // the rule would pick 32 (T = 128 .. 1024 on the 7168 x 3072 layer), and
    // under skewed loads (a fixed per-expert bias, half the experts empty,
    // which the mean over all experts hides) it is 10-15% faster at
    // T = 512 and 1024
    (void)act;
    return GemmPlan{true, mt < 4 ? 4 : mt, kTiledSplit};
  }
}

// Waves per stream workgroup (each takes 1/NW of the K steps).  GEMM1: with
// at most one item per CU (the 5120 x {640, 1152} shards at T = 1, 2: 60-252
// items) sixteen waves put four times the weight loads in flight: 10% less
// per call (v41flash I = 640, E = 128, T = 1: 28.5 -> 25.5 us); above three
// items per CU eight waves (with a step's loads issued together, eight
// against four measured 2.7% less per call on the 5120 x 640 shard at T = 8
// and equal on the 7168 x 3072 layer at T = 8 .. 64; at 2.25 items per CU,
// the 7168 x 3072 layer at T = 1, four were 0.3 us faster).  GEMM2 (K = I, a
// third of GEMM1's steps or fewer) is faster with four at every decode size
// (eight: +1% at T = 8 on 7168 x 3072, +47% at T = 64 on the 640-wide shard,
// where its waves got at most one K step each).
static int stream_waves(long items_upper, int num_cus) {
  if (items_upper <= num_cus) return 16;
  return items_upper > 3L * num_cus ? 8 : 4;
}

static unsigned persistent_grid(long items_upper, int num_cus) {
  const long cap = (long)num_cus * 4;
  return (unsigned)(items_upper < cap ? items_upper : cap);
}

// GEMM2 weight steps a wave of a fused workgroup loads before its wait
// The grid never exceeds the workgroups the device holds at once (the
// waits rely on it: see fused_kernel).
template <int FMT, int NW>
static hipError_t launch_fused_w(const GemmArgs &a, const KArgs &k, hipStream_t s) {
  static int per_cu = 0;  // resident workgroups per CU, a property of the kernel
  if (per_cu == 0) {
    int n = 0;
    const hipError_t e =
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_kernel<FMT, NW>, 64 * NW, 0);
    if (e != hipSuccess) return e;
    per_cu = n > 0 ? n : 1;
  }
  const long items = a.max_mtiles * (a.I / 32 + a.H / 64);
  const long cap = (long)per_cu * a.num_cus;
  fused_kernel<FMT, NW><<<(unsigned)(items < cap ? items : cap), 64 * NW, 0, s>>>(k);
  return hipGetLastError();
}

static hipError_t launch_fused(const GemmArgs &a, hipStream_t s) {
  const KArgs k = make_args(a, false);
  return a.act == MOE_ACT_MXFP8_E4M3 ? launch_fused_w<0, 4>(a, k, s)
                                     : launch_fused_w<4, 4>(a, k, s);
}

hipError_t launch_gemm1(const GemmArgs &a, hipStream_t s) {
  if (a.plan.fused) return launch_fused(a, s);
  const KArgs k = make_args(a, false);
  if (a.plan.tiled) return launch_tiled_gemm1(a, k, s);
  const long items = a.max_mtiles * (a.I / 32);
  const unsigned grid = persistent_grid(items, a.num_cus);
  const bool f8 = a.act == MOE_ACT_MXFP8_E4M3;
  const int nw = stream_waves(items, a.num_cus);
  if (nw == 16) {
    if (f8) gemm1_kernel<0, 16><<<grid, 1024, 0, s>>>(k);
    else gemm1_kernel<4, 16><<<grid, 1024, 0, s>>>(k);
  } else if (nw == 8) {
    if (f8) gemm1_kernel<0, 8><<<grid, 512, 0, s>>>(k);
    else gemm1_kernel<4, 8><<<grid, 512, 0, s>>>(k);
  } else {
    if (f8) gemm1_kernel<0, 4><<<grid, 256, 0, s>>>(k);
    else gemm1_kernel<4, 4><<<grid, 256, 0, s>>>(k);
  }
  return hipGetLastError();
}

hipError_t launch_gemm2(const GemmArgs &a, hipStream_t s) {
  if (a.plan.fused) return hipSuccess;  // launch_gemm1 ran both GEMMs
  const KArgs k = make_args(a, true);
  if (a.plan.tiled) return launch_tiled_gemm2(a, k, s);
  if (gemm2_writes_y(a)) {
    // token-major with the combine folded in: one item per (token, 32
    // columns).  32-column items measured at or below 64-column ones at every
    // decode size (T = 1: 58.5 against 61.1 us per call; they give 224 items
    // per token instead of 112 for the device's 256 CUs)
    const long items = (long)a.T * (a.H / 32);
    const long cap = 2L * a.num_cus;
    const unsigned grid = (unsigned)(items < cap ? items : cap);
    if (items <= a.num_cus) {
      if (a.act == MOE_ACT_MXFP8_E4M3) gemm2_tm_kernel<0, 16, 2><<<grid, 1024, 0, s>>>(k);
      else gemm2_tm_kernel<4, 16, 2><<<grid, 1024, 0, s>>>(k);
    } else {
      if (a.act == MOE_ACT_MXFP8_E4M3) gemm2_tm_kernel<0, 8, 2><<<grid, 512, 0, s>>>(k);
      else gemm2_tm_kernel<4, 8, 2><<<grid, 512, 0, s>>>(k);
    }
    return hipGetLastError();
  }
  const long items = a.max_mtiles * (a.H / 64);
  const unsigned grid = persistent_grid(items, a.num_cus);
  // four waves at every decode size (measurements at stream_waves)
  if (a.act == MOE_ACT_MXFP8_E4M3) gemm2_kernel<0, 4><<<grid, 256, 0, s>>>(k);
  else gemm2_kernel<4, 4><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

}  // namespace moe
