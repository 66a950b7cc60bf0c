// gemm_stream.hip -- stream (decode) variant of the expert GEMMs, the per-call
// choice between it and the tiled variant, and the GEMM launchers.
// Conventions and operand layouts: gemm_common.h.
#include "gemm_common.h"

namespace moe {

// A operand of K step s for lane group g from a row-major code row.
template <int FMT>
__device__ __forceinline__ v8i load_a(const uint8_t *__restrict__ row, int s, int g) {
  v8i a;
  if (FMT == 0) {
    const uint4 lo = *reinterpret_cast<const uint4 *>(row + 128 * s + 16 * g);
    const uint4 hi = *reinterpret_cast<const uint4 *>(row + 128 * s + 64 + 16 * g);
    a[0] = (int)lo.x; a[1] = (int)lo.y; a[2] = (int)lo.z; a[3] = (int)lo.w;
    a[4] = (int)hi.x; a[5] = (int)hi.y; a[6] = (int)hi.z; a[7] = (int)hi.w;
  } else {
    const uint4 lo = *reinterpret_cast<const uint4 *>(row + 64 * s + 16 * g);
    a[0] = (int)lo.x; a[1] = (int)lo.y; a[2] = (int)lo.z; a[3] = (int)lo.w;
    a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
  }
  return a;
}

// acc[q] += A(rows of this lane's m-tile) x B(prepacked tile q of one quad)
// over the K steps [s0, s1), four steps per unrolled group.
template <int FMT>
__device__ __forceinline__ void mma_4tiles(v4f acc[4], const uint8_t *__restrict__ arow,
                                           const uint8_t *__restrict__ asrow,
                                           const uint8_t *__restrict__ wt,
                                           const uint32_t *__restrict__ wsq, int s0, int s1,
                                           int lane) {
  const int g = lane >> 4;
  for (int s4 = s0; s4 < s1; s4 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s4 + u;
      if (s < s1) {
        const v8i a = load_a<FMT>(arow, s, g);
        const int sa = asrow[4 * s + g];
        const int sb = (int)wsq[(size_t)s * 64 + lane];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 bq = *reinterpret_cast<const uint4 *>(wt + (size_t)s * 4096 + q * 1024 +
                                                           lane * 16);
          v8i b;
          b[0] = (int)bq.x; b[1] = (int)bq.y; b[2] = (int)bq.z; b[3] = (int)bq.w;
          b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
          acc[q] = mfma_q<FMT>(q, a, b, acc[q], sa, sb);
        }
      }
    }
  }
}

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
  const size_t a2row = FMT == 0 ? (size_t)p.I : (size_t)p.I / 2;
  const size_t nquads = (size_t)(2 * p.I) / 64;
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    const int j = (int)(w / n_mt), mt = (int)(w % n_mt);
    const int e = uniform(p.mbexp[mt]);
    const int row0 = uniform(p.offsets[e]) + kMTile * (mt - uniform(p.mtoff[e]));
    const int nrows = min(kMTile, uniform(p.offsets[e + 1]) - row0);
    const int pr = row0 + min(lane & 15, nrows - 1);
    const int tok = p.perm[pr] / p.top_k;
    const uint8_t *arow = p.a1c + (size_t)tok * a1row;
    const uint8_t *asrow = p.a1s + (size_t)tok * (p.H / 32);
    const uint8_t *wt = p.wp + ((size_t)e * nquads + j) * (size_t)S * 4096;
    const uint32_t *wsq = p.wsp + ((size_t)e * nquads + j) * (size_t)S * 64;
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    mma_4tiles<FMT>(acc, arow, asrow, wt, wsq, s0, s1, lane);
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
      uint8_t *ar[4], *sr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (lane >> 4) + r;
        const size_t prow = (size_t)(row0 + min(m, nrows - 1));
        g0[r] = v[0 * 4 + r]; g1[r] = v[1 * 4 + r]; u0[r] = v[2 * 4 + r]; u1[r] = v[3 * 4 + r];
        ar[r] = p.a2c + prow * a2row;
        sr[r] = p.a2s + prow * (p.I / 32);
      }
      swiglu_requant_n<F, FMT, 4>(g0, g1, u0, u1, ar, sr, j, c);
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
  const size_t a2row = FMT == 0 ? (size_t)p.I : (size_t)p.I / 2;
  const size_t nquads = (size_t)p.H / 64;
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    const int nb = (int)(w / n_mt), mt = (int)(w % n_mt);
    const int e = uniform(p.mbexp[mt]);
    const int row0 = uniform(p.offsets[e]) + kMTile * (mt - uniform(p.mtoff[e]));
    const int nrows = min(kMTile, uniform(p.offsets[e + 1]) - row0);
    const size_t pr = (size_t)(row0 + min(lane & 15, nrows - 1));
    const uint8_t *arow = p.a2c + pr * a2row;
    const uint8_t *asrow = p.a2s + pr * (p.I / 32);
    const uint8_t *wt = p.wp + ((size_t)e * nquads + nb) * (size_t)S * 4096;
    const uint32_t *wsq = p.wsp + ((size_t)e * nquads + nb) * (size_t)S * 64;
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    mma_4tiles<FMT>(acc, arow, asrow, wt, wsq, s0, s1, lane);
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

// how the four waves of a tiled workgroup split a BM x 256 item: 1 = all rows
// x one quad each, 2 = half the rows x two quads each
constexpr int kTiledSplit = 1;

GemmPlan choose_plan(int T, int top_k, int E, int act) {
  // The average rows per expert decides between weight streaming (fewer than
  // 2 rows) and the pipelined tiled kernel, whose BM covers the mean plus 1.5
  // standard deviations of a binomial expert load (under uniform routing
  // most experts are then one m-block and their weights are read once).  An
  // activation tile must fill whole 1 KiB copies per wave (MXFP8: MT even;
  // MXFP4: MT a multiple of 4) and MT <= 10 keeps the accumulators in
  // registers.  Both thresholds follow the plan tuner's measurements on the
  // 7168 x 3072 (E = 384, top_k = 6) and 5120 x {640, 1152} (E = 384 x 6 and
  // 128 x 3) layers: its pick matches this rule wherever the two differ by
  // more than ~2%.
  const long N = (long)T * top_k;
  const double avg = (double)N / E;
  if (avg < 2.0) return GemmPlan{false, 1, 1};
  const double want = avg + 1.5 * sqrt(avg);
  if (act == MOE_ACT_MXFP8_E4M3) {
    int mt = (int)ceil(want / 16.0);
    mt = mt + (mt & 1);
    return GemmPlan{true, mt < 2 ? 2 : (mt > 10 ? 10 : mt), kTiledSplit};
  }
  return GemmPlan{true, want <= 64.0 ? 4 : 8, kTiledSplit};
}

// Waves per stream workgroup (each takes 1/NW of the K steps).  Measured on
// the 7168 x 3072 layer: GEMM1 runs faster with eight once there are more
// items than four per CU (below that, eight-wave workgroups at two per CU
// leave part of the items for a second round); GEMM2 (K = I, a third of
// GEMM1's steps) is faster with four at every decode size.
static int stream_waves(long items_upper, int num_cus, bool second) {
  return !second && items_upper > 4L * num_cus ? 8 : 4;
}

static unsigned persistent_grid(long items_upper, int num_cus) {
  const long cap = (long)num_cus * 4;
  return (unsigned)(items_upper < cap ? items_upper : cap);
}

hipError_t launch_gemm1(const GemmArgs &a, hipStream_t s) {
  const KArgs k = make_args(a, false);
  if (a.plan.tiled) return launch_tiled_gemm1(a, k, s);
  const long items = a.max_mtiles * (a.I / 32);
  const unsigned grid = persistent_grid(items, a.num_cus);
  const bool f8 = a.act == MOE_ACT_MXFP8_E4M3;
  if (stream_waves(items, a.num_cus, false) == 8) {
    if (f8) gemm1_kernel<0, 8><<<grid, 512, 0, s>>>(k);
    else gemm1_kernel<4, 8><<<grid, 512, 0, s>>>(k);
  } else {
    if (f8) gemm1_kernel<0, 4><<<grid, 256, 0, s>>>(k);
    else gemm1_kernel<4, 4><<<grid, 256, 0, s>>>(k);
  }
  return hipGetLastError();
}

hipError_t launch_gemm2(const GemmArgs &a, hipStream_t s) {
  const KArgs k = make_args(a, true);
  if (a.plan.tiled) return launch_tiled_gemm2(a, k, s);
  const long items = a.max_mtiles * (a.H / 64);
  const unsigned grid = persistent_grid(items, a.num_cus);
  const bool f8 = a.act == MOE_ACT_MXFP8_E4M3;
  if (stream_waves(items, a.num_cus, true) == 8) {
    if (f8) gemm2_kernel<0, 8><<<grid, 512, 0, s>>>(k);
    else gemm2_kernel<4, 8><<<grid, 512, 0, s>>>(k);
  } else {
    if (f8) gemm2_kernel<0, 4><<<grid, 256, 0, s>>>(k);
    else gemm2_kernel<4, 4><<<grid, 256, 0, s>>>(k);
  }
  return hipGetLastError();
}

}  // namespace moe
