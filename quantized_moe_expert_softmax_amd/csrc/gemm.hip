// gemm.hip -- grouped scaled-MFMA expert GEMMs of the MoE layer (gfx950).
//
// GEMM1 ("add A4W4 and FP8 P2P transport support to MegaMoE", Technical
// Details: consume FP4/FP8 activations in GEMM1, emit A2 activations and
// scales; "feat(moe): FlyDSL MegaMoE fused EP-MoE integration": interleaved
// gate/up pairing for SwiGLU): per expert, the quantised token rows routed to
// it times the expert's MXFP4 gate and up rows, FP32 accumulate, then
// h = silu(gate) * up requantised to the activation format in 1x32 blocks.
//
// GEMM2 (same page: FP4xFP4 GEMM2, weighted rows, FP32 accumulation of the
// top-k contributions): per expert, the A2 rows times the MXFP4 down rows,
// each output row scaled by its routing weight and added atomically into the
// FP32 combine buffer of its token.
//
// Both use the gfx950 block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4
// (A = activations, E4M3 or E2M1; B = weights, E2M1; one E8M0 scale per lane
// per 32-wide K block).  Operand layouts (measured on the device):
//   E2M1 operand: lane l holds row l%16, K [32*(l/16), +32), low nibble first
//   E4M3 operand: lane l holds row l%16, bytes 0..15 = K [16*(l/16), +16) and
//                 bytes 16..31 = K [64 + 16*(l/16), +16)
//   scale:        lane l gives the scale of row l%16, K block l/16
//   result:       lane l, register r holds row 4*(l/16) + r, column l%16
//
// Work is scheduled persistently: a work item is one 16-row m-tile of one
// expert (from the sort's m-tile prefix) times one 64-row weight block; the
// four waves of a workgroup split the K steps and reduce in LDS.  Padded rows
// of a partial m-tile load a valid row and never store (padding guard).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "mx_device.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct KArgs {
  int T, top_k, E, H, I;
  const uint8_t *a1c, *a1s;
  uint8_t *a2c, *a2s;
  const int32_t *perm, *offsets, *mtoff;
  const float *wts;
  const uint8_t *wp;
  const uint32_t *wsp;
  float *comb;
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Expert owning global m-tile mt: the largest e with mtoff[e] <= mt.
__device__ __forceinline__ int find_expert(const int32_t *__restrict__ mtoff, int E, int mt) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uniform(mtoff[mid]) <= mt) lo = mid;
    else hi = mid;
  }
  return lo;
}

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

// acc[q] += A(rows of this lane's m-tile) x B(prepacked tile q) over the K
// groups [g0, g1) of 4 steps each.
template <int FMT>
__device__ __forceinline__ void mma_4tiles(v4f acc[4], const uint8_t *__restrict__ arow,
                                           const uint8_t *__restrict__ asrow,
                                           const uint8_t *__restrict__ wt,
                                           const uint32_t *__restrict__ wst, size_t tile_bytes,
                                           size_t tile_dwords, int S, int g0, int g1, int lane) {
  const int g = lane >> 4;
  for (int gq = g0; gq < g1; ++gq) {
    uint32_t bs[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) bs[q] = wst[q * tile_dwords + (size_t)gq * 64 + lane];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int s = 4 * gq + jj;
      if (s < S) {
        const v8i a = load_a<FMT>(arow, s, g);
        const int sa = asrow[4 * s + g];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 bq = *reinterpret_cast<const uint4 *>(wt + q * tile_bytes +
                                                           ((size_t)s * 64 + lane) * 16);
          v8i b;
          b[0] = (int)bq.x; b[1] = (int)bq.y; b[2] = (int)bq.z; b[3] = (int)bq.w;
          b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
          acc[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a, b, acc[q], FMT, 4, 0, sa, 0, (int)((bs[q] >> (8 * jj)) & 0xffu));
        }
      }
    }
  }
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

template <int FMT>
struct ActFmt;
template <>
struct ActFmt<0> { using F = E4M3; };
template <>
struct ActFmt<4> { using F = E2M1; };

template <int FMT>
__global__ __launch_bounds__(256) void gemm1_kernel(KArgs p) {
  using F = typename ActFmt<FMT>::F;
  __shared__ float red[4][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NU = p.I / 32;
  const int n_mt = uniform(p.mtoff[p.E]);
  const long total = (long)n_mt * NU;
  const int S = p.H / 128, G = (S + 3) / 4;
  const int g0 = wave * G / 4, g1 = (wave + 1) * G / 4;
  const size_t a1row = FMT == 0 ? (size_t)p.H : (size_t)p.H / 2;
  const size_t a2row = FMT == 0 ? (size_t)p.I : (size_t)p.I / 2;
  const size_t ntiles = (size_t)(2 * p.I) / 16;
  const size_t tile_bytes = (size_t)S * 1024, tile_dwords = (size_t)G * 64;
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    const int j = (int)(w / n_mt), mt = (int)(w % n_mt);
    const int e = find_expert(p.mtoff, p.E, mt);
    const int row0 = uniform(p.offsets[e]) + kMTile * (mt - uniform(p.mtoff[e]));
    const int nrows = min(kMTile, uniform(p.offsets[e + 1]) - row0);
    const int pr = row0 + min(lane & 15, nrows - 1);
    const int tok = p.perm[pr] / p.top_k;
    const uint8_t *arow = p.a1c + (size_t)tok * a1row;
    const uint8_t *asrow = p.a1s + (size_t)tok * (p.H / 32);
    const uint8_t *wt = p.wp + ((size_t)e * ntiles + 4 * (size_t)j) * tile_bytes;
    const uint32_t *wst = p.wsp + ((size_t)e * ntiles + 4 * (size_t)j) * tile_dwords;
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    mma_4tiles<FMT>(acc, arow, asrow, wt, wst, tile_bytes, tile_dwords, S, g0, g1, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][4 * q + r][lane] = acc[q][r];
    __syncthreads();
    if (wave == 0) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = ((red[0][i][lane] + red[1][i][lane]) + red[2][i][lane]) + red[3][i][lane];
      const int c = lane & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // tiles: 0 = gate cols [32j, +16), 1 = gate [32j+16, +16), 2/3 = up
        const float hlo = silu(v[0 * 4 + r]) * v[2 * 4 + r];
        const float hhi = silu(v[1 * 4 + r]) * v[3 * 4 + r];
        uint32_t am = max(f32_bits(hlo) & 0x7fffffffu, f32_bits(hhi) & 0x7fffffffu);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
        const int X = block_exponent<F>(am);
        const uint32_t clo = encode_element<F>(f32_bits(hlo), X);
        const uint32_t chi = encode_element<F>(f32_bits(hhi), X);
        const uint32_t plo = (uint32_t)__shfl_xor((int)clo, 1);
        const uint32_t phi = (uint32_t)__shfl_xor((int)chi, 1);
        const int m = 4 * (lane >> 4) + r;
        if (m < nrows) {
          const size_t prow = (size_t)(row0 + m);
          uint8_t *dst = p.a2c + prow * a2row;
          if (FMT == 0) {
            dst[32 * j + c] = (uint8_t)clo;
            dst[32 * j + 16 + c] = (uint8_t)chi;
          } else if ((c & 1) == 0) {
            dst[16 * j + c / 2] = (uint8_t)(clo | (plo << 4));
            dst[16 * j + 8 + c / 2] = (uint8_t)(chi | (phi << 4));
          }
          if (c == 0) p.a2s[prow * (p.I / 32) + j] = (uint8_t)(X + 127);
        }
      }
    }
    __syncthreads();
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void gemm2_kernel(KArgs p) {
  __shared__ float red[4][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int NB = p.H / 64;
  const int n_mt = uniform(p.mtoff[p.E]);
  const long total = (long)n_mt * NB;
  const int S = p.I / 128, G = (S + 3) / 4;
  const int g0 = wave * G / 4, g1 = (wave + 1) * G / 4;
  const size_t a2row = FMT == 0 ? (size_t)p.I : (size_t)p.I / 2;
  const size_t ntiles = (size_t)p.H / 16;
  const size_t tile_bytes = (size_t)S * 1024, tile_dwords = (size_t)G * 64;
  for (long w = blockIdx.x; w < total; w += gridDim.x) {
    const int nb = (int)(w / n_mt), mt = (int)(w % n_mt);
    const int e = find_expert(p.mtoff, p.E, mt);
    const int row0 = uniform(p.offsets[e]) + kMTile * (mt - uniform(p.mtoff[e]));
    const int nrows = min(kMTile, uniform(p.offsets[e + 1]) - row0);
    const size_t pr = (size_t)(row0 + min(lane & 15, nrows - 1));
    const uint8_t *arow = p.a2c + pr * a2row;
    const uint8_t *asrow = p.a2s + pr * (p.I / 32);
    const uint8_t *wt = p.wp + ((size_t)e * ntiles + 4 * (size_t)nb) * tile_bytes;
    const uint32_t *wst = p.wsp + ((size_t)e * ntiles + 4 * (size_t)nb) * tile_dwords;
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    mma_4tiles<FMT>(acc, arow, asrow, wt, wst, tile_bytes, tile_dwords, S, g0, g1, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][4 * q + r][lane] = acc[q][r];
    __syncthreads();
    if (wave == 0) {
      const int c = lane & 15;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (lane >> 4) + r;
        if (m < nrows) {
          const int a = p.perm[row0 + m];
          const long t = a / p.top_k;
          const float wt_a = p.wts[a];
          float *dst = p.comb + t * (long)p.H + 64 * nb + c;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = 4 * q + r;
            const float o = ((red[0][i][lane] + red[1][i][lane]) + red[2][i][lane]) + red[3][i][lane];
            unsafeAtomicAdd(dst + 16 * q, wt_a * o);
          }
        }
      }
    }
    __syncthreads();
  }
}

static KArgs make_args(const GemmArgs &a, bool second) {
  KArgs k{};
  k.T = a.T; k.top_k = a.top_k; k.E = a.E; k.H = a.H; k.I = a.I;
  k.a1c = a.a1c; k.a1s = a.a1s; k.a2c = a.a2c; k.a2s = a.a2s;
  k.perm = a.perm; k.offsets = a.offsets; k.mtoff = a.mtoff; k.wts = a.wts;
  k.wp = second ? a.w2p : a.w13p;
  k.wsp = reinterpret_cast<const uint32_t *>(second ? a.w2sp : a.w13sp);
  k.comb = a.comb;
  return k;
}

static unsigned persistent_grid(long items_upper, int num_cus) {
  const long cap = (long)num_cus * 4;
  return (unsigned)(items_upper < cap ? items_upper : cap);
}

hipError_t launch_gemm1(const GemmArgs &a, hipStream_t s) {
  const KArgs k = make_args(a, false);
  const unsigned grid = persistent_grid(a.max_mtiles * (a.I / 32), a.num_cus);
  if (a.act == MOE_ACT_MXFP8_E4M3) gemm1_kernel<0><<<grid, 256, 0, s>>>(k);
  else gemm1_kernel<4><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

hipError_t launch_gemm2(const GemmArgs &a, hipStream_t s) {
  const KArgs k = make_args(a, true);
  const unsigned grid = persistent_grid(a.max_mtiles * (a.H / 64), a.num_cus);
  if (a.act == MOE_ACT_MXFP8_E4M3) gemm2_kernel<0><<<grid, 256, 0, s>>>(k);
  else gemm2_kernel<4><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

}  // namespace moe
