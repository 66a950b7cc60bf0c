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
// each output row scaled by its routing weight and stored as an FP32 row in
// sorted order; the combine kernel sums a token's top-k rows.
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
// Two variants, chosen per call from the rows per expert.  Stream (decode):
// a work item is one 16-row m-tile of one expert times one 64-row weight
// block; the four waves of a workgroup split the K steps and reduce in LDS.
// Tiled (prefill): see below.  Both schedule persistently from the sort's
// m-block table; padded rows of a partial m-block load a valid row and never
// store (padding guard).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "mx_device.h"

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct KArgs {
  int T, top_k, E, H, I;
  const uint8_t *a1c, *a1s;
  uint8_t *a2c, *a2s;
  const int32_t *perm, *offsets, *mtoff, *mbexp;
  const float *wts;  // [N] routing weight of sorted row p
  const uint8_t *wp;
  const uint32_t *wsp;
  float *rows;  // [N][H] weighted GEMM2 rows (sorted order)
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }


// One scaled MFMA with the weight scale taken from byte q of sb (q is a
// compile-time constant after unrolling: the byte is the MFMA's op_sel).
template <int FMT>
__device__ __forceinline__ v4f mfma_q(int q, v8i a, v8i b, v4f c, int sa, int sb) {
  switch (q) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, 4, 0, sa, 0, sb);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, 4, 0, sa, 1, sb);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, 4, 0, sa, 2, sb);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, 4, 0, sa, 3, sb);
  }
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

// silu(g) = g / (1 + exp(-g)) with the hardware exp2 and reciprocal; for very
// negative g the exponential overflows to inf and silu goes to (-)0.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Cross-lane moves within 16-lane rows (DPP, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
// maximum over the 16 lanes of a row: quad_perm [1,0,3,2], [2,3,0,1], then
// row_half_mirror and row_mirror
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, dpp<0xB1>(v));
  v = max(v, dpp<0x4E>(v));
  v = max(v, dpp<0x141>(v));
  v = max(v, dpp<0x140>(v));
  return v;
}

// GEMM1 epilogue for one accumulator register r: lane c = l%16 of row group
// l/16 holds gate/up columns 32j + c (lo) and 32j + 16 + c (hi) of one token
// row; h = silu(gate) * up; the 32 h values of the row form one 1x32 block
// (amax over the 16 lanes), requantised and stored to the A2 row.  All lanes
// call and store: the two lanes of an E2M1 byte both write it whole, all 16
// lanes write the scale byte, and a padded row (computed from the last valid
// row's data) rewrites that row's values, so no store needs a branch.
template <class F, int FMT>
__device__ __forceinline__ void swiglu_requant(float glo, float ghi, float ulo, float uhi,
                                               uint8_t *__restrict__ a2row,
                                               uint8_t *__restrict__ a2srow, int j, int c) {
  const float hlo = silu(glo) * ulo;
  const float hhi = silu(ghi) * uhi;
  const uint32_t am = row16_max(max(f32_bits(hlo) & 0x7fffffffu, f32_bits(hhi) & 0x7fffffffu));
  const int X = block_exponent<F>(am);
  const uint32_t clo = encode_element<F>(f32_bits(hlo), X);
  const uint32_t chi = encode_element<F>(f32_bits(hhi), X);
  const uint32_t plo = dpp<0xB1>(clo);  // code of lane c ^ 1
  const uint32_t phi = dpp<0xB1>(chi);
  if (FMT == 0) {
    a2row[32 * j + c] = (uint8_t)clo;
    a2row[32 * j + 16 + c] = (uint8_t)chi;
  } else {
    const bool odd = c & 1;
    a2row[16 * j + c / 2] = (uint8_t)(odd ? (plo | (clo << 4)) : (clo | (plo << 4)));
    a2row[16 * j + 8 + c / 2] = (uint8_t)(odd ? (phi | (chi << 4)) : (chi | (phi << 4)));
  }
  a2srow[j] = (uint8_t)(X + 127);
}

template <int FMT>
struct ActFmt;
template <>
struct ActFmt<0> { using F = E4M3; };
template <>
struct ActFmt<4> { using F = E2M1; };

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
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // tiles: 0 = gate cols [32j, +16), 1 = gate [32j+16, +16), 2/3 = up
        const int m = 4 * (lane >> 4) + r;
        const size_t prow = (size_t)(row0 + min(m, nrows - 1));
        swiglu_requant<F, FMT>(v[0 * 4 + r], v[1 * 4 + r], v[2 * 4 + r], v[3 * 4 + r],
                               p.a2c + prow * a2row, p.a2s + prow * (p.I / 32), j, c);
      }
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
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // a padded row recomputes the last valid row and stores the same values
        const int m = min(4 * (lane >> 4) + r, nrows - 1);
        const float wt_a = p.wts[row0 + m];
        float *dst = p.rows + (size_t)(row0 + m) * p.H + 64 * nb + c;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = 4 * q + r;
          float o = red[0][i][lane];
#pragma unroll
          for (int u = 1; u < NW; ++u) o += red[u][i][lane];
          dst[16 * q] = wt_a * o;
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Tiled variant (prefill): a work item is (expert e, 256 weight rows, BM =
// 16*MT token rows).  Wave w owns 64 weight rows (GEMM1: one gate/up unit)
// and MT x 4 accumulator tiles, so every weight fragment is read from HBM
// once per item and feeds MT MFMAs; the activation tile of a K step is
// shared by the four waves.  Every operand of a K step -- the BM activation
// rows (16-byte chunks XOR-swizzled by row), their E8M0 scales, each wave's
// four 1 KiB weight fragments and their scale dword -- is copied from
// global memory straight into LDS with global_load_lds (no register
// staging), NS steps deep, the copies of a later step interleaved with the
// MFMAs of the current one; the waits count those copies exactly (they are
// the only vector-memory instructions in the loop and issue in program
// order).  BM is picked per call so that most experts fit one m-block (each
// weight panel is then read once).  The logical workgroup index is remapped
// so consecutive items share an XCD and its L2.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *glb_ptr_t;

// lane i of the wave copies 16 (4) bytes from its own address g to
// lds_base + 16*i (4*i); lds_base must be wave-uniform
__device__ __forceinline__ void copy16_to_lds(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)g, (lds_ptr_t)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void copy4_to_lds(const void *g, void *lds_base) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)g, (lds_ptr_t)lds_base, 4, 0, 0);
}

// s_waitcnt vmcnt(N), expcnt and lgkmcnt left free (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier for the copy pipeline: LDS reads of this wave done, no
// wait on the copies still in flight (a __syncthreads would wait for all of
// them, since they write LDS).
__device__ __forceinline__ void barrier_keep_copies() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt untouched
  __builtin_amdgcn_s_barrier();
}
// LDS of the tiled kernel: a ring of NA activation stages (the BM rows of
// one K step and their scale dwords) and a ring of NB weight stages (each
// wave's four 1 KiB fragments and scale dword).  Weights stream from HBM and
// are fetched NB - 1 steps ahead, activations come from L2 and are fetched
// NA - 1 = 2 steps ahead.  (Weight rings deeper than 4 fit in 160 KiB but
// measured slower on the 7168 x 3072 layer.)
template <int FMT, int MT>
struct TileShape {
  static constexpr int BM = 16 * MT;
  static constexpr int ROWB = FMT == 0 ? 128 : 64;   // activation bytes per row per K step
  static constexpr int CH = ROWB / 16;               // 16-byte chunks per row
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int A_COPIES = A_BYTES / 4096;    // 1 KiB copies per wave per stage
  static constexpr int RPW = BM / 4;                 // scale rows copied per wave
  static constexpr int CA = A_COPIES + 1;            // activation copies per wave per step
  static constexpr int CB = 4 + 1;                   // weight copies per wave per step
  static constexpr int C = CA + CB;
  static constexpr int OFF_AS = A_BYTES;             // [4 waves][64 slots] dwords
  static constexpr int A_STAGE = OFF_AS + 1024;
  static constexpr int OFF_BS = 4 * 4096;            // after [4 waves][4 tiles] fragments
  static constexpr int B_STAGE = OFF_BS + 4 * 256;   // + [4 waves][64 lanes] scale dwords
  static constexpr int NA = 3;
  static constexpr int NB_FIT = (160 * 1024 - NA * A_STAGE) / B_STAGE;
  static constexpr int NB = NB_FIT < 4 ? NB_FIT : 4;  // deeper measured slower
  static constexpr int D = NB - NA;                  // weight lead over activations, in steps
  static constexpr int B_BASE = NA * A_STAGE;
  static constexpr int LDS = B_BASE + NB * B_STAGE;
  static_assert(A_BYTES % 4096 == 0, "activation tile must fill whole copies");
  static_assert(RPW <= 64, "scale rows per wave");
  static_assert(D >= 1, "weights must lead activations");
  static_assert((NA - 1) * CA + (NB - 1) * CB < 64, "vmcnt range");
  // LDS slot of row r's scale dword
  static __device__ __forceinline__ int sslot(int r) { return (r / RPW) * 64 + (r % RPW); }
};

template <int FMT, int MT, bool SECOND>
__global__ __launch_bounds__(256, 1) void tiled_kernel(KArgs p) {
  using F = typename ActFmt<FMT>::F;
  using TS = TileShape<FMT, MT>;
  constexpr int NA = TS::NA, NB = TS::NB, D = TS::D;
  constexpr int BM = TS::BM, ROWB = TS::ROWB, CH = TS::CH;
  __shared__ __attribute__((aligned(16))) uint8_t lds[TS::LDS];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int K = SECOND ? p.I : p.H;
  const int S = K / 128;
  const int ntiles = (SECOND ? p.H : 2 * p.I) / 16;
  const int NBLK = (ntiles + 15) / 16;  // n-blocks of 256 weight rows
  const int n_mb = uniform(p.mtoff[p.E]);
  const long total = (long)n_mb * NBLK;
  const size_t arow = FMT == 0 ? (size_t)K : (size_t)K / 2;
  const size_t srow = (size_t)K / 32;
  const size_t a2row = FMT == 0 ? (size_t)p.I : (size_t)p.I / 2;
  const size_t quad_bytes = (size_t)S * 4096, quad_dwords = (size_t)S * 64;
  const uint8_t *__restrict__ A = SECOND ? p.a2c : p.a1c;
  const uint8_t *__restrict__ As = SECOND ? p.a2s : p.a1s;
  const int G = gridDim.x;
  const int L = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);
  // per-lane constant LDS offsets of the swizzled activation fragments
  const int swz = (FMT == 0) ? (r16 & 7) : (r16 & 3);
  const int aoff_lo = r16 * ROWB + 16 * (g ^ swz);
  const int aoff_hi = r16 * ROWB + 16 * ((4 + g) ^ swz);

  for (long w = L; w < total; w += G) {
    // item w = (global m-block, n-block), n-block minor: consecutive items
    // (neighbouring CUs of one XCD) share the activation tile through L2
    const int gmb = (int)(w / NBLK), nb = (int)(w % NBLK);
    const int e = uniform(p.mbexp[gmb]);
    const int mb = gmb - uniform(p.mtoff[e]);
    const int row0 = uniform(p.offsets[e]) + BM * mb;
    const int nrows = min(BM, uniform(p.offsets[e + 1]) - row0);

    // global sources of this lane's copies (the K-step offset is added later)
    const uint8_t *asrc[TS::A_COPIES];
#pragma unroll
    for (int i = 0; i < TS::A_COPIES; ++i) {
      const int ci = (wave * TS::A_COPIES + i) * 64 + lane;  // LDS chunk this lane fills
      const int row = ci / CH, slot = ci % CH;
      const int rr = min(row, nrows - 1);
      const size_t ridx = SECOND ? (size_t)(row0 + rr) : (size_t)(p.perm[row0 + rr] / p.top_k);
      asrc[i] = A + ridx * arow + 16 * (slot ^ (row & (CH - 1)));
    }
    const uint8_t *ssrc;
    {
      const int row = wave * TS::RPW + (lane % TS::RPW);
      const int rr = min(row, nrows - 1);
      const size_t ridx = SECOND ? (size_t)(row0 + rr) : (size_t)(p.perm[row0 + rr] / p.top_k);
      ssrc = As + ridx * srow;
    }
    const int tile0 = 16 * nb + 4 * wave;
    const bool active = tile0 < ntiles;
    const size_t qbase = (size_t)e * (ntiles / 4) + (active ? tile0 / 4 : 0);
    const uint8_t *wsrc = p.wp + qbase * quad_bytes + (size_t)lane * 16;
    const uint32_t *wssrc = p.wsp + qbase * quad_dwords + lane;

    // Copy group p = the weight copies of K step p + D (the weights run D
    // steps further ahead), then the activation copies of step p.  Copies of
    // a step past the last are issued from one fixed address (every lane
    // reads the same 16 bytes) into a ring slot no step reads any more, so
    // every group has C copies and one wait count fits all.  Copies retire
    // in issue order, so "at most N outstanding" names exactly what landed;
    // the weight copies (from HBM) go first so that they have the longest
    // time to land before a wait covers them.
    const uint8_t *dummy = p.wp + qbase * quad_bytes;
    // weight copy i (0 <= i < CB) of K step sb: four fragments, scale dword
    auto issue_b = [&](int sb, int i) __attribute__((always_inline)) {
      const bool real = sb < S;
      uint8_t *sw = lds + TS::B_BASE + (sb % NB) * TS::B_STAGE;
      if (i < 4)
        copy16_to_lds(real ? wsrc + (size_t)sb * 4096 + i * 1024 : dummy,
                      sw + wave * 4096 + i * 1024);
      else
        copy4_to_lds(real ? (const void *)(wssrc + (size_t)sb * 64) : (const void *)dummy,
                     sw + TS::OFF_BS + wave * 256);
    };
    // copy i (0 <= i < C) of group p: the four weight fragments, the weight
    // scale dword, the activation chunks, the activation scale dword
    auto issue_one = [&](int pg, int i) __attribute__((always_inline)) {
      if (i < TS::CB) {
        issue_b(pg + D, i);
      } else {
        const int ia = i - TS::CB;
        const bool real = pg < S;
        uint8_t *st = lds + (pg % NA) * TS::A_STAGE;
        if (ia < TS::A_COPIES)
          copy16_to_lds(real ? asrc[ia] + (size_t)ROWB * pg : dummy,
                        st + (wave * TS::A_COPIES + ia) * 1024);
        else
          copy4_to_lds(real ? ssrc + 4 * pg : dummy, st + TS::OFF_AS + wave * 256);
      }
    };

    v4f acc[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[m][q] = v4f{0.f, 0.f, 0.f, 0.f};

    auto read_a = [&](const uint8_t *st, int m) __attribute__((always_inline)) {
      v8i a;
      const uint8_t *base = st + m * 16 * ROWB;
      const u32x4 lo = *reinterpret_cast<const u32x4 *>(base + aoff_lo);
      a[0] = (int)lo[0]; a[1] = (int)lo[1]; a[2] = (int)lo[2]; a[3] = (int)lo[3];
      if (FMT == 0) {
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(base + aoff_hi);
        a[4] = (int)hi[0]; a[5] = (int)hi[1]; a[6] = (int)hi[2]; a[7] = (int)hi[3];
      } else {
        a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
      }
      return a;
    };
    // the scale operands are read as single bytes, so the MFMA takes the load
    // result as it is and no VALU op waits on the read inside the sequence
    auto read_sa = [&](const uint8_t *st, int m) __attribute__((always_inline)) {
      return (int)st[TS::OFF_AS + 4 * TS::sslot(16 * m + r16) + g];
    };

    // prologue: the weight lead (steps 0 .. D-1), then groups 0 .. NA-2
#pragma unroll
    for (int sb = 0; sb < D; ++sb)
#pragma unroll
      for (int i = 0; i < TS::CB; ++i) issue_b(sb, i);
#pragma unroll
    for (int pg = 0; pg < NA - 1; ++pg)
#pragma unroll
      for (int i = 0; i < TS::C; ++i) issue_one(pg, i);
    // step 0 has landed: what may still be in flight is issued after its
    // activation copies (groups 1 .. NA-2)
    wait_vm<(NA - 2) * TS::C>();
    __syncthreads();

    for (int s = 0; s < S; ++s) {
      // the copies of group s + NA - 1 are spread over the MFMA sequence of
      // step s, so the wave never stalls on a full memory queue with the
      // matrix cores idle
      {  // inactive waves (past the last weight tile) compute on valid data and never store
        const uint8_t *st = lds + (s % NA) * TS::A_STAGE;
        const uint8_t *sw = lds + TS::B_BASE + (s % NB) * TS::B_STAGE;
        v8i b[4];
        const int sb = *reinterpret_cast<const int *>(sw + TS::OFF_BS + wave * 256 + lane * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v = *reinterpret_cast<const u32x4 *>(sw + wave * 4096 + q * 1024 +
                                                          lane * 16);
          b[q][0] = (int)v[0]; b[q][1] = (int)v[1]; b[q][2] = (int)v[2]; b[q][3] = (int)v[3];
          b[q][4] = 0; b[q][5] = 0; b[q][6] = 0; b[q][7] = 0;
        }
        // activation fragment m+1 is read from LDS while the MFMAs of m run
        v8i acur = read_a(st, 0);
        int sacur = read_sa(st, 0);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int i = m * TS::C / MT; i < (m + 1) * TS::C / MT; ++i) issue_one(s + NA - 1, i);
          v8i anext = acur;
          int sanext = sacur;
          if (m + 1 < MT) {
            anext = read_a(st, m + 1);
            sanext = read_sa(st, m + 1);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[m][q] = mfma_q<FMT>(q, acur, b[q], acc[m][q], sacur, sb);
          __builtin_amdgcn_sched_barrier(0);
          acur = anext;
          sacur = sanext;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<(NA - 2) * TS::C>();  // step s+1 has landed
      barrier_keep_copies();
    }

    if (active) {
      if (!SECOND) {
        const int j = tile0 / 4;  // unit: h columns [32j, 32j + 32)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int mrow = 16 * m + 4 * g + r;
            const size_t prow = (size_t)(row0 + min(mrow, nrows - 1));
            swiglu_requant<F, FMT>(acc[m][0][r], acc[m][1][r], acc[m][2][r], acc[m][3][r],
                                   p.a2c + prow * a2row,
                                   p.a2s + prow * (p.I / 32), j, r16);
          }
        }
      } else {
        // a padded row (loaded from the last valid row) stores the same
        // values as that row, so every store is unconditional
        float wa[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) wa[m][r] = p.wts[row0 + min(16 * m + 4 * g + r, nrows - 1)];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int mrow = min(16 * m + 4 * g + r, nrows - 1);
            float *d = p.rows + (size_t)(row0 + mrow) * p.H + 16 * (size_t)tile0 + r16;
#pragma unroll
            for (int q = 0; q < 4; ++q) d[16 * q] = wa[m][r] * acc[m][q][r];
          }
        }
      }
    }
  }
}

GemmPlan choose_plan(int T, int top_k, int E, int act) {
  // The average rows per expert decides between weight streaming (few rows)
  // and the pipelined tiled kernel.  The tiled kernel's BM covers the mean
  // plus 2.5 standard deviations of a binomial expert load, so that under
  // uniform routing nearly every expert is one m-block and its weights are
  // read once; an activation tile must fill whole 4 KiB copies (MXFP8: MT
  // even; MXFP4: MT a multiple of 4), and MT <= 10 keeps the accumulators
  // in registers.
  const long N = (long)T * top_k;
  const double avg = (double)N / E;
  if (avg < 6.0) return GemmPlan{false, 1};
  const double want = avg + 2.5 * sqrt(avg);
  if (act == MOE_ACT_MXFP8_E4M3) {
    int mt = (int)ceil(want / 16.0);
    mt = mt + (mt & 1);
    return GemmPlan{true, mt < 2 ? 2 : (mt > 10 ? 10 : mt)};
  }
  return GemmPlan{true, want <= 64.0 ? 4 : 8};
}

static KArgs make_args(const GemmArgs &a, bool second) {
  KArgs k{};
  k.T = a.T; k.top_k = a.top_k; k.E = a.E; k.H = a.H; k.I = a.I;
  k.a1c = a.a1c; k.a1s = a.a1s; k.a2c = a.a2c; k.a2s = a.a2s;
  k.perm = a.perm; k.offsets = a.offsets; k.mtoff = a.mtoff; k.mbexp = a.mbexp; k.wts = a.wts;
  k.wp = second ? a.w2p : a.w13p;
  k.wsp = reinterpret_cast<const uint32_t *>(second ? a.w2sp : a.w13sp);
  k.rows = a.rows;
  return k;
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

template <bool SECOND>
static hipError_t launch_tiled(const GemmArgs &a, const KArgs &k, hipStream_t s) {
  const unsigned grid = (unsigned)(a.num_cus / 8 * 8);  // one workgroup per CU
  const bool f8 = a.act == MOE_ACT_MXFP8_E4M3;
  if (f8) {
    switch (a.plan.mt) {
      case 2: tiled_kernel<0, 2, SECOND><<<grid, 256, 0, s>>>(k); break;
      case 4: tiled_kernel<0, 4, SECOND><<<grid, 256, 0, s>>>(k); break;
      case 6: tiled_kernel<0, 6, SECOND><<<grid, 256, 0, s>>>(k); break;
      case 8: tiled_kernel<0, 8, SECOND><<<grid, 256, 0, s>>>(k); break;
      case 10: tiled_kernel<0, 10, SECOND><<<grid, 256, 0, s>>>(k); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.plan.mt) {
      case 4: tiled_kernel<4, 4, SECOND><<<grid, 256, 0, s>>>(k); break;
      case 8: tiled_kernel<4, 8, SECOND><<<grid, 256, 0, s>>>(k); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm1(const GemmArgs &a, hipStream_t s) {
  const KArgs k = make_args(a, false);
  if (a.plan.tiled) return launch_tiled<false>(a, k, s);
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
  if (a.plan.tiled) return launch_tiled<true>(a, k, s);
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
