// gemm_common.h -- shared pieces of the grouped scaled-MFMA expert GEMMs
// (gemm_stream.hip: decode variant; gemm_tiled.hip: prefill variant).
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
// quad; the four or eight waves of a workgroup split the K steps and reduce
// in LDS.  Tiled (prefill): gemm_tiled.hip.  Both schedule persistently from
// the sort's m-block table; the padded rows of a partial m-block load the
// last valid row, compute its values again and store them to that row.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

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
  const int2 *mbrows;  // m-block mt's first sorted row and row count
  const float *wts;  // [N] routing weight of sorted row p
  const uint8_t *wp;
  const uint32_t *wsp;
  float *rows;  // [N][H] weighted GEMM2 rows (sorted order; layout by combine)
  int combine;  // moe_combine transport
  // fused launch only: the down weights beside the gate/up ones in wp/wsp,
  // and the zeroed sync region (kSyncHead)
  const uint8_t *w2p;
  const uint32_t *w2sp;
  int32_t *sync;
  // token-major GEMM2 only: routing by assignment and the output
  const int32_t *ids, *inv;
  const float *wts_a;
  uint16_t *y;
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A2 layout.  The SwiGLU codes GEMM1 writes and GEMM2 reads are stored
// K-step-major: K step s of GEMM2 (columns [128 s, 128 s + 128) of I) holds
// the N = T * top_k sorted rows' bytes of that step one after another --
// codes [I/128][N][128] (E4M3) or [I/128][N][64] (packed E2M1), scales
// [I/128][N][4] (the step's four E8M0 block bytes) -- so the rows of an
// m-block, which GEMM2 reads one step at a time, are one contiguous run per
// step.  (From row-major rows the tiled GEMM2's copies of a step gathered
// 16-row pieces and one scale dword per row from separate cache lines:
// 8.7% slower per GEMM2 at A4W4, T = 16384.)
template <int FMT>
__device__ __forceinline__ size_t a2c_at(size_t row, int s, size_t N) {
  return ((size_t)s * N + row) * (FMT == 0 ? 128 : 64);
}
__device__ __forceinline__ size_t a2s_at(size_t row, int s, size_t N) {
  return ((size_t)s * N + row) * 4;
}

// A weight fragment (16 bytes of a lane) or scale dword of the stream GEMMs,
// loaded with the non-temporal hint: each is read once per call, and
// streaming them past the caches leaves those to the activation rows
// (measured on the 7168 x 3072 decode layer: -5 to -10% per call at
// T = 2 .. 64, GEMM1 at T = 64 from 939 to 860 us).
__device__ __forceinline__ u32x4 load_weights16(const uint8_t *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ int load_weight_scales(const uint32_t *p) {
  return (int)__builtin_nontemporal_load(p);
}


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

// silu(g) = g / (1 + exp(-g)) in FP32 with the library exponential (about one
// ulp) and a correctly rounded division, so h tracks an FP32 evaluation of
// the same formula to an ulp or two (the hardware exp2 of -g * log2(e) and an
// approximate reciprocal were several ulps off for |g| of a few units, which
// moved requantised A2 codes across rounding boundaries more often); for very
// negative g the exponential overflows to inf and silu goes to (-)0.
__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// Cross-lane moves within 16-lane rows (DPP, no LDS traffic).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  // all rows and banks enabled: every lane is written, so no old value is kept
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// 16-lane row maximum of NR independent values (quad_perm [1,0,3,2],
// [2,3,0,1], then row_half_mirror and row_mirror), the NR chains advanced in
// lock-step so that each DPP read follows other chains' work instead of
// waiting out its own producer (a DPP operand written by the previous VALU
// op needs wait states).
template <int NR>
__device__ __forceinline__ void row16_max_n(uint32_t (&v)[NR]) {
#pragma unroll
  for (int i = 0; i < NR; ++i) v[i] = max(v[i], dpp<0xB1>(v[i]));
#pragma unroll
  for (int i = 0; i < NR; ++i) v[i] = max(v[i], dpp<0x4E>(v[i]));
#pragma unroll
  for (int i = 0; i < NR; ++i) v[i] = max(v[i], dpp<0x141>(v[i]));
#pragma unroll
  for (int i = 0; i < NR; ++i) v[i] = max(v[i], dpp<0x140>(v[i]));
}

// A byte store; COH: a device-coherent one (an agent-scope relaxed atomic
// store, which writes through to the level all XCDs share), for data another
// workgroup of the same launch reads.
template <bool COH>
__device__ __forceinline__ void store_u8(uint8_t *p, uint32_t v) {
  if (COH)
    __hip_atomic_store(p, (uint8_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = (uint8_t)v;
}

// GEMM1 epilogue for NR accumulator rows at once: for row i, lane c = l%16
// holds gate/up columns 32j + c (lo) and 32j + 16 + c (hi) of one token row.
// The element codes (clo: column c, chi: column 16 + c) and block exponent
// of NR rows' h = silu(gate) * up blocks (amax over the 16 lanes of a row).
template <class F, int NR>
__device__ __forceinline__ void swiglu_codes_n(const float (&glo)[NR], const float (&ghi)[NR],
                                               const float (&ulo)[NR], const float (&uhi)[NR],
                                               uint32_t (&clo)[NR], uint32_t (&chi)[NR],
                                               int (&X)[NR]) {
  float hlo[NR], hhi[NR];
  uint32_t am[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    hlo[i] = silu(glo[i]) * ulo[i];
    hhi[i] = silu(ghi[i]) * uhi[i];
    am[i] = max(f32_bits(hlo[i]) & 0x7fffffffu, f32_bits(hhi[i]) & 0x7fffffffu);
  }
  row16_max_n<NR>(am);
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    X[i] = block_exponent<F>(am[i]);
    encode_pair<F>(hlo[i], hhi[i], X[i], clo[i], chi[i]);
  }
}

// h = silu(gate) * up; the 32 h values of the row form one 1x32 block (amax
// over the 16 lanes), requantised and stored as block j of sorted row rows[i]
// of A2 (N rows; block j is block j % 4 of K step j / 4).  All lanes call
// and store: the two lanes of an E2M1 byte both write it whole, all 16 lanes
// write the scale byte, and a padded row (computed from the last valid row's
// data) rewrites that row's values, so no store needs a branch.
template <class F, int FMT, int NR, bool COH = false>
__device__ __forceinline__ void swiglu_requant_n(const float (&glo)[NR], const float (&ghi)[NR],
                                                 const float (&ulo)[NR], const float (&uhi)[NR],
                                                 uint8_t *a2c, uint8_t *a2s,
                                                 const size_t (&rows)[NR], size_t N, int j, int c) {
  uint32_t clo[NR], chi[NR];
  int X[NR];
  swiglu_codes_n<F, NR>(glo, ghi, ulo, uhi, clo, chi, X);
  const int s = j >> 2, jb = j & 3;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    uint8_t *cr = a2c + a2c_at<FMT>(rows[i], s, N);
    if (FMT == 0) {
      store_u8<COH>(cr + 32 * jb + c, clo[i]);
      store_u8<COH>(cr + 32 * jb + 16 + c, chi[i]);
    } else {
      const uint32_t plo = dpp<0xB1>(clo[i]);  // code of lane c ^ 1
      const uint32_t phi = dpp<0xB1>(chi[i]);
      const bool odd = c & 1;
      store_u8<COH>(cr + 16 * jb + c / 2, odd ? (plo | (clo[i] << 4)) : (clo[i] | (plo << 4)));
      store_u8<COH>(cr + 16 * jb + 8 + c / 2, odd ? (phi | (chi[i] << 4)) : (chi[i] | (phi << 4)));
    }
    store_u8<COH>(a2s + a2s_at(rows[i], s, N) + jb, (uint32_t)(X[i] + 127));
  }
}

template <int FMT>
struct ActFmt;
template <>
struct ActFmt<0> { using F = E4M3; };
template <>
struct ActFmt<4> { using F = E2M1; };

inline KArgs make_args(const GemmArgs &a, bool second) {
  KArgs k{};
  k.T = a.T; k.top_k = a.top_k; k.E = a.E; k.H = a.H; k.I = a.I;
  k.a1c = a.a1c; k.a1s = a.a1s; k.a2c = a.a2c; k.a2s = a.a2s;
  k.perm = a.perm; k.offsets = a.offsets; k.mtoff = a.mtoff; k.mbexp = a.mbexp; k.wts = a.wts;
  k.mbrows = reinterpret_cast<const int2 *>(a.mbrows);
  k.wp = second ? a.w2p : a.w13p;
  k.wsp = reinterpret_cast<const uint32_t *>(second ? a.w2sp : a.w13sp);
  k.rows = a.rows;
  k.combine = a.combine;
  k.w2p = a.w2p;
  k.w2sp = reinterpret_cast<const uint32_t *>(a.w2sp);
  k.sync = a.sync;
  k.ids = a.ids; k.inv = a.inv; k.wts_a = a.wts_a; k.y = a.y;
  return k;
}

// GEMM2 epilogue store of NR row pieces: for piece i, lane c = l%16 of a row
// group holds the weighted outputs t[i][q] of sorted row prow[i], columns
// col0 + c + 16q (q = 0..3; col0 a multiple of 64), written in the row
// transport's format.  All 16 lanes of the row group call (the MXFP8
// transport's block amax is a DPP max across them); blocks of 32 columns are
// (q0, q1) and (q2, q3).
template <int NR>
__device__ __forceinline__ void stage_store_n(const KArgs &p, const size_t (&prow)[NR], int col0,
                                              int c, const float (&t)[NR][4]) {
  const size_t H = (size_t)p.H;
  if (p.combine == MOE_COMBINE_FP32) {
    // non-temporal: the combine reads the rows only after the whole GEMM2
    // (per call, against plain stores: 5120 x 640 T = 32768 -2.9%, GEMM2
    // -3.6% and the combine -5%; 7168 x 3072 A4W4 T = 16384 -0.5%; decode
    // T = 64 -0.8%)
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      float *d = p.rows + prow[i] * H + col0 + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) __builtin_nontemporal_store(t[i][q], d + 16 * q);
    }
  } else if (p.combine == MOE_COMBINE_BF16) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      uint16_t *d = reinterpret_cast<uint16_t *>(p.rows) + prow[i] * H + col0 + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) d[16 * q] = f32_to_bf16(t[i][q]);
    }
  } else {
    uint8_t *base = reinterpret_cast<uint8_t *>(p.rows);
    const size_t scale0 = (size_t)p.T * p.top_k * H + col0 / 32;
    uint32_t am[2 * NR];
#pragma unroll
    for (int i = 0; i < NR; ++i)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        am[2 * i + b] = max(f32_bits(t[i][2 * b]) & 0x7fffffffu,
                            f32_bits(t[i][2 * b + 1]) & 0x7fffffffu);
    row16_max_n<2 * NR>(am);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      uint8_t *d = base + prow[i] * H + col0 + c;
      uint8_t *sc = base + scale0 + prow[i] * (H / 32);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int X = block_exponent<E4M3>(am[2 * i + b]);
        uint32_t c0, c1;
        encode_pair<E4M3>(t[i][2 * b], t[i][2 * b + 1], X, c0, c1);
        d[32 * b] = (uint8_t)c0;
        d[32 * b + 16] = (uint8_t)c1;
        sc[b] = (uint8_t)(X + 127);  // every lane writes the same byte
      }
    }
  }
}

// 4 x 4 byte transpose across the four lanes of a quad (lanes 4k .. 4k+3;
// j = lane & 3) by two DPP exchanges (lanes j ^ 2, then j ^ 1): on entry byte
// r of lane j's dword is M[r][j], on exit M[j][r].
__device__ __forceinline__ uint32_t quad_transpose_bytes(uint32_t d, int j) {
  const uint32_t x = dpp<0x4E>(d);
  d = (j & 2) == 0 ? (d & 0xffffu) | (x << 16) : (x >> 16) | (d & 0xffff0000u);
  const uint32_t y = dpp<0xB1>(d);
  return (j & 1) == 0 ? (d & 0x00ff00ffu) | ((y & 0x00ff00ffu) << 8)
                      : ((y >> 8) & 0x00ff00ffu) | (d & 0xff00ff00u);
}

// GEMM1 epilogue with dword stores (MXFP8 A2): for the four rows 4g + r of
// a row group, lane c = 4k + jq holds the codes of columns 32 unit + c and
// 32 unit + 16 + c; after a byte transpose in each quad, lane (k, jq) holds
// row 4g + jq's codes of columns 4k .. 4k+3 (and 16 + 4k ..), stored as two
// dwords, plus the row's scale byte (the four lanes of a row write the same
// byte).  crow / srow: the lane's row's A2 codes and scale dword of the K
// step holding the unit; jb = unit % 4, the unit's block in that step.
__device__ __forceinline__ void swiglu_store_f8_t(const float (&glo)[4], const float (&ghi)[4],
                                                  const float (&ulo)[4], const float (&uhi)[4],
                                                  uint8_t *crow, uint8_t *srow, int jb, int c) {
  uint32_t clo[4], chi[4];
  int X[4];
  swiglu_codes_n<E4M3, 4>(glo, ghi, ulo, uhi, clo, chi, X);
  const int jq = c & 3;
  const uint32_t lo = quad_transpose_bytes(clo[0] | (clo[1] << 8) | (clo[2] << 16) | (clo[3] << 24), jq);
  const uint32_t hi = quad_transpose_bytes(chi[0] | (chi[1] << 8) | (chi[2] << 16) | (chi[3] << 24), jq);
  const int Xr = jq == 0 ? X[0] : jq == 1 ? X[1] : jq == 2 ? X[2] : X[3];
  *reinterpret_cast<uint32_t *>(crow + 32 * jb + 4 * (c >> 2)) = lo;
  *reinterpret_cast<uint32_t *>(crow + 32 * jb + 16 + 4 * (c >> 2)) = hi;
  srow[jb] = (uint8_t)(Xr + 127);
}

// Tiled (prefill) variant, in gemm_tiled.hip.
hipError_t launch_tiled_gemm1(const GemmArgs &a, const KArgs &k, hipStream_t s);
hipError_t launch_tiled_gemm2(const GemmArgs &a, const KArgs &k, hipStream_t s);

}  // namespace moe
