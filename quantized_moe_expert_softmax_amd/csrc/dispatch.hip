// dispatch.hip -- routing, expert sort, activation quantisation and the
// FP32 top-k combine of the MoE layer (gfx950).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"
#include "mx_device.h"

namespace moe {

// ---------------------------------------------------------------------------
// Step 1: top-k softmax routing ("[HIP] gfx950 A8W4 fused_moe configs for
// DSv4.1 TP-sharded experts", Changes: the top-k softmax kernel).  One wave
// per token: each lane holds E/64 logits in registers; top_k rounds of a
// wave-wide arg-max (larger logit first, equal logits by lower index) pick
// the experts; the weights are exp(l_j - max) normalised over the picks,
// which equals the full softmax renormalised over the picks (the softmax
// denominator over all E cancels).
// ---------------------------------------------------------------------------
// Lane l of a wave holds logits l, l + 64, ... of one token row.  Positions
// past E load logit E - 1 (route_values ignores them): every load is
// unconditional, so all NV are in flight at once (a load under a per-lane
// branch was waited for before the next one issued).
template <int NV>
__device__ __forceinline__ void load_logits(const float *__restrict__ row, int E, int lane,
                                            float v[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = row[min(lane + 64 * i, E - 1)];
}

// Selection key of a logit: its float bits mapped to an unsigned order
// (negative values flipped whole, positive ones above them), with -0 taken
// as +0 (a strict logit compare treats them as equal).  Keys of real logits
// are at least 1 (only one NaN pattern maps to 0, raised to 1), so 0 marks
// an expert that is taken or past E.
__device__ __forceinline__ uint32_t route_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);  // -0 + 0 = +0
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return o > 1u ? o : 1u;
}
__device__ __forceinline__ float route_key_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// The wave's largest key, in every lane, with VALU cross-lane moves only:
// DPP within each 16-lane row (quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror: every lane then holds its row's largest
// key), then v_permlane16_swap (rows 0 with 1, 2 with 3) and
// v_permlane32_swap (the two halves).  (A __shfl_xor butterfly is a chain of
// dependent ds_bpermute round trips through LDS, about 0.6 us per pick.)
__device__ __forceinline__ uint32_t wave_max_key(uint32_t key) {
  auto dpp_step = [&](auto ctrl) __attribute__((always_inline)) {
    constexpr int C = decltype(ctrl)::value;
    const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)key, C, 0xF, 0xF, false);
    key = o > key ? o : key;
  };
  dpp_step(std::integral_constant<int, 0xB1>{});
  dpp_step(std::integral_constant<int, 0x4E>{});
  dpp_step(std::integral_constant<int, 0x141>{});
  dpp_step(std::integral_constant<int, 0x140>{});
  {
    const auto r = __builtin_amdgcn_permlane16_swap(key, key, false, false);
    key = r[0] > r[1] ? r[0] : r[1];
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(key, key, false, false);
    key = r[0] > r[1] ? r[0] : r[1];
  }
  return key;
}

// One wave routes the token whose logits it holds (load_logits); lanes <
// top_k write ids[j], w[j].  The whole wave must be active.  A pick is the
// wave's largest 32-bit key M; of the experts holding M the lowest index
// wins: the first register position i (ascending) at which any lane holds
// M, then the lowest such lane (expert lane + 64 i), both read from ballots.
template <int NV>
__device__ __forceinline__ void route_values(const float v[NV], int E, int top_k, int lane,
                                             int32_t *__restrict__ ids, float *__restrict__ wts) {
  uint32_t key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = lane + 64 * i < E ? route_key(v[i]) : 0u;
  float sel0 = 0.0f, mine = 0.0f;  // the largest logit; lane j: pick j's logit
  int myid = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < top_k) {
      uint32_t m = key[0];
#pragma unroll
      for (int i = 1; i < NV; ++i) m = key[i] > m ? key[i] : m;
      const uint32_t M = __builtin_amdgcn_readfirstlane(wave_max_key(m));
      int wl = -1, wi = 0;  // winning lane and register position
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const uint64_t b = __ballot(key[i] == M);
        if (wl < 0 && b != 0) {
          wl = __builtin_ctzll(b);
          wi = i;
        }
      }
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i == wi && lane == wl) key[i] = 0u;
      const float val = route_key_value(M);
      if (j == 0) sel0 = val;
      if (j == lane) {
        mine = val;
        myid = wl + 64 * wi;
      }
    }
  }
  // weights: exp(l_j - l_0) / sum_j' exp(l_j' - l_0); l_0 is the largest logit.
  // Evaluated in double (the difference of two floats is exact there), then
  // rounded once to float: lane j evaluates pick j's exponential, and every
  // lane adds them in slot order.
  const double ex = lane < top_k ? exp((double)mine - (double)sel0) : 0.0;
  double sum = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < top_k) {
      const uint64_t b = __double_as_longlong(ex);
      const uint64_t r = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), j)
                          << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, j);
      sum += __longlong_as_double((long long)r);
    }
  }
  if (lane < top_k) {
    ids[lane] = myid;
    wts[lane] = (float)(ex / sum);
  }
}

template <int NV>
__global__ __launch_bounds__(256) void route_kernel(const float *__restrict__ logits, int T, int E,
                                                    int top_k, int32_t *__restrict__ ids,
                                                    float *__restrict__ wts) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * 4 + wave;
  if (t >= T) return;  // wave-uniform; no barriers below
  float v[NV];
  load_logits<NV>(logits + t * E, E, lane, v);
  route_values<NV>(v, E, top_k, lane, ids + t * top_k, wts + t * top_k);
}

hipError_t launch_route(const float *logits, int T, int E, int top_k, int32_t *ids, float *w,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(T, 4)), block(256);
  const int nv = ceil_div(E, 64);
#define ROUTE_CASE(NV_)                                                                   \
  case NV_:                                                                               \
    route_kernel<NV_><<<grid, block, 0, s>>>(logits, T, E, top_k, ids, w);                \
    break;
  switch (nv) {
    ROUTE_CASE(1) ROUTE_CASE(2) ROUTE_CASE(3) ROUTE_CASE(4) ROUTE_CASE(5) ROUTE_CASE(6)
    ROUTE_CASE(7) ROUTE_CASE(8) ROUTE_CASE(9) ROUTE_CASE(10) ROUTE_CASE(11) ROUTE_CASE(12)
    ROUTE_CASE(13) ROUTE_CASE(14) ROUTE_CASE(15) ROUTE_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef ROUTE_CASE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Step 2: dispatch as an on-device, deterministic counting sort of the
// assignments a = t*top_k + j by expert ("add A4W4 and FP8 P2P transport
// support to MegaMoE", Technical Details: dispatch of the quantised payloads;
// on one device the experts all live here, so dispatch is a permutation).
//   hist:    per 256-token block, the number of assignments of each expert
//   scan:    per expert, exclusive prefix over blocks (relative to the
//            expert's first row); counts, offsets (exclusive prefix over
//            experts), the prefix of bm-row m-blocks per expert and the
//            expert of every m-block, which the GEMMs schedule from
//   scatter: within a block, the rank of a token among the tokens routed to
//            the same expert comes from 64-bit per-wave masks (LDS atomic
//            OR is order-free; popcount of the lanes below gives the rank),
//            so the order within an expert is ascending token, i.e.
//            ascending a (a token's top_k experts are distinct).
// ---------------------------------------------------------------------------
// The slot count K is a template argument: a token's K ids are loaded
// together (from a clamped token row, so the loads are unconditional) before
// the first is used.
template <int K>
__global__ __launch_bounds__(256) void sort_hist_kernel(const int32_t *__restrict__ ids, int T,
                                                        int E, int32_t *__restrict__ hist) {
  extern __shared__ int32_t lhist[];
  for (int e = threadIdx.x; e < E; e += 256) lhist[e] = 0;
  const long t = (long)blockIdx.x * kSortBlock + threadIdx.x;
  const long tc = t < T ? t : (long)T - 1;
  uint32_t id[K];
#pragma unroll
  for (int j = 0; j < K; ++j) id[j] = (uint32_t)ids[tc * K + j];
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (id[j] < (uint32_t)E) atomicAdd(&lhist[id[j]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(long)blockIdx.x * E + e] = lhist[e];
}

// Inclusive prefix sum of x over the wave's 64 lanes with VALU moves only:
// DPP row_shr 1, 2, 4, 8 within each 16-lane row (a lane with no source lane
// in its row adds 0), then each row adds the totals of the rows before it
// (lanes 15, 31, 47 read with readlane).  (The __shfl_up ladder it replaces
// is six dependent ds_bpermute round trips per value.)
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// The m-blocks of an expert with c rows from sorted row r0: m-block i (table
// entry mb0 + i) holds rows [r0 + bm i, + min(bm, c - bm i)).  Writes the
// expert of each and, when mbrows is not null, its first row and row count
// (one load gives a GEMM item both; from offsets they are a second
// dependent load).
__device__ __forceinline__ void write_mblocks(int32_t *__restrict__ mbexp,
                                              int32_t *__restrict__ mbrows, int e, int mb0,
                                              int m, int r0, int c, int bm) {
  for (int i = 0; i < m; ++i) {
    mbexp[mb0 + i] = e;
    if (mbrows)
      reinterpret_cast<int2 *>(mbrows)[mb0 + i] = make_int2(r0 + bm * i, min(bm, c - bm * i));
  }
}

__global__ __launch_bounds__(1024) void sort_scan_kernel(int32_t *__restrict__ hist, int nb, int E,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ mtoff,
                                                         int32_t *__restrict__ mbexp,
                                                         int32_t *__restrict__ mbrows, int bm,
                                                         int32_t *__restrict__ sync, int nsync) {
  __shared__ int32_t sc[1024];
  __shared__ int32_t sm[1024];
  __shared__ int32_t wtot[16][2];
  const int e = threadIdx.x;
  for (int i = e; i < nsync; i += 1024) sync[i] = 0;
  int run = 0;
  if (e < E) {
    // the blocks' counts are loaded 16 at a time so that the loads overlap
    // (one dependent L2 round trip per block would dominate at large T)
    constexpr int U = 16;
    int b = 0;
    for (; b + U <= nb; b += U) {
      int v[U];
#pragma unroll
      for (int i = 0; i < U; ++i) v[i] = hist[(long)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        hist[(long)(b + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; b < nb; ++b) {
      const int v = hist[(long)b * E + e];
      hist[(long)b * E + e] = run;
      run += v;
    }
    counts[e] = run;
  }
  const int c = e < E ? run : 0;
  const int m = e < E ? (run + bm - 1) / bm : 0;
  // inclusive prefix sums over the experts: within each wave, then plus the
  // totals of the lower waves
  const int wave = e >> 6, lane = e & 63;
  int ic = wave_inclusive_scan(c, lane), im = wave_inclusive_scan(m, lane);
  if (lane == 63) {
    wtot[wave][0] = ic;
    wtot[wave][1] = im;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    ic += wtot[w][0];
    im += wtot[w][1];
  }
  sc[e] = ic;
  sm[e] = im;
  if (e < E) {
    const int base = sc[e] - c;
    offsets[e] = base;
    mtoff[e] = sm[e] - m;
    if (e == E - 1) {
      offsets[E] = sc[e];
      mtoff[E] = sm[e];
    }
    write_mblocks(mbexp, mbrows, e, sm[e] - m, m, base, c, bm);
  }
}

template <int K>
__global__ __launch_bounds__(256) void sort_scatter_kernel(const int32_t *__restrict__ ids, int T,
                                                           int E,
                                                           const int32_t *__restrict__ base,
                                                           const int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ perm,
                                                           int32_t *__restrict__ inv,
                                                           const float *__restrict__ w,
                                                           float *__restrict__ wsorted) {
  extern __shared__ unsigned long long masks[];  // [4 waves][E]
  for (int i = threadIdx.x; i < 4 * E; i += 256) masks[i] = 0ull;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * kSortBlock + threadIdx.x;
  const long tc = t < T ? t : (long)T - 1;
  const unsigned long long bit = 1ull << lane;
  uint32_t id[K];
  float wt[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    id[j] = (uint32_t)ids[tc * K + j];
    wt[j] = wsorted ? w[tc * K + j] : 0.0f;
  }
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (id[j] < (uint32_t)E) atomicOr(&masks[wave * E + id[j]], bit);
  }
  // each slot's expert start row (all loads issued before the first use;
  // ids past E read expert 0's and are skipped below)
  int32_t start[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const uint32_t e = id[j] < (uint32_t)E ? id[j] : 0u;
    start[j] = offsets[e] + base[(long)blockIdx.x * E + e];
  }
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t e = id[j];
      if (e >= (uint32_t)E) continue;
      int r = __popcll(masks[wave * E + e] & (bit - 1ull));
      for (int v = 0; v < wave; ++v) r += __popcll(masks[v * E + e]);
      const int32_t pos = start[j] + r;
      perm[pos] = (int32_t)(t * K + j);
      inv[t * K + j] = pos;
      if (wsorted) wsorted[pos] = wt[j];
    }
  }
}

hipError_t launch_sort_hist(const int32_t *ids, int T, int E, int top_k, int32_t *hist, int nb,
                            hipStream_t s) {
  switch (top_k) {
#define HIST_CASE(K) \
    case K: sort_hist_kernel<K><<<nb, 256, (size_t)E * 4, s>>>(ids, T, E, hist); break;
    HIST_CASE(1) HIST_CASE(2) HIST_CASE(3) HIST_CASE(4)
    HIST_CASE(5) HIST_CASE(6) HIST_CASE(7) HIST_CASE(8)
#undef HIST_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sort_scan(int32_t *hist, int nb, int E, int32_t *counts, int32_t *offsets,
                            int32_t *mtoff, int32_t *mbexp, int32_t *mbrows, int bm,
                            int32_t *sync, int nsync, hipStream_t s) {
  sort_scan_kernel<<<1, 1024, 0, s>>>(hist, nb, E, counts, offsets, mtoff, mbexp, mbrows, bm,
                                      sync, nsync);
  return hipGetLastError();
}

hipError_t launch_sort_scatter(const int32_t *ids, int T, int E, int top_k, const int32_t *hist,
                               const int32_t *offsets, int32_t *perm, int32_t *inv,
                               const float *w, float *wsorted, hipStream_t s) {
  const int nb = ceil_div(T, kSortBlock);
  switch (top_k) {
#define SCATTER_CASE(K)                                                                  \
    case K:                                                                              \
      sort_scatter_kernel<K><<<nb, 256, (size_t)E * 4 * 8, s>>>(ids, T, E, hist, offsets, \
                                                                perm, inv, w, wsorted);  \
      break;
    SCATTER_CASE(1) SCATTER_CASE(2) SCATTER_CASE(3) SCATTER_CASE(4)
    SCATTER_CASE(5) SCATTER_CASE(6) SCATTER_CASE(7) SCATTER_CASE(8)
#undef SCATTER_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Step 3: 1x32 MX quantisation of BF16 rows (FlyDSL #972 Technical Details:
// BF16 activations to MXFP4 -- or MXFP8 on the A8W4 path -- with per-1x32
// E8M0 scales, once per token before dispatch).  One thread per 32-element
// block: amax over the bit patterns, block exponent, RNE encode.
// ---------------------------------------------------------------------------
// 1x32 block b of the row-major bf16 matrix x (the element codes by the
// scaled conversion instructions, encode_pair).
template <class F>
__device__ __forceinline__ void quant_block(const uint16_t *__restrict__ x, long b,
                                            uint8_t *__restrict__ codes,
                                            uint8_t *__restrict__ scales) {
  const uint4 *src = reinterpret_cast<const uint4 *>(x + b * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 q = src[i];
    w[4 * i + 0] = q.x;
    w[4 * i + 1] = q.y;
    w[4 * i + 2] = q.z;
    w[4 * i + 3] = q.w;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t lo = (w[i] << 16) & 0x7fffffffu, hi = w[i] & 0x7fff0000u;
    amax = max(amax, max(lo, hi));
  }
  const int X = block_exponent<F>(amax);
  if (F::kBits == 8) {
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t c0, c1, c2, c3;
      encode_pair<F>(__uint_as_float(w[2 * i] << 16), __uint_as_float(w[2 * i] & 0xffff0000u), X,
                     c0, c1);
      encode_pair<F>(__uint_as_float(w[2 * i + 1] << 16),
                     __uint_as_float(w[2 * i + 1] & 0xffff0000u), X, c2, c3);
      out[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(codes + b * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  } else {
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t d = 0;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t word = w[4 * i + h];
        uint32_t c0, c1;
        encode_pair<F>(__uint_as_float(word << 16), __uint_as_float(word & 0xffff0000u), X, c0, c1);
        d |= (c0 | (c1 << 4)) << (8 * h);
      }
      out[i] = d;
    }
    *reinterpret_cast<uint4 *>(codes + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  }
  scales[b] = (uint8_t)(X + 127);
}

template <class F>
__global__ __launch_bounds__(256) void quant_kernel(const uint16_t *__restrict__ x, long nblocks,
                                                    uint8_t *__restrict__ codes,
                                                    uint8_t *__restrict__ scales) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;
  if (b < nblocks) quant_block<F>(x, b, codes, scales);
}

hipError_t launch_quant(const uint16_t *x, long rows, int K, int act, uint8_t *codes,
                        uint8_t *scales, hipStream_t s) {
  const long nblocks = rows * (K / 32);
  if (nblocks == 0) return hipSuccess;
  const unsigned grid = (unsigned)((nblocks + 255) / 256);
  if (act == MOE_ACT_MXFP8_E4M3)
    quant_kernel<E4M3><<<grid, 256, 0, s>>>(x, nblocks, codes, scales);
  else
    quant_kernel<E2M1><<<grid, 256, 0, s>>>(x, nblocks, codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Steps 1-3 in one launch for T <= kSortBlock tokens, where separate launches
// would cost more than the work: workgroup 0 routes every token (one wave per
// token; the forward does so up to kFrontMaxT tokens) or, with null logits,
// takes the ids and weights the router kernel wrote, and sorts the
// assignments exactly as the hist/scan/scatter kernels do for a single sort
// block; workgroups 1.. quantise the token rows.  The outputs are the same as
// those kernels' outputs.
// ---------------------------------------------------------------------------
template <int NV>
__global__ __launch_bounds__(1024) void front_kernel(FrontArgs p) {
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    const long nblocks = (long)p.T * (p.H / 32);
    const long stride = (long)(gridDim.x - 1) * 1024;
    for (long b = (long)(blockIdx.x - 1) * 1024 + tid; b < nblocks; b += stride) {
      if (p.act == MOE_ACT_MXFP8_E4M3)
        quant_block<E4M3>(p.x, b, p.codes, p.scales);
      else
        quant_block<E2M1>(p.x, b, p.codes, p.scales);
    }
    return;
  }
  __shared__ int32_t sid[kSortBlock * 8];
  __shared__ float sw[kSortBlock * 8];
  __shared__ int32_t cnt[1024], sc[1024], sm[1024];
  __shared__ int32_t wtot[16][2];
  __shared__ unsigned long long masks[4][1024];
  const int wave = tid >> 6, lane = tid & 63;
  const int T = p.T, E = p.E, k = p.top_k, N = T * k;
  for (int i = tid; i < p.nsync; i += 1024) p.sync[i] = 0;
  for (int e = tid; e < E; e += 1024) {
    cnt[e] = 0;
    masks[0][e] = 0ull; masks[1][e] = 0ull; masks[2][e] = 0ull; masks[3][e] = 0ull;
  }
  if (p.logits) {
    // wave w routes tokens w, w + 16, ...; the logits of four of them are
    // loaded before the first is routed
    for (int t0 = wave; t0 < T; t0 += 64) {
      float v[4][NV];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (t0 + 16 * u < T) load_logits<NV>(p.logits + (long)(t0 + 16 * u) * E, E, lane, v[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + 16 * u;
        if (t < T) route_values<NV>(v[u], E, k, lane, sid + t * k, sw + t * k);
      }
    }
  } else {
    // routed by the router kernel earlier on the stream
    for (int a = tid; a < N; a += 1024) {
      sid[a] = p.ids[a];
      sw[a] = p.wts[a];
    }
  }
  __syncthreads();
  for (int a = tid; a < N; a += 1024) {
    if (p.logits) {
      p.ids[a] = sid[a];
      p.wts[a] = sw[a];
    }
    atomicAdd(&cnt[sid[a]], 1);
  }
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  const int m = (c + p.bm - 1) / p.bm;
  // inclusive prefix sums over the experts: within each wave, then plus the
  // totals of the lower waves
  int ic = wave_inclusive_scan(c, lane), im = wave_inclusive_scan(m, lane);
  if (lane == 63) {
    wtot[wave][0] = ic;
    wtot[wave][1] = im;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    ic += wtot[w][0];
    im += wtot[w][1];
  }
  sc[tid] = ic;
  sm[tid] = im;
  if (tid < E) {
    p.counts[tid] = c;
    p.offsets[tid] = sc[tid] - c;
    p.mtoff[tid] = sm[tid] - m;
    if (tid == E - 1) {
      p.offsets[E] = sc[tid];
      p.mtoff[E] = sm[tid];
    }
    write_mblocks(p.mbexp, p.mbrows, tid, sm[tid] - m, m, sc[tid] - c, c, p.bm);
  }
  const unsigned long long bit = 1ull << lane;
  if (tid < T)
    for (int j = 0; j < k; ++j) atomicOr(&masks[wave][sid[tid * k + j]], bit);
  __syncthreads();
  if (tid < T) {
    for (int j = 0; j < k; ++j) {
      const int a = tid * k + j, e = sid[a];
      int r = __popcll(masks[wave][e] & (bit - 1ull));
      for (int w = 0; w < wave; ++w) r += __popcll(masks[w][e]);
      const int pos = sc[e] - cnt[e] + r;
      p.perm[pos] = a;
      p.inv[a] = pos;
      p.wsorted[pos] = sw[a];
    }
  }
}

// Steps 1-3 for decode batches (T <= kFrontMaxT, so T * top_k <= 128): one
// 256-thread workgroup routes every token (one wave per token), counts the
// assignments per expert in LDS, turns the counts into offsets, m-block
// prefixes and the m-block table with one wave-level scan per wave (each
// thread owns four consecutive experts) and three barriers, and ranks each
// assignment among the lower assignments of its expert (at most 127 LDS
// compares); workgroups 1.. quantise the token rows.  The same outputs as the
// separate kernels (and front_kernel), with far fewer block-wide steps than
// front_kernel's 1024-wide scans, which the decode sizes do not need.
template <int NV, int BS>
__global__ __launch_bounds__(BS) void front_small_kernel(FrontArgs p) {
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    const long nblocks = (long)p.T * (p.H / 32);
    const long stride = (long)(gridDim.x - 1) * BS;
    for (long b = (long)(blockIdx.x - 1) * BS + tid; b < nblocks; b += stride) {
      if (p.act == MOE_ACT_MXFP8_E4M3)
        quant_block<E4M3>(p.x, b, p.codes, p.scales);
      else
        quant_block<E2M1>(p.x, b, p.codes, p.scales);
    }
    return;
  }
  __shared__ int32_t sid[kFrontMaxT * 8];
  __shared__ float sw[kFrontMaxT * 8];
  __shared__ int32_t base[1024];  // per expert: count, then first sorted row
  __shared__ int32_t wsum[BS / 64][2];
  const int wave = tid >> 6, lane = tid & 63;
  const int T = p.T, E = p.E, k = p.top_k, N = T * k;
  for (int i = tid; i < p.nsync; i += BS) p.sync[i] = 0;
  for (int e = tid; e < E; e += BS) base[e] = 0;
  // wave w routes tokens w, w + BS / 64, ...
  for (int t = wave; t < T; t += BS / 64) {
    float v[NV];
    load_logits<NV>(p.logits + (long)t * E, E, lane, v);
    route_values<NV>(v, E, k, lane, sid + t * k, sw + t * k);
  }
  __syncthreads();
  for (int a = tid; a < N; a += BS) {
    p.ids[a] = sid[a];
    p.wts[a] = sw[a];
    atomicAdd(&base[sid[a]], 1);
  }
  __syncthreads();
  // exclusive prefix sums of the counts and of the m-blocks per expert (the
  // first 256 threads own four experts each, E <= 1024; the others scan zeros)
  int c[4], m[4], lc = 0, lm = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    c[i] = e < E ? base[e] : 0;
    m[i] = (c[i] + p.bm - 1) / p.bm;
    lc += c[i];
    lm += m[i];
  }
  const int ic = wave_inclusive_scan(lc, lane), im = wave_inclusive_scan(lm, lane);
  if (lane == 63) {
    wsum[wave][0] = ic;
    wsum[wave][1] = im;
  }
  __syncthreads();
  int oc = ic - lc, om = im - lm;
  for (int w = 0; w < wave; ++w) {
    oc += wsum[w][0];
    om += wsum[w][1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * tid + i;
    if (e < E) {
      p.counts[e] = c[i];
      p.offsets[e] = oc;
      p.mtoff[e] = om;
      write_mblocks(p.mbexp, p.mbrows, e, om, m[i], oc, c[i], p.bm);
      base[e] = oc;
    }
    oc += c[i];
    om += m[i];
  }
  if (4 * tid <= E - 1 && E - 1 < 4 * tid + 4) {  // the owner of the last expert
    p.offsets[E] = oc;
    p.mtoff[E] = om;
  }
  __syncthreads();
  // assignment a's row: its expert's first row plus the number of lower
  // assignments of the same expert (ascending a within an expert)
  for (int a = tid; a < N; a += BS) {
    const int e = sid[a];
    int r = 0;
    for (int b = 0; b < a; ++b) r += sid[b] == e;
    const int pos = base[e] + r;
    p.perm[pos] = a;
    p.inv[a] = pos;
    p.wsorted[pos] = sw[a];
  }
}

hipError_t launch_front(const FrontArgs &a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.T > kSortBlock || a.E > 1024 || a.top_k > 8) return hipErrorInvalidValue;
  if (a.logits && a.T <= kFrontMaxT) {
    // one wave routes each token: 16 waves above 4 tokens (T = 16 with four:
    // each wave routed four tokens in turn, 12.8 us of routing)
    const int bs = a.T > 4 ? 1024 : 256;
    const long nq = a.x ? ((long)a.T * (a.H / 32) + bs - 1) / bs : 0;
    const dim3 grid((unsigned)(1 + nq)), block(bs);
#define FRONT_SMALL_CASE(NV_)                                                   \
  case NV_:                                                                     \
    if (bs == 1024) front_small_kernel<NV_, 1024><<<grid, block, 0, s>>>(a);    \
    else front_small_kernel<NV_, 256><<<grid, block, 0, s>>>(a);                \
    break;
    switch (ceil_div(a.E, 64)) {
      FRONT_SMALL_CASE(1) FRONT_SMALL_CASE(2) FRONT_SMALL_CASE(3) FRONT_SMALL_CASE(4)
      FRONT_SMALL_CASE(5) FRONT_SMALL_CASE(6) FRONT_SMALL_CASE(7) FRONT_SMALL_CASE(8)
      FRONT_SMALL_CASE(9) FRONT_SMALL_CASE(10) FRONT_SMALL_CASE(11) FRONT_SMALL_CASE(12)
      FRONT_SMALL_CASE(13) FRONT_SMALL_CASE(14) FRONT_SMALL_CASE(15) FRONT_SMALL_CASE(16)
      default: return hipErrorInvalidValue;
    }
#undef FRONT_SMALL_CASE
    return hipGetLastError();
  }
  // no quantisation workgroups when the caller passes MX codes (x null)
  const long nq = a.x ? ((long)a.T * (a.H / 32) + 1023) / 1024 : 0;
  const dim3 grid((unsigned)(1 + nq)), block(1024);
#define FRONT_CASE(NV_)                                \
  case NV_:                                            \
    front_kernel<NV_><<<grid, block, 0, s>>>(a);       \
    break;
  switch (ceil_div(a.E, 64)) {
    FRONT_CASE(1) FRONT_CASE(2) FRONT_CASE(3) FRONT_CASE(4) FRONT_CASE(5) FRONT_CASE(6)
    FRONT_CASE(7) FRONT_CASE(8) FRONT_CASE(9) FRONT_CASE(10) FRONT_CASE(11) FRONT_CASE(12)
    FRONT_CASE(13) FRONT_CASE(14) FRONT_CASE(15) FRONT_CASE(16)
    default: return hipErrorInvalidValue;
  }
#undef FRONT_CASE
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine ("add A4W4 and FP8 P2P transport support to MegaMoE", Technical
// Details: accumulate the top-k contributions in FP32): y[t] = bf16 of the
// FP32 sum, in slot order j = 0..top_k-1, of the weighted GEMM2 rows of the
// token's assignments (row inv[t*top_k + j]), rounded once to nearest even.
// The rows arrive in the call's transport (FP32, BF16, or MXFP8 codes with
// one E8M0 scale per 32 columns).  One thread per 8 outputs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// Every slot's row piece is requested before the first is summed (the slot
// count is a template argument, so the loads are straight-line code and all
// of a thread's rows are in flight at once).
template <int MODE, int K>
__global__ __launch_bounds__(256) void combine_kernel(const void *__restrict__ rows,
                                                      const int32_t *__restrict__ inv, long n8,
                                                      int H, long N, uint16_t *__restrict__ y) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const long t = i / (H / 8);
  const int h = (int)(i % (H / 8)) * 8;
  size_t p[K];
#pragma unroll
  for (int j = 0; j < K; ++j) p[j] = (size_t)inv[t * K + j];
  float v[K][8];
  if (MODE == MOE_COMBINE_FP32) {
    float4 a[K], b[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float4 *r = reinterpret_cast<const float4 *>(static_cast<const float *>(rows) +
                                                         p[j] * H + h);
      a[j] = r[0];
      b[j] = r[1];
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      v[j][0] = a[j].x; v[j][1] = a[j].y; v[j][2] = a[j].z; v[j][3] = a[j].w;
      v[j][4] = b[j].x; v[j][5] = b[j].y; v[j][6] = b[j].z; v[j][7] = b[j].w;
    }
  } else if (MODE == MOE_COMBINE_BF16) {
    uint4 a[K];
#pragma unroll
    for (int j = 0; j < K; ++j)
      a[j] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(rows) + p[j] * H + h);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t w[4] = {a[j].x, a[j].y, a[j].z, a[j].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[j][2 * k] = __uint_as_float(w[k] << 16);
        v[j][2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  } else {
    const uint8_t *base = static_cast<const uint8_t *>(rows);
    uint2 a[K];
    int sx[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a[j] = *reinterpret_cast<const uint2 *>(base + p[j] * H + h);
      sx[j] = base[(size_t)N * H + p[j] * (H / 32) + h / 32];
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const uint32_t w[2] = {a[j].x, a[j].y};
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[j][k] = ldexpf(e4m3_value((w[k / 4] >> (8 * (k % 4))) & 0xffu), sx[j] - 127);
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < K; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += v[j][k];
  uint4 o;
  o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
  reinterpret_cast<uint4 *>(y)[i] = o;
}

template <int MODE>
hipError_t launch_combine_k(const void *rows, const int32_t *inv, long n8, int H, int top_k,
                            long N, uint16_t *y, hipStream_t s) {
  const unsigned grid = (unsigned)((n8 + 255) / 256);
  switch (top_k) {
#define COMBINE_CASE(K) \
    case K: combine_kernel<MODE, K><<<grid, 256, 0, s>>>(rows, inv, n8, H, N, y); break;
    COMBINE_CASE(1) COMBINE_CASE(2) COMBINE_CASE(3) COMBINE_CASE(4)
    COMBINE_CASE(5) COMBINE_CASE(6) COMBINE_CASE(7) COMBINE_CASE(8)
#undef COMBINE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void *rows, const int32_t *inv, int T, int H, int top_k,
                          int combine, uint16_t *y, hipStream_t s) {
  const long n8 = (long)T * H / 8;
  if (n8 == 0) return hipSuccess;
  const long N = (long)T * top_k;
  switch (combine) {
    case MOE_COMBINE_FP32:
      return launch_combine_k<MOE_COMBINE_FP32>(rows, inv, n8, H, top_k, N, y, s);
    case MOE_COMBINE_BF16:
      return launch_combine_k<MOE_COMBINE_BF16>(rows, inv, n8, H, top_k, N, y, s);
    case MOE_COMBINE_FP8:
      return launch_combine_k<MOE_COMBINE_FP8>(rows, inv, n8, H, top_k, N, y, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
