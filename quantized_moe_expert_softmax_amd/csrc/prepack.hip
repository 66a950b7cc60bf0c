// prepack.hip -- load-time repack of the canonical MXFP4 expert weights into
// the scaled-MFMA operand layout the expert GEMMs stream (layout: PackDims).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Weight repack (load time; "feat(moe): FlyDSL MegaMoE fused EP-MoE
// integration", summary bullets: gate/up weights are shuffled into the
// interleaved layout the fused SwiGLU needs).  Canonical MXFP4 rows become
// 1 KiB scaled-MFMA B fragments (see PackDims); for the gate/up matrix the
// 16-row tiles are ordered gate[32j, +16), gate[32j+16, +16), up[32j, +16),
// up[32j+16, +16) so that one GEMM1 work unit holds the gate and up columns
// of one 32-wide requantisation block of h.
// ---------------------------------------------------------------------------
__device__ __forceinline__ long packed_row(int tile, int c, int half_rows, bool gate_up) {
  if (!gate_up) return (long)tile * 16 + c;
  const int j = tile >> 2, q = tile & 3;
  return (long)((q >> 1) ? half_rows : 0) + 32 * j + 16 * (q & 1) + c;
}

__global__ __launch_bounds__(256) void prepack_codes_kernel(const uint8_t *__restrict__ src,
                                                            long total, int R, int K, bool gate_up,
                                                            uint8_t *__restrict__ dst) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int steps = K / 128, nquad = R / 64;
  const int lane = (int)(idx & 63);
  const int q = (int)((idx >> 6) & 3);
  const long rest = idx >> 8;
  const int s = (int)(rest % steps);
  const long rest2 = rest / steps;
  const int u = (int)(rest2 % nquad);
  const long e = rest2 / nquad;
  const long row = packed_row(4 * u + q, lane & 15, R / 2, gate_up);
  const uint8_t *p = src + (e * R + row) * (long)(K / 2) + 64 * s + 16 * (lane >> 4);
  *reinterpret_cast<uint4 *>(dst + idx * 16) = *reinterpret_cast<const uint4 *>(p);
}

__global__ __launch_bounds__(256) void prepack_scales_kernel(const uint8_t *__restrict__ src,
                                                             long total, int R, int K,
                                                             bool gate_up,
                                                             uint32_t *__restrict__ dst) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int steps = K / 128, nquad = R / 64;
  const int lane = (int)(idx & 63);
  const long rest = idx >> 6;
  const int s = (int)(rest % steps);
  const long rest2 = rest / steps;
  const int u = (int)(rest2 % nquad);
  const long e = rest2 / nquad;
  uint32_t d = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const long row = packed_row(4 * u + q, lane & 15, R / 2, gate_up);
    d |= (uint32_t)src[(e * R + row) * (long)(K / 32) + 4 * s + (lane >> 4)] << (8 * q);
  }
  dst[idx] = d;
}

hipError_t launch_prepack(const uint8_t *codes, const uint8_t *scales, int E, int R, int K,
                          bool gate_up, uint8_t *pcodes, uint8_t *pscales, hipStream_t s) {
  const PackDims d = pack_dims(R, K);
  const long nc = (long)E * (R / 64) * d.steps * 256;
  const long ns = (long)E * (R / 64) * d.steps * 64;
  prepack_codes_kernel<<<(unsigned)((nc + 255) / 256), 256, 0, s>>>(codes, nc, R, K, gate_up,
                                                                   pcodes);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  prepack_scales_kernel<<<(unsigned)((ns + 255) / 256), 256, 0, s>>>(
      scales, ns, R, K, gate_up, reinterpret_cast<uint32_t *>(pscales));
  return hipGetLastError();
}

}  // namespace moe
