/* Drives every entry point of the CPU oracle on small pseudo-random inputs so
 * that a build with host sanitizers (address, undefined behaviour) checks its
 * memory accesses and arithmetic; tests/test_oracle_sanitized.py compiles and
 * runs it.  Inputs come from a fixed linear congruential generator. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_mx_quantize(const float *v, long rows, int K, int fmt, uint8_t *codes, uint8_t *scales);
void oracle_mx_quantize_bf16(const uint16_t *x, long rows, int K, int fmt, uint8_t *codes,
                             uint8_t *scales);
void oracle_mx_dequantize(const uint8_t *codes, const uint8_t *scales, long rows, int K, int fmt,
                          float *out);
double oracle_code_value(int fmt, unsigned code);
void oracle_float_to_bf16(const float *f, long n, uint16_t *out);
void oracle_route(const float *logits, int T, int E, int top_k, int32_t *ids, float *w);
void oracle_sort(const int32_t *ids, int T, int E, int top_k, int32_t *counts, int32_t *offsets,
                 int32_t *perm);
void oracle_forward(const uint16_t *x, const float *logits, int T, int H, int I, int E, int top_k,
                    int fmt, const uint8_t *w13, const uint8_t *w13s, const uint8_t *w2,
                    const uint8_t *w2s, int acc_double, int combine, uint16_t *y, float *y_f32,
                    uint8_t *a2_codes, uint8_t *a2_scales, const int32_t *expert_map);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(state >> 32);
}
static float next_gauss(void) { /* sum of uniforms: roughly N(0, 1) */
  float s = 0.f;
  for (int i = 0; i < 12; ++i) s += (float)next_u32() / 4294967296.0f;
  return s - 6.0f;
}
static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) { fprintf(stderr, "oom\n"); exit(2); }
  return p;
}

int main(void) {
  /* codec: every code of both formats, scaled blocks including special values */
  for (unsigned c = 0; c < 256; ++c) (void)oracle_code_value(0, c);
  for (unsigned c = 0; c < 16; ++c) (void)oracle_code_value(1, c);
  const int K = 96, R = 5;
  float *v = xmalloc(sizeof(float) * K * R);
  for (int i = 0; i < K * R; ++i) v[i] = next_gauss() * (float)(1 << (i % 7));
  v[0] = 0.f; v[1] = -0.f; v[2] = 1e-30f; v[3] = 6.0e4f;
  for (int k = 32; k < 64; ++k) v[k] = 0.f; /* an all-zero block */
  uint16_t *xb = xmalloc(sizeof(uint16_t) * K * R);
  oracle_float_to_bf16(v, (long)K * R, xb);
  for (int fmt = 0; fmt <= 1; ++fmt) { /* 0: E4M3, 1: E2M1 */
    uint8_t *codes = xmalloc((size_t)K * R), *scales = xmalloc((size_t)K / 32 * R);
    float *back = xmalloc(sizeof(float) * K * R);
    oracle_mx_quantize(v, R, K, fmt, codes, scales);
    oracle_mx_dequantize(codes, scales, R, K, fmt, back);
    oracle_mx_quantize_bf16(xb, R, K, fmt, codes, scales);
    free(codes); free(scales); free(back);
  }

  /* routing and sort, including top_k = E and ties */
  const int T = 9, E = 6;
  float *lg = xmalloc(sizeof(float) * T * E);
  for (int i = 0; i < T * E; ++i) lg[i] = next_gauss();
  lg[E] = lg[E + 1]; /* a tie */
  for (int k = 1; k <= E; ++k) {
    int32_t *ids = xmalloc(sizeof(int32_t) * T * k), *perm = xmalloc(sizeof(int32_t) * T * k);
    int32_t *counts = xmalloc(sizeof(int32_t) * E), *offsets = xmalloc(sizeof(int32_t) * (E + 1));
    float *w = xmalloc(sizeof(float) * T * k);
    oracle_route(lg, T, E, k, ids, w);
    oracle_sort(ids, T, E, k, counts, offsets, perm);
    free(ids); free(perm); free(counts); free(offsets); free(w);
  }

  /* the layer: both formats, every combine transport, fp32 and double
   * accumulation, with the A2 and FP32 outputs, full and compact expert sets */
  const int H = 128, I = 64, k = 2;
  uint16_t *x = xmalloc(sizeof(uint16_t) * T * H);
  for (int i = 0; i < T * H; ++i) {
    float f = next_gauss();
    oracle_float_to_bf16(&f, 1, &x[i]);
  }
  uint8_t *w13 = xmalloc((size_t)E * 2 * I * H / 2), *w13s = xmalloc((size_t)E * 2 * I * H / 32);
  uint8_t *w2 = xmalloc((size_t)E * H * I / 2), *w2s = xmalloc((size_t)E * H * I / 32);
  for (size_t i = 0; i < (size_t)E * 2 * I * H / 2; ++i) w13[i] = (uint8_t)next_u32();
  for (size_t i = 0; i < (size_t)E * 2 * I * H / 32; ++i) w13s[i] = (uint8_t)(120 + next_u32() % 6);
  for (size_t i = 0; i < (size_t)E * H * I / 2; ++i) w2[i] = (uint8_t)next_u32();
  for (size_t i = 0; i < (size_t)E * H * I / 32; ++i) w2s[i] = (uint8_t)(120 + next_u32() % 6);
  int32_t emap[6] = {5, 4, 3, 2, 1, 0};
  uint16_t *y = xmalloc(sizeof(uint16_t) * T * H);
  float *yf = xmalloc(sizeof(float) * T * H);
  uint8_t *a2c = xmalloc((size_t)T * k * I), *a2s = xmalloc((size_t)T * k * I / 32);
  for (int fmt = 0; fmt <= 1; ++fmt)
    for (int combine = 0; combine < 3; ++combine)
      for (int dbl = 0; dbl < 2; ++dbl)
        for (int m = 0; m < 2; ++m)
          oracle_forward(x, lg, T, H, I, E, k, fmt, w13, w13s, w2, w2s, dbl, combine, y, yf, a2c,
                         a2s, m ? emap : NULL);
  free(v); free(xb); free(lg); free(x); free(w13); free(w13s); free(w2); free(w2s);
  free(y); free(yf); free(a2c); free(a2s);
  printf("ok\n");
  return 0;
}
