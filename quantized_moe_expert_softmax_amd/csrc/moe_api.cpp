// moe_api.cpp -- the C-ABI of the MoE layer: validation, the handle, the
// workspace plan and the launch sequence of one forward call.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

using namespace moe;

struct moe_layer {
  int E, H, I;
  int device;
  int num_cus;
  uint8_t *w13p, *w13sp, *w2p, *w2sp;  // the weight set forward calls read (null: none bound)
  uint8_t *own[4];                     // packed weights the handle allocated (moe_prepare_weights)
  std::vector<moe_plan> plans;  // per-layer plan table (moe_set_plans)
  // kernel timing (benchmarks only)
  bool profiling;
  int prof_max, prof_calls;
  std::vector<hipEvent_t> events;  // [prof_max][MOE_K_NUM + 1]
};

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status hip_fail(hipError_t e, const char *what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool bad_dims(int E, int H, int I, std::string *why) {
  char b[160];
  if (E < 1 || E > 1024) { snprintf(b, sizeof b, "E=%d outside [1, 1024]", E); *why = b; return true; }
  if (H <= 0 || H % 128) { snprintf(b, sizeof b, "H=%d is not a positive multiple of 128", H); *why = b; return true; }
  if (I <= 0 || I % 128) { snprintf(b, sizeof b, "I=%d is not a positive multiple of 128", I); *why = b; return true; }
  if (H > (1 << 16) || I > (1 << 16)) { snprintf(b, sizeof b, "H=%d or I=%d above 65536", H, I); *why = b; return true; }
  return false;
}

bool misaligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

moe_status check_call(moe_layer_t L, int T, int top_k, int act) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "null layer handle");
  if (T < 0 || T > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, 2^20]", T);
  const int kmax = L->E < 8 ? L->E : 8;
  if (top_k < 1 || top_k > kmax)
    return fail(MOE_ERR_INVALID_ARG, "top_k=%d outside [1, %d]", top_k, kmax);
  if (act != MOE_ACT_MXFP8_E4M3 && act != MOE_ACT_MXFP4_E2M1)
    return fail(MOE_ERR_INVALID_ARG, "unknown activation dtype %d", act);
  return MOE_OK;
}

// Device in use must be gfx950 and must be the handle's device.
moe_status check_device(int *dev_out, int *cus_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MOE_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  if (dev_out) *dev_out = dev;
  if (cus_out) *cus_out = prop.multiProcessorCount;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_OOM: return "MOE_ERR_OOM";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_prepare_weights(int E, int H, int I, const void *w13, const void *w13_scale,
                               const void *w2, const void *w2_scale, hipStream_t s,
                               moe_layer_t *out) {
  std::string why;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "null output handle pointer");
  *out = nullptr;
  if (bad_dims(E, H, I, &why)) return fail(MOE_ERR_INVALID_ARG, "%s", why.c_str());
  if (!w13 || !w13_scale || !w2 || !w2_scale) return fail(MOE_ERR_INVALID_ARG, "null weight pointer");
  if (misaligned(w13, 16) || misaligned(w2, 16))
    return fail(MOE_ERR_INVALID_ARG, "weight code buffers must be 16-byte aligned");
  int dev = 0, cus = 0;
  moe_status st = check_device(&dev, &cus);
  if (st != MOE_OK) return st;
  void *scratch = nullptr;  // set-up of moe_forward_noalloc's array on this device
  hipError_t e = noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "static scratch lookup");

  const PackDims d13 = pack_dims(2 * I, H), d2 = pack_dims(H, I);
  moe_layer *L = new moe_layer();
  L->E = E; L->H = H; L->I = I; L->device = dev; L->num_cus = cus;
  L->profiling = false; L->prof_max = 0; L->prof_calls = 0;
  const size_t b13 = (size_t)E * d13.code_bytes(), s13 = (size_t)E * d13.scale_bytes();
  const size_t b2 = (size_t)E * d2.code_bytes(), s2 = (size_t)E * d2.scale_bytes();
  e = hipMalloc(&L->own[0], b13);
  if (e == hipSuccess) e = hipMalloc(&L->own[1], s13);
  if (e == hipSuccess) e = hipMalloc(&L->own[2], b2);
  if (e == hipSuccess) e = hipMalloc(&L->own[3], s2);
  L->w13p = L->own[0]; L->w13sp = L->own[1]; L->w2p = L->own[2]; L->w2sp = L->own[3];
  if (e != hipSuccess) {
    (void)hipGetLastError();
    moe_destroy(L);
    return fail(MOE_ERR_OOM, "hipMalloc of %zu bytes of packed weights failed",
                b13 + s13 + b2 + s2);
  }
  e = launch_prepack(static_cast<const uint8_t *>(w13), static_cast<const uint8_t *>(w13_scale),
                     E, 2 * I, H, true, L->w13p, L->w13sp, s);
  if (e == hipSuccess)
    e = launch_prepack(static_cast<const uint8_t *>(w2), static_cast<const uint8_t *>(w2_scale),
                       E, H, I, false, L->w2p, L->w2sp, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    moe_destroy(L);
    return hip_fail(e, "weight repack");
  }
  *out = L;
  return MOE_OK;
}

void moe_destroy(moe_layer_t L) {
  if (!L) return;
  (void)hipDeviceSynchronize();
  for (hipEvent_t ev : L->events) (void)hipEventDestroy(ev);
  for (uint8_t *p : L->own)
    if (p) (void)hipFree(p);
  delete L;
}

moe_status moe_packed_weight_bytes(int E, int H, int I, size_t bytes[4]) {
  std::string why;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "null output array");
  if (bad_dims(E, H, I, &why)) return fail(MOE_ERR_INVALID_ARG, "%s", why.c_str());
  const PackDims d13 = pack_dims(2 * I, H), d2 = pack_dims(H, I);
  bytes[0] = (size_t)E * d13.code_bytes();
  bytes[1] = (size_t)E * d13.scale_bytes();
  bytes[2] = (size_t)E * d2.code_bytes();
  bytes[3] = (size_t)E * d2.scale_bytes();
  return MOE_OK;
}

moe_status moe_pack_weights(int E, int H, int I, const void *w13, const void *w13_scale,
                            const void *w2, const void *w2_scale, const moe_packed_weights *dst,
                            hipStream_t s) {
  std::string why;
  if (bad_dims(E, H, I, &why)) return fail(MOE_ERR_INVALID_ARG, "%s", why.c_str());
  if (!w13 || !w13_scale || !w2 || !w2_scale || !dst) return fail(MOE_ERR_INVALID_ARG, "null pointer");
  if (!dst->w13 || !dst->w13_scale || !dst->w2 || !dst->w2_scale)
    return fail(MOE_ERR_INVALID_ARG, "null packed weight pointer");
  if (misaligned(w13, 16) || misaligned(w2, 16))
    return fail(MOE_ERR_INVALID_ARG, "weight code buffers must be 16-byte aligned");
  if (misaligned(dst->w13, 16) || misaligned(dst->w13_scale, 16) || misaligned(dst->w2, 16) ||
      misaligned(dst->w2_scale, 16))
    return fail(MOE_ERR_INVALID_ARG, "packed weight buffers must be 16-byte aligned");
  moe_status st = check_device(nullptr, nullptr);
  if (st != MOE_OK) return st;
  hipError_t e = launch_prepack(static_cast<const uint8_t *>(w13),
                                static_cast<const uint8_t *>(w13_scale), E, 2 * I, H, true,
                                static_cast<uint8_t *>(dst->w13),
                                static_cast<uint8_t *>(dst->w13_scale), s);
  if (e == hipSuccess)
    e = launch_prepack(static_cast<const uint8_t *>(w2), static_cast<const uint8_t *>(w2_scale), E,
                       H, I, false, static_cast<uint8_t *>(dst->w2),
                       static_cast<uint8_t *>(dst->w2_scale), s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "weight repack");
}

moe_status moe_create_layer(int E, int H, int I, moe_layer_t *out) {
  std::string why;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "null output handle pointer");
  *out = nullptr;
  if (bad_dims(E, H, I, &why)) return fail(MOE_ERR_INVALID_ARG, "%s", why.c_str());
  int dev = 0, cus = 0;
  moe_status st = check_device(&dev, &cus);
  if (st != MOE_OK) return st;
  void *scratch = nullptr;  // set-up of moe_forward_noalloc's array on this device
  const hipError_t e = noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "static scratch lookup");
  moe_layer *L = new moe_layer();
  L->E = E; L->H = H; L->I = I; L->device = dev; L->num_cus = cus;
  *out = L;
  return MOE_OK;
}

moe_status moe_bind_weights(moe_layer_t L, const moe_packed_weights *w) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "null layer handle");
  if (!w) {
    L->w13p = L->own[0]; L->w13sp = L->own[1]; L->w2p = L->own[2]; L->w2sp = L->own[3];
    return MOE_OK;
  }
  if (!w->w13 || !w->w13_scale || !w->w2 || !w->w2_scale)
    return fail(MOE_ERR_INVALID_ARG, "null packed weight pointer");
  if (misaligned(w->w13, 16) || misaligned(w->w13_scale, 16) || misaligned(w->w2, 16) ||
      misaligned(w->w2_scale, 16))
    return fail(MOE_ERR_INVALID_ARG, "packed weight buffers must be 16-byte aligned");
  L->w13p = static_cast<uint8_t *>(w->w13);
  L->w13sp = static_cast<uint8_t *>(w->w13_scale);
  L->w2p = static_cast<uint8_t *>(w->w2);
  L->w2sp = static_cast<uint8_t *>(w->w2_scale);
  return MOE_OK;
}

size_t moe_workspace_bytes(moe_layer_t L, int T, int top_k, moe_act_dtype act) {
  if (check_call(L, T, top_k, act) != MOE_OK) return 0;
  return ws_layout(T, top_k, L->E, L->H, L->I, act).total;
}

moe_status moe_workspace_offsets(moe_layer_t L, int T, int top_k, moe_act_dtype act,
                                 size_t *offs) {
  moe_status st = check_call(L, T, top_k, act);
  if (st != MOE_OK) return st;
  if (!offs) return fail(MOE_ERR_INVALID_ARG, "null offsets array");
  const WsLayout W = ws_layout(T, top_k, L->E, L->H, L->I, act);
  for (int i = 0; i < MOE_WS_NUM; ++i) offs[i] = W.off[i];
  return MOE_OK;
}

extern "C++" {  // internal helpers: C++ linkage inside the C-ABI block
namespace {

GemmPlan plan_for(const moe_layer *L, int T, int top_k, int act) {
  for (const moe_plan &p : L->plans)
    if (p.act == act && p.top_k == top_k && T <= p.t_max)
      return p.variant == MOE_PLAN_TILED
                 ? GemmPlan{true, p.rows / 16, kTiledSplit}
                 : GemmPlan{false, 1, 1, p.variant == MOE_PLAN_FUSED,
                            p.variant == MOE_PLAN_DECODE};
  return choose_plan(T, top_k, L->E, act);
}

}  // namespace
}  // extern "C++"

moe_status moe_set_plans(moe_layer_t L, const moe_plan *plans, int n) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "null layer handle");
  if (n < 0 || n > 256) return fail(MOE_ERR_INVALID_ARG, "plan count %d outside [0, 256]", n);
  if (n > 0 && !plans) return fail(MOE_ERR_INVALID_ARG, "null plan array");
  for (int i = 0; i < n; ++i) {
    const moe_plan &p = plans[i];
    if (p.act != MOE_ACT_MXFP8_E4M3 && p.act != MOE_ACT_MXFP4_E2M1)
      return fail(MOE_ERR_INVALID_ARG, "plan %d: act %d", i, p.act);
    if (p.top_k < 1 || p.top_k > 8 || p.top_k > L->E)
      return fail(MOE_ERR_INVALID_ARG, "plan %d: top_k %d", i, p.top_k);
    if (p.t_max < 1) return fail(MOE_ERR_INVALID_ARG, "plan %d: t_max %d", i, p.t_max);
    if (p.variant == MOE_PLAN_STREAM || p.variant == MOE_PLAN_FUSED ||
        p.variant == MOE_PLAN_DECODE) {
      if (p.rows != 16)
        return fail(MOE_ERR_INVALID_ARG, "plan %d: stream, fused and decode rows must be 16", i);
    } else if (p.variant == MOE_PLAN_TILED) {
      if (p.rows % 16 != 0 || !tiled_mt_built(p.act, p.rows / 16))
        return fail(MOE_ERR_INVALID_ARG, "plan %d: no tiled kernel with %d rows for act %d", i,
                    p.rows, p.act);
    } else {
      return fail(MOE_ERR_INVALID_ARG, "plan %d: variant %d", i, p.variant);
    }
  }
  L->plans.assign(plans, plans + n);
  return MOE_OK;
}

moe_status moe_get_plan(moe_layer_t L, int T, int top_k, moe_act_dtype act, moe_plan *out) {
  moe_status st = check_call(L, T, top_k, act);
  if (st != MOE_OK) return st;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "null output");
  const GemmPlan g = plan_for(L, T, top_k, act);
  *out = moe_plan{(int32_t)act, top_k, T,
                  g.tiled ? MOE_PLAN_TILED
                          : (g.fused ? MOE_PLAN_FUSED : (g.tm ? MOE_PLAN_DECODE : MOE_PLAN_STREAM)),
                  g.tiled ? 16 * g.mt : 16};
  return MOE_OK;
}

moe_status moe_forward(moe_layer_t L, const void *x, const float *logits, int T, int top_k,
                       moe_act_dtype act, void *y, void *ws, size_t ws_bytes, hipStream_t s) {
  return moe_forward_ex(L, x, logits, T, top_k, act, 0u, y, ws, ws_bytes, s);
}

// The whole layer, from bf16 rows x (quantised here) or, when prequant, from
// the caller's MX codes xq and scales xqs.
static moe_status forward_impl(moe_layer_t L, bool prequant, const void *x, const uint8_t *xq,
                               const uint8_t *xqs, const float *logits, int T, int top_k,
                               moe_act_dtype act, uint32_t flags, void *y, void *ws,
                               size_t ws_bytes, hipStream_t s) {
  moe_status st = check_call(L, T, top_k, act);
  if (st != MOE_OK) return st;
  if (flags != MOE_COMBINE_FP32 && flags != MOE_COMBINE_BF16 && flags != MOE_COMBINE_FP8)
    return fail(MOE_ERR_INVALID_ARG, "flags 0x%x: not a moe_combine value", flags);
  if (T == 0) return MOE_OK;
  if (!L->w13p) return fail(MOE_ERR_INVALID_ARG, "no weights bound to the layer");
  if ((prequant ? (!xq || !xqs) : !x) || !logits || !y || !ws)
    return fail(MOE_ERR_INVALID_ARG, "null data pointer");
  if (misaligned(y, 16) || misaligned(logits, 4))
    return fail(MOE_ERR_INVALID_ARG, "y must be 16-byte aligned, logits 4-byte aligned");
  if (prequant ? (misaligned(xq, 16) || misaligned(xqs, 4)) : misaligned(x, 16))
    return fail(MOE_ERR_INVALID_ARG,
                "x must be 16-byte aligned (codes 16-byte, scales 4-byte aligned)");
  if (misaligned(ws, 256)) return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (!prequant && x == y) return fail(MOE_ERR_INVALID_ARG, "y must not alias x");
  const WsLayout W = ws_layout(T, top_k, L->E, L->H, L->I, act);
  if (ws_bytes < W.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, W.total);

  uint8_t *base = static_cast<uint8_t *>(ws);
  int32_t *ids = reinterpret_cast<int32_t *>(base + W.off[MOE_WS_IDS]);
  float *wts = reinterpret_cast<float *>(base + W.off[MOE_WS_WEIGHTS]);
  int32_t *counts = reinterpret_cast<int32_t *>(base + W.off[MOE_WS_COUNTS]);
  int32_t *offsets = reinterpret_cast<int32_t *>(base + W.off[MOE_WS_OFFSETS]);
  int32_t *mtoff = reinterpret_cast<int32_t *>(base + W.mtoff);
  int32_t *mbexp = reinterpret_cast<int32_t *>(base + W.mbexp);
  int32_t *mbrows = reinterpret_cast<int32_t *>(base + W.mbrows);
  int32_t *hist = reinterpret_cast<int32_t *>(base + W.hist);
  int32_t *perm = reinterpret_cast<int32_t *>(base + W.off[MOE_WS_PERM]);
  uint8_t *a1c = base + W.off[MOE_WS_A1_CODES];
  uint8_t *a1s = base + W.off[MOE_WS_A1_SCALES];
  // GEMM1 reads the activation codes from here
  const uint8_t *g1c = prequant ? xq : a1c, *g1s = prequant ? xqs : a1s;
  uint8_t *a2c = base + W.off[MOE_WS_A2_CODES];
  uint8_t *a2s = base + W.off[MOE_WS_A2_SCALES];
  float *rows = reinterpret_cast<float *>(base + W.off[MOE_WS_ROWS]);
  int32_t *inv = reinterpret_cast<int32_t *>(base + W.off[MOE_WS_SLOT]);
  float *wsorted = reinterpret_cast<float *>(base + W.wsorted);

  GemmArgs g{};
  g.T = T; g.top_k = top_k; g.E = L->E; g.H = L->H; g.I = L->I; g.act = act;
  g.plan = plan_for(L, T, top_k, act);
  {  // each non-empty expert adds at most one partial m-block
    const long N = (long)T * top_k;
    g.max_mtiles = (N + g.plan.bm() - 1) / g.plan.bm() + (N < L->E ? N : L->E);
  }
  g.num_cus = L->num_cus;
  g.a1c = g1c; g.a1s = g1s; g.a2c = a2c; g.a2s = a2s;
  g.perm = perm; g.offsets = offsets; g.mtoff = mtoff; g.mbexp = mbexp; g.wts = wsorted;
  g.mbrows = mbrows;
  g.w13p = L->w13p; g.w13sp = L->w13sp; g.w2p = L->w2p; g.w2sp = L->w2sp;
  g.rows = rows;
  g.combine = (int)flags;
  g.ids = ids; g.inv = inv; g.wts_a = wts; g.y = static_cast<uint16_t *>(y);
  // the fused launch's counters, zeroed by the route/sort launch before it
  g.sync = reinterpret_cast<int32_t *>(base + W.sync);
  // the routing launch clears the give-up flag on every call (moe_fused_status
  // reads it) and, for the fused plan, its per-m-tile counts
  const int nsync = g.plan.fused ? (int)(kSyncHead + g.max_mtiles) : kSyncHead;

  const bool prof = L->profiling && L->prof_calls < L->prof_max;
  hipEvent_t *ev = prof ? &L->events[(size_t)L->prof_calls * (MOE_K_NUM + 1)] : nullptr;
  int stage = 0;
  hipError_t e = hipSuccess;
  auto mark = [&]() {
    if (prof && e == hipSuccess) e = hipEventRecord(ev[stage], s);
    ++stage;
  };
  mark();
  // the fused front launch's arguments; routed_logits null: the router
  // kernel has already written ids and wts
  auto front_args = [&](const float *routed_logits) {
    FrontArgs f{};
    f.logits = routed_logits; f.x = static_cast<const uint16_t *>(x);
    f.T = T; f.E = L->E; f.top_k = top_k; f.H = L->H; f.act = act; f.bm = g.plan.bm();
    f.ids = ids; f.wts = wts; f.counts = counts; f.offsets = offsets; f.mtoff = mtoff;
    f.mbexp = mbexp; f.mbrows = mbrows; f.perm = perm; f.inv = inv; f.wsorted = wsorted; f.codes = a1c;
    f.scales = a1s;
    f.sync = g.sync;
    f.nsync = nsync;
    return f;
  };
  if (T <= kFrontMaxT) {
    // small decode batches: route, sort and quantisation in one launch (its
    // time is recorded as the route stage; the sort and quant stages record
    // ~0).  One workgroup routes every token there, which is slower than
    // the separate kernels beyond a few tens of tokens.
    if (e == hipSuccess) e = launch_front(front_args(logits), s);
    for (int i = 0; i < 5; ++i) mark();
  } else if (T <= kSortBlock) {
    // up to one sort block: the router kernel, then sort and quantisation in
    // one launch (recorded as the sort_hist stage; the scan, scatter and
    // quant stages record ~0)
    if (e == hipSuccess) e = launch_route(logits, T, L->E, top_k, ids, wts, s);
    mark();
    if (e == hipSuccess) e = launch_front(front_args(nullptr), s);
    for (int i = 0; i < 4; ++i) mark();
  } else {
    if (e == hipSuccess) e = launch_route(logits, T, L->E, top_k, ids, wts, s);
    mark();
    if (e == hipSuccess) e = launch_sort_hist(ids, T, L->E, top_k, hist, W.nb, s);
    mark();
    if (e == hipSuccess)
      e = launch_sort_scan(hist, W.nb, L->E, counts, offsets, mtoff, mbexp, mbrows, g.plan.bm(),
                           g.sync, nsync, s);
    mark();
    if (e == hipSuccess)
      e = launch_sort_scatter(ids, T, L->E, top_k, hist, offsets, perm, inv, wts, wsorted, s);
    mark();
    if (e == hipSuccess && !prequant)
      e = launch_quant(static_cast<const uint16_t *>(x), T, L->H, act, a1c, a1s, s);
    mark();
  }
  if (e == hipSuccess) e = launch_gemm1(g, s);
  mark();
  if (e == hipSuccess) e = launch_gemm2(g, s);
  mark();
  if (e == hipSuccess && !gemm2_writes_y(g))
    e = launch_combine(rows, inv, T, L->H, top_k, (int)flags, static_cast<uint16_t *>(y), s);
  mark();
  if (e != hipSuccess) return hip_fail(e, "moe_forward launch");
  if (prof) ++L->prof_calls;
  return MOE_OK;
}

moe_status moe_forward_ex(moe_layer_t L, const void *x, const float *logits, int T, int top_k,
                          moe_act_dtype act, uint32_t flags, void *y, void *ws, size_t ws_bytes,
                          hipStream_t s) {
  return forward_impl(L, false, x, nullptr, nullptr, logits, T, top_k, act, flags, y, ws,
                      ws_bytes, s);
}

moe_status moe_forward_noalloc(moe_layer_t L, const void *x, const float *logits, int T,
                               int top_k, moe_act_dtype act, uint32_t flags, void *y,
                               hipStream_t s) {
  moe_status st = check_call(L, T, top_k, act);
  if (st != MOE_OK) return st;
  const size_t need = ws_layout(T, top_k, L->E, L->H, L->I, act).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "T=%d top_k=%d needs %zu bytes of workspace; the static scratch of "
                "moe_forward_noalloc holds %zu (use moe_forward_ex with a workspace)",
                T, top_k, need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_fail(e, "moe_forward_noalloc scratch lookup");
  return forward_impl(L, false, x, nullptr, nullptr, logits, T, top_k, act, flags, y, ws,
                      MOE_NOALLOC_SCRATCH_BYTES, s);
}

moe_status moe_forward_prequant(moe_layer_t L, const uint8_t *x_codes, const uint8_t *x_scales,
                                const float *logits, int T, int top_k, moe_act_dtype act,
                                uint32_t flags, void *y, void *ws, size_t ws_bytes,
                                hipStream_t s) {
  return forward_impl(L, true, nullptr, x_codes, x_scales, logits, T, top_k, act, flags, y, ws,
                      ws_bytes, s);
}

moe_status moe_fused_status(moe_layer_t L, const void *ws, int T, int top_k, moe_act_dtype act,
                            hipStream_t s, int32_t *gave_up) {
  moe_status st = check_call(L, T, top_k, act);
  if (st != MOE_OK) return st;
  if (!ws || !gave_up) return fail(MOE_ERR_INVALID_ARG, "null pointer");
  *gave_up = 0;
  if (T == 0) return MOE_OK;  // a T = 0 call launches nothing
  const WsLayout W = ws_layout(T, top_k, L->E, L->H, L->I, act);
  int32_t flag = 0;
  hipError_t e = hipMemcpyAsync(&flag, static_cast<const uint8_t *>(ws) + W.sync, sizeof flag,
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "moe_fused_status");
  *gave_up = flag != 0;
  return MOE_OK;
}

moe_status moe_route(const float *logits, int T, int E, int top_k, int32_t *ids, float *w,
                     hipStream_t s) {
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "E=%d outside [1, 1024]", E);
  const int kmax = E < 8 ? E : 8;
  if (top_k < 1 || top_k > kmax) return fail(MOE_ERR_INVALID_ARG, "top_k=%d outside [1, %d]", top_k, kmax);
  if (T < 0 || T > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, 2^20]", T);
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !w) return fail(MOE_ERR_INVALID_ARG, "null data pointer");
  moe_status st = check_device(nullptr, nullptr);
  if (st != MOE_OK) return st;
  hipError_t e = launch_route(logits, T, E, top_k, ids, w, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "route launch");
}

size_t moe_sort_workspace_bytes(int T, int E, int top_k) {
  if (T < 0 || T > (1 << 20) || E < 1 || E > 1024 || top_k < 1 || top_k > 8) return 0;
  return sort_ws_layout(T, E, top_k).total;
}

moe_status moe_sort(const int32_t *ids, int T, int E, int top_k, int32_t *counts,
                    int32_t *offsets, int32_t *perm, void *ws, size_t ws_bytes, hipStream_t s) {
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "E=%d outside [1, 1024]", E);
  const int kmax = E < 8 ? E : 8;
  if (top_k < 1 || top_k > kmax) return fail(MOE_ERR_INVALID_ARG, "top_k=%d outside [1, %d]", top_k, kmax);
  if (T < 0 || T > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, 2^20]", T);
  if (!ids || !counts || !offsets || !perm || !ws) return fail(MOE_ERR_INVALID_ARG, "null data pointer");
  if (misaligned(ws, 256)) return fail(MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const SortWs W = sort_ws_layout(T, E, top_k);
  if (ws_bytes < W.total) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, W.total);
  moe_status st = check_device(nullptr, nullptr);
  if (st != MOE_OK) return st;
  uint8_t *base = static_cast<uint8_t *>(ws);
  int32_t *hist = reinterpret_cast<int32_t *>(base + W.hist);
  int32_t *mtoff = reinterpret_cast<int32_t *>(base + W.mtoff);
  int32_t *mbexp = reinterpret_cast<int32_t *>(base + W.mbexp);
  int32_t *inv = reinterpret_cast<int32_t *>(base + W.inv);
  const int nb = ceil_div(T, kSortBlock);
  hipError_t e = hipSuccess;
  if (nb > 0) e = launch_sort_hist(ids, T, E, top_k, hist, nb, s);
  if (e == hipSuccess)
    e = launch_sort_scan(hist, nb, E, counts, offsets, mtoff, mbexp, nullptr, kMTile, nullptr, 0,
                         s);
  if (e == hipSuccess && nb > 0)
    e = launch_sort_scatter(ids, T, E, top_k, hist, offsets, perm, inv, nullptr, nullptr, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "sort launch");
}

moe_status moe_quant_act(const void *x, int T, int H, moe_act_dtype act, uint8_t *codes,
                         uint8_t *scales, hipStream_t s) {
  if (T < 0 || T > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "T=%d outside [0, 2^20]", T);
  if (H <= 0 || H % 128) return fail(MOE_ERR_INVALID_ARG, "H=%d is not a positive multiple of 128", H);
  if (act != MOE_ACT_MXFP8_E4M3 && act != MOE_ACT_MXFP4_E2M1)
    return fail(MOE_ERR_INVALID_ARG, "unknown activation dtype %d", act);
  if (T == 0) return MOE_OK;
  if (!x || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "null data pointer");
  if (misaligned(x, 16) || misaligned(codes, 16))
    return fail(MOE_ERR_INVALID_ARG, "x and codes must be 16-byte aligned");
  moe_status st = check_device(nullptr, nullptr);
  if (st != MOE_OK) return st;
  hipError_t e = launch_quant(static_cast<const uint16_t *>(x), T, H, act, codes, scales, s);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "quant launch");
}

moe_status moe_profile_enable(moe_layer_t L, int enable, int max_calls) {
  if (!L) return fail(MOE_ERR_INVALID_ARG, "null layer handle");
  if (enable && (max_calls < 1 || max_calls > 100000))
    return fail(MOE_ERR_INVALID_ARG, "max_calls=%d outside [1, 100000]", max_calls);
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  for (hipEvent_t ev : L->events) (void)hipEventDestroy(ev);
  L->events.clear();
  L->profiling = false;
  L->prof_calls = 0;
  L->prof_max = 0;
  if (!enable) return MOE_OK;
  L->events.resize((size_t)max_calls * (MOE_K_NUM + 1));
  for (size_t i = 0; i < L->events.size(); ++i) {
    e = hipEventCreate(&L->events[i]);
    if (e != hipSuccess) {
      for (size_t k = 0; k < i; ++k) (void)hipEventDestroy(L->events[k]);
      L->events.clear();
      return hip_fail(e, "hipEventCreate");
    }
  }
  L->prof_max = max_calls;
  L->profiling = true;
  return MOE_OK;
}

moe_status moe_profile_read(moe_layer_t L, float *ms, int *ncalls) {
  if (!L || !ms || !ncalls) return fail(MOE_ERR_INVALID_ARG, "null argument");
  for (int k = 0; k < MOE_K_NUM; ++k) ms[k] = 0.0f;
  *ncalls = L->prof_calls;
  for (int c = 0; c < L->prof_calls; ++c) {
    hipEvent_t *ev = &L->events[(size_t)c * (MOE_K_NUM + 1)];
    hipError_t e = hipEventSynchronize(ev[MOE_K_NUM]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    for (int k = 0; k < MOE_K_NUM; ++k) {
      float t = 0.0f;
      e = hipEventElapsedTime(&t, ev[k], ev[k + 1]);
      if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
      ms[k] += t;
    }
  }
  return MOE_OK;
}

}  // extern "C"
