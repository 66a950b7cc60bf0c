/*
 * moe.h -- C-ABI of the MI355X (gfx950) routed-expert MoE layer.
 *
 * The layer (sources: "add A4W4 and FP8 P2P transport support to MegaMoE",
 * ROCm/FlyDSL #972, Motivation and Technical Details; "feat(moe): FlyDSL
 * MegaMoE fused EP-MoE integration", ROCm/ATOM #1666, summary bullets;
 * "[HIP] gfx950 A8W4 fused_moe configs for DSv4.1 TP-sharded experts",
 * ROCm/aiter #6125, Motivation and Changes):
 *
 *   1. top-k softmax routing of router logits [T, E];
 *   2. dispatch: the T*top_k (token, slot) assignments grouped by expert
 *      (one device holds every expert, so dispatch is a permutation);
 *   3. BF16 activations quantised once per token to MXFP8 (E4M3, "A8W4") or
 *      MXFP4 (E2M1, "A4W4") with one E8M0 scale per 1x32 block;
 *   4. GEMM1 against the MXFP4 gate/up weights of each assignment's expert,
 *      SwiGLU h = silu(gate) * up, h re-quantised to the activation format;
 *   5. GEMM2 against the MXFP4 down weights, each row scaled by its routing
 *      weight; the top_k rows of a token summed in FP32 in slot order and
 *      rounded once to BF16.
 *
 * Conventions (all calls):
 *   - Every pointer argument is a DEVICE pointer on the current HIP device
 *     unless stated otherwise; the caller owns it.  Calls only enqueue work on
 *     the given stream (0 = the legacy default stream) unless stated.
 *   - Errors are returned as moe_status; nothing aborts.  Arguments are
 *     validated before anything is enqueued; a failing call enqueues nothing
 *     (HIP launch failures excepted: then MOE_ERR_HIP).  moe_last_error()
 *     returns a thread-local description of the last failure.
 *   - MX layouts at the ABI are canonical: E2M1 codes are packed two per byte,
 *     the even element in the low nibble; E4M3 codes take one byte (OCP
 *     E4M3FN); E8M0 scales are one byte per 1x32 block along the contraction
 *     dimension, row-major, value 2^(byte - 127).
 *   - Limits: 1 <= E <= 1024, 1 <= top_k <= min(E, 8), H and I positive
 *     multiples of 128, 0 <= T <= 2^20; byte offsets are 64-bit throughout.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_layer *moe_layer_t;

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, size out of range, bad enum    */
    MOE_ERR_UNSUPPORTED = -2, /* not a gfx950 device                           */
    MOE_ERR_WORKSPACE = -3,   /* workspace smaller than moe_workspace_bytes()  */
    MOE_ERR_OOM = -4,         /* device allocation failed (prepare only)       */
    MOE_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed     */
} moe_status;

/* Activation format of one forward call (chosen per call against the same
 * MXFP4 weights; aiter #6125 Motivation: A8W4 vs A4W4). */
typedef enum {
    MOE_ACT_MXFP8_E4M3 = 0, /* A8W4 */
    MOE_ACT_MXFP4_E2M1 = 1  /* A4W4 */
} moe_act_dtype;

/*
 * Copy and repack one layer's canonical MXFP4 expert weights into memory the
 * layer owns (ATOM #1666 summary: weights are shuffled once at build time; the
 * expert count is stored explicitly, never inferred from shapes).
 *
 *   E, H, I    experts, hidden size, intermediate size (per expert)
 *   w13        [E][2I][H/2] E2M1 pairs; rows [0, I) are the gate rows and
 *              rows [I, 2I) the up rows of each expert (the gate/up pairing
 *              that SwiGLU needs is kept by the repack)
 *   w13_scale  [E][2I][H/32] E8M0
 *   w2         [E][H][I/2]  E2M1 pairs (down projection, contraction over I)
 *   w2_scale   [E][H][I/32] E8M0
 *   s          stream for the repack; the call synchronises s before
 *              returning, after which the canonical buffers may be freed
 *   out        host pointer receiving the handle
 *
 * This is the only call that allocates device memory (about the canonical
 * size: E*I*H*(3/2 + 3/32) bytes).  Returns MOE_ERR_OOM if that fails.
 */
moe_status moe_prepare_weights(int E, int H, int I, const void *w13, const void *w13_scale,
                               const void *w2, const void *w2_scale, hipStream_t s,
                               moe_layer_t *out);

/* ---- weight sets owned by the caller, swapped per layer -------------------
 * The pages run one fused MoE object for every layer of the model and swap
 * its stage-1 weight pointers per layer ("FlyDSL MegaMoE fused EP-MoE
 * integration", summary: the per-layer weight swap targets the fused
 * kernel's runtime weight pointers).  Here: weights packed once into device
 * memory the caller owns, and a handle (plan table, device properties) whose
 * forward calls read the weight set last bound to it. */
typedef struct {
    void *w13;        /* packed gate/up codes,  bytes[0] of moe_packed_weight_bytes */
    void *w13_scale;  /* packed gate/up scales, bytes[1]                            */
    void *w2;         /* packed down codes,     bytes[2]                            */
    void *w2_scale;   /* packed down scales,    bytes[3]                            */
} moe_packed_weights;

/* Host out bytes[4]: the sizes of the four packed buffers of an (E, H, I)
 * expert set (equal to the canonical buffers' sizes).  MOE_ERR_INVALID_ARG on
 * dimensions moe_prepare_weights rejects. */
moe_status moe_packed_weight_bytes(int E, int H, int I, size_t bytes[4]);

/* Repack canonical weights (layouts as in moe_prepare_weights) into the
 * caller's device buffers dst (16-byte aligned, sizes from
 * moe_packed_weight_bytes, not overlapping the sources).  Enqueue only: no
 * allocation, no synchronisation; the sources must stay valid until the
 * repack on s has run. */
moe_status moe_pack_weights(int E, int H, int I, const void *w13, const void *w13_scale,
                            const void *w2, const void *w2_scale, const moe_packed_weights *dst,
                            hipStream_t s);

/* A handle for (E, H, I) layers that owns no weights: forward calls fail
 * with MOE_ERR_INVALID_ARG until moe_bind_weights has given it a set.
 * Allocates no device memory. */
moe_status moe_create_layer(int E, int H, int I, moe_layer_t *out);

/* Point the handle's later calls at the packed set w (device pointers,
 * copied into the handle; the memory stays the caller's and must outlive
 * the calls that read it).  w == NULL returns a handle made by
 * moe_prepare_weights to its own weights (and unbinds a moe_create_layer
 * handle).  A forward call reads the pointers bound when it is enqueued, so
 * rebinding between calls on one stream, or between HIP-graph captures, is
 * safe; it mutates the handle, so it is not concurrent with calls enqueuing
 * on the same handle from other threads. */
moe_status moe_bind_weights(moe_layer_t layer, const moe_packed_weights *w);

/* Release a handle and its device memory (synchronises the device first).
 * NULL is ignored. */
void moe_destroy(moe_layer_t layer);

/* Bytes of workspace moe_forward needs for (T, top_k, act); 0 on invalid
 * arguments (see moe_last_error). */
size_t moe_workspace_bytes(moe_layer_t layer, int T, int top_k, moe_act_dtype act);

/*
 * One forward pass of the layer.
 *
 *   x        [T][H] bf16 tokens
 *   logits   [T][E] fp32 router logits
 *   top_k    experts per token
 *   act      activation format
 *   y        [T][H] bf16 output (may not alias x)
 *   ws       device workspace of at least moe_workspace_bytes(layer, T,
 *            top_k, act) bytes, 256-byte aligned; its contents need not be
 *            initialised and are overwritten
 *
 * Only enqueues kernels on s: no allocation, no host synchronisation and no
 * memcpy, so the call can be captured into a HIP graph.  T == 0 is a no-op.
 * Calls sharing a workspace must be ordered (same stream); different
 * workspaces may run concurrently against one handle, except that a call
 * running the fused plan (MOE_PLAN_FUSED, opt-in) needs the device's compute
 * units to itself: beside other long-running work its bounded waits can give
 * up, which moe_fused_status reports.
 */
moe_status moe_forward(moe_layer_t layer, const void *x, const float *logits, int T, int top_k,
                       moe_act_dtype act, void *y, void *ws, size_t ws_bytes, hipStream_t s);

/* How the weighted GEMM2 rows travel to the FP32 top-k sum ("add A4W4 and FP8
 * P2P transport support to MegaMoE", Technical Details: the combine payload
 * is BF16 or fp8 1x32 blockwise).  FP32 (the default) adds no rounding; BF16
 * rounds each weighted row element to nearest even; FP8 quantises each row
 * along H in 1x32 blocks exactly as the activation quantiser does (E4M3,
 * E8M0 block exponent floor(log2 amax) - 8) and dequantises it in the
 * combine.  The staging buffer shrinks from 4 to 2 or 33/32 bytes per
 * element; the sum stays FP32 in slot order and is rounded once to BF16. */
typedef enum {
    MOE_COMBINE_FP32 = 0,
    MOE_COMBINE_BF16 = 1,
    MOE_COMBINE_FP8 = 2
} moe_combine;

/* moe_forward with the combine transport in flags (a moe_combine value; other
 * bits must be zero).  moe_forward(...) == moe_forward_ex(..., 0, ...). */
moe_status moe_forward_ex(moe_layer_t layer, const void *x, const float *logits, int T, int top_k,
                          moe_act_dtype act, uint32_t flags, void *y, void *ws, size_t ws_bytes,
                          hipStream_t s);

/* The layer fed with activations that are already MX-quantised (the pages
 * benchmark this "prequant" end to end beside the BF16 entry: "add A4W4 and
 * FP8 P2P transport support to MegaMoE", Test Plan).  Steps 1, 2 and 4-7 run
 * as in moe_forward_ex; step 3 is skipped and GEMM1 reads
 *   x_codes  [T][H] E4M3 bytes (act MXFP8) or [T][H/2] packed E2M1 (MXFP4,
 *            element 2c in the low nibble of byte c), 16-byte aligned
 *   x_scales [T][H/32] E8M0 bytes, 4-byte aligned
 * in the layout moe_quant_act writes, so moe_quant_act followed by this call
 * gives exactly moe_forward_ex's output.  The buffers are read, never
 * written; the workspace is the one moe_forward takes (its activation-code
 * region is left unused).  Errors as for moe_forward_ex.  E4M3 codes 0x7F and
 * 0xFF are NaN in OCP E4M3FN (moe_quant_act never writes them): they are not
 * valid input, and the output rows of a token holding one are unspecified
 * (NaN propagates through that token's experts). */
moe_status moe_forward_prequant(moe_layer_t layer, const uint8_t *x_codes, const uint8_t *x_scales,
                                const float *logits, int T, int top_k, moe_act_dtype act,
                                uint32_t flags, void *y, void *ws, size_t ws_bytes,
                                hipStream_t s);

/* Whether a forward call on workspace ws (for T, top_k, act) had a wait of
 * the fused plan give up (MOE_PLAN_FUSED: a GEMM2 work item waits, with a
 * bound, for the GEMM1 items of its rows; past the bound it goes on with
 * whatever rows it reads, so that call's output is unreliable).  Every
 * forward call clears the flag in its routing launch, so read it after the
 * call and before the next call on the same workspace.  Waits for stream s,
 * copies the flag to *gave_up (host): 0 = no wait gave up (always so for the
 * stream and tiled plans), 1 = at least one did.  Not graph-capturable (it
 * synchronises). */
moe_status moe_fused_status(moe_layer_t layer, const void *ws, int T, int top_k,
                            moe_act_dtype act, hipStream_t s, int32_t *gave_up);

/* ---- a forward call that allocates nothing --------------------------------
 * For callers that cannot allocate device memory or pass a workspace of their
 * own (code under HIP-graph capture, tight serving loops, harnesses that
 * forbid allocation): moe_forward_ex with the forward workspace in a static
 * device array of the library, MOE_NOALLOC_SCRATCH_BYTES on every device the
 * library runs on (held until the process ends; its device address is looked
 * up once per device, when a layer is made there or at the first call).
 * Arguments and results as for moe_forward_ex, without ws / ws_bytes.  A call
 * whose workspace (moe_workspace_bytes) exceeds the array fails with
 * MOE_ERR_WORKSPACE before anything is enqueued (64 MiB holds, e.g., the
 * 7168 x 3072, top_k = 6 layer up to T = 300 with the FP32 transport).  The
 * call allocates nothing (no hipMalloc, no allocating library routine).
 * Every call on a device shares that device's array and leaves it holding
 * its intermediate results; calls that overlap on one device (other streams,
 * other threads, other handles) race on it and must be ordered by the
 * caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(moe_layer_t layer, const void *x, const float *logits, int T,
                               int top_k, moe_act_dtype act, uint32_t flags, void *y,
                               hipStream_t s);

/* Regions of the forward workspace, for inspection after a call (all device
 * pointers into ws; layouts as listed). */
typedef enum {
    MOE_WS_IDS = 0,     /* [T][top_k] int32 expert ids, slot order           */
    MOE_WS_WEIGHTS,     /* [T][top_k] fp32 routing weights                   */
    MOE_WS_COUNTS,      /* [E] int32 assignments per expert                  */
    MOE_WS_OFFSETS,     /* [E+1] int32 exclusive prefix sum of counts        */
    MOE_WS_PERM,        /* [T*top_k] int32 assignment ids t*top_k+j, grouped
                           by expert, ascending within an expert             */
    MOE_WS_A1_CODES,    /* [T][H] (E4M3) or [T][H/2] (E2M1) token codes      */
    MOE_WS_A1_SCALES,   /* [T][H/32] E8M0                                    */
    MOE_WS_A2_CODES,    /* SwiGLU codes of sorted row p (the assignment
                           perm[p]), K-step-major: [I/128][T*top_k][128]
                           E4M3 or [I/128][T*top_k][64] packed E2M1 (K step
                           s of every row, then step s + 1)                 */
    MOE_WS_A2_SCALES,   /* [I/128][T*top_k][4] E8M0, the same rows and steps
                           (the four 1x32 blocks of a step)                 */
    MOE_WS_ROWS,        /* [T*top_k][H] GEMM2 rows times their routing weight,
                           row p is the assignment perm[p]: fp32 (FP32
                           transport), bf16 (BF16), or E4M3 codes followed by
                           [T*top_k][H/32] E8M0 scales (FP8)                */
    MOE_WS_SLOT,        /* [T*top_k] int32: row of assignment a in perm    */
    MOE_WS_NUM
} moe_ws_region;

/* Byte offsets of each region inside the workspace (offs has MOE_WS_NUM
 * entries, host memory). */
moe_status moe_workspace_offsets(moe_layer_t layer, int T, int top_k, moe_act_dtype act,
                                 size_t *offs);

/* ---- stage entry points: the same kernels moe_forward launches ---------- */

/* Step 1 (aiter #6125 Changes: the top-k softmax kernel).  For each token the
 * top_k largest logits are taken, larger first, equal logits by lower expert
 * index; w[t][j] = exp(l_j - m) / sum over the picks of exp(l - m), which is
 * the softmax over all E renormalised over the picks.  Logits are finite or
 * infinite; with a NaN logit in a row the picks of that row are unspecified
 * (they are still distinct experts below E).
 *   logits [T][E] fp32 -> ids [T][top_k] int32, w [T][top_k] fp32. */
moe_status moe_route(const float *logits, int T, int E, int top_k, int32_t *ids, float *w,
                     hipStream_t s);

/* Workspace bytes moe_sort needs for (T, E, top_k). */
size_t moe_sort_workspace_bytes(int T, int E, int top_k);

/* Step 2 (FlyDSL #972 Technical Details: dispatch).  ids [T][top_k] int32 ->
 * counts [E], offsets [E+1] (exclusive prefix sum), perm [T*top_k]: the flat
 * assignment ids a = t*top_k + j grouped by ascending expert and ascending a
 * within an expert (a deterministic, stable order).  Every id must lie in
 * [0, E) and a token's top_k ids must be distinct (as routing produces). */
moe_status moe_sort(const int32_t *ids, int T, int E, int top_k, int32_t *counts,
                    int32_t *offsets, int32_t *perm, void *ws, size_t ws_bytes, hipStream_t s);

/* Step 3 (FlyDSL #972 Technical Details: quantise BF16 activations with
 * per-1x32 E8M0 scales).  x [T][H] bf16 -> codes [T][H] (E4M3) or [T][H/2]
 * (E2M1), scales [T][H/32].  Block exponent floor(log2(amax)) - emax (8 for
 * E4M3, 2 for E2M1) clamped to [-127, 127] (an all-zero block gets byte 0);
 * elements rounded to nearest even and saturated, the sign of zero kept. */
moe_status moe_quant_act(const void *x, int T, int H, moe_act_dtype act, uint8_t *codes,
                         uint8_t *scales, hipStream_t s);

/* ---- per-layer plan table ---------------------------------------------------
 * The GEMM variant and tile height of a forward call follow a table keyed by
 * token count, like the tuned configuration tables the pages keep per token
 * bucket ("[HIP] gfx950 A8W4 fused_moe configs for DSv4.1 TP-sharded
 * experts", Changes: tuned entries per token count; "add A4W4 and FP8 P2P
 * transport support to MegaMoE", Technical Details: BM profiles chosen by
 * token count).  A layer starts with an empty table; calls no entry matches
 * use the built-in choice (at most 4 rows per expert: decode for T <= 2, else
 * stream; otherwise tiled with BM from the expected expert load, at least 64
 * rows).  Every plan computes the same result
 * (parity is tested per plan); plans differ only in speed. */
typedef enum {
    MOE_PLAN_STREAM = 0, /* 16-row m-tiles, K split over the waves, weights to VGPRs */
    MOE_PLAN_TILED = 1,  /* BM-row m-blocks staged in LDS, 256 weight rows per item */
    MOE_PLAN_FUSED = 2,  /* the stream items of both GEMMs in one persistent launch
                            (the pages' MegaMoE runs Stage1 and Stage2 as one
                            launch: "add A4W4 and FP8 P2P transport support to
                            MegaMoE"); a GEMM2 item waits on a device-side count
                            for its 16 rows' SwiGLU activations.  The launch
                            sizes its grid to the workgroups the device holds at
                            once; work on other streams (or another fused call)
                            that keeps CUs busy for seconds can make its bounded
                            waits give up, and then the call's output is wrong:
                            moe_fused_status reports it.  Opt-in: never the
                            built-in choice, nor the tuner's unless asked */
    MOE_PLAN_DECODE = 3  /* the stream GEMM1, then GEMM2 token-major: a work item
                            is (token, 32 output columns) over all its top_k
                            experts, which sums the token's weighted rows in
                            FP32 in slot order and writes y itself (no combine
                            launch; "feat(moe): FlyDSL MegaMoE fused EP-MoE
                            integration", summary: one fused operation).  With
                            the BF16 or FP8 combine transport the call runs the
                            stream plan instead */
} moe_plan_variant;

typedef struct {
    int32_t act;     /* moe_act_dtype the entry applies to                        */
    int32_t top_k;   /* top_k the entry applies to                                */
    int32_t t_max;   /* applies to calls with T <= t_max; the first matching entry
                        in table order is used                                    */
    int32_t variant; /* moe_plan_variant                                          */
    int32_t rows;    /* token rows per work item: 16 for MOE_PLAN_STREAM,
                        MOE_PLAN_FUSED and MOE_PLAN_DECODE; for
                        MOE_PLAN_TILED 32, 64, 96, 128, 160 or 192 (both
                        activation formats)                                       */
} moe_plan;

/* Replace the layer's table with plans[0 .. n-1] (host array, copied; at most
 * 256 entries; n == 0 clears it).  Every entry is validated first; on an
 * invalid one the table is left unchanged and MOE_ERR_INVALID_ARG returned.
 * Mutates the handle: not concurrent with forward calls on the same layer. */
moe_status moe_set_plans(moe_layer_t layer, const moe_plan *plans, int n);

/* The plan a forward call (T, top_k, act) on this layer uses (host out). */
moe_status moe_get_plan(moe_layer_t layer, int T, int top_k, moe_act_dtype act, moe_plan *out);

/* ---- kernel timing for benchmarks (not thread-safe; mutates the handle) -- */

/* Kernels moe_forward launches, in order. */
typedef enum {
    MOE_K_ROUTE = 0, MOE_K_SORT_HIST, MOE_K_SORT_SCAN, MOE_K_SORT_SCATTER, MOE_K_QUANT,
    MOE_K_GEMM1, MOE_K_GEMM2, MOE_K_COMBINE, MOE_K_NUM
} moe_kernel_id;

/* When enabled, each moe_forward records HIP events around every kernel on
 * its stream (up to max_calls calls are kept; later calls are not timed).
 * Enabling resets the record.  Events are created here, not in forward. */
moe_status moe_profile_enable(moe_layer_t layer, int enable, int max_calls);

/* Waits for the recorded events and writes, per moe_kernel_id, the summed
 * milliseconds (ms[MOE_K_NUM], host) over *ncalls timed calls. */
moe_status moe_profile_read(moe_layer_t layer, float *ms, int *ncalls);

/* ---- errors --------------------------------------------------------------- */
const char *moe_status_str(moe_status st);
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
