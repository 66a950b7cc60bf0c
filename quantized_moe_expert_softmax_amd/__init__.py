"""MI355X (gfx950) routed-expert MoE layer with MXFP4 weights and MXFP8/MXFP4
activations -- Python binding of the C-ABI in include/moe.h.

The binding only marshals arguments: every step of the layer runs in the HIP
kernels of libmoe_mi355x.so (built in-tree by ``build.py``).  If that library
is missing, every call raises; there is no fallback.

PyTorch is used for device memory and streams: tensors are passed by data
pointer, the stream is torch's current stream unless one is given.

Names mirror the C-ABI: moe_prepare_weights, moe_workspace_bytes,
moe_forward, moe_destroy, moe_route, moe_sort, moe_quant_act, plus
moe_workspace_offsets and the kernel-timing calls.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_OOM = -4
MOE_ERR_HIP = -5

MOE_ACT_MXFP8_E4M3 = 0  # A8W4
MOE_ACT_MXFP4_E2M1 = 1  # A4W4

(MOE_WS_IDS, MOE_WS_WEIGHTS, MOE_WS_COUNTS, MOE_WS_OFFSETS, MOE_WS_PERM, MOE_WS_A1_CODES,
 MOE_WS_A1_SCALES, MOE_WS_A2_CODES, MOE_WS_A2_SCALES, MOE_WS_ROWS, MOE_WS_SLOT,
 MOE_WS_NUM) = range(12)

KERNELS = ("route", "sort_hist", "sort_scan", "sort_scatter", "quant", "gemm1", "gemm2",
           "combine")
MOE_K_NUM = len(KERNELS)

EXPORTS = ("moe_prepare_weights", "moe_destroy", "moe_workspace_bytes", "moe_forward",
           "moe_forward_ex", "moe_forward_prequant", "moe_packed_weight_bytes",
           "moe_pack_weights", "moe_create_layer", "moe_bind_weights",
           "moe_workspace_offsets", "moe_route", "moe_sort_workspace_bytes", "moe_sort",
           "moe_quant_act", "moe_set_plans", "moe_get_plan", "moe_profile_enable",
           "moe_profile_read", "moe_status_str", "moe_last_error", "moe_fused_status",
           "moe_forward_noalloc")
# bytes of the static workspace moe_forward_noalloc uses (MOE_NOALLOC_SCRATCH_BYTES)
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

MOE_COMBINE_FP32 = 0  # transport of the weighted GEMM2 rows into the FP32 top-k sum
MOE_COMBINE_BF16 = 1
MOE_COMBINE_FP8 = 2

MOE_PLAN_STREAM = 0
MOE_PLAN_TILED = 1
MOE_PLAN_FUSED = 2
MOE_PLAN_DECODE = 3


class MoePlan(ctypes.Structure):
    """One plan-table entry (moe_plan in include/moe.h)."""
    _fields_ = [("act", ctypes.c_int32), ("top_k", ctypes.c_int32), ("t_max", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("rows", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}

_lock = threading.Lock()
_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (status, msg))
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libmoe_mi355x.so (raises if it was not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("HIP library %s is missing; run quantized_moe_expert_softmax_amd."
                               "build.build() first (there is no CPU fallback)" % path)
        import torch  # noqa: F401  (loads the HIP runtime the library links against)
        lib = ctypes.CDLL(path)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.moe_prepare_weights.argtypes = [I, I, I, P, P, P, P, P, ctypes.POINTER(P)]
        lib.moe_destroy.argtypes = [P]
        lib.moe_destroy.restype = None
        lib.moe_workspace_bytes.argtypes = [P, I, I, I]
        lib.moe_workspace_bytes.restype = Z
        lib.moe_forward.argtypes = [P, P, P, I, I, I, P, P, Z, P]
        lib.moe_forward_ex.argtypes = [P, P, P, I, I, I, ctypes.c_uint32, P, P, Z, P]
        lib.moe_forward_prequant.argtypes = [P, P, P, P, I, I, I, ctypes.c_uint32, P, P, Z, P]
        lib.moe_forward_noalloc.argtypes = [P, P, P, I, I, I, ctypes.c_uint32, P, P]
        lib.moe_packed_weight_bytes.argtypes = [I, I, I, P]
        lib.moe_pack_weights.argtypes = [I, I, I, P, P, P, P, P, P]
        lib.moe_create_layer.argtypes = [I, I, I, ctypes.POINTER(P)]
        lib.moe_bind_weights.argtypes = [P, P]
        lib.moe_workspace_offsets.argtypes = [P, I, I, I, P]
        lib.moe_fused_status.argtypes = [P, P, I, I, I, P, P]
        lib.moe_route.argtypes = [P, I, I, I, P, P, P]
        lib.moe_sort_workspace_bytes.argtypes = [I, I, I]
        lib.moe_sort_workspace_bytes.restype = Z
        lib.moe_sort.argtypes = [P, I, I, I, P, P, P, P, Z, P]
        lib.moe_quant_act.argtypes = [P, I, I, I, P, P, P]
        lib.moe_set_plans.argtypes = [P, P, I]
        lib.moe_get_plan.argtypes = [P, I, I, I, P]
        lib.moe_profile_enable.argtypes = [P, I, I]
        lib.moe_profile_read.argtypes = [P, P, P]
        lib.moe_status_str.argtypes = [I]
        lib.moe_status_str.restype = ctypes.c_char_p
        lib.moe_last_error.argtypes = []
        lib.moe_last_error.restype = ctypes.c_char_p
        for name in ("moe_prepare_weights", "moe_forward", "moe_forward_ex", "moe_forward_noalloc",
                     "moe_forward_prequant", "moe_packed_weight_bytes", "moe_pack_weights",
                     "moe_create_layer", "moe_bind_weights", "moe_workspace_offsets",
                     "moe_fused_status", "moe_route",
                     "moe_sort", "moe_quant_act", "moe_set_plans", "moe_get_plan",
                     "moe_profile_enable", "moe_profile_read"):
            getattr(lib, name).restype = I
        _lib = lib
        return lib


def _check(status: int):
    if status != MOE_OK:
        lib = load_library()
        raise MoeError(status, lib.moe_last_error().decode())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _require(t, dtype_bytes, shape, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.element_size() != dtype_bytes:
        raise TypeError("%s must have %d-byte elements, got %s" % (name, dtype_bytes, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


class MoeLayer:
    """Owner of a moe_layer_t handle (repacked weights of one layer)."""

    def __init__(self, handle, E, H, I):
        self.handle = handle
        self.E, self.H, self.I = E, H, I

    def __del__(self):
        self.close()

    def close(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.moe_destroy(h)
        self.handle = None


def moe_prepare_weights(E, H, I, w13, w13_scale, w2, w2_scale, stream=None) -> MoeLayer:
    """Repack canonical MXFP4 weights (uint8 device tensors) into a layer handle.

    w13 [E, 2I, H/2] (gate rows then up rows), w13_scale [E, 2I, H/32],
    w2 [E, H, I/2], w2_scale [E, H, I/32].  Synchronises the stream.
    """
    lib = load_library()
    _require(w13, 1, (E, 2 * I, H // 2), "w13")
    _require(w13_scale, 1, (E, 2 * I, H // 32), "w13_scale")
    _require(w2, 1, (E, H, I // 2), "w2")
    _require(w2_scale, 1, (E, H, I // 32), "w2_scale")
    h = ctypes.c_void_p()
    _check(lib.moe_prepare_weights(E, H, I, _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                                   _stream(stream), ctypes.byref(h)))
    return MoeLayer(h, E, H, I)


class PackedWeights(ctypes.Structure):
    """moe_packed_weights: device pointers of one packed weight set."""
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


def moe_packed_weight_bytes(E: int, H: int, I: int):
    """Sizes of the four packed buffers (w13, w13_scale, w2, w2_scale) in bytes."""
    out = (ctypes.c_size_t * 4)()
    _check(load_library().moe_packed_weight_bytes(E, H, I, out))
    return list(out)


def moe_pack_weights(E, H, I, w13, w13_scale, w2, w2_scale, stream=None):
    """Repack canonical weights into four new uint8 device tensors (the caller
    owns them; keep them alive while a layer is bound to them).  Enqueue only."""
    import torch
    lib = load_library()
    _require(w13, 1, (E, 2 * I, H // 2), "w13")
    _require(w13_scale, 1, (E, 2 * I, H // 32), "w13_scale")
    _require(w2, 1, (E, H, I // 2), "w2")
    _require(w2_scale, 1, (E, H, I // 32), "w2_scale")
    bufs = [torch.empty(n, dtype=torch.uint8, device=w13.device)
            for n in moe_packed_weight_bytes(E, H, I)]
    dst = PackedWeights(*(b.data_ptr() for b in bufs))
    _check(lib.moe_pack_weights(E, H, I, _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                                ctypes.byref(dst), _stream(stream)))
    return bufs


def moe_create_layer(E: int, H: int, I: int) -> MoeLayer:
    """A handle with no weights of its own (bind a packed set before calling)."""
    h = ctypes.c_void_p()
    _check(load_library().moe_create_layer(E, H, I, ctypes.byref(h)))
    return MoeLayer(h, E, H, I)


def moe_bind_weights(layer: MoeLayer, packed=None):
    """Point the layer's later calls at a packed set (the four tensors from
    moe_pack_weights), or back to its own weights with None."""
    lib = load_library()
    if packed is None:
        _check(lib.moe_bind_weights(layer.handle, None))
        return
    w = PackedWeights(*(b.data_ptr() for b in packed))
    _check(lib.moe_bind_weights(layer.handle, ctypes.byref(w)))


def moe_workspace_bytes(layer: MoeLayer, T: int, top_k: int, act: int) -> int:
    n = load_library().moe_workspace_bytes(layer.handle, T, top_k, act)
    if n == 0 and T >= 0:
        _check(MOE_ERR_INVALID_ARG)
    return n


def alloc_workspace(layer: MoeLayer, T: int, top_k: int, act: int, device=None):
    import torch
    n = moe_workspace_bytes(layer, T, top_k, act)
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def moe_forward(layer: MoeLayer, x, logits, top_k: int, act: int, y=None, ws=None, stream=None,
                combine: int = MOE_COMBINE_FP32):
    """y [T, H] bf16 = MoE(x [T, H] bf16, logits [T, E] fp32); enqueue only.
    combine: transport of the weighted rows into the FP32 top-k sum
    (MOE_COMBINE_FP32 -> moe_forward, else moe_forward_ex)."""
    import torch
    lib = load_library()
    T = x.shape[0]
    _require(x, 2, (T, layer.H), "x")
    _require(logits, 4, (T, layer.E), "logits")
    if y is None:
        y = torch.empty((T, layer.H), dtype=torch.bfloat16, device=x.device)
    _require(y, 2, (T, layer.H), "y")
    if ws is None:
        ws = alloc_workspace(layer, T, top_k, act, x.device)
    if combine == MOE_COMBINE_FP32:
        _check(lib.moe_forward(layer.handle, _ptr(x), _ptr(logits), T, top_k, act, _ptr(y),
                               _ptr(ws), ws.numel(), _stream(stream)))
    else:
        _check(lib.moe_forward_ex(layer.handle, _ptr(x), _ptr(logits), T, top_k, act, combine,
                                  _ptr(y), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def moe_forward_noalloc(layer: MoeLayer, x, logits, top_k: int, act: int, y,
                        combine: int = MOE_COMBINE_FP32, stream=None):
    """moe_forward with the library's static device workspace (no workspace
    argument, nothing allocated by the call; y [T, H] bf16 must be given).
    Calls on one device share that workspace: order them.  Enqueue only."""
    lib = load_library()
    T = x.shape[0]
    _require(x, 2, (T, layer.H), "x")
    _require(logits, 4, (T, layer.E), "logits")
    _require(y, 2, (T, layer.H), "y")
    _check(lib.moe_forward_noalloc(layer.handle, _ptr(x), _ptr(logits), T, top_k, act, combine,
                                   _ptr(y), _stream(stream)))
    return y


def moe_forward_prequant(layer: MoeLayer, codes, scales, logits, top_k: int, act: int, y=None,
                         ws=None, stream=None, combine: int = MOE_COMBINE_FP32):
    """y [T, H] bf16 = MoE of MX-quantised activations: codes [T, H] (MXFP8) or
    [T, H/2] (MXFP4) uint8 and scales [T, H/32] uint8, as moe_quant_act writes
    them; logits [T, E] fp32.  Enqueue only."""
    import torch
    lib = load_library()
    T = codes.shape[0]
    _require(codes, 1, (T, layer.H if act == MOE_ACT_MXFP8_E4M3 else layer.H // 2), "codes")
    _require(scales, 1, (T, layer.H // 32), "scales")
    _require(logits, 4, (T, layer.E), "logits")
    if y is None:
        y = torch.empty((T, layer.H), dtype=torch.bfloat16, device=codes.device)
    _require(y, 2, (T, layer.H), "y")
    if ws is None:
        ws = alloc_workspace(layer, T, top_k, act, codes.device)
    _check(lib.moe_forward_prequant(layer.handle, _ptr(codes), _ptr(scales), _ptr(logits), T,
                                    top_k, act, combine, _ptr(y), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return y


def moe_fused_status(layer: MoeLayer, ws, T: int, top_k: int, act: int, stream=None) -> int:
    """1 if a bounded wait of the fused plan gave up in the last forward call on
    workspace ws (that call's output is unreliable), else 0.  Synchronises."""
    out = ctypes.c_int32()
    _check(load_library().moe_fused_status(layer.handle, _ptr(ws), T, top_k, act,
                                           _stream(stream), ctypes.byref(out)))
    return out.value


def moe_workspace_offsets(layer: MoeLayer, T: int, top_k: int, act: int):
    lib = load_library()
    arr = (ctypes.c_size_t * MOE_WS_NUM)()
    _check(lib.moe_workspace_offsets(layer.handle, T, top_k, act, arr))
    return list(arr)


def moe_route(logits, top_k: int, stream=None):
    """ids [T, k] int32 and weights [T, k] fp32 from logits [T, E] fp32."""
    import torch
    lib = load_library()
    T, E = logits.shape
    _require(logits, 4, (T, E), "logits")
    ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _check(lib.moe_route(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(w), _stream(stream)))
    return ids, w


def moe_sort(ids, E: int, stream=None):
    """counts [E], offsets [E+1], perm [T*k] (int32) from ids [T, k] int32."""
    import torch
    lib = load_library()
    T, k = ids.shape
    _require(ids, 4, (T, k), "ids")
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    n = lib.moe_sort_workspace_bytes(T, E, k)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    _check(lib.moe_sort(_ptr(ids), T, E, k, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(ws),
                        ws.numel(), _stream(stream)))
    return counts, offsets, perm


def moe_quant_act(x, act: int, stream=None):
    """codes [T, H] (E4M3) or [T, H/2] (E2M1 pairs) and scales [T, H/32] uint8."""
    import torch
    lib = load_library()
    T, H = x.shape
    _require(x, 2, (T, H), "x")
    codes = torch.empty((T, H if act == MOE_ACT_MXFP8_E4M3 else H // 2), dtype=torch.uint8,
                        device=x.device)
    scales = torch.empty((T, H // 32), dtype=torch.uint8, device=x.device)
    _check(lib.moe_quant_act(_ptr(x), T, H, act, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def moe_set_plans(layer: MoeLayer, plans):
    """Install a plan table: a sequence of dicts (or MoePlan) with keys act, top_k,
    t_max, variant, rows; [] clears it."""
    arr = (MoePlan * max(len(plans), 1))()
    for i, pl in enumerate(plans):
        d = pl.as_dict() if isinstance(pl, MoePlan) else pl
        arr[i] = MoePlan(int(d["act"]), int(d["top_k"]), int(d["t_max"]), int(d["variant"]),
                         int(d["rows"]))
    _check(load_library().moe_set_plans(layer.handle, arr, len(plans)))


def moe_get_plan(layer: MoeLayer, T: int, top_k: int, act: int) -> dict:
    """The plan a forward call (T, top_k, act) uses, as a dict."""
    out = MoePlan()
    _check(load_library().moe_get_plan(layer.handle, T, top_k, act, ctypes.byref(out)))
    return out.as_dict()


def moe_profile_enable(layer: MoeLayer, enable: bool = True, max_calls: int = 1024):
    _check(load_library().moe_profile_enable(layer.handle, int(bool(enable)), max_calls))


def moe_profile_read(layer: MoeLayer):
    """{kernel name: summed ms}, number of timed calls."""
    lib = load_library()
    ms = (ctypes.c_float * MOE_K_NUM)()
    n = ctypes.c_int()
    _check(lib.moe_profile_read(layer.handle, ms, ctypes.byref(n)))
    return dict(zip(KERNELS, list(ms))), n.value
