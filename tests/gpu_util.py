"""Shared helpers of the GPU parity tests (device transfer, comparisons)."""
import numpy as np

# Final-output criteria (relative L2 norm over the compared rows and the
# largest per-row relative L2 error): the FP32 accumulation order of the
# GPU differs from the oracle's, which moves a few requantised SwiGLU codes
# across rounding boundaries.
REL_L2_TOL = 1e-2
ROW_REL_TOL = 3e-2
# Routing weights: the GPU evaluates exp(l_j - l_0) / sum over the picks in
# FP32 (a few roundings); the oracle rounds the exact value once.
ROUTE_ULP_TOL = 4


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    import torch
    return dev(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def host(t):
    return t.detach().cpu().numpy()


def bf16_host_bits(t):
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_diff(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def output_errors(y_bits, ref_bits):
    y = bf16_to_f64(y_bits)
    r = bf16_to_f64(ref_bits)
    rel = np.linalg.norm(y - r) / max(np.linalg.norm(r), 1e-30)
    rown = np.linalg.norm(r, axis=1)
    rowe = np.linalg.norm(y - r, axis=1)
    row_rel = np.where(rown > 0, rowe / np.maximum(rown, 1e-30), rowe)
    return rel, float(row_rel.max())


def assert_output_close(y_bits, ref_bits, what=""):
    rel, row = output_errors(y_bits, ref_bits)
    assert rel <= REL_L2_TOL and row <= ROW_REL_TOL, \
        "%s: rel L2 %.3g (tol %.0e), max row rel %.3g (tol %.0e)" % (what, rel, REL_L2_TOL, row,
                                                                      ROW_REL_TOL)
    return rel, row


def ws_view(ws, offs, region, nbytes, dtype=np.uint8):
    """Host copy of a workspace region."""
    import torch
    o = offs[region]
    return ws[o:o + nbytes].cpu().numpy().view(dtype)


def unpack_fp4(packed):
    packed = np.asarray(packed)
    out = np.zeros(packed.shape[:-1] + (packed.shape[-1] * 2,), np.int64)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out
