"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects invalid arguments before touching a device."""
import ctypes
import os
import re

import pytest

import quantized_moe_expert_softmax_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from quantized_moe_expert_softmax_amd import build
        build.build()
    return moe.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_calls():
    names = header_functions()
    for n in ("moe_prepare_weights", "moe_forward", "moe_workspace_bytes", "moe_destroy",
              "moe_route", "moe_sort", "moe_quant_act"):
        assert n in names
    assert sorted(names) == sorted(moe.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for n in header_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for st, name in ((0, "MOE_OK"), (-1, "MOE_ERR_INVALID_ARG"), (-3, "MOE_ERR_WORKSPACE"),
                     (-4, "MOE_ERR_OOM"), (-5, "MOE_ERR_HIP"), (-2, "MOE_ERR_UNSUPPORTED")):
        assert lib.moe_status_str(st).decode() == name


def _err(lib):
    return lib.moe_last_error().decode()


def test_prepare_rejects_bad_dims(lib):
    h = ctypes.c_void_p()
    p = ctypes.c_void_p(256)  # never dereferenced: validation fails first
    for E, H, I in ((0, 256, 128), (1025, 256, 128), (8, 100, 128), (8, 256, 96), (8, -128, 128)):
        st = lib.moe_prepare_weights(E, H, I, p, p, p, p, None, ctypes.byref(h))
        assert st == moe.MOE_ERR_INVALID_ARG, (E, H, I)
        assert h.value is None
    assert "I=96" in _err(lib) or "H=" in _err(lib)
    st = lib.moe_prepare_weights(8, 256, 128, None, p, p, p, None, ctypes.byref(h))
    assert st == moe.MOE_ERR_INVALID_ARG and "null" in _err(lib)
    st = lib.moe_prepare_weights(8, 256, 128, p, p, p, p, None, None)
    assert st == moe.MOE_ERR_INVALID_ARG


def test_forward_rejects_null_handle(lib):
    p = ctypes.c_void_p(256)
    st = lib.moe_forward(None, p, p, 4, 2, 0, p, p, 1 << 20, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "handle" in _err(lib)
    st = lib.moe_forward_ex(None, p, p, 4, 2, 0, 1, p, p, 1 << 20, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "handle" in _err(lib)
    st = lib.moe_forward_prequant(None, p, p, p, 4, 2, 0, 0, p, p, 1 << 20, None)
    assert st == moe.MOE_ERR_INVALID_ARG and "handle" in _err(lib)
    assert lib.moe_workspace_bytes(None, 4, 2, 0) == 0
    offs = (ctypes.c_size_t * moe.MOE_WS_NUM)()
    assert lib.moe_workspace_offsets(None, 4, 2, 0, offs) == moe.MOE_ERR_INVALID_ARG


def test_stage_calls_validate(lib):
    p = ctypes.c_void_p(256)
    assert lib.moe_route(p, 4, 2000, 2, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(p, 4, 8, 9, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(p, 4, 4, 5, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(p, -1, 8, 2, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route(p, 0, 8, 2, p, p, None) == moe.MOE_OK  # T == 0: nothing to do
    assert lib.moe_quant_act(p, 4, 100, 0, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quant_act(p, 4, 256, 7, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_quant_act(p, 0, 256, 0, p, p, None) == moe.MOE_OK
    assert lib.moe_quant_act(ctypes.c_void_p(8), 4, 256, 0, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_sort(p, 4, 0, 1, p, p, p, p, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_sort(p, 4, 8, 2, p, p, p, p, 16, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_sort(p, 4, 8, 2, p, p, p, ctypes.c_void_p(300), 1 << 20, None) == \
        moe.MOE_ERR_INVALID_ARG


def test_sort_workspace_size(lib):
    # [E+1] m-block prefix, [ceil(T/256)][E] block histograms, [N/16 + E + 1]
    # m-block experts, [N] inverse permutation; each region 256-byte aligned
    al = lambda n: -(-n // 256) * 256
    for T, E, k in ((1, 8, 2), (32768, 384, 6), (1000, 128, 3)):
        N = T * k
        want = al((E + 1) * 4) + al(-(-T // 256) * E * 4) + al((N // 16 + E + 1) * 4) + al(N * 4)
        assert lib.moe_sort_workspace_bytes(T, E, k) == want
    assert lib.moe_sort_workspace_bytes(4, 0, 1) == 0
    assert lib.moe_sort_workspace_bytes(4, 8, 9) == 0


def test_profile_calls_validate(lib):
    assert lib.moe_profile_enable(None, 1, 10) == moe.MOE_ERR_INVALID_ARG
    ms = (ctypes.c_float * moe.MOE_K_NUM)()
    n = ctypes.c_int()
    assert lib.moe_profile_read(None, ms, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG


def test_product_path_has_no_oracle_dependency():
    """The package never imports the oracle (which is test infrastructure)."""
    pkg = os.path.dirname(moe.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(root, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "moe_oracle" not in src and "liboracle" not in src, f


def test_plan_calls_validate(lib):
    entry = (moe.MoePlan * 1)(moe.MoePlan(0, 2, 16, moe.MOE_PLAN_STREAM, 16))
    assert lib.moe_set_plans(None, entry, 1) == moe.MOE_ERR_INVALID_ARG and "handle" in _err(lib)
    out = moe.MoePlan()
    assert lib.moe_get_plan(None, 4, 2, 0, ctypes.byref(out)) == moe.MOE_ERR_INVALID_ARG


def test_packed_weight_bytes_equal_canonical_sizes(lib):
    """The packed layout holds exactly the canonical bytes (host-only call)."""
    for E, H, I in ((8, 256, 128), (384, 7168, 3072), (1, 128, 128), (128, 5120, 640)):
        assert moe.moe_packed_weight_bytes(E, H, I) == [
            E * 2 * I * H // 2, E * 2 * I * H // 32, E * H * I // 2, E * H * I // 32]
    out = (ctypes.c_size_t * 4)()
    for E, H, I in ((0, 256, 128), (8, 100, 128), (8, 256, 96)):
        assert lib.moe_packed_weight_bytes(E, H, I, out) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_packed_weight_bytes(8, 256, 128, None) == moe.MOE_ERR_INVALID_ARG


def test_weight_binding_calls_validate(lib):
    p = ctypes.c_void_p(256)
    h = ctypes.c_void_p()
    assert lib.moe_create_layer(0, 256, 128, ctypes.byref(h)) == moe.MOE_ERR_INVALID_ARG
    assert h.value is None
    assert lib.moe_create_layer(8, 256, 128, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_bind_weights(None, None) == moe.MOE_ERR_INVALID_ARG
    dst = moe.PackedWeights(256, 256, 0, 256)
    st = lib.moe_pack_weights(8, 256, 128, p, p, p, p, ctypes.byref(dst), None)
    assert st == moe.MOE_ERR_INVALID_ARG and "null" in _err(lib)
    dst = moe.PackedWeights(256, 256, 264, 256)
    st = lib.moe_pack_weights(8, 256, 128, p, p, p, p, ctypes.byref(dst), None)
    assert st == moe.MOE_ERR_INVALID_ARG and "aligned" in _err(lib)
    assert lib.moe_pack_weights(8, 256, 128, p, p, p, p, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_pack_weights(8, 100, 128, p, p, p, p, ctypes.byref(dst), None) == \
        moe.MOE_ERR_INVALID_ARG
