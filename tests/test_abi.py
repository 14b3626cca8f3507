"""C-ABI library: loads, exports every symbol the header declares, and rejects
bad arguments on the host before any HIP call.  CPU only (no compute calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_moe_relu_amd as dm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dm.LIB_PATH):
        from sparse_moe_relu_amd.build import build_library
        build_library(verbose=False)
    return dm.load_library()


def _declared_functions():
    with open(os.path.join(ROOT, "include", "deco_moe.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(deco_moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(dm.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings(lib):
    for st in (dm.DECO_OK, dm.DECO_ERR_INVALID_ARG, dm.DECO_ERR_UNSUPPORTED, dm.DECO_ERR_OUT_OF_MEMORY,
               dm.DECO_ERR_HIP):
        assert dm.status_string(st) and dm.status_string(st) != "unknown status"
    assert dm.status_string(12345) == "unknown status"


@pytest.mark.parametrize("kw,expect", [
    (dict(), dm.DECO_OK),
    (dict(d=2048, E=56, F=128, Fs=1024), dm.DECO_OK),
    (dict(d=4096, E=112, F=128, Fs=2048), dm.DECO_OK),
    (dict(E=256), dm.DECO_OK),
    (dict(F=256, Fs=32), dm.DECO_OK),
    (dict(d=0), dm.DECO_ERR_INVALID_ARG),
    (dict(E=0), dm.DECO_ERR_INVALID_ARG),
    (dict(T=0), dm.DECO_ERR_INVALID_ARG),
    (dict(eps=-1.0), dm.DECO_ERR_INVALID_ARG),
    (dict(eps=float("nan")), dm.DECO_ERR_INVALID_ARG),
    (dict(d=96), dm.DECO_ERR_UNSUPPORTED),
    (dict(E=257), dm.DECO_ERR_UNSUPPORTED),
    (dict(F=48), dm.DECO_ERR_UNSUPPORTED),
    (dict(F=512), dm.DECO_ERR_UNSUPPORTED),
    (dict(Fs=48), dm.DECO_ERR_UNSUPPORTED),
    (dict(T=(1 << 20) + 1), dm.DECO_ERR_UNSUPPORTED),
    (dict(top_k=1), dm.DECO_OK),
    (dict(top_k=8), dm.DECO_OK),
    (dict(top_k=9), dm.DECO_ERR_INVALID_ARG),
    (dict(top_k=-1), dm.DECO_ERR_INVALID_ARG),
    # every packed matrix stays below 2 GiB (32-bit buffer offsets)
    (dict(d=32768, Fs=16384, dtype="bf16"), dm.DECO_OK),              # 1 GiB
    (dict(d=32768, Fs=16352), dm.DECO_OK),                            # fp32, 2 GiB - 4 MiB
    (dict(d=32768, Fs=16384), dm.DECO_ERR_UNSUPPORTED),               # fp32, exactly 2 GiB
])
def test_check_config(lib, kw, expect):
    a = dict(d=64, E=8, F=32, Fs=64, T=16, dtype="f32", eps=1e-6, top_k=0)
    a.update(kw)
    cfg = dm.make_config(a["d"], a["E"], a["F"], a["Fs"], a["T"], a["dtype"], a["eps"], a["top_k"])
    assert dm.check_config(cfg) == expect


def test_shared_workspace_flag_range(lib):
    cfg = dm.make_config(64, 8, 32, 64, 16, "f32", shared_workspace=True)
    assert cfg.shared_workspace == 1 and dm.check_config(cfg) == dm.DECO_OK
    cfg.shared_workspace = 2
    assert dm.check_config(cfg) == dm.DECO_ERR_INVALID_ARG


def test_bad_dtype_is_unsupported(lib):
    cfg = dm.make_config(64, 8, 32, 64, 16, "f32")
    cfg.dtype = 7
    assert dm.check_config(cfg) == dm.DECO_ERR_UNSUPPORTED
    assert lib.deco_moe_check_config(None) == dm.DECO_ERR_INVALID_ARG


def test_host_side_rejections_touch_no_device(lib):
    cfg = dm.make_config(64, 8, 32, 64, 16, "f32")
    h = ctypes.c_void_p(1234)
    # null weight pointer: rejected before any HIP call, *out_layer cleared
    st = lib.deco_moe_load_weights(ctypes.byref(cfg), None, None, None, None, None, None, None, None,
                                   ctypes.byref(h))
    assert st == dm.DECO_ERR_INVALID_ARG and not h.value
    # invalid config is reported before the pointer checks
    bad = dm.make_config(96, 8, 32, 64, 16, "f32")
    assert lib.deco_moe_load_weights(ctypes.byref(bad), None, None, None, None, None, None, None, None,
                                     ctypes.byref(h)) == dm.DECO_ERR_UNSUPPORTED
    assert lib.deco_moe_load_weights(ctypes.byref(cfg), None, None, None, None, None, None, None, None,
                                     None) == dm.DECO_ERR_INVALID_ARG
    # gated loader: same order of checks; a missing up-projection is rejected too
    st = lib.deco_moe_load_weights_gated(ctypes.byref(cfg), *([None] * 9), ctypes.byref(h))
    assert st == dm.DECO_ERR_INVALID_ARG and not h.value
    h.value = 1234
    assert lib.deco_moe_load_weights_gated(ctypes.byref(bad), *([None] * 9),
                                           ctypes.byref(h)) == dm.DECO_ERR_UNSUPPORTED and not h.value
    assert lib.deco_moe_load_weights_gated(ctypes.byref(cfg), *([None] * 9), None) == dm.DECO_ERR_INVALID_ARG
    # null layer
    assert lib.deco_moe_forward(None, None, 0, None, None) == dm.DECO_ERR_INVALID_ARG
    assert lib.deco_moe_forward_path(None, None, 4, None, None, 1) == dm.DECO_ERR_INVALID_ARG
    assert lib.deco_moe_copy_routing(None, 1, None, None, None) == dm.DECO_ERR_INVALID_ARG
    assert lib.deco_moe_copy_mean_up(None, None, None) == dm.DECO_ERR_INVALID_ARG
    assert lib.deco_moe_read_error_flags(None, None) == dm.DECO_ERR_INVALID_ARG
    lib.deco_moe_free(None)
    assert lib.deco_moe_timing_read(-1, None, None, None) == dm.DECO_ERR_INVALID_ARG


def test_product_path_has_no_oracle_dependency():
    # the binding and the HIP sources never reference the oracle package
    pkg = os.path.join(ROOT, "sparse_moe_relu_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(dirpath, fn), encoding="utf-8") as f:
                    src = f.read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), fn
                assert "oracle/" not in src, fn


def test_backward_flag_and_host_side_backward_calls(lib):
    cfg = dm.make_config(64, 8, 32, 64, 16, "f32", backward=True)
    assert dm.check_config(cfg) == dm.DECO_OK
    cfg.backward = 2
    assert dm.check_config(cfg) == dm.DECO_ERR_INVALID_ARG
    # null layer / grads: rejected before any HIP call
    g = dm.DecoGrads()
    assert lib.deco_moe_backward(None, None, None, 4, 0.0, ctypes.byref(g), None) == dm.DECO_ERR_INVALID_ARG
    assert lib.deco_moe_backward(None, None, None, 4, 0.0, None, None) == dm.DECO_ERR_INVALID_ARG


@pytest.mark.parametrize("ratio,target", [(0.25, 0.2), (0.15, 0.2), (0.2, 0.2), (0.0, 0.05)])
def test_sparsity_coef_update_matches_the_oracle_rule(lib, ratio, target):
    import oracle
    for coef in (1.0, 0.37, 3e-3):
        got = dm.sparsity_coef_update(coef, ratio, target, 1.002)
        want = oracle.sparsity_coef_update(np.float32(coef), np.float32(ratio), np.float32(target),
                                           np.float32(1.002))
        assert np.float32(got) == np.float32(want)


def test_ablation_switches_are_validated(lib):
    cfg = dm.make_config(64, 8, 32, 64, 16, "f32", backward=True, shared_rms=True)
    assert dm.check_config(cfg) == dm.DECO_ERR_UNSUPPORTED   # the backward covers the DECO layer only
    cfg = dm.make_config(64, 8, 32, 64, 16, "f32", normsilu_mean=False, normsilu_rms=False, scalar_lambda=True)
    assert dm.check_config(cfg) == dm.DECO_OK and cfg.normsilu == 3
    for field, bad in (("normsilu", 4), ("normsilu", -1), ("scalar_lambda", 2), ("shared_rms", 7)):
        c = dm.make_config(64, 8, 32, 64, 16, "f32")
        setattr(c, field, bad)
        assert dm.check_config(c) == dm.DECO_ERR_INVALID_ARG, field


def test_backward_needs_two_routed_experts(lib):
    # with one routed expert the mean term equals its projection (h~ = 0)
    assert dm.check_config(dm.make_config(64, 1, 32, 64, 16, "bf16", backward=True)) == dm.DECO_ERR_UNSUPPORTED
    assert dm.check_config(dm.make_config(64, 2, 32, 64, 16, "bf16", backward=True)) == dm.DECO_OK
    assert dm.check_config(dm.make_config(64, 1, 32, 64, 16, "bf16")) == dm.DECO_OK
