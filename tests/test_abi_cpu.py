"""The C-ABI library without a GPU: it loads, exports every symbol that
include/moe_layer.h declares, and rejects bad arguments on the host before
any device work (no compute call is made here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_layer.h")


def _lib():
    from moe_ffn_amd import layer
    if not os.path.exists(layer.LIB_PATH):
        pytest.fail("libmoe_layer.so is not built (python -m moe_ffn_amd.build)")
    return layer.load_library(), layer


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(["moe_abi_version", "moe_last_error", "moe_layer_create",
                            "moe_layer_create_fp8", "moe_layer_create_w8a8",
                            "moe_fp8_quantize_rows",
                            "moe_layer_forward", "moe_layer_set_bias", "moe_layer_get_bias",
                            "moe_layer_update_bias",
                            "moe_layer_timing_start", "moe_layer_timing_stop",
                            "moe_layer_destroy", "moe_stack_create", "moe_stack_forward",
                            "moe_stack_capture", "moe_stack_replay", "moe_stack_destroy",
                            "moe_stack_set_eda", "moe_stack_forward_routing",
                            "moe_layer_forward_static"])


def test_library_exports_every_declared_symbol():
    lib, layer = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"missing export {name}"
    assert set(layer.EXPORTS) == set(declared_functions())
    assert lib.moe_abi_version() == 6


def test_abi_structs_match_header_sizes():
    _, layer = _lib()
    assert ctypes.sizeof(layer.LayerConfig) == 7 * 4
    assert ctypes.sizeof(layer.LayerWeights) == 6 * 8
    assert ctypes.sizeof(layer.RoutingOut) == 6 * 8
    assert ctypes.sizeof(layer.Fp8Scales) == 3 * 8


def _cfg(layer, **kw):
    base = dict(d_model=2048, d_ff=3072, n_experts=16, top_k=1, dtype=1, rms_eps=1e-6,
                max_tokens=64)
    base.update(kw)
    return layer.LayerConfig(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 1), (dict(d_model=0), 1), (dict(top_k=0), 1), (dict(top_k=17), 1),
    (dict(max_tokens=0), 1), (dict(rms_eps=-1.0), 1), (dict(rms_eps=float("nan")), 1),
    (dict(n_experts=65, top_k=1), 4), (dict(n_experts=16, top_k=9), 4),
    (dict(d_model=2000), 4), (dict(d_ff=3000), 4), (dict(max_tokens=(1 << 20) + 1), 4),
    (dict(d_model=65536 + 256), 4), (dict(d_ff=65536 + 128), 4),
    (dict(dtype=0, d_model=6), 4),
])
def test_create_rejects_bad_configs_on_host(kw, status):
    lib, layer = _lib()
    cfg = _cfg(layer, **kw)
    w = layer.LayerWeights(16, 16, 16, 16, 16, 16)  # never dereferenced: config fails first
    h = ctypes.c_void_p(123)
    st = lib.moe_layer_create(ctypes.byref(cfg), ctypes.byref(w), None, ctypes.byref(h))
    assert st == status, lib.moe_last_error()
    assert h.value is None
    assert lib.moe_last_error()


def test_create_rejects_null_and_misaligned_weights_on_host():
    lib, layer = _lib()
    cfg = _cfg(layer)
    h = ctypes.c_void_p()
    assert lib.moe_layer_create(None, None, None, ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_create(ctypes.byref(cfg), None, None, None) == layer.MOE_ERR_INVALID_ARG
    w = layer.LayerWeights(16, 0, 16, 16, 16, 16)
    assert lib.moe_layer_create(ctypes.byref(cfg), ctypes.byref(w), None,
                                ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    w = layer.LayerWeights(16, 24, 16, 16, 16, 16)
    assert lib.moe_layer_create(ctypes.byref(cfg), ctypes.byref(w), None,
                                ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    assert b"aligned" in lib.moe_last_error()


def test_create_fp8_rejects_bad_scales_and_dtype_on_host():
    lib, layer = _lib()
    cfg = _cfg(layer)
    w = layer.LayerWeights(16, 16, 16, 16, 16, 16)
    h = ctypes.c_void_p(123)
    assert lib.moe_layer_create_fp8(ctypes.byref(cfg), ctypes.byref(w), None, None,
                                    ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    assert h.value is None and b"scales" in lib.moe_last_error()
    sc = layer.Fp8Scales(16, 0, 16)
    assert lib.moe_layer_create_fp8(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(sc), None,
                                    ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    sc = layer.Fp8Scales(16, 18, 16)
    assert lib.moe_layer_create_fp8(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(sc), None,
                                    ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    sc = layer.Fp8Scales(16, 16, 16)
    cfg32 = _cfg(layer, dtype=0)
    assert lib.moe_layer_create_fp8(ctypes.byref(cfg32), ctypes.byref(w), ctypes.byref(sc), None,
                                    ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    assert b"BF16" in lib.moe_last_error()


def test_create_w8a8_and_quantize_rows_reject_bad_arguments_on_host():
    lib, layer = _lib()
    cfg = _cfg(layer)
    w = layer.LayerWeights(16, 16, 16, 16, 16, 16)
    h = ctypes.c_void_p(123)
    assert lib.moe_layer_create_w8a8(ctypes.byref(cfg), ctypes.byref(w), None, None,
                                     ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    assert h.value is None and b"scales" in lib.moe_last_error()
    sc = layer.Fp8Scales(16, 16, 16)
    cfg32 = _cfg(layer, dtype=0)
    assert lib.moe_layer_create_w8a8(ctypes.byref(cfg32), ctypes.byref(w), ctypes.byref(sc),
                                     None, ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    q = lib.moe_fp8_quantize_rows
    assert q(16, 4, 12, 16, 16, None) == layer.MOE_ERR_INVALID_ARG      # K % 8 != 0
    assert q(16, -1, 8, 16, 16, None) == layer.MOE_ERR_INVALID_ARG      # R < 0
    assert q(None, 4, 8, 16, 16, None) == layer.MOE_ERR_INVALID_ARG     # NULL x
    assert q(24, 4, 8, 16, 16, None) == layer.MOE_ERR_INVALID_ARG       # x not 16-byte aligned
    assert b"aligned" in lib.moe_last_error()
    assert q(None, 0, 8, None, None, None) == layer.MOE_OK              # nothing to do


def test_entry_points_reject_bad_handles_and_destroy_is_null_safe():
    lib, layer = _lib()
    assert lib.moe_layer_forward(None, None, 1, None, None, None) == layer.MOE_ERR_INVALID_ARG
    bogus = (ctypes.c_uint32 * 64)()
    assert lib.moe_layer_forward(ctypes.addressof(bogus), None, 1, None, None,
                                 None) == layer.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_set_bias(None, None, None) == layer.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_update_bias(None, None, 0.01, None) == layer.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_get_bias(None, None, None) == layer.MOE_ERR_INVALID_ARG
    assert lib.moe_stack_forward(None, None, 1, None, None) == layer.MOE_ERR_INVALID_ARG
    assert lib.moe_stack_replay(None, None) == layer.MOE_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert lib.moe_stack_create(0, None, 1, ctypes.byref(h)) == layer.MOE_ERR_INVALID_ARG
    lib.moe_stack_destroy(None)
    assert lib.moe_layer_update_bias(ctypes.addressof(bogus), None, 0.01,
                                     None) == layer.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_timing_start(None, 4) == layer.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_timing_stop(None, None, None) == layer.MOE_ERR_INVALID_ARG
    lib.moe_layer_destroy(None)
    lib.moe_layer_destroy(ctypes.addressof(bogus))  # wrong magic: ignored


def test_binding_checks_caller_outputs():
    """The binding refuses an `out` tensor the library would write past or
    misread (it writes T * d elements through the pointer without a size)."""
    import torch
    from moe_ffn_amd.layer import _out_like
    h = torch.zeros((8, 64), dtype=torch.bfloat16)
    assert _out_like(h, None).shape == h.shape
    ok = torch.empty_like(h)
    assert _out_like(h, ok) is ok
    for bad in (torch.zeros((7, 64), dtype=torch.bfloat16), torch.zeros((8, 64)),
                torch.zeros((64, 8), dtype=torch.bfloat16).t()):
        with pytest.raises(ValueError):
            _out_like(h, bad)
