"""The C-ABI library loads, exports every entry point include/bw.h declares, and rejects bad
arguments on the host side before touching a GPU. No GPU needed."""
import ctypes
import os
import re

import pytest

import memory_bound_autoregressive_amd as bw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "bw.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(bw_\w+)\s*\(", text, flags=re.M)))


def _lib():
    if not os.path.exists(bw.LIB_PATH):
        pytest.skip("libbw.so is not built")
    return bw.lib()


def test_header_declares_the_step_api():
    names = _declared()
    for n in ("bw_model_load_synthetic", "bw_kv_pool_create", "bw_decode_step", "bw_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert set(_declared()) == set(bw.EXPORTS)


def test_null_and_shape_errors_are_reported_without_a_gpu():
    L = _lib()
    assert L.bw_decode_step(None, None, None, None, None, 1, 1, 1, None, None, None) == bw.BW_EINVAL
    assert "null" in bw.bw_last_error()
    assert L.bw_model_load_synthetic(None, 0, None) == bw.BW_EINVAL
    out = ctypes.c_void_p()
    cfg = bw.make_config(dict(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=96, ffn_dim=1024,
                              vocab=1024), 64, 1)
    assert L.bw_model_load_synthetic(ctypes.byref(cfg), 1, ctypes.byref(out)) == bw.BW_EINVAL
    assert "head_dim" in bw.bw_last_error()
    cfg = bw.make_config(dict(n_layers=1, d_model=256, n_q_heads=3, n_kv_heads=2, head_dim=64, ffn_dim=1024,
                              vocab=1024), 64, 1)
    assert L.bw_model_load_synthetic(ctypes.byref(cfg), 1, ctypes.byref(out)) == bw.BW_EINVAL
    assert L.bw_kv_pool_create(None, 4, ctypes.byref(out)) == bw.BW_EINVAL
    assert L.bw_model_free(None) == bw.BW_OK
    assert L.bw_kv_pool_free(None) == bw.BW_OK
    assert L.bw_check_device_error(None, None, None) == bw.BW_EINVAL
    assert L.bw_debug_kv_round(3, None, 1, None, None, None) == bw.BW_EINVAL
    # both pool-synthesis forms refuse a null pool or array before touching the GPU
    assert L.bw_kv_pool_synthesize(None, 1, None, None, None, 1, 1) == bw.BW_EINVAL
    assert L.bw_kv_pool_synthesize_async(None, 1, None, None, None, 1, 1, None) == bw.BW_EINVAL
    assert "null" in bw.bw_last_error()
    cfg = bw.make_config(dict(n_layers=1, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn_dim=1024,
                              vocab=1024), 64, 1)
    cfg.kv_dtype = 4
    assert L.bw_model_load_synthetic(ctypes.byref(cfg), 1, ctypes.byref(out)) == bw.BW_EINVAL
    assert "kv_dtype" in bw.bw_last_error()


def test_binding_raises_when_library_is_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(bw, "_lib", None)
    monkeypatch.setattr(bw, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError):
        bw.lib()
