"""CPU-runnable checks of the C-ABI library: it loads, exports every function
include/oscar_kv.h declares, and rejects bad arguments before touching the GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar_kv.h")


@pytest.fixture(scope="module")
def ok():
    from bit_attention_oscar_amd import oscar_kv
    return oscar_kv


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_\w+)\s*\(", text)))


def test_header_symbols_exported(ok):
    names = declared_functions()
    assert {"oscar_kv_create", "oscar_kv_append", "oscar_int2_decode_attn", "oscar_kv_destroy"} <= set(names)
    lib = C.CDLL(ok.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(ok.EXPORTED)


def _cfg(ok, **kw):
    base = dict(num_layers=1, max_batch=1, num_q_heads=4, num_kv_heads=1, head_dim=128, max_context=64,
                sink_tokens=4, recent_tokens=8, group_size=128, k_clip=0.96, v_clip=0.92, k_dtype=0,
                v_dtype=0, rot_k=None, rot_v=None, device=0)
    base.update(kw)
    c = ok.oscar_kv_config()
    for k, v in base.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("field,value,code", [
    ("num_layers", 0, -1), ("max_batch", 0, -1), ("num_kv_heads", 3, -1), ("num_kv_heads", 0, -1),
    ("head_dim", 96, -5), ("head_dim", 256, -5), ("group_size", 64, -5), ("max_context", 0, -1),
    ("sink_tokens", -1, -1), ("recent_tokens", -3, -1), ("k_clip", 0.0, -1), ("v_clip", 1.5, -1),
    ("k_dtype", 7, -1), ("num_q_heads", 64, -5), ("absorb_v_rotation", 2, -1),
    ("in_quant_hadamard", 64, -1), ("in_quant_hadamard", 1, -1), ("codebook", 2, -1), ("codebook", -1, -1),
])
def test_create_rejects_bad_config(ok, field, value, code):
    cfg = _cfg(ok, **{field: value})
    h = C.c_void_p()
    rc = ok._lib.oscar_kv_create(C.byref(cfg), C.byref(h))
    assert rc == code, (rc, ok.oscar_last_error())
    assert h.value is None
    assert ok.oscar_last_error()


def test_null_arguments(ok):
    lib = ok._lib
    assert lib.oscar_kv_create(None, None) == ok.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_kv_destroy(None) == ok.OSCAR_OK
    assert lib.oscar_kv_append(None, 0, None, None, 1, 1, None) == ok.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_int2_decode_attn(None, 0, None, None, 0, 1, 0.0, None) == ok.OSCAR_ERR_INVALID_ARG
    t = C.c_int32()
    assert lib.oscar_kv_length(None, 0, C.byref(t)) == ok.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_kv_set_num_splits(None, 1) == ok.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_kv_export(None, 0, 0, None, None, None, None) == ok.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_kv_profile_enable(None, 1) == ok.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_prefill_attn(None, 0, None, None, 0, 1, 1, 0.0, None) == ok.OSCAR_ERR_INVALID_ARG
    assert lib.oscar_kv_decode_step(None, 0, None, None, None, None, 0, 1, 0.0, None) == ok.OSCAR_ERR_INVALID_ARG


@pytest.mark.parametrize("rows,D,G,clip,code", [
    (-1, 128, 128, 0.96, -1), (4, 96, 128, -0.5, -5), (4, 128, 64, 0.96, -5), (4, 128, 128, 0.0, -1),
    (4, 128, 128, 1.01, -1), (4, 128, 128, 0.96, -1),   # NULL pointers with rows > 0
])
def test_quantize_rows_rejects(ok, rows, D, G, clip, code):
    rc = ok._lib.oscar_quantize_rows(None, rows, D, G, clip, None, None, None)
    assert rc == code, ok.oscar_last_error()


@pytest.mark.parametrize("ratio,lm_ratio_code", [(0.0, -1), (-1.0, -1), (16.5, -1), (float("nan"), -1)])
def test_lloyd_max_ratio_rejected(ok, ratio, lm_ratio_code):
    """LM_RATIO outside (0, 16] is refused by create and by the quantizer hook;
    with the Lloyd-Max codebook the clip ratios are not checked."""
    cfg = _cfg(ok, codebook=1, lm_ratio=ratio, k_clip=0.0, v_clip=0.0)
    h = C.c_void_p()
    assert ok._lib.oscar_kv_create(C.byref(cfg), C.byref(h)) == lm_ratio_code
    assert h.value is None
    assert ok._lib.oscar_quantize_rows_lloyd_max(None, 4, 128, 128, ratio, None, None, None) == -1


def test_lloyd_max_config_passes_validation(ok):
    """A valid Lloyd-Max config (clip ratios zero: unused) gets past the argument
    checks to device set-up."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    cfg = _cfg(ok, codebook=1, lm_ratio=1.16, k_clip=0.0, v_clip=0.0)
    h = C.c_void_p()
    assert ok._lib.oscar_kv_create(C.byref(cfg), C.byref(h)) == ok.OSCAR_ERR_HIP
    assert ok._lib.oscar_quantize_rows_lloyd_max(None, 0, 128, 128, 1.16, None, None, None) == ok.OSCAR_OK


def test_quantize_rows_zero_rows_is_noop(ok):
    assert ok._lib.oscar_quantize_rows(None, 0, 128, 128, 0.96, None, None, None) == ok.OSCAR_OK


def test_create_without_gpu_fails_cleanly(ok):
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    cfg = _cfg(ok)
    h = C.c_void_p()
    rc = ok._lib.oscar_kv_create(C.byref(cfg), C.byref(h))
    assert rc in (ok.OSCAR_ERR_HIP, ok.OSCAR_ERR_INVALID_ARG)
    assert h.value is None
