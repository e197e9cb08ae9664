"""ctypes binding of liboscar_kv.so: argument marshalling only.

The functions carry the C ABI's names; every step of the append and decode path
runs in the library's gfx950 kernels.  torch supplies device memory and the
stream handle.  Importing this module loads the library and raises if it has
not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; OSCAR_KV_LIBRARY selects another build of the same library
# (the sanitized host build of the CPU tests)
LIB_PATH = os.environ.get("OSCAR_KV_LIBRARY") or os.path.join(_HERE, "liboscar_kv.so")

OSCAR_OK = 0
OSCAR_ERR_INVALID_ARG = -1
OSCAR_ERR_OUT_OF_MEMORY = -2
OSCAR_ERR_CAPACITY = -3
OSCAR_ERR_HIP = -4
OSCAR_ERR_UNSUPPORTED = -5
KV_INT2 = 0
KV_BF16 = 1
OUT_F32 = 0
OUT_BF16 = 1
OUT_F16 = 2
CODEBOOK_UNIFORM = 0
CODEBOOK_LLOYD_MAX = 1

EXPORTED = [
    "oscar_kv_create", "oscar_kv_append", "oscar_int2_decode_attn", "oscar_kv_destroy",
    "oscar_last_error", "oscar_kv_length", "oscar_kv_device_bytes", "oscar_kv_set_num_splits",
    "oscar_kv_set_decode_impl", "oscar_kv_export", "oscar_kv_append_dump", "oscar_quantize_rows",
    "oscar_kv_profile_enable", "oscar_kv_profile_read", "oscar_stream_copy", "oscar_stream_read",
    "oscar_kv_decode_step", "oscar_prefill_attn", "oscar_int2_decode_attn_noalloc",
    "oscar_quantize_rows_lloyd_max", "oscar_kv_append_seq", "oscar_kv_reset_seq", "oscar_kv_seq_length",
    "oscar_kv_set_one_round",
]


class OscarError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"oscar status {code}: {msg}")
        self.code = code


class oscar_kv_config(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32), ("max_batch", C.c_int32), ("num_q_heads", C.c_int32),
        ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("max_context", C.c_int32),
        ("sink_tokens", C.c_int32), ("recent_tokens", C.c_int32), ("group_size", C.c_int32),
        ("k_clip", C.c_float), ("v_clip", C.c_float), ("k_dtype", C.c_int32),
        ("v_dtype", C.c_int32), ("rot_k", C.POINTER(C.c_float)), ("rot_v", C.POINTER(C.c_float)),
        ("device", C.c_int32), ("absorb_v_rotation", C.c_int32), ("in_quant_hadamard", C.c_int32),
        ("codebook", C.c_int32), ("lm_ratio", C.c_float),
    ]


def load_library(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build the HIP library first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = C.CDLL(path)
    vp, i32, f32 = C.c_void_p, C.c_int32, C.c_float
    sig = {
        "oscar_kv_create": ([C.POINTER(oscar_kv_config), C.POINTER(vp)], C.c_int),
        "oscar_kv_append": ([vp, i32, vp, vp, i32, i32, vp], C.c_int),
        "oscar_int2_decode_attn": ([vp, i32, vp, vp, i32, i32, f32, vp], C.c_int),
        "oscar_int2_decode_attn_noalloc": ([vp, i32, vp, vp, i32, i32, f32, vp], C.c_int),
        "oscar_kv_destroy": ([vp], C.c_int),
        "oscar_last_error": ([], C.c_char_p),
        "oscar_kv_length": ([vp, i32, C.POINTER(i32)], C.c_int),
        "oscar_kv_device_bytes": ([vp, C.POINTER(C.c_size_t)], C.c_int),
        "oscar_kv_set_num_splits": ([vp, i32], C.c_int),
        "oscar_kv_set_decode_impl": ([vp, i32], C.c_int),
        "oscar_kv_set_one_round": ([vp, i32], C.c_int),
        "oscar_kv_export": ([vp, i32, i32, vp, vp, vp, vp], C.c_int),
        "oscar_kv_append_dump": ([vp, i32, vp, vp, i32, i32, vp, vp, vp], C.c_int),
        "oscar_quantize_rows": ([vp, i32, i32, i32, f32, vp, vp, vp], C.c_int),
        "oscar_quantize_rows_lloyd_max": ([vp, i32, i32, i32, f32, vp, vp, vp], C.c_int),
        "oscar_kv_append_seq": ([vp, i32, i32, vp, vp, i32, vp], C.c_int),
        "oscar_kv_reset_seq": ([vp, i32, vp], C.c_int),
        "oscar_kv_seq_length": ([vp, i32, i32, C.POINTER(i32)], C.c_int),
        "oscar_kv_profile_enable": ([vp, i32], C.c_int),
        "oscar_kv_profile_read": ([vp, i32, C.POINTER(C.c_double), C.POINTER(C.c_int64)], C.c_int),
        "oscar_stream_copy": ([vp, vp, C.c_size_t, vp], C.c_int),
        "oscar_stream_read": ([vp, C.c_size_t, vp, vp], C.c_int),
        "oscar_kv_decode_step": ([vp, i32, vp, vp, vp, vp, i32, i32, f32, vp], C.c_int),
        "oscar_prefill_attn": ([vp, i32, vp, vp, i32, i32, i32, f32, vp], C.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = load_library()


def _check(rc: int):
    if rc != OSCAR_OK:
        raise OscarError(rc, _lib.oscar_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------- C-ABI names

def oscar_last_error() -> str:
    return _lib.oscar_last_error().decode()


def oscar_kv_create(cfg: oscar_kv_config) -> int:
    h = C.c_void_p()
    _check(_lib.oscar_kv_create(C.byref(cfg), C.byref(h)))
    return h.value


def oscar_kv_append(kv, layer, k, v, batch, n_new, stream=None):
    _check(_lib.oscar_kv_append(kv, layer, _ptr(k), _ptr(v), batch, n_new, _stream(stream)))


def oscar_int2_decode_attn(kv, layer, q, out, out_dtype, batch, softmax_scale=0.0, stream=None):
    _check(_lib.oscar_int2_decode_attn(kv, layer, _ptr(q), _ptr(out), out_dtype, batch,
                                       float(softmax_scale), _stream(stream)))


def oscar_int2_decode_attn_noalloc(kv, layer, q, out, out_dtype, batch, softmax_scale=0.0, stream=None):
    _check(_lib.oscar_int2_decode_attn_noalloc(kv, layer, _ptr(q), _ptr(out), out_dtype, batch,
                                               float(softmax_scale), _stream(stream)))


def oscar_kv_decode_step(kv, layer, k, v, q, out, out_dtype, batch, softmax_scale=0.0, stream=None):
    _check(_lib.oscar_kv_decode_step(kv, layer, _ptr(k), _ptr(v), _ptr(q), _ptr(out), out_dtype, batch,
                                     float(softmax_scale), _stream(stream)))


def oscar_prefill_attn(kv, layer, q, out, out_dtype, batch, n_q, softmax_scale=0.0, stream=None):
    _check(_lib.oscar_prefill_attn(kv, layer, _ptr(q), _ptr(out), out_dtype, batch, n_q,
                                   float(softmax_scale), _stream(stream)))


def oscar_kv_destroy(kv):
    _check(_lib.oscar_kv_destroy(kv))


def oscar_kv_length(kv, layer) -> int:
    t = C.c_int32()
    _check(_lib.oscar_kv_length(kv, layer, C.byref(t)))
    return t.value


def oscar_kv_device_bytes(kv) -> int:
    n = C.c_size_t()
    _check(_lib.oscar_kv_device_bytes(kv, C.byref(n)))
    return n.value


def oscar_kv_set_num_splits(kv, n):
    _check(_lib.oscar_kv_set_num_splits(kv, n))


def oscar_kv_set_decode_impl(kv, impl):
    _check(_lib.oscar_kv_set_decode_impl(kv, impl))


def oscar_kv_set_one_round(kv, blocks):
    _check(_lib.oscar_kv_set_one_round(kv, blocks))


def oscar_kv_append_dump(kv, layer, k, v, batch, n_new, k_rot, v_rot, stream=None):
    _check(_lib.oscar_kv_append_dump(kv, layer, _ptr(k), _ptr(v), batch, n_new, _ptr(k_rot),
                                     _ptr(v_rot), _stream(stream)))


def oscar_quantize_rows(x, rows, D, G, clip, codes, meta, stream=None):
    _check(_lib.oscar_quantize_rows(_ptr(x), rows, D, G, float(clip), _ptr(codes), _ptr(meta),
                                    _stream(stream)))


def oscar_kv_append_seq(kv, layer, seq, k, v, n_new, stream=None):
    _check(_lib.oscar_kv_append_seq(kv, layer, seq, _ptr(k), _ptr(v), n_new, _stream(stream)))


def oscar_kv_reset_seq(kv, seq, stream=None):
    _check(_lib.oscar_kv_reset_seq(kv, seq, _stream(stream)))


def oscar_kv_seq_length(kv, layer, seq):
    t = C.c_int32()
    _check(_lib.oscar_kv_seq_length(kv, layer, seq, C.byref(t)))
    return t.value


def oscar_quantize_rows_lloyd_max(x, rows, D, G, ratio, codes, meta, stream=None):
    _check(_lib.oscar_quantize_rows_lloyd_max(_ptr(x), rows, D, G, float(ratio), _ptr(codes), _ptr(meta),
                                              _stream(stream)))


def oscar_kv_profile_enable(kv, enable):
    _check(_lib.oscar_kv_profile_enable(kv, 1 if enable else 0))


def oscar_kv_profile_read(kv, kernel_class):
    """-> (total_ms, launches) of the HIP events recorded for a kernel class."""
    ms, n = C.c_double(), C.c_int64()
    _check(_lib.oscar_kv_profile_read(kv, kernel_class, C.byref(ms), C.byref(n)))
    return ms.value, n.value


def oscar_stream_copy(src, dst, nbytes, stream=None):
    _check(_lib.oscar_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def oscar_stream_read(src, nbytes, xor_out, stream=None):
    _check(_lib.oscar_stream_read(_ptr(src), nbytes, _ptr(xor_out), _stream(stream)))


def oscar_kv_export(kv, layer, which, codes, meta, sink, ring):
    """numpy arrays (or None) receive the canonical host copy."""
    p = lambda a: None if a is None else a.ctypes.data
    _check(_lib.oscar_kv_export(kv, layer, which, p(codes), p(meta), p(sink), p(ring)))


# ---------------------------------------------------------------- convenience


class KVCache:
    """Owning wrapper of one oscar_kv handle."""

    def __init__(self, num_layers, max_batch, num_q_heads, num_kv_heads, head_dim, max_context,
                 sink_tokens, recent_tokens, group_size=128, k_clip=0.96, v_clip=0.92,
                 k_dtype=KV_INT2, v_dtype=KV_INT2, rot_k=None, rot_v=None, device=0, absorb_v_rotation=0,
                 in_quant_hadamard=0, codebook=CODEBOOK_UNIFORM, lm_ratio=1.16):
        self.num_layers, self.max_batch = num_layers, max_batch
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.max_context, self.N, self.M, self.G = max_context, sink_tokens, recent_tokens, group_size
        self.k_dtype, self.v_dtype = k_dtype, v_dtype
        self._rk = None if rot_k is None else np.ascontiguousarray(rot_k, np.float32)
        self._rv = None if rot_v is None else np.ascontiguousarray(rot_v, np.float32)
        fp = lambda a: None if a is None else a.ctypes.data_as(C.POINTER(C.c_float))
        cfg = oscar_kv_config(num_layers, max_batch, num_q_heads, num_kv_heads, head_dim,
                              max_context, sink_tokens, recent_tokens, group_size, k_clip, v_clip,
                              k_dtype, v_dtype, fp(self._rk), fp(self._rv), device, absorb_v_rotation,
                              in_quant_hadamard, codebook, lm_ratio)
        self.handle = oscar_kv_create(cfg)

    def close(self):
        if self.handle:
            oscar_kv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def length(self, layer):
        return oscar_kv_length(self.handle, layer)

    def append(self, layer, k, v, stream=None):
        B, n = k.shape[0], k.shape[1]
        oscar_kv_append(self.handle, layer, k, v, B, n, stream)

    def append_seq(self, layer, seq, k, v, stream=None):
        """k, v: [n_new, Hkv, D] of sequence seq, appended at its own length."""
        oscar_kv_append_seq(self.handle, layer, seq, k, v, k.shape[0], stream)

    def reset_seq(self, seq, stream=None):
        oscar_kv_reset_seq(self.handle, seq, stream)

    def seq_length(self, layer, seq):
        return oscar_kv_seq_length(self.handle, layer, seq)

    def append_dump(self, layer, k, v, k_rot, v_rot, stream=None):
        B, n = k.shape[0], k.shape[1]
        oscar_kv_append_dump(self.handle, layer, k, v, B, n, k_rot, v_rot, stream)

    def decode_attn(self, layer, q, out, out_dtype=OUT_F32, softmax_scale=0.0, stream=None):
        oscar_int2_decode_attn(self.handle, layer, q, out, out_dtype, q.shape[0], softmax_scale, stream)

    def decode_attn_noalloc(self, layer, q, out, out_dtype=OUT_F32, softmax_scale=0.0, stream=None):
        oscar_int2_decode_attn_noalloc(self.handle, layer, q, out, out_dtype, q.shape[0], softmax_scale, stream)

    def prefill_attn(self, layer, q, out, out_dtype=OUT_F32, softmax_scale=0.0, stream=None):
        """Causal attention of the last q.shape[1] cached positions' queries over the cache."""
        oscar_prefill_attn(self.handle, layer, q, out, out_dtype, q.shape[0], q.shape[1], softmax_scale, stream)

    def decode_step(self, layer, k, v, q, out, out_dtype=OUT_F32, softmax_scale=0.0, stream=None):
        """append(k, v) of one token then decode_attn(q) -> out, fused where possible."""
        oscar_kv_decode_step(self.handle, layer, k, v, q, out, out_dtype, q.shape[0], softmax_scale, stream)

    def set_num_splits(self, n):
        oscar_kv_set_num_splits(self.handle, n)

    def set_decode_impl(self, impl):
        oscar_kv_set_decode_impl(self.handle, impl)

    def set_one_round(self, blocks):
        oscar_kv_set_one_round(self.handle, blocks)

    def device_bytes(self):
        return oscar_kv_device_bytes(self.handle)

    def profile_enable(self, enable=True):
        oscar_kv_profile_enable(self.handle, enable)

    def profile_read(self, kernel_class):
        return oscar_kv_profile_read(self.handle, kernel_class)

    def export(self, layer, which):
        """Canonical host copy of plane `which` (0 K, 1 V) for max_batch sequences."""
        T = self.length(layer)
        B, H, D, G = self.max_batch, self.num_kv_heads, self.head_dim, self.G
        bf16 = (self.v_dtype if which else self.k_dtype) == KV_BF16
        if bf16:
            full = np.zeros((B, H, T, D), np.uint16)
            oscar_kv_export(self.handle, layer, which, full, None, None, None)
            return {"full": full}
        codes = np.zeros((B, H, T, D // 4), np.uint8)
        meta = np.zeros((B, H, T, D // G, 2), np.uint16)
        sink = np.zeros((B, H, self.N, D), np.uint16)
        ring = np.zeros((B, H, self.M, D), np.uint16)
        oscar_kv_export(self.handle, layer, which, codes, meta, sink, ring)
        return {"codes": codes, "s16": meta[..., 0].view(np.float16), "z16": meta[..., 1].view(np.float16),
                "sink": sink, "ring": ring}
