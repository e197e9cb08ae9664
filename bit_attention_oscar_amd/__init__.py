"""OSCAR INT2 KV cache for MI355X (gfx950): append (rotate, clip, INT2 quantize,
pack) and fused mixed-precision split-K decode attention, behind a C ABI
(include/oscar_kv.h).  The binding lives in `oscar_kv`; importing it loads the
built library and fails loudly when it is missing."""

__all__ = ["oscar_kv", "build"]
