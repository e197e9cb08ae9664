"""Shared helpers of the GPU tests: build a cache on both sides from the same
seeded inputs and compare.  The oracle side never sees a value computed by the
HIP path except where a test states it works on the identical (exported) cache
or on the GPU's own fp32 rotated vectors."""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass

import numpy as np

import oracle as orc
import synth


ATTN_TOL = 2e-3       # attention output against the oracle, relative L2


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def row_errors(got, want) -> np.ndarray:
    """Relative L2 error of every output row (one query head of one sequence,
    or of one query position), over the last axis."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    g = g.reshape(-1, g.shape[-1])
    w = w.reshape(-1, w.shape[-1])
    return np.linalg.norm(g - w, axis=1) / np.maximum(np.linalg.norm(w, axis=1), 1e-300)


def oracle_err(got, want, tol: float = ATTN_TOL) -> float:
    """Relative L2 error of the whole output against the oracle's; asserts
    on the way that every row is within tol on its own (a small error confined
    to one head cannot hide in the norm of many)."""
    rows = row_errors(got, want)
    worst = float(rows.max())
    assert worst <= tol, f"row {int(rows.argmax())}: rel L2 {worst:.3e} > {tol:.1e}"
    return rel_l2(got, want)


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


@dataclass
class Shape:
    L: int = 1
    B: int = 1
    Hq: int = 4
    Hkv: int = 1
    D: int = 128
    N: int = 64
    M: int = 256
    k_clip: float = 0.96
    v_clip: float = 0.92
    k_dtype: int = 0
    v_dtype: int = 0
    outliers: str = "fixed"
    dist: str = "normal"
    seed: int = 0
    outlier_scale: float = 8.0
    codebook: int = 0          # 0: min/max with the clip ratios; 1: Lloyd-Max with lm_ratio
    lm_ratio: float = 1.16


def make_rotations(shape: Shape, kind: str):
    D, L = shape.D, shape.L
    if kind == "identity":
        return None, None
    if kind == "haar":
        return synth.rotations(L, D, shape.seed, "rot_k"), synth.rotations(L, D, shape.seed, "rot_v")
    if kind == "exact":
        # bit-reversal permutation (K) and a signed permutation (V): the rotated
        # vectors are exact in fp32, so every stored bit is fixed by the inputs
        pbr = orc.bit_reversal_permutation(D)
        g = synth.rng(shape.seed, 0, "rot_v")
        perm = g.permutation(D)
        sp = np.zeros((D, D), np.float32)
        sp[np.arange(D), perm] = np.where(g.random(D) < 0.5, -1.0, 1.0)
        return np.stack([pbr] * L), np.stack([sp] * L)
    if kind == "exact_layers":
        # a different signed permutation per layer for K and for V: exact in
        # fp32, so every stored bit of every layer is fixed by the inputs, and
        # a layer that read another layer's rotation would differ
        out = []
        for role in ("rot_k", "rot_v"):
            mats = []
            for l in range(L):
                g = synth.rng(shape.seed, l, role)
                m = np.zeros((D, D), np.float32)
                m[np.arange(D), g.permutation(D)] = np.where(g.random(D) < 0.5, -1.0, 1.0)
                mats.append(m)
            out.append(np.stack(mats))
        return out[0], out[1]
    raise ValueError(kind)


def inputs(shape: Shape, T: int, layer: int = 0, chunk: int = 0):
    mask = synth.outlier_mask(shape.D, shape.Hkv, shape.seed, layer, shape.outliers)
    k = synth.kv_bits(shape.B, T, shape.Hkv, shape.D, shape.seed, layer, "k", mask, shape.dist, chunk,
                      shape.outlier_scale)
    v = synth.kv_bits(shape.B, T, shape.Hkv, shape.D, shape.seed, layer, "v", mask, shape.dist, chunk,
                      shape.outlier_scale)
    return k, v, mask


def query(shape: Shape, mask, layer: int = 0, step: int = 0):
    return synth.q_bits(shape.B, shape.Hq, shape.Hkv, shape.D, shape.seed, layer, mask, shape.dist, step,
                        shape.outlier_scale)


def compare_planes(gp, op, T, N, M, label):
    """GPU export (canonical) vs oracle logical planes, bit for bit."""
    if "full" in gp:
        np.testing.assert_array_equal(gp["full"], op.win, err_msg=f"{label} bf16 plane")
        return
    np.testing.assert_array_equal(gp["codes"], orc.pack_codes(op.codes), err_msg=f"{label} codes")
    np.testing.assert_array_equal(gp["s16"].view(np.uint16), op.s16.view(np.uint16), err_msg=f"{label} s16")
    np.testing.assert_array_equal(gp["z16"].view(np.uint16), op.z16.view(np.uint16), err_msg=f"{label} z16")
    for t in range(min(N, T)):
        np.testing.assert_array_equal(gp["sink"][:, :, t], op.win[:, :, t], err_msg=f"{label} sink {t}")
    if M > 0:
        for t in range(max(N, T - M), T):
            np.testing.assert_array_equal(gp["ring"][:, :, t % M], op.win[:, :, t], err_msg=f"{label} ring {t}")


def gpu_cache(ok, shape: Shape, rk, rv, max_context: int, absorb_v: int = 0, hadamard: int = 0):
    return ok.KVCache(shape.L, shape.B, shape.Hq, shape.Hkv, shape.D, max_context, shape.N, shape.M,
                      128, shape.k_clip, shape.v_clip, shape.k_dtype, shape.v_dtype, rk, rv, 0, absorb_v,
                      hadamard, shape.codebook, shape.lm_ratio)


def oracle_cache(shape: Shape, rk, rv):
    cfg = orc.OracleConfig(num_layers=shape.L, batch=shape.B, num_q_heads=shape.Hq,
                           num_kv_heads=shape.Hkv, head_dim=shape.D, sink_tokens=shape.N,
                           recent_tokens=shape.M, k_clip=shape.k_clip, v_clip=shape.v_clip,
                           k_dtype=shape.k_dtype, v_dtype=shape.v_dtype, codebook=shape.codebook,
                           lm_ratio=shape.lm_ratio)
    return orc.OracleKVCache(cfg, rk, rv)


def planes_from_export(exp: dict, T: int, N: int, M: int, codebook: int = 0):
    if "full" in exp:
        return orc.planes_from_storage(None, None, None, None, None, T, N, M, full_bits=exp["full"])
    return orc.planes_from_storage(exp["codes"], exp["s16"], exp["z16"], exp["sink"], exp["ring"], T, N, M,
                                   codebook=codebook)


def oracle_on_exported(cache, layer, q_bits, shape: Shape, rk, rv, batch_idx=None, absorb_v=False):
    """Oracle attention over the cache exported from the GPU (identical cache)."""
    T = cache.length(layer)
    ek, ev = cache.export(layer, 0), cache.export(layer, 1)
    sel = slice(None) if batch_idx is None else batch_idx
    sub = lambda e: {k: v[sel] for k, v in e.items()}
    kp = planes_from_export(sub(ek), T, shape.N, shape.M, shape.codebook)
    vp = planes_from_export(sub(ev), T, shape.N, shape.M, shape.codebook)
    D = shape.D
    Rk = rk[layer] if rk is not None else np.eye(D, dtype=np.float32)
    Rv = rv[layer] if rv is not None else np.eye(D, dtype=np.float32)
    qb = q_bits if batch_idx is None else q_bits[batch_idx]
    return orc.decode_attention(qb, kp, vp, Rk, Rv, shape.Hkv, shape.N, shape.M, 128,
                                shape.k_dtype, shape.v_dtype, absorb_v=absorb_v)
