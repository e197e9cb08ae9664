"""A model, on the CPU, of how the matrix-core decode kernels round their
operands, checked against the oracle's exact attention.

The kernels feed the 2-bit codes to fp16 matrix-core products as exact
operands; the other operand of QK^T is the rotated query and that of PV is the
softmax weight times the V scale.  Those two are rounded to fp16.  This module
repeats that rounding on top of the oracle's arithmetic (oracle functions only,
nothing from the HIP library) and measures the attention error it causes over a
sweep of outlier scales (outlier channels are the premise of the method:
"OSCAR: 2-bit KV Cache Quantization for SGLang and llama.cpp", "How the offline
rotation is fit from Q/K/V covariance"):

  * one fp16 piece (11 significant bits) per operand exceeds the 2e-3 bar on
    some rows of the tiny workload's shape, because a score's absolute error
    grows with its size and the softmax exponentiates it;
  * two pieces per operand, hi = fp16(x) and lo = fp16(x - hi) (22 bits), as
    the kernels now use, stay orders of magnitude inside it.
"""
import math

import numpy as np
import pytest

import oracle as orc
import synth

LOG2E = 1.4426950408889634
TOL = 2e-3


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def _pieces(x, n):
    """x rounded to n fp16 pieces (1: fp16(x); 2: hi + fp16(x - hi))."""
    hi = _f16(x)
    return hi if n == 1 else hi + _f16(np.asarray(x, np.float32) - np.asarray(hi, np.float32))


def kernel_model_attention(q_bits, kp, vp, rk, rv, num_kv_heads, N, M, q_pieces, p_pieces, heads=None):
    """Decode attention as the matrix-core kernels round it (one split):
      * q_rot in units of log2 (scale 1/sqrt(D) folded in), scaled per head by
        2^eq so that max |q| < 2^15, times 4^-(d % 4) (the code's bit position),
        rounded to q_pieces fp16 pieces, used against the exact codes;
        score = s_K (q . c) + z_K sum(q_rot) on INT2 positions, q_rot . k on
        window positions (fp32 window arithmetic, exact here);
      * p = 2^(score - max); on INT2 positions the PV operand s_V p 2^ev
        (2^ev from the largest V scale) is rounded to p_pieces fp16 pieces,
        and sum p z_V, sum p are exact.
    Returns the un-rotated output [B, Hq, D] (rows outside `heads` zero)."""
    B, Hq, D = q_bits.shape
    Gq = Hq // num_kv_heads
    T = kp.x32.shape[2]
    qr = orc.rotate_f64(q_bits, rk) * (LOG2E / math.sqrt(D))
    hp = orc.high_precision_mask(T, N, M)
    s4 = 4.0 ** -(np.arange(D) % 4)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        for h in range(num_kv_heads):
            Kw = orc.mixed_values(kp, b, h, T, N, M, 128, 0)
            Vw = orc.mixed_values(vp, b, h, T, N, M, 128, 0)
            ck = kp.codes[b, h, :T].astype(np.float64)
            cv = vp.codes[b, h, :T].astype(np.float64)
            sk, zk = kp.s16[b, h, :T, 0].astype(np.float64), kp.z16[b, h, :T, 0].astype(np.float64)
            sv, zv = vp.s16[b, h, :T, 0].astype(np.float64), vp.z16[b, h, :T, 0].astype(np.float64)
            ev = 15 - math.frexp(sv.max())[1]
            for j in range(h * Gq, (h + 1) * Gq):
                if heads is not None and j not in heads:
                    continue
                q = qr[b, j]
                eq = 15 - math.frexp(np.abs(q).max())[1]
                qo = _pieces(q * 2.0 ** eq * s4, q_pieces) / s4 / 2.0 ** eq
                s = np.where(hp, Kw @ q, sk * (ck @ qo) + zk * q.sum())
                p = np.exp2(s - s.max())
                po = _pieces(p * sv * 2.0 ** ev, p_pieces) / 2.0 ** ev
                o = (np.where(hp, p, 0.0)[:, None] * Vw).sum(0)
                o += (np.where(hp, 0.0, po)[:, None] * cv).sum(0) + np.where(hp, 0.0, p * zv).sum()
                out[b, j] = o / p.sum()
    return out @ np.asarray(rv, np.float64).T


def _case(B, Hq, Hkv, D, N, M, T, mode, seed, scale):
    mask = synth.outlier_mask(D, Hkv, seed, 0, mode)
    k = synth.kv_bits(B, T, Hkv, D, seed, 0, "k", mask, outlier_scale=scale)
    v = synth.kv_bits(B, T, Hkv, D, seed, 0, "v", mask, outlier_scale=scale)
    q = synth.q_bits(B, Hq, Hkv, D, seed, 0, mask, outlier_scale=scale)
    rk, rv = synth.rotations(1, D, seed, "rot_k"), synth.rotations(1, D, seed, "rot_v")
    oc = orc.OracleKVCache(orc.OracleConfig(1, B, Hq, Hkv, D, N, M), rk, rv)
    oc.append(0, k, v)
    return q, oc, rk[0], rv[0]


def _row_err(got, want, heads=None):
    g, w = got.reshape(-1, got.shape[-1]), want.reshape(-1, want.shape[-1])
    r = np.linalg.norm(g - w, axis=1) / np.linalg.norm(w, axis=1)
    if heads is not None:
        r = r[list(heads)]
    return float(r.max())


def test_two_piece_operands_hold_the_bar_tiny_sweep():
    """Tiny workload's shape (1 kv head, 4 query heads, 4 outlier channels,
    1025 tokens, sink 64, recent 256), six seeds, outlier scales 8 to 32."""
    worst1, worst2 = 0.0, 0.0
    for seed in range(6):
        for scale in (8.0, 16.0, 24.0, 32.0):
            q, oc, rk, rv = _case(1, 4, 1, 128, 64, 256, 1025, "fixed", seed, scale)
            want = oc.attend(0, q)
            one = kernel_model_attention(q, oc.k[0], oc.v[0], rk, rv, 1, 64, 256, 1, 1)
            two = kernel_model_attention(q, oc.k[0], oc.v[0], rk, rv, 1, 64, 256, 2, 2)
            worst1 = max(worst1, _row_err(one, want))
            worst2 = max(worst2, _row_err(two, want))
    print(f"worst row: one piece {worst1:.2e}, two pieces {worst2:.2e}")
    assert worst1 > TOL          # one fp16 piece is not enough at these ranges
    assert worst2 < TOL / 20     # two pieces: well inside the bar


@pytest.mark.parametrize("scale", [8.0, 32.0])
def test_two_piece_operands_hold_the_bar_16k(scale):
    """The 16k batch-1 shape (32 query heads, 8 kv heads, 16384 tokens, sink
    512, recent 2048, 1% outlier channels), query heads of two kv heads."""
    q, oc, rk, rv = _case(1, 32, 8, 128, 512, 2048, 16384, "percent", 0, scale)
    heads = range(0, 8)
    want = oc.attend(0, q)
    two = kernel_model_attention(q, oc.k[0], oc.v[0], rk, rv, 8, 512, 2048, 2, 2, heads=heads)
    one_p = kernel_model_attention(q, oc.k[0], oc.v[0], rk, rv, 8, 512, 2048, 2, 1, heads=heads)
    e2, e1 = _row_err(two, want, heads), _row_err(one_p, want, heads)
    print(f"x{scale}: worst row two pieces {e2:.2e}; one-piece softmax weights {e1:.2e}")
    assert e2 < TOL / 20
    assert e1 > 10 * e2          # the weights' second piece matters too
