"""Pins for the CPU oracle: each test checks the oracle against something other
than itself (a library routine, a closed form, a hand-worked example, brute
force on tiny inputs, or an invariant the mathematics fixes)."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows[key] = vals
    return rows


# --------------------------------------------------------------------------- formats


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 10,
        g.standard_normal(2000).astype(np.float32) * 1e-30,
        # exact ties: low half exactly 0x8000 with both parities of the kept lsb
        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38], np.float32),
    ])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(orc.f32_to_bf16_bits(x), want)
    back = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(orc.bf16_bits_to_f32(want), back)


def test_canonical_zero():
    z = orc.canonical_zero(np.array([-0.0, 0.0, -1.5], np.float32))
    assert z.view(np.uint32)[0] == 0 and z.view(np.uint32)[1] == 0 and z[2] == -1.5


# --------------------------------------------------------------------------- packing


def test_pack_golden_examples():
    with open(os.path.join(GOLDEN, "pack_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            lhs, rhs = line.split("->")
            codes = np.array([int(v) for v in lhs.split()], np.uint8)[None]
            assert orc.pack_codes(codes)[0, 0] == int(rhs.strip(), 16)


def test_pack_roundtrip():
    g = np.random.default_rng(2)
    c = g.integers(0, 4, size=(37, 512)).astype(np.uint8)
    p = orc.pack_codes(c)
    assert p.shape == (37, 128)
    np.testing.assert_array_equal(orc.unpack_codes(p), c)
    # each code occupies exactly its own two bits: compare against bit reads
    for j in (0, 1, 2, 3, 4, 127, 511):
        np.testing.assert_array_equal((p[:, j // 4] >> (2 * (j % 4))) & 3, c[:, j])


# --------------------------------------------------------------------------- quantizer


def test_quant_worked_example():
    gd = _read_golden("quant_worked_example.txt")
    G = int(gd["group"][0])
    x = np.array([float(v) for v in gd["x"]], np.float32)[None]
    q = orc.quantize_rows(x, G, float(gd["clip"][0]))
    assert float(q.s16[0, 0]) == float(gd["scale"][0])
    assert float(q.z16[0, 0]) == float(gd["zero"][0])
    np.testing.assert_array_equal(q.codes[0], [int(v) for v in gd["codes"]])
    np.testing.assert_array_equal(orc.pack_codes(q.codes)[0], [int(v, 16) for v in gd["packed"]])


def _rand_rows(n=512, D=256, seed=3):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, D)).astype(np.float32)
    x[:, 5] *= 8.0
    x[7] = np.abs(x[7]) + 0.5          # one-signed group
    x[8] = -np.abs(x[8]) - 0.5
    return x


@pytest.mark.parametrize("clip", [0.96, 0.92, 1.0])
def test_quant_codes_are_nearest_levels(clip):
    """Brute force: every code is the nearest of the 4 levels z + c*s (exact
    fp64 distances) for values inside [z, z + 3s]; outside they clamp."""
    G = 128
    x = _rand_rows()
    q = orc.quantize_rows(x, G, clip)
    assert q.codes.max() <= 3
    s = q.s16.astype(np.float64).repeat(G, axis=1)
    z = q.z16.astype(np.float64).repeat(G, axis=1)
    xd = x.astype(np.float64)
    levels = z[..., None] + np.arange(4)[None, None, :] * s[..., None]
    dist = np.abs(xd[..., None] - levels)
    best = dist.argmin(-1)
    d_sorted = np.sort(dist, axis=-1)
    near_tie = (d_sorted[..., 1] - d_sorted[..., 0]) <= 1e-6 * np.maximum(s, 1e-30)
    ok = (q.codes == best) | near_tie
    assert ok.all(), np.argwhere(~ok)[:5]
    # clamping: below the lowest level -> 0, above the highest -> 3
    assert np.all(q.codes[xd < z] == 0)
    assert np.all(q.codes[xd > z + 3 * s] == 3)


def test_quant_clip_one_hits_extremes():
    """clip = 1: the group minimum gets code 0 and the maximum code 3."""
    G = 128
    x = _rand_rows()
    q = orc.quantize_rows(x, G, 1.0)
    g = x.reshape(x.shape[0], -1, G)
    c = q.codes.reshape(g.shape)
    rows = np.arange(g.shape[0])[:, None]
    grp = np.arange(g.shape[1])[None, :]
    assert np.all(c[rows, grp, g.argmin(-1)] == 0)
    assert np.all(c[rows, grp, g.argmax(-1)] == 3)


@pytest.mark.parametrize("clip", [0.96, 0.92])
def test_quant_range_is_clipped_min_max(clip):
    """Dequantized range [z, z + 3s] equals [r*min, r*max] up to fp16 rounding:
    pins the ratio, the divisor 3 and which extreme feeds the zero."""
    G = 128
    x = _rand_rows()
    q = orc.quantize_rows(x, G, clip)
    g = x.reshape(x.shape[0], -1, G).astype(np.float64)
    lo = clip * g.min(-1)
    hi = clip * g.max(-1)
    z = q.z16.astype(np.float64)
    s = q.s16.astype(np.float64)
    tol = 2.0 ** -10 * (np.abs(lo) + np.abs(hi)) + 1e-7
    assert np.all(np.abs(z - lo) <= tol)
    assert np.all(np.abs(z + 3 * s - hi) <= 4 * tol)


def test_quant_error_bound():
    """|x - x_hat| <= s/2 (plus fp16 slack) for values inside the clipped range."""
    G = 128
    x = _rand_rows()
    q = orc.quantize_rows(x, G, 0.96)
    xh = orc.dequantize_rows(q.codes, q.s16, q.z16, G)
    s = q.s16.astype(np.float64).repeat(G, axis=1)
    z = q.z16.astype(np.float64).repeat(G, axis=1)
    inside = (x >= z) & (x <= z + 3 * s)
    err = np.abs(x - xh)
    assert np.all(err[inside] <= 0.5 * s[inside] * (1 + 1e-6) + 1e-12)


def test_quant_degenerate_groups():
    x = np.zeros((3, 128), np.float32)
    x[1] = 2.5
    x[2] = -0.0
    q = orc.quantize_rows(x, 128, 0.96)
    assert np.all(q.codes == 0)
    assert np.all(q.s16 == 0)
    assert float(q.z16[1, 0]) == float(np.float16(np.float32(0.96) * np.float32(2.5)))
    # -0.0 canonicalised: zero bits are +0
    assert q.z16[2].view(np.uint16)[0] == 0


# --------------------------------------------------------------------------- Lloyd-Max codebook


def test_lloyd_max_levels_match_max_table():
    """Lloyd's iteration on a unit Gaussian converges to the published 4-level
    quantizer (Max 1960: levels +-0.4528, +-1.510; thresholds 0, +-0.9816;
    mean squared error 0.1175), which the oracle's codebook constants carry."""
    y, t, mse = orc.lloyd_max_gaussian()
    np.testing.assert_allclose(y, _LM_TABLE, atol=6e-5)
    np.testing.assert_allclose(t, [-0.9816, 0.0, 0.9816], atol=6e-5)
    assert abs(mse - 0.1175) < 1e-4
    np.testing.assert_array_equal(orc.LLOYD_MAX_LEVELS, _LM_TABLE)
    assert orc.LLOYD_MAX_THRESHOLD == 0.9816
    # the thresholds are the midpoints of the constants' levels
    assert abs(0.5 * (_LM_TABLE[2] + _LM_TABLE[3]) - orc.LLOYD_MAX_THRESHOLD) < 1e-12


def test_gaussian_quantizer_mse_closed_form():
    """The closed-form error against numerical integration, and a local
    minimum at the Lloyd-Max levels (perturbing any level raises it)."""
    from scipy import integrate, stats
    y = np.array(_LM_TABLE)
    t = 0.5 * (y[1:] + y[:-1])
    q = lambda x: y[np.searchsorted(t, x)]
    num = integrate.quad(lambda x: (x - q(x)) ** 2 * stats.norm.pdf(x), -12, 12,
                         points=list(t), limit=200)[0]
    assert abs(orc.gaussian_quantizer_mse(y, t) - num) < 1e-9
    y0, t0, m0 = orc.lloyd_max_gaussian()
    for k in range(4):
        for dv in (-0.01, 0.01):
            yy = y0.copy()
            yy[k] += dv
            assert orc.gaussian_quantizer_mse(yy, t0) > m0


def test_lloyd_max_worked_example():
    gd = _read_golden("lloyd_max_worked_example.txt")
    G = int(gd["group"][0])
    x = np.array([float(v) for v in gd["x"]], np.float32)[None]
    q = orc.quantize_rows_lloyd_max(x, G, float(gd["ratio"][0]))
    assert float(q.s16[0, 0]) == float(gd["scale"][0])
    assert float(q.z16[0, 0]) == float(gd["zero"][0])
    np.testing.assert_array_equal(q.codes[0], [int(v) for v in gd["codes"]])
    xh = orc.dequantize_rows_lloyd_max(q.codes, q.s16, q.z16, G)[0]
    np.testing.assert_allclose(xh, [float(v) for v in gd["dequant"]], atol=6e-6)


@pytest.mark.parametrize("ratio", [1.16, 1.0, 0.5])
def test_lloyd_max_codes_are_nearest_levels(ratio):
    """Brute force: every code is the nearest of z + s*level (fp64 distances,
    the table's levels), s and z the stored fp16 values."""
    G = 128
    x = _rand_rows()
    q = orc.quantize_rows_lloyd_max(x, G, ratio)
    assert q.codes.max() <= 3
    s = q.s16.astype(np.float64).repeat(G, axis=1)
    z = q.z16.astype(np.float64).repeat(G, axis=1)
    levels = z[..., None] + s[..., None] * np.array(_LM_TABLE)[None, None, :]
    dist = np.abs(x.astype(np.float64)[..., None] - levels)
    best = dist.argmin(-1)
    d_sorted = np.sort(dist, axis=-1)
    near_tie = (d_sorted[..., 1] - d_sorted[..., 0]) <= 1e-6 * np.maximum(s, 1e-30)
    ok = (q.codes == best) | near_tie
    assert ok.all(), np.argwhere(~ok)[:5]


def test_lloyd_max_statistics():
    """mu and the step against float64 mean and (population) standard
    deviation: equal within fp32 rounding before the fp16 store."""
    G = 128
    x = _rand_rows()
    ratio = 1.16
    q = orc.quantize_rows_lloyd_max(x, G, ratio)
    g = x.reshape(x.shape[0], -1, G).astype(np.float64)
    mu, sd = g.mean(-1), g.std(-1)
    scale = np.abs(g).max(-1)
    assert np.all(np.abs(q.z16.astype(np.float64) - mu) <= 2.0 ** -11 * np.abs(mu) + 1e-6 * scale)
    s = q.s16.astype(np.float64)
    assert np.all(np.abs(s - ratio * sd) <= 2.0 ** -11 * ratio * sd + 1e-5 * scale)
    # population (divide by G), not sample (G - 1), deviation
    assert np.median(np.abs(s / (ratio * g.std(-1, ddof=1)) - 1)) > 2e-3


def test_lloyd_max_error_matches_gaussian_theory():
    """On Gaussian groups the mean squared dequantization error per unit
    variance is the quantizer's closed form for levels scaled by the ratio
    (0.1175 at ratio 1): pins levels, step and dequantization together."""
    g = np.random.default_rng(17)
    x = g.standard_normal((4000, 128)).astype(np.float32) * 3.0 + 1.5
    for ratio in (1.0, 1.16):
        q = orc.quantize_rows_lloyd_max(x, 128, ratio)
        xh = orc.dequantize_rows_lloyd_max(q.codes, q.s16, q.z16, 128)
        err = np.mean((xh - x.astype(np.float64)) ** 2) / 9.0
        y = ratio * np.array(_LM_TABLE)
        want = orc.gaussian_quantizer_mse(y, 0.5 * (y[1:] + y[:-1]))
        assert abs(err - want) < 0.004, (ratio, err, want)
    assert want > 0.1175


def test_lloyd_max_degenerate_groups():
    x = np.zeros((3, 128), np.float32)
    x[1] = 2.5
    x[2] = -0.0
    q = orc.quantize_rows_lloyd_max(x, 128, 1.16)
    assert np.all(q.codes == 0)
    assert np.all(q.s16 == 0)
    assert float(q.z16[1, 0]) == 2.5
    assert q.z16[2].view(np.uint16)[0] == 0


def test_lloyd_max_group_size():
    """Two groups per row are quantized independently."""
    x = _rand_rows(n=16, D=256)
    q = orc.quantize_rows_lloyd_max(x, 128, 1.16)
    for gi in range(2):
        qq = orc.quantize_rows_lloyd_max(np.ascontiguousarray(x[:, 128 * gi:128 * (gi + 1)]), 128, 1.16)
        np.testing.assert_array_equal(q.codes[:, 128 * gi:128 * (gi + 1)], qq.codes)
        np.testing.assert_array_equal(q.s16[:, gi], qq.s16[:, 0])


# --------------------------------------------------------------------------- windows


@pytest.mark.parametrize("T,N,M", [(10, 3, 4), (7, 3, 4), (8, 3, 4), (5, 0, 2), (5, 2, 0),
                                   (2, 3, 4), (0, 3, 4), (1025, 64, 256)])
def test_window_sets(T, N, M):
    hp = orc.high_precision_mask(T, N, M)
    brute = np.array([t < N or t >= T - M for t in range(T)], bool)
    np.testing.assert_array_equal(hp, brute)
    n_int2 = int((~hp).sum())
    assert n_int2 == max(0, T - N - M)
    if T == N + M + 1:
        assert np.flatnonzero(~hp).tolist() == [N]


# --------------------------------------------------------------------------- attention


def _mk_cache(T, Hq=4, Hkv=2, D=128, N=3, M=4, seed=5, rot=True, k_dtype=0, v_dtype=0,
              dist="normal", batch=2, codebook=0, lm_ratio=1.16):
    cfg = orc.OracleConfig(num_layers=1, batch=batch, num_q_heads=Hq, num_kv_heads=Hkv,
                           head_dim=D, sink_tokens=N, recent_tokens=M,
                           k_dtype=k_dtype, v_dtype=v_dtype, codebook=codebook, lm_ratio=lm_ratio)
    rk = synth.rotations(1, D, seed, "rot_k") if rot else None
    rv = synth.rotations(1, D, seed, "rot_v") if rot else None
    c = orc.OracleKVCache(cfg, rk, rv)
    mask = synth.outlier_mask(D, Hkv, seed, 0, "fixed", 2)
    k = synth.kv_bits(batch, T, Hkv, D, seed, 0, "k", mask, dist)
    v = synth.kv_bits(batch, T, Hkv, D, seed, 0, "v", mask, dist)
    c.append(0, k[:, : T // 2], v[:, : T // 2])
    c.append(0, k[:, T // 2:], v[:, T // 2:])
    q = synth.q_bits(batch, Hq, Hkv, D, seed, 0, mask, dist)
    return c, q, k, v, rk, rv


def _sdpa_f64(q, K, V, scale):
    """torch's scaled_dot_product_attention in float64 on the CPU; q [B,H,D], K/V [B,H,T,D]."""
    qt = torch.from_numpy(q)[:, :, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.from_numpy(K), torch.from_numpy(V), scale=scale)
    return out[:, :, 0, :].numpy()


@pytest.mark.parametrize("rot", [False, True])
def test_all_window_equals_library_attention(rot):
    """N + M >= T: every token is read at bf16; with R = I the result must equal a
    library attention over the bf16 K/V; with random R, library attention over
    bf16(x R) with q R, un-rotated by R_V^T."""
    T, Hq, Hkv, D = 12, 4, 2, 128
    c, q, k, v, rk, rv = _mk_cache(T, Hq, Hkv, D, N=5, M=7, rot=rot)
    got = c.attend(0, q)
    eye = np.eye(D)
    Rk = rk[0].astype(np.float64) if rot else eye
    Rv = rv[0].astype(np.float64) if rot else eye
    kk = orc.bf16_bits_to_f64(k) @ Rk            # [B, T, Hkv, D]
    vv = orc.bf16_bits_to_f64(v) @ Rv
    kw = torch.from_numpy(kk.astype(np.float32)).to(torch.bfloat16).double().numpy()
    vw = torch.from_numpy(vv.astype(np.float32)).to(torch.bfloat16).double().numpy()
    Gq = Hq // Hkv
    K = np.repeat(np.transpose(kw, (0, 2, 1, 3)), Gq, axis=1)
    V = np.repeat(np.transpose(vw, (0, 2, 1, 3)), Gq, axis=1)
    qr = orc.bf16_bits_to_f64(q) @ Rk
    want = _sdpa_f64(qr, K, V, 1.0 / math.sqrt(D)) @ Rv.T
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_rotation_invariance_without_quantization():
    """Orthogonal R_K, R_V leave attention unchanged when nothing is rounded:
    softmax((qR)(KR)^T) (VR) R^T == softmax(q K^T) V."""
    g = np.random.default_rng(9)
    D, T = 128, 300
    q = g.standard_normal(D)
    K = g.standard_normal((T, D))
    V = g.standard_normal((T, D))
    Rk = synth.haar_rotation(D, 11, 0, "rot_k").astype(np.float64)
    Rv = synth.haar_rotation(D, 11, 0, "rot_v").astype(np.float64)
    # fp32-stored Haar rotations are orthogonal to ~1e-7; use the exact polar
    # factor of each so the identity is exact in fp64
    u, _, vt = np.linalg.svd(Rk)
    Rk = u @ vt
    u, _, vt = np.linalg.svd(Rv)
    Rv = u @ vt
    sc = 1 / math.sqrt(D)
    a = orc.softmax_attention_f64(q @ Rk, K @ Rk, V @ Rv, sc) @ Rv.T
    b = orc.softmax_attention_f64(q, K, V, sc)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11)
    # and the fp32 rotation the GPU receives is orthogonal to fp32 precision
    R32 = synth.haar_rotation(D, 11, 0, "rot_k").astype(np.float64)
    assert np.abs(R32 @ R32.T - np.eye(D)).max() < 1e-6


def test_absorbed_v_rotation_output():
    """With the V rotation absorbed into the caller's output projection the
    library returns o' (the V-rotated basis): o' @ R_V^T is the ordinary output
    and, with R_V orthogonal, o' = o @ R_V; the brute-force loops agree."""
    T, Hq, Hkv, D, N, M = 11, 4, 2, 128, 2, 3
    c, qb, kb, vb, rk, rv = _mk_cache(T, Hq, Hkv, D, N=N, M=M, batch=1, seed=23)
    o = c.attend(0, qb)
    oa = orc.decode_attention(qb, c.k[0], c.v[0], rk[0], rv[0], Hkv, N, M, 128, 0, 0, absorb_v=True)
    Rv = rv[0].astype(np.float64)
    np.testing.assert_allclose(oa @ Rv.T, o, rtol=1e-10, atol=1e-12)
    assert np.abs(oa - o).max() > 1e-3                  # the rotation is not the identity
    want = _brute_attention(qb, kb, vb, rk[0], rv[0], Hkv, N, M, 128, 0.96, 0.92)
    np.testing.assert_allclose(oa @ Rv.T, want, rtol=1e-9, atol=1e-9)


def _pairwise_f32(vals):
    """fp32 sum of a power-of-two list, element i with i + n/2, halves again."""
    a = [np.float32(v) for v in vals]
    while len(a) > 1:
        h = len(a) // 2
        a = [np.float32(a[i] + a[i + h]) for i in range(h)]
    return a[0]


# the Gaussian Lloyd-Max levels as Max's table prints them (4 decimals)
_LM_TABLE = (-1.5104, -0.4528, 0.4528, 1.5104)


def _brute_attention(q_bits, k_bits, v_bits, rk, rv, Hkv, N, M, G, kclip, vclip, ntok=None,
                     lm_ratio=None):
    """Pure-Python loops for tiny shapes, written straight from the definition.
    The windows are those of the full length T; the query attends over the
    first ntok positions (all T by default).  lm_ratio set: the Lloyd-Max
    codebook (nearest of mu + s*level, s = ratio * sd) instead of min/max."""
    B, Hq, D = q_bits.shape
    T = k_bits.shape[1]
    ntok = T if ntok is None else ntok
    Gq = Hq // Hkv
    f = lambda bits: float(orc.bf16_bits_to_f64(np.array([bits], np.uint16))[0])
    out = np.zeros((B, Hq, D))

    def rot(xbits, R):
        x = [f(b) for b in xbits]
        return [sum(x[e] * float(R[e][d]) for e in range(D)) for d in range(D)]

    def vec_for(xbits, R, t, clip):
        xr = np.array(rot(xbits, R), np.float64).astype(np.float32)
        if t < N or t >= T - M:                     # high precision
            return [f(b) for b in orc.f32_to_bf16_bits(orc.canonical_zero(xr))]
        res = []
        for g0 in range(0, D, G):
            grp = [float(v) + 0.0 for v in orc.canonical_zero(xr[g0:g0 + G])]
            if lm_ratio is not None:
                mu = np.float32(_pairwise_f32(grp) * np.float32(1.0 / G))
                var = np.float32(_pairwise_f32([np.float32(np.float32(v - mu) * np.float32(v - mu))
                                                for v in grp]) * np.float32(1.0 / G))
                s = float(np.float16(np.float32(np.float32(lm_ratio) * np.float32(math.sqrt(var)))))
                z = float(np.float16(mu))
                lv = [float(np.float32(l)) for l in _LM_TABLE]
                for val in grp:
                    if s == 0.0:
                        c = 0
                    else:
                        # nearest level, equal distances to the higher one
                        d = [abs(val - (z + s * lv[cc])) for cc in range(4)]
                        c = min(range(4), key=lambda cc: (d[cc], -cc))
                    res.append(z + s * lv[c])
                continue
            r = np.float32(clip)
            hi = np.float32(r * np.float32(max(grp)))
            lo = np.float32(r * np.float32(min(grp)))
            s = float(np.float16(np.float32(np.float32(hi - lo) / np.float32(3))))
            z = float(np.float16(lo))
            for val in grp:
                if s == 0.0:
                    c = 0
                else:
                    # nearest level among z + c*s, ties to the even code
                    d = [abs(val - (z + cc * s)) for cc in range(4)]
                    c = min(range(4), key=lambda cc: (d[cc], cc % 2))
                res.append(s * c + z)
        return res

    for b in range(B):
        for j in range(Hq):
            h = j // Gq
            qv = rot(q_bits[b, j], rk)
            Ks = [vec_for(k_bits[b, t, h], rk, t, kclip) for t in range(ntok)]
            Vs = [vec_for(v_bits[b, t, h], rv, t, vclip) for t in range(ntok)]
            sc = [sum(qv[d] * Kt[d] for d in range(D)) / math.sqrt(D) for Kt in Ks]
            mx = max(sc)
            w = [math.exp(s_ - mx) for s_ in sc]
            tot = sum(w)
            o = [sum(w[t] * Vs[t][d] for t in range(ntok)) / tot for d in range(D)]
            out[b, j] = [sum(o[e] * float(rv[d][e]) for e in range(D)) for d in range(D)]
    return out


def test_brute_force_tiny():
    """T <= 16, some INT2 tokens, random rotations: vectorised oracle == loops.
    (The loop picks nearest levels with an explicit argmin instead of the
    division-and-rint route, so ties aside the two agree exactly.)"""
    T, Hq, Hkv, D, N, M = 11, 4, 2, 128, 2, 3
    c, q, k, v, rk, rv = _mk_cache(T, Hq, Hkv, D, N=N, M=M, batch=1, seed=21)
    got = c.attend(0, q)
    want = _brute_attention(q, k, v, rk[0], rv[0], Hkv, N, M, 128, 0.96, 0.92)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("ratio", [1.16, 1.0])
def test_brute_force_tiny_lloyd_max(ratio):
    """Lloyd-Max codebook, T <= 16, INT2 tokens present: vectorised oracle ==
    loops that pick the nearest level by distance (not by the thresholds)."""
    T, Hq, Hkv, D, N, M = 11, 4, 2, 128, 2, 3
    c, q, k, v, rk, rv = _mk_cache(T, Hq, Hkv, D, N=N, M=M, batch=1, seed=23,
                                   codebook=orc.CODEBOOK_LLOYD_MAX, lm_ratio=ratio)
    got = c.attend(0, q)
    want = _brute_attention(q, k, v, rk[0], rv[0], Hkv, N, M, 128, 0.96, 0.92, lm_ratio=ratio)
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-9)
    # and the codebook matters: the min/max quantizer gives another result
    c2, *_ = _mk_cache(T, Hq, Hkv, D, N=N, M=M, batch=1, seed=23)
    assert not np.allclose(c2.attend(0, q), got, rtol=1e-6, atol=0)


# --------------------------------------------------------------------------- ragged batches


def _ragged(lengths, Hq=4, Hkv=2, D=128, N=2, M=3, seed=31):
    cfg = orc.OracleConfig(num_layers=1, batch=len(lengths), num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           sink_tokens=N, recent_tokens=M)
    rk = synth.rotations(1, D, seed, "rot_k")
    rv = synth.rotations(1, D, seed, "rot_v")
    rc = orc.OracleRaggedCache(cfg, rk, rv)
    mask = synth.outlier_mask(D, Hkv, seed, 0, "fixed", 2)
    T = max(lengths)
    k = synth.kv_bits(len(lengths), T, Hkv, D, seed, 0, "k", mask)
    v = synth.kv_bits(len(lengths), T, Hkv, D, seed, 0, "v", mask)
    for b, Tb in enumerate(lengths):
        rc.append_seq(0, b, k[b, :Tb // 2], v[b, :Tb // 2])
        rc.append_seq(0, b, k[b, Tb // 2:Tb], v[b, Tb // 2:Tb])
    q = synth.q_bits(len(lengths), Hq, Hkv, D, seed, 0, mask)
    return rc, q, k, v, rk, rv


def test_ragged_equal_lengths_equals_batch():
    """Equal lengths: the ragged cache is the batched cache, bit for bit."""
    rc, q, k, v, rk, rv = _ragged([9, 9, 9])
    cfg = orc.OracleConfig(num_layers=1, batch=3, num_q_heads=4, num_kv_heads=2, head_dim=128,
                           sink_tokens=2, recent_tokens=3)
    c = orc.OracleKVCache(cfg, rk, rv)
    c.append(0, k[:, :4], v[:, :4])
    c.append(0, k[:, 4:], v[:, 4:])
    np.testing.assert_array_equal(rc.attend(0, q), c.attend(0, q))


def test_ragged_each_sequence_brute_force():
    """Lengths below, at and above N + M: every row equals pure-Python loops
    over that sequence alone, with the windows of its own length."""
    lengths = [3, 6, 11, 5]                      # N + M = 5: all-window, one INT2, several, none
    rc, q, k, v, rk, rv = _ragged(lengths)
    got = rc.attend(0, q)
    for b, Tb in enumerate(lengths):
        want = _brute_attention(q[b:b + 1], k[b:b + 1, :Tb], v[b:b + 1, :Tb], rk[0], rv[0], 2, 2, 3, 128,
                                0.96, 0.92)
        np.testing.assert_allclose(got[b:b + 1], want, rtol=1e-9, atol=1e-9)


def test_ragged_windows_follow_own_length():
    """Sequence 1 holds N + M + 1 tokens: its token N is its only INT2 token,
    so changing that token's codes changes sequence 1's output and no other."""
    rc, q, *_ = _ragged([4, 6, 11])
    base = rc.attend(0, q)
    kp = rc.seqs[1].k[0]
    kp.codes[:, :, 2] = (kp.codes[:, :, 2] + 1) % 4
    after = rc.attend(0, q)
    assert not np.allclose(after[1], base[1], rtol=0, atol=0)
    np.testing.assert_array_equal(after[[0, 2]], base[[0, 2]])
    kp.codes[:, :, 2] = (kp.codes[:, :, 2] + 3) % 4
    kp.codes[:, :, 3] = (kp.codes[:, :, 3] + 1) % 4         # token 3 is in the recent window
    np.testing.assert_array_equal(rc.attend(0, q), base)


def test_ragged_reset_sequence():
    rc, q, k, v, *_ = _ragged([7, 10])
    base = rc.attend(0, q)
    rc.reset_seq(0)
    assert rc.length(0, 0) == 0 and rc.length(0, 1) == 10
    rc.append_seq(0, 0, k[0, :7], v[0, :7])
    np.testing.assert_array_equal(rc.attend(0, q), base)


def test_gqa_equals_replicated_mha():
    T, Hq, Hkv, D = 40, 8, 2, 128
    c, q, k, v, rk, rv = _mk_cache(T, Hq, Hkv, D, N=4, M=6)
    got = c.attend(0, q)
    Gq = Hq // Hkv
    cfg = orc.OracleConfig(num_layers=1, batch=2, num_q_heads=Hq, num_kv_heads=Hq,
                           head_dim=D, sink_tokens=4, recent_tokens=6)
    c2 = orc.OracleKVCache(cfg, rk, rv)
    c2.append(0, np.repeat(k, Gq, axis=2), np.repeat(v, Gq, axis=2))
    want = c2.attend(0, q)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_window_boundary_effects():
    """T = N+M+1: exactly token N is INT2 -> changing its codes changes the
    output; changing codes of window tokens does not."""
    N, M, T = 3, 4, 8
    c, q, *_ = _mk_cache(T, N=N, M=M, batch=1)
    base = c.attend(0, q)
    kp = c.k[0]
    for t, should_change in [(N, True), (0, False), (T - 1, False), (N + 1, False)]:
        old = kp.codes[:, :, t].copy()
        kp.codes[:, :, t] = (old + 1) % 4
        changed = not np.allclose(c.attend(0, q), base, rtol=0, atol=0)
        kp.codes[:, :, t] = old
        assert changed == should_change, (t, changed)


def test_bf16_v_variant_reads_window_everywhere():
    T = 30
    c, q, k, v, rk, rv = _mk_cache(T, N=2, M=3, v_dtype=orc.KV_BF16)
    got = c.attend(0, q)
    # same as an all-window V: replace V planes with INT2 ones but N+M large
    assert c.v[0].codes is None
    vv = orc.bf16_bits_to_f64(c.v[0].win)
    hp = orc.high_precision_mask(T, 2, 3)
    Kh = np.where(hp[None, None, :, None], orc.bf16_bits_to_f64(c.k[0].win),
                  orc.dequantize_rows(c.k[0].codes.reshape(-1, 128), c.k[0].s16.reshape(-1, 1),
                                      c.k[0].z16.reshape(-1, 1), 128).reshape(vv.shape))
    qr = orc.rotate_f64(q, rk[0])
    want = np.zeros_like(got)
    for b in range(2):
        for j in range(4):
            want[b, j] = orc.softmax_attention_f64(qr[b, j], Kh[b, j // 2], vv[b, j // 2],
                                                   1 / math.sqrt(128))
    want = want @ rv[0].astype(np.float64).T
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_storage_import_roundtrip():
    """planes_from_storage(sink, ring) reproduces the logical window values."""
    T, N, M = 23, 3, 5
    c, q, *_ = _mk_cache(T, N=N, M=M)
    kp = c.k[0]
    B, H, _, D = kp.win.shape
    sink = kp.win[:, :, :N]
    ring = np.zeros((B, H, M, D), np.uint16)
    for t in range(T):
        ring[:, :, t % M] = kp.win[:, :, t]          # the last write per slot wins
    imp = orc.planes_from_storage(orc.pack_codes(kp.codes), kp.s16, kp.z16, sink, ring, T, N, M)
    hp = orc.high_precision_mask(T, N, M)
    np.testing.assert_array_equal(imp.win[:, :, hp], kp.win[:, :, hp])
    np.testing.assert_array_equal(imp.codes, kp.codes)


def test_compression_ratio_matches_pages():
    """2-bit codes + fp16 scale and zero per 128-group: 36 B vs 256 B of bf16
    per 128 values = 7.11x, consistent with the ~7x the RotationZoo card states."""
    b = orc.compressed_bytes_per_token_head(128, 128)
    assert b == 36
    assert abs(256 / b - 7.11) < 0.01


def test_bit_reversal_permutation():
    P = orc.bit_reversal_permutation(128)
    assert np.array_equal(P @ P, np.eye(128))      # an involution
    x = np.arange(128, dtype=np.float64)
    y = x @ P
    assert y[1] == 64 and y[64] == 1 and y[3] == 96 and y[127] == 127


# --------------------------------------------------------------------------- in-quant Hadamard


def _fwht(x):
    """Walsh-Hadamard butterflies over the last axis (length a power of two),
    orthonormal scaling; independent of the matrix form."""
    y = np.array(x, np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = y[..., i:i + h].copy()
            b = y[..., i + h:i + 2 * h].copy()
            y[..., i:i + h] = a + b
            y[..., i + h:i + 2 * h] = a - b
        h *= 2
    return y / math.sqrt(n)


def test_block_hadamard_matches_library_and_recursion():
    """The order-128 matrix is scipy's Sylvester Hadamard scaled to unit rows;
    it is orthogonal; order 256 is the two-block recursion of order 128; a
    head_dim of 512 repeats the order-128 block along the diagonal."""
    import scipy.linalg
    H = orc.block_hadamard(128)
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(128) / math.sqrt(128))
    np.testing.assert_allclose(H @ H.T, np.eye(128), atol=1e-14)
    H256 = orc.block_hadamard(256, 256)
    np.testing.assert_allclose(H256, np.block([[H, H], [H, -H]]) / math.sqrt(2), atol=1e-15)
    Hb = orc.block_hadamard(512)
    for g in range(4):
        for g2 in range(4):
            blk = Hb[128 * g:128 * (g + 1), 128 * g2:128 * (g2 + 1)]
            np.testing.assert_array_equal(blk, H if g == g2 else np.zeros((128, 128)))
    e0 = np.zeros(128)
    e0[0] = 1.0
    np.testing.assert_allclose(e0 @ H, np.full(128, 1 / math.sqrt(128)), atol=1e-16)


@pytest.mark.parametrize("D", [128, 512])
def test_in_quant_hadamard_rotation(D):
    """fp32(R @ H): the identity rotation gives the Hadamard itself; the product
    stays orthogonal to fp32 accuracy; applied to a vector it equals the
    rotation followed by butterflies over each 128-group."""
    R = synth.rotations(1, D, 5, "rot_k")[0]
    RH = orc.with_in_quant_hadamard(R)
    assert RH.dtype == np.float32 and RH.shape == (D, D)
    np.testing.assert_array_equal(orc.with_in_quant_hadamard(np.eye(D, dtype=np.float32)),
                                  orc.block_hadamard(D).astype(np.float32))
    P = RH.astype(np.float64)
    np.testing.assert_allclose(P @ P.T, np.eye(D), atol=1e-6)
    x = np.random.default_rng(3).standard_normal((5, D))
    via_fwht = _fwht((x @ R.astype(np.float64)).reshape(5, D // 128, 128)).reshape(5, D)
    np.testing.assert_allclose(x @ P, via_fwht, rtol=0, atol=1e-5)


def test_in_quant_hadamard_spreads_an_outlier():
    """Closed form: a group whose energy sits in one channel j comes out of the
    transform flat, entry i = x_j (-1)^popcount(i & j) / sqrt(128), so the
    quantizer sees two levels instead of one outlier over zeros."""
    D, j, amp = 128, 7, 48.0
    x = np.zeros((1, D), np.float32)
    x[0, j] = amp
    bits = orc.f32_to_bf16_bits(x)
    I = np.eye(D, dtype=np.float32)
    xh = orc.rotated_fp32(bits, orc.with_in_quant_hadamard(I))[0].astype(np.float64)
    signs = np.array([(-1.0) ** bin(i & j).count("1") for i in range(D)])
    np.testing.assert_allclose(xh, amp * signs / math.sqrt(D), rtol=1e-6)
    q = orc.quantize_rows(xh.astype(np.float32)[None], 128, 1.0)
    assert set(np.unique(q.codes)) == {0, 3}


# --------------------------------------------------------------------------- chunked-prefill attention


def _prefill_queries(batch, n, Hq, Hkv, D, seed, mask=None):
    mask = synth.outlier_mask(D, Hkv, seed, 0, "fixed", 2) if mask is None else mask
    return np.stack([synth.q_bits(batch, Hq, Hkv, D, seed, 0, mask, "normal", step=i) for i in range(n)], axis=1)


def test_prefill_attention_single_query_is_decode():
    """n = 1: the one query sits at position T - 1 and attends over the whole
    cache, which is the decode step."""
    T, Hq, Hkv, D = 30, 4, 2, 128
    c, q, k, v, rk, rv = _mk_cache(T, Hq, Hkv, D, N=3, M=5)
    got = orc.prefill_attention(q[:, None], c.k[0], c.v[0], rk[0], rv[0], Hkv, 3, 5, 128, 0, 0)
    np.testing.assert_allclose(got[:, 0], c.attend(0, q), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("rot", [False, True])
def test_prefill_attention_all_window_equals_library(rot):
    """N + M >= T: every position is read at bf16, and the chunk's queries
    (the last n positions) equal a library attention over the bf16 K/V under
    an explicit causal mask (query i sees keys 0 .. T - n + i), with q R_K and
    the output un-rotated by R_V^T."""
    T, n, Hq, Hkv, D = 12, 5, 4, 2, 128
    c, _, k, v, rk, rv = _mk_cache(T, Hq, Hkv, D, N=5, M=7, rot=rot)
    qb = _prefill_queries(2, n, Hq, Hkv, D, 5)
    got = orc.prefill_attention(qb, c.k[0], c.v[0], rk[0] if rot else np.eye(D, dtype=np.float32),
                                rv[0] if rot else np.eye(D, dtype=np.float32), Hkv, 5, 7, 128, 0, 0)
    eye = np.eye(D)
    Rk = rk[0].astype(np.float64) if rot else eye
    Rv = rv[0].astype(np.float64) if rot else eye
    kw = torch.from_numpy((orc.bf16_bits_to_f64(k) @ Rk).astype(np.float32)).to(torch.bfloat16).double().numpy()
    vw = torch.from_numpy((orc.bf16_bits_to_f64(v) @ Rv).astype(np.float32)).to(torch.bfloat16).double().numpy()
    Gq = Hq // Hkv
    K = torch.from_numpy(np.repeat(np.transpose(kw, (0, 2, 1, 3)), Gq, axis=1))      # [B, Hq, T, D]
    V = torch.from_numpy(np.repeat(np.transpose(vw, (0, 2, 1, 3)), Gq, axis=1))
    qr = torch.from_numpy(np.transpose(orc.bf16_bits_to_f64(qb) @ Rk, (0, 2, 1, 3)).copy())  # [B, Hq, n, D]
    allowed = torch.from_numpy(np.arange(T)[None, :] <= (T - n + np.arange(n))[:, None])  # [n, T]
    want = torch.nn.functional.scaled_dot_product_attention(qr, K, V, attn_mask=allowed, scale=1.0 / math.sqrt(D))
    want = np.transpose(want.numpy(), (0, 2, 1, 3)) @ Rv.T
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_prefill_attention_brute_force_tiny():
    """INT2 positions inside the chunk and before it, random rotations: every
    query equals the pure-Python loops over its causal prefix, with the
    windows of the full length."""
    T, n, Hq, Hkv, D, N, M = 11, 4, 4, 2, 128, 2, 3
    c, _, k, v, rk, rv = _mk_cache(T, Hq, Hkv, D, N=N, M=M, batch=1, seed=21)
    qb = _prefill_queries(1, n, Hq, Hkv, D, 21)
    got = orc.prefill_attention(qb, c.k[0], c.v[0], rk[0], rv[0], Hkv, N, M, 128, 0, 0)
    for i in range(n):
        want = _brute_attention(qb[:, i], k, v, rk[0], rv[0], Hkv, N, M, 128, 0.96, 0.92, ntok=T - n + i + 1)
        np.testing.assert_allclose(got[:, i], want, rtol=1e-9, atol=1e-9)


def test_prefill_attention_query_subset():
    """Listed queries only: the same values as the full computation's rows."""
    T, n, Hq, Hkv, D, N, M = 40, 9, 4, 2, 128, 3, 7
    c, _, k, v, rk, rv = _mk_cache(T, Hq, Hkv, D, N=N, M=M, batch=2, seed=31)
    qb = _prefill_queries(2, n, Hq, Hkv, D, 31)
    full = orc.prefill_attention(qb, c.k[0], c.v[0], rk[0], rv[0], Hkv, N, M, 128, 0, 0)
    sub = orc.prefill_attention(qb, c.k[0], c.v[0], rk[0], rv[0], Hkv, N, M, 128, 0, 0, query_ids=[8, 0, 4])
    np.testing.assert_array_equal(sub, full[:, [8, 0, 4]])
