"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: codes, scales/zeros and bf16 windows bit-exact given identical fp32
rotated inputs (and end to end where the rotation is exact in fp32);
attention output within 2e-3 relative L2 of the oracle on the identical cache.
"""
import numpy as np
import pytest

import oracle as orc
import synth
from tests.gpu_util import (ATTN_TOL, Shape, compare_planes, gpu_cache, inputs, make_rotations, oracle_cache,
                            oracle_err, oracle_on_exported, planes_from_export, query, rel_l2, say)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ok():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_attention_oscar_amd import oscar_kv
    return oscar_kv


def dev(bits):
    return synth.bits_to_torch_bf16(bits, "cuda")


# ------------------------------------------------------------------ quantizer


def _quant_rows(D, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((300, D)).astype(np.float32)
    x[:, 3] *= 8.0
    x[10] = 0.0                              # degenerate: constant zero
    x[11] = 1.25                             # degenerate: constant
    x[12] = -0.0
    x[13] = np.abs(x[13]) + 1                # one-signed groups
    x[14] = -np.abs(x[14]) - 1
    x[15, ::2] = -0.0
    x[16] *= 1e-6                            # tiny range: fp16 denormal scales
    x[17] *= 3000.0                          # large range
    # exact ties of (x - z)/s at k + 1/2 under r = 1: group [0, 3] -> s = 1, z = 0
    x[18] = np.tile(np.array([0.0, 3.0, 0.5, 1.5, 2.5, 1.0, 2.0, 0.25], np.float32), D // 8)
    # near ties under r = 1: groups [0, mx] give z = 0 and s = fp16(mx / 3);
    # values within a few ulps of (k + 1/2) s on both sides, where a quotient
    # through an approximate reciprocal can land on the other side of the tie
    for row, mx in zip(range(20, 26), (9.0, 2.1, 7.3, 0.77, 5.5, 100.3)):
        sf = np.float32(np.float16(np.float32(np.float32(mx) / np.float32(3.0))))
        vals = [0.0, mx]
        for k in (0.5, 1.5, 2.5):
            c = np.float32(np.float32(k) * sf)
            for n in range(-3, 4):
                v = c
                for _ in range(abs(n)):
                    v = np.nextafter(v, np.float32(np.inf if n > 0 else -np.inf), dtype=np.float32)
                vals.append(v)
        vals = np.array(vals, np.float32)
        x[row] = np.resize(vals, D)
    return x


def _double_rounding_min(clip, seed=0):
    """A group minimum whose clipped value r*min rounds to a different fp16 via
    fp32 (the specified two roundings) than straight from the exact product:
    a quantizer that fuses the multiply into the fp16 conversion fails on it."""
    r = np.float32(clip)
    g = np.random.default_rng(seed)
    while True:
        mn = np.float32(-g.uniform(0.5, 4.0))
        if np.float16(np.float32(r * mn)) != np.float16(float(r) * float(mn)):
            return mn


@pytest.mark.parametrize("D", [128, 512])
@pytest.mark.parametrize("clip", [0.96, 0.92, 1.0])
def test_quantize_rows_bitexact(ok, D, clip):
    say(f"[quantize_rows] D={D} clip={clip}")
    x = _quant_rows(D, 7 + D)
    if clip != 1.0:
        x[19] = np.clip(x[19], -0.4, 0.4)
        x[19, 5::128] = _double_rounding_min(clip)
    rows = x.shape[0]
    xd = torch.from_numpy(x).cuda()
    codes = torch.zeros((rows, D // 4), dtype=torch.uint8, device="cuda")
    meta = torch.zeros((rows, D // 128, 2), dtype=torch.int16, device="cuda")
    ok.oscar_quantize_rows(xd, rows, D, 128, clip, codes, meta)
    torch.cuda.synchronize()
    q = orc.quantize_rows(x, 128, clip)
    np.testing.assert_array_equal(codes.cpu().numpy(), orc.pack_codes(q.codes))
    m = meta.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(m[..., 0], q.s16.view(np.uint16))
    np.testing.assert_array_equal(m[..., 1], q.z16.view(np.uint16))


# ------------------------------------------------------------------ append


@pytest.mark.parametrize("shape,chunks", [
    (Shape(B=2, Hq=4, Hkv=1, D=128, N=64, M=256), [1000, 1, 23, 1]),
    (Shape(B=1, Hq=8, Hkv=2, D=128, N=5, M=7), [3, 1, 1, 9, 64, 1]),
    (Shape(B=2, Hq=4, Hkv=2, D=512, N=16, M=40), [77, 1, 2]),
    (Shape(B=1, Hq=4, Hkv=1, D=128, N=0, M=0), [130, 1]),
    (Shape(B=1, Hq=4, Hkv=1, D=128, N=8, M=16, v_dtype=1), [50, 1]),
])
def test_append_exact_rotation_bitexact(ok, shape, chunks):
    """Rotations exact in fp32 (bit-reversal permutation for K, a signed
    permutation for V): codes, scales, zeros and windows bit-exact end to end."""
    say(f"[append exact] {shape} chunks={chunks}")
    rk, rv = make_rotations(shape, "exact")
    T = sum(chunks)
    k, v, _ = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 5)
    oc = oracle_cache(shape, rk, rv)
    t = 0
    for n in chunks:
        gc.append(0, dev(k[:, t:t + n]), dev(v[:, t:t + n]))
        oc.append(0, k[:, t:t + n], v[:, t:t + n])
        t += n
    torch.cuda.synchronize()
    assert gc.length(0) == T
    compare_planes(gc.export(0, 0), oc.k[0], T, shape.N, shape.M, "K")
    compare_planes(gc.export(0, 1), oc.v[0], T, shape.N, shape.M, "V")
    gc.close()


@pytest.mark.parametrize("D", [128, 512])
def test_append_random_rotation_dump(ok, D):
    """Random Haar rotations: the GPU's fp32 rotated vectors are within fp32
    accumulation error of the fp64 rotation, and the stored codes/metadata/
    windows equal the oracle quantizer applied to those same fp32 vectors."""
    shape = Shape(B=2, Hq=4, Hkv=2, D=D, N=3, M=9)
    say(f"[append dump] {shape}")
    rk, rv = make_rotations(shape, "haar")
    T = 70
    k, v, _ = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T)
    kr = torch.zeros((shape.B, T, shape.Hkv, D), dtype=torch.float32, device="cuda")
    vr = torch.zeros_like(kr)
    gc.append_dump(0, dev(k), dev(v), kr, vr)
    torch.cuda.synchronize()
    kr, vr = kr.cpu().numpy(), vr.cpu().numpy()
    for xr, bits, R, clip, which in ((kr, k, rk[0], 0.96, 0), (vr, v, rv[0], 0.92, 1)):
        ref = orc.rotate_f64(bits, R)
        err = np.abs(xr - ref).max() / np.abs(ref).max()
        say(f"  which={which} max rel rotation err {err:.2e}")
        assert err < 1e-5
        x32 = np.ascontiguousarray(np.transpose(xr, (0, 2, 1, 3)))            # [B, H, T, D]
        q = orc.quantize_rows(x32.reshape(-1, D), 128, clip)
        exp = gc.export(0, which)
        np.testing.assert_array_equal(exp["codes"].reshape(-1, D // 4), orc.pack_codes(q.codes))
        np.testing.assert_array_equal(exp["s16"].reshape(-1, D // 128).view(np.uint16), q.s16.view(np.uint16))
        np.testing.assert_array_equal(exp["z16"].reshape(-1, D // 128).view(np.uint16), q.z16.view(np.uint16))
        win = orc.f32_to_bf16_bits(orc.canonical_zero(x32))
        np.testing.assert_array_equal(exp["sink"], win[:, :, :shape.N])
        for t in range(max(shape.N, T - shape.M), T):
            np.testing.assert_array_equal(exp["ring"][:, :, t % shape.M], win[:, :, t])
    gc.close()


# ------------------------------------------------------------------ decode


def _decode(ok, gc, layer, qbits, impl=0, splits=0, out_dtype=0):
    gc.set_decode_impl(impl)
    gc.set_num_splits(splits)
    B, Hq, D = qbits.shape
    dt = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}[out_dtype]
    out = torch.zeros((B, Hq, D), dtype=dt, device="cuda")
    gc.decode_attn(layer, dev(qbits), out, out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _fill(ok, shape, T, rot="haar", extra=8, chunks=None):
    rk, rv = make_rotations(shape, rot)
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + extra)
    chunks = chunks or [T]
    t = 0
    for n in chunks:
        gc.append(0, dev(k[:, t:t + n]), dev(v[:, t:t + n]))
        t += n
    return gc, rk, rv, k, v, mask


@pytest.mark.parametrize("impl", [0, 1, 2, 3])
def test_decode_tiny_identical_cache(ok, impl):
    """Tiny workload: 1 layer, B=1, Hq=4, Hkv=1, D=128, 1024 tokens appended,
    then one decode step with its append; attention vs the oracle over the
    exported cache."""
    shape = Shape()
    say(f"[decode tiny] impl={impl}")
    gc, rk, rv, k, v, mask = _fill(ok, shape, 1024, chunks=[512, 512])
    k1, v1, _ = inputs(shape, 1, chunk=1)
    gc.append(0, dev(k1), dev(v1))
    qb = query(shape, mask)
    got = _decode(ok, gc, 0, qb, impl=impl)
    want = oracle_on_exported(gc, 0, qb, shape, rk, rv)
    e = oracle_err(got, want)
    say(f"  rel L2 {e:.3e}")
    assert e <= ATTN_TOL
    gc.close()


def test_decode_end_to_end_vs_oracle_cache(ok):
    """Against the oracle's own cache (fp64 rotation on its side): reported;
    code flips from fp32-vs-fp64 rotation are allowed, so the gate is looser."""
    shape = Shape()
    say("[decode end-to-end]")
    T = 1025
    gc, rk, rv, k, v, mask = _fill(ok, shape, T)
    oc = oracle_cache(shape, rk, rv)
    oc.append(0, k, v)
    qb = query(shape, mask)
    got = _decode(ok, gc, 0, qb)
    want = oc.attend(0, qb)
    e = rel_l2(got, want)
    say(f"  end-to-end rel L2 {e:.3e}")
    assert e <= 1e-2
    # with exact rotations the two caches are identical, so the bar is the tight one
    gc2, rk2, rv2, *_ = _fill(ok, shape, T, rot="exact")
    oc2 = oracle_cache(shape, rk2, rv2)
    oc2.append(0, k, v)
    e2 = oracle_err(_decode(ok, gc2, 0, qb), oc2.attend(0, qb))
    say(f"  end-to-end exact-rotation rel L2 {e2:.3e}")
    assert e2 <= ATTN_TOL
    gc.close()
    gc2.close()


@pytest.mark.parametrize("T,N,M", [
    (1, 64, 256), (40, 64, 256), (320, 64, 256), (321, 64, 256), (385, 64, 256),
    (1000, 0, 256), (1000, 64, 0), (1000, 0, 0), (777, 13, 29), (64, 0, 0), (65, 1, 0),
])
@pytest.mark.parametrize("gq", [2, 4, 8])
def test_decode_window_edges(ok, T, N, M, gq):
    """1, 2 and 4 query heads per kv head: the general kernel and the
    one-launch matrix-core kernel (4 and 8), fewer tokens than the sink
    included."""
    shape = Shape(B=2, Hq=2 * gq, Hkv=2, N=N, M=M)
    say(f"[decode edges] T={T} N={N} M={M} gq={gq}")
    gc, rk, rv, k, v, mask = _fill(ok, shape, T)
    qb = query(shape, mask)
    want = oracle_on_exported(gc, 0, qb, shape, rk, rv)
    got = {}
    for impl in (0, 1, 2, 3):
        got[impl] = _decode(ok, gc, 0, qb, impl=impl)
        e = oracle_err(got[impl], want)
        say(f"  impl={impl} rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    # q records from the prologue launch or q rotated in every block: the same
    # arithmetic, the same bits
    np.testing.assert_array_equal(got[2], got[3])
    gc.close()


@pytest.mark.parametrize("T,N,M,gq,vdt", [
    (1, 64, 256, 2, 0), (40, 64, 256, 2, 0), (321, 64, 256, 2, 0), (700, 300, 300, 2, 0), (1000, 0, 256, 2, 0),
    (1000, 64, 0, 2, 0), (1000, 0, 0, 1, 0), (777, 13, 29, 4, 0), (64, 0, 0, 2, 0), (65, 1, 0, 1, 0),
    (2000, 40, 600, 2, 0),
    (1, 64, 256, 2, 1), (321, 64, 256, 2, 1), (1000, 0, 0, 1, 1), (777, 13, 29, 4, 1), (2000, 40, 600, 2, 1),
])
def test_decode_wide_window_edges(ok, T, N, M, gq, vdt):
    """head_dim 512 (three-launch matrix-core path) at the window edges, the
    ring past its wrap, 1, 2 and 4 query heads per kv head, V INT2 or kept
    bf16; the VALU kernel on the same cache as a second check."""
    shape = Shape(B=2, Hq=2 * gq, Hkv=2, D=512, N=N, M=M, v_dtype=vdt)
    say(f"[decode wide edges] T={T} N={N} M={M} gq={gq} v_dtype={vdt}")
    gc, rk, rv, k, v, mask = _fill(ok, shape, T, chunks=[T // 2, T - T // 2] if T > 1 else None)
    qb = query(shape, mask)
    want = oracle_on_exported(gc, 0, qb, shape, rk, rv)
    for impl in (0, 1):
        e = oracle_err(_decode(ok, gc, 0, qb, impl=impl), want)
        say(f"  impl={impl} rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    gc.close()


@pytest.mark.parametrize("impl,tol", [
    (1, 1e-5),        # VALU kernel: fp32 throughout, only summation order changes
    (0, 2 ** -12),    # matrix-core kernel: p*s_V enters as fp16 relative to each
                      # split's running max, so splits move its rounding points;
                      # bounded by fp16's half-ulp
    (2, 2 ** -12),    # the same with q records from a launch of their own
    (3, 2 ** -12),    # the same with q rotated in every block
])
@pytest.mark.parametrize("gq,D,vdt", [(4, 128, 0), (8, 128, 0), (2, 512, 0), (2, 512, 1)])
def test_split_invariance(ok, impl, tol, gq, D, vdt):
    shape = Shape(B=2, Hq=2 * gq, Hkv=2, D=D, N=64, M=256, v_dtype=vdt)
    say(f"[split invariance] impl={impl} gq={gq} D={D} v_dtype={vdt}")
    gc, rk, rv, k, v, mask = _fill(ok, shape, 5000)
    qb = query(shape, mask)
    ref = _decode(ok, gc, 0, qb, impl=impl, splits=1)
    for s in (2, 7, 64, 200):
        e = rel_l2(_decode(ok, gc, 0, qb, impl=impl, splits=s), ref)
        say(f"  splits={s} vs 1: {e:.2e}")
        assert e <= tol
    want = oracle_on_exported(gc, 0, qb, shape, rk, rv)
    assert oracle_err(ref, want) <= ATTN_TOL
    gc.close()


@pytest.mark.parametrize("shape", [
    Shape(B=2, Hq=2, Hkv=2, N=8, M=16),                         # MHA
    Shape(B=1, Hq=16, Hkv=2, N=8, M=16),                        # GQA 8
    Shape(B=2, Hq=4, Hkv=2, D=512, N=16, M=32),                 # wide head, GQA 2
    Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=32, v_dtype=1),      # V kept bf16
    Shape(B=1, Hq=4, Hkv=1, D=128, N=16, M=32, v_dtype=1),
    Shape(B=2, Hq=8, Hkv=2, D=128, N=16, M=32, dist="student_t3", outliers="none"),
])
def test_decode_shapes(ok, shape):
    say(f"[decode shapes] {shape}")
    gc, rk, rv, k, v, mask = _fill(ok, shape, 700)
    qb = query(shape, mask)
    want = oracle_on_exported(gc, 0, qb, shape, rk, rv)
    e = oracle_err(_decode(ok, gc, 0, qb), want)
    say(f"  rel L2 {e:.3e}")
    assert e <= ATTN_TOL
    gc.close()


def test_gqa_equals_replicated_heads(ok):
    """GQA with Hkv=2, Gq=4 equals MHA over K/V replicated per query head."""
    s1 = Shape(B=1, Hq=8, Hkv=2, N=8, M=16)
    s2 = Shape(B=1, Hq=8, Hkv=8, N=8, M=16)
    say("[gqa replicate]")
    rk, rv = make_rotations(s1, "haar")
    T = 300
    k, v, mask = inputs(s1, T)
    g1 = gpu_cache(ok, s1, rk, rv, T)
    g2 = gpu_cache(ok, s2, rk, rv, T)
    g1.append(0, dev(k), dev(v))
    g2.append(0, dev(np.repeat(k, 4, axis=2)), dev(np.repeat(v, 4, axis=2)))
    qb = query(s1, mask)
    a = _decode(ok, g1, 0, qb)
    b = _decode(ok, g2, 0, qb)
    assert rel_l2(a, b) <= ATTN_TOL
    g1.close()
    g2.close()


def test_output_dtypes(ok):
    shape = Shape(B=2, Hq=4, Hkv=1)
    say("[out dtypes]")
    gc, rk, rv, k, v, mask = _fill(ok, shape, 900)
    qb = query(shape, mask)
    f32 = _decode(ok, gc, 0, qb, out_dtype=0)
    for od, tol in ((1, 2 ** -8), (2, 2 ** -11)):
        o = _decode(ok, gc, 0, qb, out_dtype=od)
        assert np.all(np.abs(o - f32) <= tol * np.abs(f32) + 1e-30)
    gc.close()


def test_decode_after_many_single_appends(ok):
    """Decode loop shape: token-by-token appends crossing tile and 8-token
    group boundaries, attention after each."""
    shape = Shape(B=2, Hq=4, Hkv=1, N=4, M=20)
    say("[decode loop]")
    gc, rk, rv, k, v, mask = _fill(ok, shape, 60, extra=40)
    kk, vv, _ = inputs(shape, 30, chunk=3)
    for i in range(30):
        gc.append(0, dev(kk[:, i:i + 1]), dev(vv[:, i:i + 1]))
        if i % 7 == 0 or i == 29:
            qb = query(shape, mask, step=i)
            want = oracle_on_exported(gc, 0, qb, shape, rk, rv)
            e = oracle_err(_decode(ok, gc, 0, qb), want)
            assert e <= ATTN_TOL, (i, e)
    gc.close()


# ------------------------------------------------------------------ fused decode step


def _step(ok, gc, layer, kb, vb, qbits, out_dtype=0):
    B, Hq, D = qbits.shape
    dt = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}[out_dtype]
    out = torch.zeros((B, Hq, D), dtype=dt, device="cuda")
    gc.decode_step(layer, dev(kb), dev(vb), dev(qbits), out, out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _exports_equal(g1, g2, layer, N, M):
    """Every stored bit of positions [0, T) equal; sink rows past T and ring
    slots not yet written hold no data and are skipped."""
    T = g1.length(layer)
    assert g2.length(layer) == T
    for which in (0, 1):
        e1, e2 = g1.export(layer, which), g2.export(layer, which)
        assert sorted(e1) == sorted(e2)
        for key in e1:
            a, b = e1[key], e2[key]
            if key == "sink":
                a, b = a[:, :, :min(N, T)], b[:, :, :min(N, T)]
            elif key == "ring":
                slots = [t % M for t in range(max(N, T - M), T)]
                a, b = a[:, :, slots], b[:, :, slots]
            np.testing.assert_array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8),
                                          err_msg=f"plane {which} {key}")


@pytest.mark.parametrize("shape,T0,steps", [
    (Shape(B=2, Hq=4, Hkv=1, N=64, M=256), 1000, 5),           # INT2 range + both windows
    (Shape(B=1, Hq=8, Hkv=2, N=4, M=68), 60, 80),              # ring wraps, tiles and 8-groups crossed
    (Shape(B=2, Hq=8, Hkv=2, N=8, M=64), 0, 90),               # from an empty cache: sink, ring, INT2 range
    (Shape(B=1, Hq=16, Hkv=2, N=4, M=64), 0, 80),              # the same with two head groups per kv head
    (Shape(B=3, Hq=12, Hkv=3, N=16, M=100), 400, 5),           # 9 (sequence, kv head) pairs: blocks of one on several XCDs
    (Shape(B=1, Hq=4, Hkv=1, N=64, M=256), 300, 4),            # every token still bf16
    (Shape(B=2, Hq=16, Hkv=2, N=8, M=64), 700, 6),             # GQA 8: two head groups per kv head
    (Shape(B=2, Hq=4, Hkv=2, N=8, M=16), 0, 30),               # ring under a tile: the append in the q-record launch
    (Shape(B=1, Hq=4, Hkv=1, N=0, M=1), 130, 3),               # window = the new token only (append in the q-record launch)
    (Shape(B=1, Hq=8, Hkv=1, N=3, M=5), 66, 40),               # GQA 8, ring wraps, tile edges crossed (the same)
    (Shape(B=2, Hq=4, Hkv=2, D=512, N=8, M=16), 0, 40),        # head_dim 512 from an empty cache, ring wraps
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=8, M=16, v_dtype=1), 60, 10),  # head_dim 512, V kept bf16
])
def test_decode_step_equals_append_then_decode(ok, shape, T0, steps):
    """The step (at head_dim 128 and these sizes: one launch that also appends,
    with a ring of at least a tile; else the q-record launch appends) against
    the two separate calls on a twin cache: identical stored cache bit for
    bit, output within the matrix-core kernel's fp16 half-ulp, and within the
    attention bar of the oracle over the exported cache."""
    say(f"[decode step] {shape} T0={T0} steps={steps}")
    rk, rv = make_rotations(shape, "haar")
    k, v, mask = inputs(shape, T0 + steps)
    g1 = gpu_cache(ok, shape, rk, rv, T0 + steps + 3)
    g2 = gpu_cache(ok, shape, rk, rv, T0 + steps + 3)
    if T0:
        for g in (g1, g2):
            g.append(0, dev(k[:, :T0]), dev(v[:, :T0]))
    worst = 0.0
    for i in range(steps):
        t = T0 + i
        qb = query(shape, mask, step=i)
        got = _step(ok, g1, 0, k[:, t:t + 1], v[:, t:t + 1], qb)
        g2.append(0, dev(k[:, t:t + 1]), dev(v[:, t:t + 1]))
        ref = _decode(ok, g2, 0, qb)
        assert g1.length(0) == g2.length(0) == t + 1
        e = rel_l2(got, ref)
        worst = max(worst, e)
        assert e <= 2 ** -12, (i, e)
        if i == 0 or i == steps - 1 or i % 16 == 0:
            _exports_equal(g1, g2, 0, shape.N, shape.M)
            want = oracle_on_exported(g1, 0, qb, shape, rk, rv)
            eo = oracle_err(got, want)
            assert eo <= ATTN_TOL, (i, eo)
    say(f"  worst step-vs-separate rel L2 {worst:.2e}")
    g1.close()
    g2.close()


@pytest.mark.parametrize("shape,T0,steps", [
    (Shape(B=2, Hq=8, Hkv=2, N=8, M=64), 0, 90),               # sink, ring, its wrap, INT2 range
    (Shape(B=3, Hq=24, Hkv=3, N=16, M=100), 300, 6),           # two head groups, 9 (sequence, kv head) pairs
])
def test_decode_step_both_launch_forms(ok, shape, T0, steps):
    """The step as one launch (q rotated in every block, the append by the
    window block holding the token) against the q-record launch followed by
    the attention launch, on twin caches: the stored caches identical bit for
    bit (V scales included, through the next steps' outputs), outputs within
    the fp16 half-ulp (the one launch scales V by the running maximum from
    before its own token)."""
    say(f"[decode step forms] {shape} T0={T0} steps={steps}")
    rk, rv = make_rotations(shape, "haar")
    k, v, mask = inputs(shape, T0 + steps)
    g3 = gpu_cache(ok, shape, rk, rv, T0 + steps + 3)
    g2 = gpu_cache(ok, shape, rk, rv, T0 + steps + 3)
    g3.set_decode_impl(3)
    g2.set_decode_impl(2)
    if T0:
        for g in (g2, g3):
            g.append(0, dev(k[:, :T0]), dev(v[:, :T0]))
    worst = 0.0
    for i in range(steps):
        t = T0 + i
        qb = query(shape, mask, step=i)
        o3 = _step(ok, g3, 0, k[:, t:t + 1], v[:, t:t + 1], qb)
        o2 = _step(ok, g2, 0, k[:, t:t + 1], v[:, t:t + 1], qb)
        e = rel_l2(o3, o2)
        worst = max(worst, e)
        assert e <= 2 ** -12, (i, e)
        if i == steps - 1 or i % 32 == 0:
            _exports_equal(g3, g2, 0, shape.N, shape.M)
            assert oracle_err(o3, oracle_on_exported(g3, 0, qb, shape, rk, rv)) <= ATTN_TOL
    # decode attention after the steps: the same running V maximum on both
    qb = query(shape, mask, step=steps)
    np.testing.assert_array_equal(_decode(ok, g3, 0, qb, impl=2), _decode(ok, g2, 0, qb, impl=2))
    say(f"  worst one-launch vs two-launch rel L2 {worst:.2e}")
    g2.close()
    g3.close()


def test_decode_step_exact_rotation_bitexact(ok):
    """Fused steps with rotations exact in fp32: the stored cache equals the
    oracle's bit for bit, and the output is within the bar of the oracle's
    own attention."""
    shape = Shape(B=2, Hq=4, Hkv=1, N=6, M=10)
    say("[decode step exact]")
    rk, rv = make_rotations(shape, "exact")
    T0, steps = 70, 12
    k, v, mask = inputs(shape, T0 + steps)
    gc = gpu_cache(ok, shape, rk, rv, T0 + steps)
    oc = oracle_cache(shape, rk, rv)
    gc.append(0, dev(k[:, :T0]), dev(v[:, :T0]))
    oc.append(0, k[:, :T0], v[:, :T0])
    for i in range(steps):
        t = T0 + i
        qb = query(shape, mask, step=i)
        got = _step(ok, gc, 0, k[:, t:t + 1], v[:, t:t + 1], qb)
        oc.append(0, k[:, t:t + 1], v[:, t:t + 1])
        e = oracle_err(got, oc.attend(0, qb))
        assert e <= ATTN_TOL, (i, e)
    T = T0 + steps
    compare_planes(gc.export(0, 0), oc.k[0], T, shape.N, shape.M, "K")
    compare_planes(gc.export(0, 1), oc.v[0], T, shape.N, shape.M, "V")
    gc.close()


@pytest.mark.parametrize("shape", [
    Shape(B=1, Hq=32, Hkv=2, N=8, M=16),                       # GQA 16: separate launches
    Shape(B=1, Hq=4, Hkv=2, N=8, M=16),                        # GQA 2
    Shape(B=2, Hq=4, Hkv=2, D=512, N=16, M=32),                # wide head
    Shape(B=1, Hq=4, Hkv=1, N=8, M=0),                         # no recent window
    Shape(B=1, Hq=4, Hkv=1, N=8, M=16, v_dtype=1),             # V kept bf16
])
def test_decode_step_other_shapes(ok, shape):
    """Shapes the fused launch does not take: the step still equals the two
    separate calls."""
    say(f"[decode step other] {shape}")
    rk, rv = make_rotations(shape, "haar")
    T0 = 200
    k, v, mask = inputs(shape, T0 + 2)
    g1 = gpu_cache(ok, shape, rk, rv, T0 + 2)
    g2 = gpu_cache(ok, shape, rk, rv, T0 + 2)
    for g in (g1, g2):
        g.append(0, dev(k[:, :T0]), dev(v[:, :T0]))
    for i in range(2):
        t = T0 + i
        qb = query(shape, mask, step=i)
        got = _step(ok, g1, 0, k[:, t:t + 1], v[:, t:t + 1], qb)
        g2.append(0, dev(k[:, t:t + 1]), dev(v[:, t:t + 1]))
        assert rel_l2(got, _decode(ok, g2, 0, qb)) <= 1e-6
    _exports_equal(g1, g2, 0, shape.N, shape.M)
    g1.close()
    g2.close()


# ------------------------------------------------------------------ full-size samples


@pytest.mark.slow
@pytest.mark.parametrize("impl", [0, 3])
def test_full_size_32k_sampled(ok, impl):
    """The 32k-context benchmark shape (B=16, Hq=32, Hkv=8, D=128, N=64,
    M=256) on one layer, filled on the device, decoded in the benchmark's
    launch configuration (impl 0: a q-record launch first at this size) and
    as one launch whose blocks rotate q themselves (impl 3: more blocks than
    are resident, the window blocks running last); sequences 0 and 15 checked
    against the oracle over the exported cache."""
    from bench import fill_layer_device
    shape = Shape(B=16, Hq=32, Hkv=8, D=128, N=64, M=256, outliers="percent")
    T = 32768
    say("[full 32k] filling")
    rk, rv = make_rotations(shape, "haar")
    gc = gpu_cache(ok, shape, rk, rv, T + 64)
    fill_layer_device(gc, 0, shape.B, shape.Hkv, shape.D, T, seed=0, dist="normal", outliers="percent")
    mask = synth.outlier_mask(shape.D, shape.Hkv, 0, 0, "percent")
    k1, v1, _ = inputs(shape, 1, chunk=99)
    qb = query(shape, mask, step=1)
    # the step (what the benchmark times), then the attention call alone
    gc.set_decode_impl(impl)
    got_step = _step(ok, gc, 0, k1, v1, qb)
    got = _decode(ok, gc, 0, qb, impl=impl)
    say(f"  step vs attention call: {rel_l2(got_step, got):.2e}")
    assert rel_l2(got_step, got) <= 2 ** -12
    for b in (0, 15):
        want = oracle_on_exported(gc, 0, qb, shape, rk, rv, batch_idx=slice(b, b + 1))
        e = oracle_err(got[b:b + 1], want)
        say(f"  seq {b}: rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    gc.close()


@pytest.mark.slow
@pytest.mark.parametrize("impl", [0, 2])
def test_full_size_16k_batch1_sampled(ok, impl):
    """The 16k-context batch-1 shape (B=1, Hq=32, Hkv=8, D=128, N=512,
    M=2048) on one layer, filled on the device, then several steps in the
    benchmark's launch configuration (impl 0: one launch at this size) and
    with a q-record launch first (impl 2); every head against the oracle over
    the exported cache after the last step."""
    from bench import fill_layer_device
    shape = Shape(B=1, Hq=32, Hkv=8, D=128, N=512, M=2048, outliers="percent")
    T = 16384
    say("[full 16k batch 1] filling")
    rk, rv = make_rotations(shape, "haar")
    gc = gpu_cache(ok, shape, rk, rv, T + 64)
    fill_layer_device(gc, 0, shape.B, shape.Hkv, shape.D, T, seed=0, dist="normal", outliers="percent")
    mask = synth.outlier_mask(shape.D, shape.Hkv, 0, 0, "percent")
    gc.set_decode_impl(impl)
    for i in range(4):
        k1, v1, _ = inputs(shape, 1, chunk=90 + i)
        qb = query(shape, mask, step=i)
        got = _step(ok, gc, 0, k1, v1, qb)
    want = oracle_on_exported(gc, 0, qb, shape, rk, rv)
    e = oracle_err(got, want)
    say(f"  after 4 steps (T={gc.length(0)}): rel L2 {e:.3e}")
    assert e <= ATTN_TOL
    gc.close()


@pytest.mark.slow
@pytest.mark.parametrize("D,B,vdt", [(128, 16, 0), (512, 4, 0), (512, 4, 1)])
def test_prefill_chunk_full_size(ok, D, B, vdt):
    """A 4096-token prefill append at the benchmark shapes (head_dim 128, B=16
    and head_dim 512, B=4; 8 kv heads), behind 4096 stored tokens so the
    chunk starts mid-cache: the GPU's fp32 rotated rows (dump hook) are within
    fp32 accumulation error of the fp64 rotation, and for sampled (sequence,
    kv head) pairs every stored code, scale, zero and window value of the
    chunk equals the oracle quantizer applied to those rows."""
    from bench import fill_layer_device
    shape = Shape(B=B, Hq=2 * 8, Hkv=8, D=D, N=512, M=2048, outliers="percent", v_dtype=vdt)
    n, T0 = 4096, 4096
    say(f"[prefill chunk full size] D={D} B={B} v_dtype={vdt}")
    rk, rv = make_rotations(shape, "haar")
    gc = gpu_cache(ok, shape, rk, rv, T0 + n + 64)
    fill_layer_device(gc, 0, B, 8, D, T0, seed=0, dist="normal", outliers="percent")
    k, v, _ = inputs(shape, n, chunk=77)
    kr = torch.zeros((B, n, 8, D), dtype=torch.float32, device="cuda")
    vr = torch.zeros_like(kr)
    gc.append_dump(0, dev(k), dev(v), kr, vr)
    torch.cuda.synchronize()
    ek, ev = gc.export(0, 0), gc.export(0, 1)
    pairs = [(0, 0), (B - 1, 7), (B // 2, 3)]
    T = T0 + n
    for xr_dev, bits, R, clip, exp, which in ((kr, k, rk[0], 0.96, ek, 0), (vr, v, rv[0], 0.92, ev, 1)):
        for b, h in pairs:
            xr = xr_dev[b, :, h].cpu().numpy()                                    # [n, D]
            ref = orc.rotate_f64(bits[b:b + 1, :, h:h + 1], R)[0, :, 0]
            err = np.abs(xr - ref).max() / np.abs(ref).max()
            assert err < 1e-5, (which, b, h, err)
            win = orc.f32_to_bf16_bits(orc.canonical_zero(xr))
            if "full" in exp:
                np.testing.assert_array_equal(exp["full"][b, h, T0:T], win)
                continue
            q = orc.quantize_rows(np.ascontiguousarray(xr), 128, clip)
            np.testing.assert_array_equal(exp["codes"][b, h, T0:T], orc.pack_codes(q.codes))
            np.testing.assert_array_equal(exp["s16"][b, h, T0:T].view(np.uint16), q.s16.view(np.uint16))
            np.testing.assert_array_equal(exp["z16"][b, h, T0:T].view(np.uint16), q.z16.view(np.uint16))
            for t in range(max(shape.N, T - shape.M), T):
                np.testing.assert_array_equal(exp["ring"][b, h, t % shape.M], win[t - T0])
        say(f"  which={which}: sampled pairs bit-exact")
    gc.close()


@pytest.mark.slow
def test_prefill_attn_full_size_16k_sampled(ok):
    """Chunked-prefill attention in the benchmark's configuration: 4096 queries
    of the last 4096 positions at the 16k batch-1 shape (Hq=32, Hkv=8, sink
    512, recent 2048); the first, middle and last queries of the chunk, every
    head, against the oracle over the exported cache."""
    from bench import fill_layer_device
    shape = Shape(B=1, Hq=32, Hkv=8, D=128, N=512, M=2048, outliers="percent")
    T, n = 16384, 4096
    say("[full prefill attention 16k] filling")
    rk, rv = make_rotations(shape, "haar")
    gc = gpu_cache(ok, shape, rk, rv, T + 64)
    fill_layer_device(gc, 0, shape.B, shape.Hkv, shape.D, T, seed=0, dist="normal", outliers="percent")
    mask = synth.outlier_mask(shape.D, shape.Hkv, 0, 0, "percent")
    qb = _prefill_q(shape, mask, n)
    got = _prefill_gpu(gc, qb)
    ids = [0, 1, n // 2, n - 2, n - 1]
    kp = planes_from_export(gc.export(0, 0), T, shape.N, shape.M)
    vp = planes_from_export(gc.export(0, 1), T, shape.N, shape.M)
    want = orc.prefill_attention(qb, kp, vp, rk[0], rv[0], shape.Hkv, shape.N, shape.M, 128, 0, 0,
                                 query_ids=ids)
    e = oracle_err(got[:, ids], want)
    say(f"  sampled queries {ids}: rel L2 {e:.3e}")
    assert e <= ATTN_TOL
    gc.close()


@pytest.mark.slow
def test_prefill_attn_wide_16k_sampled(ok):
    """Chunked-prefill attention at head_dim 512 with the wide-head model's
    heads and windows (Hq=16, Hkv=8, sink 512, recent 2048) at 16k context,
    batch 1: 256 queries of the last positions; the first, middle and last
    queries of the chunk, every head, against the oracle over the exported
    cache."""
    from bench import fill_layer_device
    shape = Shape(B=1, Hq=16, Hkv=8, D=512, N=512, M=2048, outliers="percent")
    T, n = 16384, 256
    say("[prefill attention wide 16k] filling")
    rk, rv = make_rotations(shape, "haar")
    gc = gpu_cache(ok, shape, rk, rv, T + 64)
    fill_layer_device(gc, 0, shape.B, shape.Hkv, shape.D, T, seed=0, dist="normal", outliers="percent")
    mask = synth.outlier_mask(shape.D, shape.Hkv, 0, 0, "percent")
    qb = _prefill_q(shape, mask, n)
    got = _prefill_gpu(gc, qb)
    ids = [0, 1, n // 2, n - 2, n - 1]
    kp = planes_from_export(gc.export(0, 0), T, shape.N, shape.M)
    vp = planes_from_export(gc.export(0, 1), T, shape.N, shape.M)
    want = orc.prefill_attention(qb, kp, vp, rk[0], rv[0], shape.Hkv, shape.N, shape.M, 128, 0, 0,
                                 query_ids=ids)
    e = oracle_err(got[:, ids], want)
    say(f"  sampled queries {ids}: rel L2 {e:.3e}")
    assert e <= ATTN_TOL
    gc.close()


@pytest.mark.slow
def test_full_size_128k_gqa8_sampled(ok):
    """The 128k-context GQA-8 shape (B=8, Hq=64, Hkv=8, D=128, N=64, M=256,
    Student-t(3) values) on one layer, filled on the device, one fused step
    in the benchmark's launch configuration; sequences 0 and 7 checked against
    the oracle over the exported cache."""
    from bench import fill_layer_device
    shape = Shape(B=8, Hq=64, Hkv=8, D=128, N=64, M=256, dist="student_t3", outliers="none")
    T = 131072
    say("[full 128k gqa8] filling")
    rk, rv = make_rotations(shape, "haar")
    gc = gpu_cache(ok, shape, rk, rv, T + 64)
    fill_layer_device(gc, 0, shape.B, shape.Hkv, shape.D, T, seed=0, dist="student_t3", outliers="none")
    mask = synth.outlier_mask(shape.D, shape.Hkv, 0, 0, "none")
    k1, v1, _ = inputs(shape, 1, chunk=99)
    qb = query(shape, mask, step=1)
    got_step = _step(ok, gc, 0, k1, v1, qb)
    got = _decode(ok, gc, 0, qb)
    say(f"  step vs attention call: {rel_l2(got_step, got):.2e}")
    assert rel_l2(got_step, got) <= 2 ** -12
    for b in (0, 7):
        want = oracle_on_exported(gc, 0, qb, shape, rk, rv, batch_idx=slice(b, b + 1))
        e = oracle_err(got[b:b + 1], want)
        say(f"  seq {b}: rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    gc.close()


@pytest.mark.slow
def test_full_size_wide_64k_sampled(ok):
    """The wide-head shape (B=4, Hq=16, Hkv=8, D=512, N=512, M=2048) at 64k
    context on one layer, filled on the device, decoded in the benchmark's
    launch configuration; sequences 0 and 3 checked against the oracle over
    the exported cache."""
    from bench import fill_layer_device
    shape = Shape(B=4, Hq=16, Hkv=8, D=512, N=512, M=2048, outliers="percent")
    T = 65536
    say("[full wide 64k] filling")
    rk, rv = make_rotations(shape, "haar")
    gc = gpu_cache(ok, shape, rk, rv, T + 64)
    fill_layer_device(gc, 0, shape.B, shape.Hkv, shape.D, T, seed=0, dist="normal", outliers="percent")
    mask = synth.outlier_mask(shape.D, shape.Hkv, 0, 0, "percent")
    k1, v1, _ = inputs(shape, 1, chunk=99)
    qb = query(shape, mask, step=1)
    _step(ok, gc, 0, k1, v1, qb)
    got = _decode(ok, gc, 0, qb)
    for b in (0, 3):
        want = oracle_on_exported(gc, 0, qb, shape, rk, rv, batch_idx=slice(b, b + 1))
        e = oracle_err(got[b:b + 1], want)
        say(f"  seq {b}: rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    gc.close()


def test_stream_read_calibration(ok):
    """The read-only calibration kernel reads every word once: its XOR equals
    the host XOR of the buffer (odd and even sizes of the grid-stride tail)."""
    rng = np.random.default_rng(7)
    for nwords in (4, 4 * 1000 + 4, 4 * (1 << 18)):
        host = rng.integers(0, 2 ** 31 - 1, size=nwords, dtype=np.int64).astype(np.int32)
        src = torch.from_numpy(host).cuda()
        acc = torch.zeros(8192, dtype=torch.int32, device="cuda")
        ok.oscar_stream_read(src, nwords * 4, acc)
        torch.cuda.synchronize()
        want = np.bitwise_xor.reduce(host.view(np.uint32))
        got = np.bitwise_xor.reduce(acc.cpu().numpy().view(np.uint32))
        assert int(got) == int(want), nwords


@pytest.mark.slow
def test_full_size_wide_64k_vbf16_sampled(ok):
    """The wide-head shape with V kept bf16 (INT2 K only) at 64k context on
    one layer; sequences 0 and 3 against the oracle over the exported cache."""
    from bench import fill_layer_device
    shape = Shape(B=4, Hq=16, Hkv=8, D=512, N=512, M=2048, outliers="percent", v_dtype=1)
    T = 65536
    say("[full wide 64k bf16 V] filling")
    rk, rv = make_rotations(shape, "haar")
    gc = gpu_cache(ok, shape, rk, rv, T + 64)
    fill_layer_device(gc, 0, shape.B, shape.Hkv, shape.D, T, seed=0, dist="normal", outliers="percent")
    mask = synth.outlier_mask(shape.D, shape.Hkv, 0, 0, "percent")
    k1, v1, _ = inputs(shape, 1, chunk=99)
    qb = query(shape, mask, step=1)
    _step(ok, gc, 0, k1, v1, qb)
    got = _decode(ok, gc, 0, qb)
    for b in (0, 3):
        want = oracle_on_exported(gc, 0, qb, shape, rk, rv, batch_idx=slice(b, b + 1))
        e = oracle_err(got[b:b + 1], want)
        say(f"  seq {b}: rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    gc.close()


@pytest.mark.parametrize("shape,impl", [
    (Shape(B=2, Hq=8, Hkv=2, N=16, M=64), 0),                   # fused matrix-core step, 4 heads per kv head
    (Shape(B=1, Hq=16, Hkv=2, N=16, M=64), 0),                  # 8 heads per kv head
    (Shape(B=2, Hq=8, Hkv=2, N=16, M=64), 1),                   # VALU kernel + standalone merge
    (Shape(B=2, Hq=4, Hkv=2, D=512, N=16, M=64), 0),            # head_dim 512
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64, v_dtype=1), 0), # head_dim 512, bf16 V
])
def test_absorbed_v_rotation(ok, shape, impl):
    """absorb_v_rotation = 1: the output is o' (V-rotated basis), within the bar
    of the oracle's o', and o' @ R_V^T matches an ordinary cache's output."""
    say(f"[absorbed V rotation] {shape} impl={impl}")
    rk, rv = make_rotations(shape, "haar")
    T = 900
    k, v, mask = inputs(shape, T)
    ga = gpu_cache(ok, shape, rk, rv, T + 4, absorb_v=1)
    gn = gpu_cache(ok, shape, rk, rv, T + 4)
    for g in (ga, gn):
        g.append(0, dev(k[:, :T - 1]), dev(v[:, :T - 1]))
    qb = query(shape, mask)
    # one fused step each (the merge paths of the step), then plain decodes
    got_a = _step(ok, ga, 0, k[:, T - 1:T], v[:, T - 1:T], qb)
    got_n = _step(ok, gn, 0, k[:, T - 1:T], v[:, T - 1:T], qb)
    want = oracle_on_exported(ga, 0, qb, shape, rk, rv, absorb_v=True)
    e = oracle_err(got_a, want)
    say(f"  step: rel L2 vs oracle o' {e:.3e}")
    assert e <= ATTN_TOL
    Rv = rv[0].astype(np.float64)
    assert rel_l2(got_a.astype(np.float64) @ Rv.T, got_n) <= 1e-5
    got_a = _decode(ok, ga, 0, qb, impl=impl)
    got_n = _decode(ok, gn, 0, qb, impl=impl)
    e = oracle_err(got_a, want)
    say(f"  decode impl={impl}: rel L2 vs oracle o' {e:.3e}")
    assert e <= ATTN_TOL
    assert rel_l2(got_a.astype(np.float64) @ Rv.T, got_n) <= 1e-5
    ga.close()
    gn.close()


@pytest.mark.parametrize("shape", [
    Shape(B=2, Hq=8, Hkv=2, N=16, M=64),                        # fused matrix-core step, 4 heads per kv head
    Shape(B=1, Hq=16, Hkv=2, N=16, M=64),                       # 8 heads per kv head
    Shape(B=2, Hq=4, Hkv=2, D=512, N=16, M=64),                 # head_dim 512: four 128-blocks
    Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64, v_dtype=1),      # head_dim 512, bf16 V
])
def test_in_quant_hadamard(ok, shape):
    """in_quant_hadamard = 128 on the GPU against the oracle run with the
    rotations fp32(R @ H): the GPU's fp32 rotated vectors are within fp32
    accumulation error of x @ R @ H in fp64, its codes and metadata equal the
    oracle quantizer on those vectors, and attention (one fused step, then a
    plain decode) is within the bar over the identical cache."""
    say(f"[in-quant Hadamard] {shape}")
    rk, rv = make_rotations(shape, "haar")
    rkh = np.stack([orc.with_in_quant_hadamard(r) for r in rk])
    rvh = np.stack([orc.with_in_quant_hadamard(r) for r in rv])
    T = 600
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 4, hadamard=128)
    D = shape.D
    kr = torch.zeros((shape.B, T - 1, shape.Hkv, D), dtype=torch.float32, device="cuda")
    vr = torch.zeros_like(kr)
    gc.append_dump(0, dev(k[:, :T - 1]), dev(v[:, :T - 1]), kr, vr)
    torch.cuda.synchronize()
    kr, vr = kr.cpu().numpy(), vr.cpu().numpy()
    planes = ((kr, k, rk[0], 0.96, 0),) + (((vr, v, rv[0], 0.92, 1),) if shape.v_dtype == 0 else ())
    for xr, bits, R, clip, which in planes:
        ref = orc.rotate_f64(bits[:, :T - 1], R) @ orc.block_hadamard(D)
        err = np.abs(xr - ref).max() / np.abs(ref).max()
        say(f"  which={which} max rel rotation err vs x R H {err:.2e}")
        assert err < 1e-5
        x32 = np.ascontiguousarray(np.transpose(xr, (0, 2, 1, 3)))            # [B, H, T, D]
        q = orc.quantize_rows(x32.reshape(-1, D), 128, clip)
        exp = gc.export(0, which)
        np.testing.assert_array_equal(exp["codes"].reshape(-1, D // 4), orc.pack_codes(q.codes))
        np.testing.assert_array_equal(exp["s16"].reshape(-1, D // 128).view(np.uint16), q.s16.view(np.uint16))
        np.testing.assert_array_equal(exp["z16"].reshape(-1, D // 128).view(np.uint16), q.z16.view(np.uint16))
    qb = query(shape, mask)
    got = _step(ok, gc, 0, k[:, T - 1:T], v[:, T - 1:T], qb)
    want = oracle_on_exported(gc, 0, qb, shape, rkh, rvh)
    e = oracle_err(got, want)
    say(f"  step: rel L2 vs oracle over the identical cache {e:.3e}")
    assert e <= ATTN_TOL
    got = _decode(ok, gc, 0, qb)
    e = oracle_err(got, want)
    say(f"  decode: rel L2 {e:.3e}")
    assert e <= ATTN_TOL
    oc = oracle_cache(shape, rkh, rvh)
    oc.append(0, k, v)
    e2e = rel_l2(got, oc.attend(0, qb))
    say(f"  end to end vs the oracle's own cache: rel L2 {e2e:.3e}")
    assert e2e <= 1e-2
    if D == 128:                      # chunked-prefill attention reads the same rotations
        qp = _prefill_q(shape, mask, 50)
        gotp = _prefill_gpu(gc, qp)
        wantp = _prefill_oracle(gc, qp, shape, rkh, rvh)
        e = oracle_err(gotp, wantp)
        say(f"  prefill attention: rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    gc.close()


# ------------------------------------------------------------------ chunked-prefill attention


def _prefill_q(shape, mask, n, step0=0):
    return np.stack([query(shape, mask, step=step0 + i) for i in range(n)], axis=1)   # [B, n, Hq, D]


def _prefill_gpu(gc, qb, out_dtype=0):
    B, n, Hq, D = qb.shape
    dt = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}[out_dtype]
    out = torch.zeros((B, n, Hq, D), dtype=dt, device="cuda")
    gc.prefill_attn(0, dev(qb), out, out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _prefill_oracle(gc, qb, shape, rk, rv, absorb_v=False):
    T = gc.length(0)
    kp = planes_from_export(gc.export(0, 0), T, shape.N, shape.M)
    vp = planes_from_export(gc.export(0, 1), T, shape.N, shape.M)
    D = shape.D
    Rk = rk[0] if rk is not None else np.eye(D, dtype=np.float32)
    Rv = rv[0] if rv is not None else np.eye(D, dtype=np.float32)
    return orc.prefill_attention(qb, kp, vp, Rk, Rv, shape.Hkv, shape.N, shape.M, 128,
                                 shape.k_dtype, shape.v_dtype, absorb_v=absorb_v)


@pytest.mark.parametrize("shape,T0,n", [
    (Shape(B=2, Hq=8, Hkv=2, N=16, M=64), 500, 200),            # 4 query heads per kv head, INT2 inside the chunk
    (Shape(B=1, Hq=16, Hkv=2, N=16, M=64), 300, 130),           # 8 per kv head
    (Shape(B=2, Hq=2, Hkv=2, N=16, M=64), 200, 70),             # 1 per kv head
    (Shape(B=1, Hq=8, Hkv=2, N=16, M=64, v_dtype=1), 300, 100), # bf16 V plane
    (Shape(B=1, Hq=8, Hkv=2, N=0, M=0), 150, 67),               # no windows: INT2 everywhere
    (Shape(B=1, Hq=8, Hkv=2, N=40, M=60), 0, 100),              # the whole sequence is the chunk, all window
    (Shape(B=1, Hq=8, Hkv=2, N=3, M=500), 700, 129),            # recent window longer than the chunk
    (Shape(B=1, Hq=32, Hkv=2, N=16, M=64), 250, 37),            # 16 query heads per kv head (4 queries per block)
    (Shape(B=1, Hq=8, Hkv=2, N=16, M=64, k_dtype=1), 300, 90),  # bf16 K plane, INT2 V
    (Shape(B=1, Hq=8, Hkv=2, N=16, M=64, k_dtype=1, v_dtype=1), 300, 90),  # both planes bf16
    (Shape(B=3, Hq=8, Hkv=2, N=16, M=64, outliers="percent", dist="student_t3"), 1000, 300),  # heavy tails
    # key tiles that end at or before a block's first query position skip the
    # causal compare: the first block's first query sits at the edge of tile 0
    (Shape(B=1, Hq=8, Hkv=2, N=16, M=64), 63, 80),              # at position 63: tile 0 unmasked, exactly full
    (Shape(B=1, Hq=8, Hkv=2, N=16, M=64), 62, 81),              # at position 62: tile 0 still masked
    (Shape(B=2, Hq=2, Hkv=2, N=0, M=0), 127, 64),               # 1 head, at position 127: two unmasked INT2 tiles first
    # head_dim 512 (16 query rows per block, 32-token key tiles)
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64), 300, 70),      # 2 query heads per kv head
    (Shape(B=2, Hq=2, Hkv=2, D=512, N=16, M=64), 200, 33),      # 1 per kv head
    (Shape(B=1, Hq=8, Hkv=2, D=512, N=16, M=64, v_dtype=1), 250, 40),   # 4 per kv head, bf16 V plane
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=0, M=0), 100, 50),        # no windows
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=40, M=60), 0, 70),        # all window
    (Shape(B=1, Hq=32, Hkv=2, D=512, N=16, M=64), 120, 9),      # 16 per kv head (one query per block)
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=3, M=500), 600, 45),      # recent window longer than the chunk
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64), 31, 40),       # first query at position 31: tile 0 unmasked
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64), 30, 41),       # at position 30: tile 0 masked
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64, k_dtype=1), 150, 30),   # bf16 K plane
])
def test_prefill_attn_vs_oracle(ok, shape, T0, n):
    """Chunked-prefill attention through the C ABI against the oracle over the
    identical (exported) cache: every query of the chunk, rel L2 <= 2e-3."""
    say(f"[prefill attention] {shape} T0={T0} n={n}")
    rk, rv = make_rotations(shape, "haar")
    k, v, mask = inputs(shape, T0 + n)
    gc = gpu_cache(ok, shape, rk, rv, T0 + n + 8)
    if T0:
        gc.append(0, dev(k[:, :T0]), dev(v[:, :T0]))
    gc.append(0, dev(k[:, T0:]), dev(v[:, T0:]))
    qb = _prefill_q(shape, mask, n)
    got = _prefill_gpu(gc, qb)
    want = _prefill_oracle(gc, qb, shape, rk, rv)
    e = oracle_err(got, want)
    worst = max(rel_l2(got[:, i], want[:, i]) for i in range(n))
    say(f"  rel L2 {e:.3e} (worst query {worst:.3e})")
    assert e <= ATTN_TOL and worst <= ATTN_TOL
    gc.close()


def test_prefill_attn_last_query_is_decode(ok):
    """The chunk's last query attends over the whole cache: it equals the
    decode attention call for the same q (two kernels, one definition), and a
    chunk of one query is that call."""
    shape = Shape(B=2, Hq=8, Hkv=2, N=16, M=64)
    say("[prefill attention] last query vs decode")
    rk, rv = make_rotations(shape, "haar")
    T = 900
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 8)
    gc.append(0, dev(k), dev(v))
    qb = _prefill_q(shape, mask, 3)
    got = _prefill_gpu(gc, qb)
    dec = _decode(ok, gc, 0, qb[:, -1])
    say(f"  last query vs decode: {rel_l2(got[:, -1], dec):.2e}")
    assert rel_l2(got[:, -1], dec) <= 1e-3
    one = _prefill_gpu(gc, qb[:, -1:])
    assert rel_l2(one[:, 0], dec) <= 1e-3
    gc.close()


@pytest.mark.parametrize("D", [128, 512])
def test_prefill_attn_absorbed_and_dtypes(ok, D):
    """absorb_v_rotation = 1 returns o' (the oracle's o'); bf16 and fp16
    outputs are the fp32 output rounded."""
    shape = Shape(B=1, Hq=8, Hkv=2, D=D, N=16, M=64)
    say(f"[prefill attention] absorbed V rotation, output dtypes, D={D}")
    rk, rv = make_rotations(shape, "haar")
    T0, n = 300, 90
    k, v, mask = inputs(shape, T0 + n)
    ga = gpu_cache(ok, shape, rk, rv, T0 + n, absorb_v=1)
    ga.append(0, dev(k), dev(v))
    qb = _prefill_q(shape, mask, n)
    got = _prefill_gpu(ga, qb)
    want = _prefill_oracle(ga, qb, shape, rk, rv, absorb_v=True)
    assert oracle_err(got, want) <= ATTN_TOL
    for dt, tol in ((1, 2.0 ** -8), (2, 2.0 ** -11)):
        o = _prefill_gpu(ga, qb, dt)
        assert np.abs(o - got).max() <= tol * np.abs(got).max() + 1e-6
    ga.close()


def test_prefill_attn_rejects(ok):
    """Argument checks before anything is enqueued: n_q beyond the cached
    tokens, a batch other than the layer's, a number of query heads per kv
    head that does not divide the 16 query rows of a head_dim-512 block."""
    shape = Shape(B=1, Hq=8, Hkv=2, N=16, M=64)
    rk, rv = make_rotations(shape, "haar")
    k, v, mask = inputs(shape, 40)
    gc = gpu_cache(ok, shape, rk, rv, 64)
    gc.append(0, dev(k), dev(v))
    q = torch.zeros((1, 41, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, 41, 8, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ok.OscarError):
        gc.prefill_attn(0, q, out)
    with pytest.raises(ok.OscarError):
        ok.oscar_prefill_attn(gc.handle, 0, q, out, 0, 2, 4)
    gc.close()
    wide = Shape(B=1, Hq=6, Hkv=2, D=512, N=16, M=64)
    gw = gpu_cache(ok, wide, None, None, 64)
    kw, vw, _ = inputs(wide, 10)
    gw.append(0, dev(kw), dev(vw))
    qw = torch.zeros((1, 2, 6, 512), dtype=torch.bfloat16, device="cuda")
    ow = torch.zeros((1, 2, 6, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(ok.OscarError):
        gw.prefill_attn(0, qw, ow)
    gw.close()


def test_prefill_attn_after_decode_steps(ok):
    """A cache filled in several chunks and single-token decode steps (the
    recent ring wrapped several times), then one more chunk: its queries
    against the oracle over the identical cache."""
    shape = Shape(B=2, Hq=8, Hkv=2, N=16, M=64)
    say("[prefill attention] after decode steps")
    rk, rv = make_rotations(shape, "haar")
    T = 700
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 8)
    gc.append(0, dev(k[:, :300]), dev(v[:, :300]))
    for t in range(300, 340):
        _step(ok, gc, 0, k[:, t:t + 1], v[:, t:t + 1], query(shape, mask, step=t))
    gc.append(0, dev(k[:, 340:500]), dev(v[:, 340:500]))
    gc.append(0, dev(k[:, 500:]), dev(v[:, 500:]))
    qb = _prefill_q(shape, mask, T - 500, step0=7)
    got = _prefill_gpu(gc, qb)
    want = _prefill_oracle(gc, qb, shape, rk, rv)
    e = oracle_err(got, want)
    say(f"  rel L2 {e:.3e}")
    assert e <= ATTN_TOL
    gc.close()


@pytest.mark.parametrize("shape,impl", [
    (Shape(B=2, Hq=8, Hkv=2, N=16, M=64), 0),                   # matrix-core kernel, 4 heads per kv head
    (Shape(B=1, Hq=16, Hkv=2, N=16, M=64), 0),                  # 8 heads per kv head
    (Shape(B=2, Hq=8, Hkv=2, N=16, M=64), 1),                   # VALU kernel
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64), 0),            # head_dim 512
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64, v_dtype=1), 0), # head_dim 512, bf16 V
])
def test_softmax_scale_argument(ok, shape, impl):
    """A caller-given softmax scale (not 1/sqrt(D)) reaches every kernel: the
    fused step, the attention call and (head_dim 128) prefill attention,
    against the oracle with the same scale over the identical cache."""
    say(f"[softmax scale] {shape} impl={impl}")
    rk, rv = make_rotations(shape, "haar")
    T, sc = 700, 0.031
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 4)
    gc.append(0, dev(k[:, :T - 1]), dev(v[:, :T - 1]))
    qb = query(shape, mask)
    B, Hq, D = qb.shape
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    gc.set_decode_impl(impl)
    gc.decode_step(0, dev(k[:, T - 1:T]), dev(v[:, T - 1:T]), dev(qb), out, 0, sc)
    torch.cuda.synchronize()
    got_step = out.cpu().numpy()
    out.zero_()
    gc.decode_attn(0, dev(qb), out, 0, sc)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    T1 = gc.length(0)
    kp = planes_from_export(gc.export(0, 0), T1, shape.N, shape.M)
    vp = planes_from_export(gc.export(0, 1), T1, shape.N, shape.M)
    want = orc.decode_attention(qb, kp, vp, rk[0], rv[0], shape.Hkv, shape.N, shape.M, 128,
                                shape.k_dtype, shape.v_dtype, scale=sc)
    default = orc.decode_attention(qb, kp, vp, rk[0], rv[0], shape.Hkv, shape.N, shape.M, 128,
                                   shape.k_dtype, shape.v_dtype)
    assert rel_l2(default, want) > 1e-2                 # the scale matters on this input
    for name, g in (("step", got_step), ("call", got)):
        e = oracle_err(g, want)
        say(f"  {name}: rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    if D == 128:
        qp = _prefill_q(shape, mask, 20)
        outp = torch.zeros((B, 20, Hq, D), dtype=torch.float32, device="cuda")
        gc.prefill_attn(0, dev(qp), outp, 0, sc)
        torch.cuda.synchronize()
        wantp = orc.prefill_attention(qp, kp, vp, rk[0], rv[0], shape.Hkv, shape.N, shape.M, 128,
                                      shape.k_dtype, shape.v_dtype, scale=sc)
        e = oracle_err(outp.cpu().numpy(), wantp)
        say(f"  prefill: rel L2 {e:.3e}")
        assert e <= ATTN_TOL
    gc.close()
