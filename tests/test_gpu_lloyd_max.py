"""GPU parity of the Lloyd-Max codebook ("OSCAR: 2-bit KV Cache Quantization
for SGLang and llama.cpp": the Lloyd-Max switch of "Installing OSCAR and running
a first Qwen3-8B calibration", LM_RATIO = 1.16 of "Where OSCAR loses, and the
cases it is the wrong tool for") through the C ABI against the CPU oracle.

Bars as for the min/max codebook: codes, scales, zeros (here the group means)
and bf16 windows bit-exact given identical fp32 rotated inputs, end to end where
the rotation is exact in fp32; attention within 2e-3 relative L2 of the oracle
over the identical (exported) cache, row by row.
"""
import numpy as np
import pytest

import oracle as orc
import synth
from tests.gpu_util import (ATTN_TOL, Shape, compare_planes, gpu_cache, inputs, make_rotations, oracle_cache,
                            oracle_err, oracle_on_exported, query, rel_l2, say)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LM = orc.CODEBOOK_LLOYD_MAX


@pytest.fixture(scope="module")
def ok():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_attention_oscar_amd import oscar_kv
    return oscar_kv


def dev(bits):
    return synth.bits_to_torch_bf16(bits, "cuda")


def _near_threshold_rows(D, ratio, seed):
    """Groups with values placed within a few ulps of the decision boundaries
    z + s * {-tau, 0, tau} of their own (fp16) mean and step: a fixed-point
    iteration, since moving the values moves the statistics a little."""
    g = np.random.default_rng(seed)
    rows = []
    tau = np.float32(orc.LLOYD_MAX_THRESHOLD)
    for _ in range(24):
        x = g.standard_normal(D).astype(np.float32)
        for _ in range(4):
            q = orc.quantize_rows_lloyd_max(x[None], 128, ratio)
            for gi in range(D // 128):
                sf = np.float32(q.s16[0, gi])
                zf = np.float32(q.z16[0, gi])
                for j, k in enumerate((-tau, np.float32(0.0), tau)):
                    base = np.float32(zf + np.float32(k * sf))
                    for n in range(-2, 3):
                        v = base
                        for _ in range(abs(n)):
                            v = np.nextafter(v, np.float32(np.inf if n > 0 else -np.inf), dtype=np.float32)
                        x[128 * gi + 8 * j + n + 2] = v
        rows.append(x)
    return np.stack(rows)


def _lm_rows(D, ratio, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal((200, D)).astype(np.float32)
    x[:, 3] *= 8.0
    x[10] = 0.0                               # constant groups: step 0, codes 0
    x[11] = 1.25
    x[12] = -0.0
    x[13] = np.abs(x[13]) + 1                 # one-signed groups
    x[14, ::2] = -0.0
    x[15] *= 1e-6                             # fp16-denormal steps
    x[16] *= 3000.0                           # large range
    x[17] = g.standard_t(3, D).astype(np.float32) * 5
    # exact zeros of (x - z) / s: half the group at the (fp16-exact) mean
    x[18] = np.where(np.arange(D) % 2 == 0, 0.5, np.float32(0.5) + np.float32(2.0) * ((np.arange(D) % 4) - 2))
    return np.concatenate([x, _near_threshold_rows(D, ratio, seed + 1)])


@pytest.mark.parametrize("D", [128, 512])
@pytest.mark.parametrize("ratio", [1.16, 1.0, 0.6])
def test_quantize_rows_lloyd_max_bitexact(ok, D, ratio):
    say(f"[lm quantize_rows] D={D} ratio={ratio}")
    x = _lm_rows(D, ratio, 3 + D)
    rows = x.shape[0]
    codes = torch.zeros((rows, D // 4), dtype=torch.uint8, device="cuda")
    meta = torch.zeros((rows, D // 128, 2), dtype=torch.int16, device="cuda")
    ok.oscar_quantize_rows_lloyd_max(torch.from_numpy(x).cuda(), rows, D, 128, ratio, codes, meta)
    torch.cuda.synchronize()
    q = orc.quantize_rows_lloyd_max(x, 128, ratio)
    np.testing.assert_array_equal(codes.cpu().numpy(), orc.pack_codes(q.codes))
    m = meta.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(m[..., 0], q.s16.view(np.uint16))
    np.testing.assert_array_equal(m[..., 1], q.z16.view(np.uint16))
    assert (q.codes == 3).any() and (q.codes == 0).any()


@pytest.mark.parametrize("shape,chunks", [
    (Shape(B=2, Hq=4, Hkv=1, D=128, N=64, M=256, codebook=LM), [1000, 1, 23, 1]),
    (Shape(B=1, Hq=8, Hkv=2, D=128, N=5, M=7, codebook=LM), [3, 1, 1, 9, 300, 1]),
    (Shape(B=2, Hq=4, Hkv=2, D=512, N=16, M=40, codebook=LM), [77, 1, 300, 2]),
    (Shape(B=1, Hq=4, Hkv=1, D=128, N=8, M=16, v_dtype=1, codebook=LM, lm_ratio=1.0), [50, 1]),
])
def test_append_lloyd_max_exact_rotation_bitexact(ok, shape, chunks):
    """Rotations exact in fp32: one-token appends (VALU rotation) and chunk
    appends (matrix-core rotation, quad-wise statistics) store exactly the
    oracle's codes, steps, means and windows."""
    say(f"[lm append exact] {shape} chunks={chunks}")
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
    compare_planes(gc.export(0, 0), oc.k[0], T, shape.N, shape.M, "K")
    compare_planes(gc.export(0, 1), oc.v[0], T, shape.N, shape.M, "V")
    gc.close()


@pytest.mark.parametrize("D,n", [(128, 70), (128, 1), (512, 70), (512, 1)])
def test_append_lloyd_max_random_rotation_dump(ok, D, n):
    """Haar rotations: the stored codes and metadata equal the oracle's
    Lloyd-Max quantizer applied to the GPU's own fp32 rotated vectors."""
    shape = Shape(B=2, Hq=4, Hkv=2, D=D, N=3, M=9, codebook=LM)
    say(f"[lm append dump] D={D} n={n}")
    rk, rv = make_rotations(shape, "haar")
    k, v, _ = inputs(shape, n)
    gc = gpu_cache(ok, shape, rk, rv, n)
    kr = torch.zeros((shape.B, n, shape.Hkv, D), dtype=torch.float32, device="cuda")
    vr = torch.zeros_like(kr)
    gc.append_dump(0, dev(k), dev(v), kr, vr)
    torch.cuda.synchronize()
    for xr, which in ((kr.cpu().numpy(), 0), (vr.cpu().numpy(), 1)):
        x32 = np.ascontiguousarray(np.transpose(xr, (0, 2, 1, 3)))
        q = orc.quantize_rows_lloyd_max(x32.reshape(-1, D), 128, shape.lm_ratio)
        exp = gc.export(0, which)
        np.testing.assert_array_equal(exp["codes"].reshape(-1, D // 4), orc.pack_codes(q.codes))
        np.testing.assert_array_equal(exp["s16"].reshape(-1, D // 128).view(np.uint16), q.s16.view(np.uint16))
        np.testing.assert_array_equal(exp["z16"].reshape(-1, D // 128).view(np.uint16), q.z16.view(np.uint16))
    gc.close()


def _decode(gc, layer, qbits):
    B, Hq, D = qbits.shape
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    gc.decode_attn(layer, dev(qbits), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("shape,T", [
    (Shape(codebook=LM), 1025),                                               # the tiny shape
    (Shape(B=2, Hq=32, Hkv=8, D=128, N=64, M=256, outliers="percent", codebook=LM), 3000),
    (Shape(B=1, Hq=16, Hkv=2, D=128, N=8, M=40, codebook=LM), 700),           # 8 query heads per kv head
    (Shape(B=2, Hq=4, Hkv=2, D=512, N=16, M=64, codebook=LM), 900),           # head_dim 512
    (Shape(B=1, Hq=4, Hkv=2, D=512, N=16, M=64, v_dtype=1, codebook=LM), 500),  # V kept bf16
    (Shape(codebook=LM, outlier_scale=32.0), 1025),
    (Shape(codebook=LM, N=0, M=0), 300),                                      # every token INT2
])
def test_decode_lloyd_max_vs_oracle(ok, shape, T):
    say(f"[lm decode] {shape} T={T}")
    rk, rv = make_rotations(shape, "haar")
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 4)
    gc.append(0, dev(k[:, :T // 2]), dev(v[:, :T // 2]))
    gc.append(0, dev(k[:, T // 2:]), dev(v[:, T // 2:]))
    qb = query(shape, mask)
    got = _decode(gc, 0, qb)
    want = oracle_on_exported(gc, 0, qb, shape, rk, rv)
    e = oracle_err(got, want)
    say(f"  rel L2 {e:.3e}")
    assert e <= ATTN_TOL
    gc.close()


def test_decode_lloyd_max_end_to_end_exact(ok):
    """Exact rotations: the GPU cache equals the oracle's own, so its decode
    attention is held to the bar end to end (not only on the export)."""
    shape = Shape(B=2, Hq=8, Hkv=2, codebook=LM)
    rk, rv = make_rotations(shape, "exact")
    T = 1500
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T)
    oc = oracle_cache(shape, rk, rv)
    gc.append(0, dev(k), dev(v))
    oc.append(0, k, v)
    qb = query(shape, mask)
    e = oracle_err(_decode(gc, 0, qb), oc.attend(0, qb))
    say(f"[lm end-to-end exact] rel L2 {e:.3e}")
    # the uniform codebook gives a different cache and output
    su = Shape(B=2, Hq=8, Hkv=2)
    ou = oracle_cache(su, rk, rv)
    ou.append(0, k, v)
    assert rel_l2(ou.attend(0, qb), oc.attend(0, qb)) > 1e-2
    gc.close()


def test_decode_step_lloyd_max(ok):
    """decode_step (append one token, then attend) over many steps from an
    empty cache, ring wrapping, against the oracle over the exported cache and
    bit-exact stored planes with exact rotations."""
    shape = Shape(B=2, Hq=4, Hkv=2, N=4, M=20, codebook=LM)
    rk, rv = make_rotations(shape, "exact")
    steps = 90
    k, v, mask = inputs(shape, steps)
    gc = gpu_cache(ok, shape, rk, rv, steps)
    oc = oracle_cache(shape, rk, rv)
    for i in range(steps):
        qb = query(shape, mask, step=i)
        out = torch.zeros((shape.B, shape.Hq, shape.D), dtype=torch.float32, device="cuda")
        gc.decode_step(0, dev(k[:, i:i + 1]), dev(v[:, i:i + 1]), dev(qb), out)
        oc.append(0, k[:, i:i + 1], v[:, i:i + 1])
        if i in (0, 30, steps - 1):
            torch.cuda.synchronize()
            e = oracle_err(out.cpu().numpy(), oc.attend(0, qb))
            say(f"[lm decode step] step {i}: rel L2 {e:.3e}")
    compare_planes(gc.export(0, 0), oc.k[0], steps, shape.N, shape.M, "K")
    compare_planes(gc.export(0, 1), oc.v[0], steps, shape.N, shape.M, "V")
    gc.close()


def test_prefill_attn_lloyd_max_unsupported(ok):
    shape = Shape(codebook=LM)
    rk, rv = make_rotations(shape, "identity")
    k, v, mask = inputs(shape, 40)
    gc = gpu_cache(ok, shape, rk, rv, 64)
    gc.append(0, dev(k), dev(v))
    q = torch.zeros((1, 8, shape.Hq, shape.D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, 8, shape.Hq, shape.D), dtype=torch.float32, device="cuda")
    with pytest.raises(ok.OscarError) as ei:
        gc.prefill_attn(0, q, out)
    assert ei.value.code == ok.OSCAR_ERR_UNSUPPORTED
    gc.close()
