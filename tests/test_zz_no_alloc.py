"""The allocation-free decode call (oscar_int2_decode_attn_noalloc, working
memory in a static device array shared by every call on the GPU) against
oscar_int2_decode_attn on the same caches, through the C ABI: on every decode
path, two calls in a row with the second on a smaller input, then the larger
one again (the block counters the first call left must be zero), and the
rejection of a call whose working memory does not fit the array."""
import numpy as np
import pytest

from tests.gpu_util import Shape, gpu_cache, inputs, make_rotations, oracle_err, oracle_on_exported, query, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ok():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_attention_oscar_amd import oscar_kv
    return oscar_kv


def dev(bits):
    import synth
    return synth.bits_to_torch_bf16(bits, "cuda")


def _both(gc, qb):
    outs = []
    for fn in (gc.decode_attn, gc.decode_attn_noalloc):
        out = torch.full(qb.shape, float("nan"), dtype=torch.float32, device="cuda")
        fn(0, dev(qb), out, 0)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    return outs


@pytest.mark.parametrize("Hq,Hkv,D,vdt,impl", [
    (8, 2, 128, 0, 0),   # matrix-core kernel, 4 query heads per kv head (one launch at these sizes)
    (16, 2, 128, 0, 0),  # two head groups
    (8, 2, 128, 0, 2),   # q records in the static array, from a launch of their own
    (16, 2, 128, 0, 2),  # the same, two head groups
    (4, 2, 512, 0, 0),   # head_dim 512
    (4, 2, 512, 1, 0),   # head_dim 512, V kept bf16
    (2, 2, 128, 0, 0),   # general kernel
])
def test_noalloc_equals_decode_attn(ok, Hq, Hkv, D, vdt, impl):
    caches = []
    for B, T in ((4, 3000), (2, 500)):
        shape = Shape(B=B, Hq=Hq, Hkv=Hkv, D=D, N=64, M=256, v_dtype=vdt)
        rk, rv = make_rotations(shape, "haar")
        k, v, mask = inputs(shape, T)
        gc = gpu_cache(ok, shape, rk, rv, T)
        gc.set_decode_impl(impl)
        gc.append(0, dev(k), dev(v))
        caches.append((shape, gc, rk, rv, mask))
    for i in (0, 1, 0):                       # larger, smaller, larger again
        shape, gc, rk, rv, mask = caches[i]
        qb = query(shape, mask, step=i)
        ref, got = _both(gc, qb)
        assert np.array_equal(got, ref), f"call {i}: differs from oscar_int2_decode_attn"
        e = oracle_err(got, oracle_on_exported(gc, 0, qb, shape, rk, rv))
        say(f"[noalloc] Hq={Hq} Hkv={Hkv} D={D} v_dtype={vdt} impl={impl} B={shape.B}: identical, rel L2 {e:.3e}")
    for _, gc, *_ in caches:
        gc.close()


def test_noalloc_rejects_oversize(ok):
    """64 sequences x 64 query heads x 4 splits of 514 floats: 34 MB of
    partial results, more than the 16 MiB array holds."""
    shape = Shape(B=64, Hq=64, Hkv=8, D=512, N=0, M=0)
    gc = gpu_cache(ok, shape, None, None, 300)
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    k = torch.randn((shape.B, 300, shape.Hkv, shape.D), generator=g, device="cuda").to(torch.bfloat16)
    gc.append(0, k, k)
    q = torch.randn((shape.B, shape.Hq, shape.D), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.zeros((shape.B, shape.Hq, shape.D), dtype=torch.float32, device="cuda")
    with pytest.raises(ok.OscarError) as ei:
        gc.decode_attn_noalloc(0, q, out, 0)
    assert ei.value.code == ok.OSCAR_ERR_CAPACITY
    torch.cuda.synchronize()
    assert not bool(out.any())               # nothing was enqueued
    gc.close()
