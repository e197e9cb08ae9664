"""The head_dim-128 attention launch's one-round schedule (every block of the
launch resident at once: one INT2 split per block, the window chunks carried
by the first splits) against the oracle and against the several-round
schedule (it runs only when the test switch turns it on)."""
import numpy as np
import pytest

import synth
from tests.gpu_util import (ATTN_TOL, Shape, gpu_cache, inputs, make_rotations, oracle_err, oracle_on_exported,
                            query, rel_l2, say)

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


def _decode(gc, qb):
    out = torch.zeros(qb.shape, dtype=torch.float32, device="cuda")
    gc.decode_attn(0, dev(qb), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("gq", [4, 8])
@pytest.mark.parametrize("T,N,M", [(5000, 64, 256), (1500, 8, 700), (321, 64, 256), (40, 64, 256),
                                   (3000, 0, 0), (2000, 0, 64)])
@pytest.mark.parametrize("R", [3, 6, 16])
def test_one_round_decode(ok, gq, T, N, M, R):
    """decode_attn under the one-round schedule with R blocks per (sequence,
    kv head): within the bar of the oracle on the exported cache, and within
    the fp16 operand half-ulp of the several-round schedule."""
    shape = Shape(B=2, Hq=2 * gq, Hkv=2, N=N, M=M)
    say(f"[one round] gq={gq} T={T} N={N} M={M} R={R}")
    rk, rv = make_rotations(shape, "haar")
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 4)
    gc.append(0, dev(k), dev(v))
    qb = query(shape, mask)
    gc.set_one_round(-1)
    ref = _decode(gc, qb)
    gc.set_one_round(R)
    got = _decode(gc, qb)
    e = oracle_err(got, oracle_on_exported(gc, 0, qb, shape, rk, rv))
    d = rel_l2(got, ref)
    say(f"  rel L2 {e:.3e}, vs several rounds {d:.2e}")
    assert d <= 2 ** -12
    gc.close()


@pytest.mark.parametrize("gq,R,M", [(4, 3, 24), (4, 6, 64), (8, 5, 64), (4, 16, 24), (8, 3, 70)])
def test_one_round_decode_steps(ok, gq, R, M):
    """Decode steps from an empty cache through the sink, the ring's wrap and
    into the INT2 range (a ring of at least a tile: the append by producer
    blocks of the attention launch; under a tile: in a launch of its own): the
    stored cache bit-equal to a twin filled by separate calls, outputs within
    the bar."""
    shape = Shape(B=2, Hq=2 * gq, Hkv=2, N=8, M=M)
    say(f"[one round steps] gq={gq} R={R} M={M}")
    rk, rv = make_rotations(shape, "haar")
    steps = 100
    k, v, mask = inputs(shape, steps)
    g1 = gpu_cache(ok, shape, rk, rv, steps)
    g2 = gpu_cache(ok, shape, rk, rv, steps)
    g1.set_one_round(R)
    g2.set_one_round(-1)
    worst = 0.0
    for i in range(steps):
        qb = query(shape, mask, step=i)
        o1 = torch.zeros((shape.B, shape.Hq, shape.D), dtype=torch.float32, device="cuda")
        o2 = torch.zeros_like(o1)
        g1.decode_step(0, dev(k[:, i:i + 1]), dev(v[:, i:i + 1]), dev(qb), o1)
        g2.append(0, dev(k[:, i:i + 1]), dev(v[:, i:i + 1]))
        g2.decode_attn(0, dev(qb), o2)
        torch.cuda.synchronize()
        a, b = o1.cpu().numpy(), o2.cpu().numpy()
        worst = max(worst, rel_l2(a, b))
        assert rel_l2(a, b) <= 2 ** -12, i
        if i in (0, 7, 40, steps - 1):
            oracle_err(a, oracle_on_exported(g1, 0, qb, shape, rk, rv))
    for which in (0, 1):
        e1, e2 = g1.export(0, which), g2.export(0, which)
        for key in ("codes", "s16", "z16"):
            np.testing.assert_array_equal(e1[key], e2[key])
    say(f"  worst vs separate calls {worst:.2e}")
    g1.close()
    g2.close()


def test_one_round_ragged(ok):
    """A ragged batch (lengths below N, at N + M + 1 and long) under the
    one-round schedule: every sequence within the bar of the oracle."""
    shape = Shape(B=4, Hq=8, Hkv=2, N=16, M=64)
    lengths = [5, 81, 3000, 700]
    rk, rv = make_rotations(shape, "haar")
    k, v, mask = inputs(shape, max(lengths))
    gc = gpu_cache(ok, shape, rk, rv, max(lengths) + 2)
    for b, Tb in enumerate(lengths):
        gc.append_seq(0, b, dev(k[b, :Tb]), dev(v[b, :Tb]))
    gc.set_one_round(6)
    qb = query(shape, mask)
    got = _decode(gc, qb)
    gc.set_one_round(-1)
    ref = _decode(gc, qb)
    assert rel_l2(got, ref) <= 2 ** -12
    from tests.test_gpu_ragged import oracle_ragged_on_export
    oracle_err(got, oracle_ragged_on_export(gc, 0, qb, shape, rk, rv, lengths))
    gc.close()


def test_one_round_switch_rejects(ok):
    shape = Shape()
    gc = gpu_cache(ok, shape, None, None, 16)
    for bad in (1, 2, 17, -2):
        with pytest.raises(ok.OscarError):
            gc.set_one_round(bad)
    gc.close()
