"""GPU parity of ragged batches: the sequences of a layer at their own lengths
(the requests of a serving batch: "OSCAR-RotationZoo", "How to use" step 2,
the sglang server), through the C ABI against the oracle's ragged cache (one
cache per sequence).

Bars: stored codes, scales, zeros and windows bit-exact where the rotation is
exact in fp32; attention within 2e-3 relative L2 of the oracle over the
exported cache, row by row, every sequence with the windows of its own length.
"""
import numpy as np
import pytest

import oracle as orc
import synth
from tests.gpu_util import (ATTN_TOL, Shape, compare_planes, gpu_cache, inputs, make_rotations, oracle_err,
                            planes_from_export, query, rel_l2, say)

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


def ragged_oracle(shape, rk, rv):
    cfg = orc.OracleConfig(num_layers=shape.L, batch=shape.B, num_q_heads=shape.Hq, num_kv_heads=shape.Hkv,
                           head_dim=shape.D, sink_tokens=shape.N, recent_tokens=shape.M, k_clip=shape.k_clip,
                           v_clip=shape.v_clip, k_dtype=shape.k_dtype, v_dtype=shape.v_dtype,
                           codebook=shape.codebook, lm_ratio=shape.lm_ratio)
    return orc.OracleRaggedCache(cfg, rk, rv)


def _seq_export(exp, b, Tb):
    return {k: (v[b:b + 1, :, :Tb] if k in ("codes", "s16", "z16", "full") else v[b:b + 1]) for k, v in exp.items()}


def oracle_ragged_on_export(gc, layer, qb, shape, rk, rv, lengths, absorb_v=False):
    """Oracle attention of every sequence over its own part of the exported
    cache (its first T_b positions, its windows)."""
    ek, ev = gc.export(layer, 0), gc.export(layer, 1)
    Rk = rk[layer] if rk is not None else np.eye(shape.D, dtype=np.float32)
    Rv = rv[layer] if rv is not None else np.eye(shape.D, dtype=np.float32)
    out = []
    for b, Tb in enumerate(lengths):
        kp = planes_from_export(_seq_export(ek, b, Tb), Tb, shape.N, shape.M, shape.codebook)
        vp = planes_from_export(_seq_export(ev, b, Tb), Tb, shape.N, shape.M, shape.codebook)
        out.append(orc.decode_attention(qb[b:b + 1], kp, vp, Rk, Rv, shape.Hkv, shape.N, shape.M, 128,
                                        shape.k_dtype, shape.v_dtype, absorb_v=absorb_v))
    return np.concatenate(out)


def compare_ragged_planes(gc, oc, layer, shape, lengths):
    ek, ev = gc.export(layer, 0), gc.export(layer, 1)
    for b, Tb in enumerate(lengths):
        if Tb == 0:
            continue
        compare_planes(_seq_export(ek, b, Tb), oc.seqs[b].k[layer], Tb, shape.N, shape.M, f"K seq {b}")
        compare_planes(_seq_export(ev, b, Tb), oc.seqs[b].v[layer], Tb, shape.N, shape.M, f"V seq {b}")


def _decode(gc, layer, qbits, noalloc=False):
    B, Hq, D = qbits.shape
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device="cuda")
    (gc.decode_attn_noalloc if noalloc else gc.decode_attn)(layer, dev(qbits), out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _fill_seqs(gc, oc, shape, lengths, k, v, chunk=None):
    """Per-sequence prefill with append_seq, in chunks (chunk None: one call)."""
    for b, Tb in enumerate(lengths):
        t = 0
        while t < Tb:
            n = Tb - t if chunk is None else min(chunk, Tb - t)
            gc.append_seq(0, b, dev(k[b, t:t + n]), dev(v[b, t:t + n]))
            if oc is not None:
                oc.append_seq(0, b, k[b, t:t + n], v[b, t:t + n])
            t += n


# every case: lengths below N + M, exactly N + M + 1 (one INT2 token), long,
# and a tile or 8-token group boundary crossed at different places
CASES = [
    (Shape(B=5, Hq=4, Hkv=1, D=128, N=8, M=16), [3, 25, 300, 64, 129]),          # 4 query heads per kv head
    (Shape(B=5, Hq=4, Hkv=1, D=128, N=8, M=64), [3, 25, 300, 64, 129]),          # the step's append in the attention launch
    (Shape(B=4, Hq=16, Hkv=2, D=128, N=8, M=70), [49, 700, 5, 200]),             # the same, two head groups
    (Shape(B=4, Hq=16, Hkv=2, D=128, N=8, M=40), [49, 700, 5, 200]),             # 8 query heads per kv head
    (Shape(B=3, Hq=4, Hkv=2, D=128, N=4, M=20), [25, 1, 190]),                   # 2 per kv head: general kernel
    (Shape(B=3, Hq=4, Hkv=2, D=512, N=16, M=40), [57, 400, 9]),                  # head_dim 512
    (Shape(B=3, Hq=4, Hkv=2, D=512, N=16, M=40, v_dtype=1), [57, 300, 20]),      # head_dim 512, V bf16
    (Shape(B=3, Hq=4, Hkv=1, D=128, N=8, M=16, codebook=1), [25, 200, 3]),       # Lloyd-Max codebook
]


@pytest.mark.parametrize("shape,lengths", CASES)
def test_ragged_prefill_then_decode(ok, shape, lengths):
    """Sequences prefilled one by one (append_seq, in chunks and single
    tokens), then one decode attention call over the whole ragged batch."""
    say(f"[ragged decode] {shape} lengths={lengths}")
    rk, rv = make_rotations(shape, "exact")
    T = max(lengths)
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 8)
    oc = ragged_oracle(shape, rk, rv)
    _fill_seqs(gc, oc, shape, lengths, k, v, chunk=97)
    torch.cuda.synchronize()
    assert [gc.seq_length(0, b) for b in range(shape.B)] == lengths
    assert gc.length(0) == T
    compare_ragged_planes(gc, oc, 0, shape, lengths)
    qb = query(shape, mask)
    got = _decode(gc, 0, qb)
    e = oracle_err(got, oc.attend(0, qb))            # exact rotations: the oracle's own cache
    e2 = oracle_err(got, oracle_ragged_on_export(gc, 0, qb, shape, rk, rv, lengths))
    say(f"  rel L2 {e:.3e} (oracle cache), {e2:.3e} (exported cache)")
    # each row equals that sequence decoded alone, in a batch of its own
    for b in (0, shape.B - 1):
        solo = gpu_cache(ok, Shape(**{**shape.__dict__, "B": 1}), rk, rv, T + 8)
        solo.append(0, dev(k[b:b + 1, :lengths[b]]), dev(v[b:b + 1, :lengths[b]]))
        alone = _decode(solo, 0, qb[b:b + 1])
        assert rel_l2(got[b:b + 1], alone) <= 2 ** -12, b
        solo.close()
    gc.close()


@pytest.mark.parametrize("shape,lengths", CASES)
def test_ragged_decode_steps(ok, shape, lengths):
    """Decode steps (append one token to every sequence, attend) over a ragged
    batch, windows sliding at each sequence's own length: stored planes bit-exact
    with the oracle's, attention within the bar, at several steps."""
    steps = 20
    say(f"[ragged steps] {shape} lengths={lengths}")
    rk, rv = make_rotations(shape, "exact")
    T = max(lengths) + steps
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T)
    oc = ragged_oracle(shape, rk, rv)
    _fill_seqs(gc, oc, shape, lengths, k, v)
    cur = list(lengths)
    for i in range(steps):
        kb = np.stack([k[b, cur[b]:cur[b] + 1] for b in range(shape.B)])
        vb = np.stack([v[b, cur[b]:cur[b] + 1] for b in range(shape.B)])
        qb = query(shape, mask, step=i)
        out = torch.zeros((shape.B, shape.Hq, shape.D), dtype=torch.float32, device="cuda")
        gc.decode_step(0, dev(kb), dev(vb), dev(qb), out)
        oc.append(0, kb, vb)
        cur = [c + 1 for c in cur]
        if i in (0, 7, steps - 1):
            torch.cuda.synchronize()
            e = oracle_err(out.cpu().numpy(), oc.attend(0, qb))
            say(f"  step {i}: rel L2 {e:.3e}")
    assert [gc.seq_length(0, b) for b in range(shape.B)] == cur
    compare_ragged_planes(gc, oc, 0, shape, cur)
    gc.close()


@pytest.mark.parametrize("shape,n", [
    (Shape(B=4, Hq=4, Hkv=1, D=128, N=8, M=16), 1),
    (Shape(B=4, Hq=4, Hkv=1, D=128, N=8, M=16), 77),         # matrix-core chunk append, ragged
    (Shape(B=3, Hq=4, Hkv=2, D=512, N=16, M=40), 1),
    (Shape(B=3, Hq=4, Hkv=2, D=512, N=16, M=40), 300),
])
def test_ragged_batch_append(ok, shape, n):
    """oscar_kv_append on a ragged batch: each sequence's n new tokens land at
    its own length (its own tiles, 8-token groups, windows), bit-exact."""
    lengths = [5, 250, 0, 64][:shape.B]
    say(f"[ragged batch append] {shape} n={n} lengths={lengths}")
    rk, rv = make_rotations(shape, "exact")
    T = max(lengths) + n
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T + 1)
    oc = ragged_oracle(shape, rk, rv)
    _fill_seqs(gc, oc, shape, [x for x in lengths], k, v, chunk=61)
    kb = np.stack([k[b, lengths[b]:lengths[b] + n] for b in range(shape.B)])
    vb = np.stack([v[b, lengths[b]:lengths[b] + n] for b in range(shape.B)])
    gc.append(0, dev(kb), dev(vb))
    oc.append(0, kb, vb)
    torch.cuda.synchronize()
    new = [x + n for x in lengths]
    assert [gc.seq_length(0, b) for b in range(shape.B)] == new
    compare_ragged_planes(gc, oc, 0, shape, new)
    qb = query(shape, mask)
    oracle_err(_decode(gc, 0, qb), oc.attend(0, qb))
    gc.close()


@pytest.mark.parametrize("D", [128, 512])
def test_ragged_prefill_attn(ok, D):
    """Prefill attention over a ragged batch: the last n_q positions of each
    sequence attend causally over that sequence's own tokens."""
    shape = Shape(B=3, Hq=8, Hkv=2, D=D, N=16, M=64)
    lengths = [130, 700, 90] if D == 128 else [70, 300, 45]
    n_q = 70 if D == 128 else 40
    rk, rv = make_rotations(shape, "haar")
    k, v, mask = inputs(shape, max(lengths))
    gc = gpu_cache(ok, shape, rk, rv, max(lengths))
    _fill_seqs(gc, None, shape, lengths, k, v, chunk=200)
    q = synth.q_bits(shape.B * n_q, shape.Hq, shape.Hkv, shape.D, 5, 0, mask).reshape(shape.B, n_q, shape.Hq,
                                                                                       shape.D)
    out = torch.zeros((shape.B, n_q, shape.Hq, shape.D), dtype=torch.float32, device="cuda")
    gc.prefill_attn(0, dev(q), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ek, ev = gc.export(0, 0), gc.export(0, 1)
    for b, Tb in enumerate(lengths):
        kp = planes_from_export(_seq_export(ek, b, Tb), Tb, shape.N, shape.M)
        vp = planes_from_export(_seq_export(ev, b, Tb), Tb, shape.N, shape.M)
        want = orc.prefill_attention(q[b:b + 1], kp, vp, rk[0], rv[0], shape.Hkv, shape.N, shape.M, 128, 0, 0)
        e = oracle_err(got[b:b + 1], want)
        say(f"[ragged prefill attn] seq {b} T={Tb}: rel L2 {e:.3e}")
    gc.close()


def test_ragged_reset_and_reuse(ok):
    """A finished sequence's slot is emptied and refilled with a new request
    while the others keep their tokens; then the batch decodes as a fresh
    cache would."""
    shape = Shape(B=3, Hq=4, Hkv=1, D=128, N=8, M=16)
    rk, rv = make_rotations(shape, "exact")
    k, v, mask = inputs(shape, 400)
    gc = gpu_cache(ok, shape, rk, rv, 400)
    oc = ragged_oracle(shape, rk, rv)
    _fill_seqs(gc, oc, shape, [300, 40, 120], k, v)
    gc.reset_seq(1)
    oc.reset_seq(1)
    assert gc.seq_length(0, 1) == 0
    k2, v2, _ = inputs(Shape(**{**shape.__dict__, "seed": 9}), 260)
    gc.append_seq(0, 1, dev(k2[0]), dev(v2[0]))
    oc.append_seq(0, 1, k2[0], v2[0])
    lengths = [300, 260, 120]
    compare_ragged_planes(gc, oc, 0, shape, lengths)
    qb = query(shape, mask)
    e = oracle_err(_decode(gc, 0, qb), oc.attend(0, qb))
    say(f"[ragged reset] rel L2 {e:.3e}")
    gc.close()


def test_ragged_noalloc_equals_decode_attn(ok):
    shape = Shape(B=4, Hq=8, Hkv=2, D=128, N=8, M=16)
    rk, rv = make_rotations(shape, "haar")
    lengths = [700, 30, 1, 250]
    k, v, mask = inputs(shape, max(lengths))
    gc = gpu_cache(ok, shape, rk, rv, max(lengths))
    _fill_seqs(gc, None, shape, lengths, k, v, chunk=128)
    qb = query(shape, mask)
    a = _decode(gc, 0, qb)
    b = _decode(gc, 0, qb, noalloc=True)
    np.testing.assert_array_equal(a, b)
    gc.close()


def test_ragged_rejects(ok):
    """Errors before anything is enqueued: an empty sequence in a decode batch,
    a sequence past max_batch, capacity counted per sequence."""
    shape = Shape(B=3, Hq=4, Hkv=1, D=128, N=8, M=16)
    k, v, mask = inputs(shape, 70)
    gc = gpu_cache(ok, shape, None, None, 64)
    gc.append_seq(0, 0, dev(k[0, :10]), dev(v[0, :10]))
    qb = query(shape, mask)
    with pytest.raises(ok.OscarError):
        _decode(gc, 0, qb)                                   # sequences 1 and 2 are empty
    out = _decode(gc, 0, qb[:1])                             # a batch of the first sequence alone
    assert np.isfinite(out).all()
    with pytest.raises(ok.OscarError):
        gc.append_seq(0, 3, dev(k[0, :1]), dev(v[0, :1]))    # past max_batch
    with pytest.raises(ok.OscarError) as ei:
        gc.append_seq(0, 0, dev(k[0, :60]), dev(v[0, :60]))  # 10 + 60 > 64
    assert ei.value.code == ok.OSCAR_ERR_CAPACITY
    gc.append_seq(0, 1, dev(k[1, :60]), dev(v[1, :60]))      # another sequence still has room
    assert gc.seq_length(0, 1) == 60
    gc.close()


@pytest.mark.slow
def test_ragged_full_size_32k_shape(ok):
    """The 32k workload's shape (32 query heads, 8 kv heads, head_dim 128, sink
    64, recent 256, clip 0.96 / 0.92, 1% outlier channels) with lengths below
    N + M, exactly N + M + 1, mid-range and 32768 in one batch: prefill, a
    few fused decode steps, oracle over the exported cache for every sequence."""
    shape = Shape(B=5, Hq=32, Hkv=8, D=128, N=64, M=256, outliers="percent")
    lengths = [100, 321, 32768, 4999, 1]
    rk, rv = make_rotations(shape, "haar")
    T = max(lengths) + 2
    say(f"[ragged 32k] lengths={lengths}")
    k, v, mask = inputs(shape, T)
    gc = gpu_cache(ok, shape, rk, rv, T)
    _fill_seqs(gc, None, shape, lengths, k, v, chunk=4096)
    cur = list(lengths)
    for i in range(2):
        kb = np.stack([k[b, cur[b]:cur[b] + 1] for b in range(shape.B)])
        vb = np.stack([v[b, cur[b]:cur[b] + 1] for b in range(shape.B)])
        qb = query(shape, mask, step=i)
        out = torch.zeros((shape.B, shape.Hq, shape.D), dtype=torch.float32, device="cuda")
        gc.decode_step(0, dev(kb), dev(vb), dev(qb), out)
        cur = [c + 1 for c in cur]
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle_ragged_on_export(gc, 0, qb, shape, rk, rv, cur)
    e = oracle_err(got, want)
    say(f"  rel L2 {e:.3e}")
    gc.close()
