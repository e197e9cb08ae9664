"""Plain CPU oracle for OSCAR's serving-time KV path: append (rotate, clip, INT2
quantize, pack), decode attention and chunked-prefill attention over the mixed
INT2 + BF16 cache, and the rotation variants (in-quant Hadamard, absorbed V
rotation).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  It shares no code
with the HIP library: it never imports the product package, and the product
never imports it.

Sources (web pages on OSCAR; cited by page title and section):
  [Qwen3-4B card]  "OSCAR-LLAMACPP-Qwen3-4B-Thinking-2507-INT2-KV" (ModelScope),
                   sections "Files" and "Run" (its env-var table).
  [Gemma card]     "OSCAR-LLAMACPP-Gemma-4-12B-it-INT2-KV", the "Folders" table
                   and the paragraph on the OSCAR rotation below it; "Run".
  [RotationZoo]    "OSCAR-RotationZoo" (ModelScope), sections "Available
                   rotations", "File format", "How to use" (step 2, the sglang
                   launch flags).
  [Article]        "OSCAR: 2-bit KV Cache Quantization for SGLang and llama.cpp",
                   sections "What OSCAR compresses..." and "How the offline
                   rotation is fit from Q/K/V covariance".

Precision: rotation and attention in fp64; the quantizer in IEEE fp32 with
round-to-nearest-even per operation (numpy float32 element-wise ops), fp16
metadata via numpy's RNE float32->float16 conversion.

Readings taken where the pages are silent (each is listed in the design notes):
  * row-vector convention x_rot = x @ R, R given as fp32 [D, D];
  * q is rotated by R_K inside attention, the output is un-rotated by R_V^T;
  * window values are bf16 of the rotated fp32 vector;
  * sink = first N positions, recent = last M positions, INT2 = the rest;
  * clip: hi = r*max, lo = r*min per group; asymmetric 4-level quantizer on
    [lo, hi] with fp16 scale s = (hi - lo)/3 and fp16 zero z = lo; codes use
    the stored fp16 values; ties round to even; s16 == 0 gives all-zero codes;
  * -0.0 is canonicalised to +0.0 before min/max and before the bf16 window;
  * 2-bit codes packed little-endian, 4 per byte, in head_dim order;
  * prefill attention: the queries of the last n cached positions attend
    causally over the cache as it stands (windows of the current length);
  * in-quant Hadamard: fp32(R @ H), H the orthonormal Sylvester Walsh-Hadamard
    matrix of order 128 on each 128-group;
  * Lloyd-Max codebook (the switch of [Article] "Installing OSCAR..." and the
    LM_RATIO of "Where OSCAR loses"): the 4-level quantizer of least mean
    squared error for a Gaussian source, laid on each 128-group's mean and
    standard deviation, the deviation scaled by LM_RATIO (parity unpinned
    against the real kernels, which are not available);
  * ragged batches: each sequence holds its own number of tokens and its
    windows follow its own length; a batch result is the one-sequence result
    of every row.
Parity status of every function is in the function docstring ("pinned by").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

INT2_LEVELS = 4          # 2-bit codes: 0..3  ([RotationZoo] "How to use": --kv-cache-dtype int2)
FP16_MAX = 65504.0

# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32.

    Pinned by: tests compare with torch's bfloat16 -> float32 conversion.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even.

    Finite inputs only (the cache contract excludes NaN/Inf).
    Pinned by: tests compare with torch's float32 -> bfloat16 conversion on
    random and tie-constructed values.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    assert np.all(np.isfinite(x32)), "non-finite value in bf16 rounding"
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def canonical_zero(x32: np.ndarray) -> np.ndarray:
    """Map -0.0 to +0.0 (x + 0.0 under RNE), leave every other value unchanged."""
    return (np.asarray(x32, dtype=np.float32) + np.float32(0.0)).astype(np.float32)


# ----------------------------------------------------------------------------
# rotation  ([Qwen3-4B card] "Files" note: the rotation is an orthogonal,
# post-RoPE, in-graph transform of K and V; [Gemma card] rotation paragraph:
# applied to Q/K and V; [RotationZoo] "File format": one head_dim x head_dim
# matrix per layer)
# ----------------------------------------------------------------------------


def rotate_f64(x_bits: np.ndarray, R32: np.ndarray) -> np.ndarray:
    """x_rot = x @ R in float64, with x given as bf16 bit patterns [..., D].

    The matrix is the fp32 one the GPU receives, widened exactly.
    Pinned by: orthogonal-invariance and permutation-matrix tests.
    """
    x = bf16_bits_to_f64(x_bits)
    R = np.asarray(R32, dtype=np.float32).astype(np.float64)
    return x @ R


def rotated_fp32(x_bits: np.ndarray, R32: np.ndarray) -> np.ndarray:
    """The quantizer input: fp32 RNE of the fp64 rotation, -0 canonicalised."""
    return canonical_zero(rotate_f64(x_bits, R32).astype(np.float32))


# ----------------------------------------------------------------------------
# quantizer  (group of G consecutive head_dim elements: [RotationZoo]
# "Available rotations" note on the group size and "How to use" flags
# --kv-cache-quant-group-size 128; clip ratios K 0.96 / V 0.92: [RotationZoo]
# "How to use" flags; clip applied before quantization: [Qwen3-4B card] "Run"
# env-var table; clipping bounds values before rounding: [Article] "How the
# offline rotation is fit")
# ----------------------------------------------------------------------------


@dataclass
class QuantizedRows:
    codes: np.ndarray   # uint8 [rows, D], values 0..3
    s16: np.ndarray     # float16 [rows, D // G]
    z16: np.ndarray     # float16 [rows, D // G]


def quantize_rows(x32: np.ndarray, group: int, clip: float) -> QuantizedRows:
    """Asymmetric min/max INT2 quantization of fp32 rows, one scale/zero per group.

    Per group, in IEEE fp32 with one rounding per operation:
        mx, mn = max, min of the group (after -0 -> +0)
        hi = r*mx ; lo = r*mn          (r = clip ratio as fp32)
        s  = (hi - lo) / 3
        s16, z16 = fp16(s), fp16(lo)   (stored metadata)
        c  = clamp(rint((x - z) / s), 0, 3) with z, s the stored fp16 values
             (rint = round half to even); c = 0 everywhere if s16 == 0.
    Pinned by: codes in 0..3, nearest-level brute force, clip = 1 extremes,
    [lo, hi] range closure, a hand-worked exact example in tests/golden.
    """
    x32 = canonical_zero(np.asarray(x32, dtype=np.float32))
    rows, D = x32.shape
    assert D % group == 0, "head_dim must be a multiple of the group size"
    assert np.all(np.isfinite(x32)), "non-finite quantizer input is out of contract"
    g = x32.reshape(rows, D // group, group)
    r = np.float32(clip)
    mx = g.max(axis=-1)
    mn = g.min(axis=-1)
    hi = (r * mx).astype(np.float32)
    lo = (r * mn).astype(np.float32)
    s = ((hi - lo).astype(np.float32) / np.float32(3.0)).astype(np.float32)
    assert np.all(np.abs(s) <= FP16_MAX) and np.all(np.abs(lo) <= FP16_MAX), \
        "group range beyond fp16 metadata is out of contract"
    s16 = s.astype(np.float16)
    z16 = lo.astype(np.float16)
    sf = s16.astype(np.float32)[..., None]
    zf = z16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = ((g - zf).astype(np.float32) / sf).astype(np.float32)
        c = np.clip(np.rint(t), 0, INT2_LEVELS - 1)
    c = np.where(sf == 0, 0, c)
    return QuantizedRows(codes=c.reshape(rows, D).astype(np.uint8), s16=s16, z16=z16)


def dequantize_rows(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray, group: int) -> np.ndarray:
    """x_hat = s * c + z per group, exact in float64 (fp16 inputs, c in 0..3)."""
    codes = np.asarray(codes)
    rows, D = codes.shape
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    z = np.asarray(z16, dtype=np.float16).astype(np.float64)
    c = codes.astype(np.float64).reshape(rows, D // group, group)
    return (c * s[..., None] + z[..., None]).reshape(rows, D)


# ----------------------------------------------------------------------------
# Lloyd-Max codebook ([Article] "Installing OSCAR and running a first Qwen3-8B
# calibration": the SGLANG_LLOYD_MAX switch; "Where OSCAR loses, and the cases
# it is the wrong tool for": LM_RATIO = 1.16; "OSCAR against KIVI, QuaRot and
# RotateKV on the same benchmark": OSCAR with Lloyd-Max).  The pages name the
# codebook and the ratio only; the reading here is the classical one: the
# Gaussian Lloyd-Max levels placed on the group's mean, in units of the
# group's standard deviation times the ratio.
# ----------------------------------------------------------------------------

CODEBOOK_UNIFORM = 0
CODEBOOK_LLOYD_MAX = 1

# The 4-level quantizer of least mean squared error for a unit Gaussian source
# (Max's table: levels +-0.4528 and +-1.510, decision thresholds 0 and +-0.9816,
# mean squared error 0.1175), to the four decimals the codebook uses.  The
# thresholds are the midpoints of neighbouring levels.
LLOYD_MAX_LEVELS = (-1.5104, -0.4528, 0.4528, 1.5104)
LLOYD_MAX_THRESHOLD = 0.9816


def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x):
    return 0.5 * (1.0 + np.vectorize(math.erf)(np.asarray(x, np.float64) / math.sqrt(2.0)))


def lloyd_max_gaussian(levels: int = 4, iters: int = 500):
    """Lloyd's iteration for the `levels`-level quantizer of a unit Gaussian in
    float64: thresholds = midpoints of neighbouring levels, each level = the
    mean of the Gaussian over its cell, E[X | a < X < b] = (phi(a) - phi(b)) /
    (Phi(b) - Phi(a)).  Returns (levels, thresholds, mean squared error).
    Pinned by: Max's published 4-level values, symmetry, and a local minimum
    of the error against perturbed levels."""
    y = np.linspace(-1.5, 1.5, levels)
    for _ in range(iters):
        t = 0.5 * (y[1:] + y[:-1])
        a = np.concatenate([[-np.inf], t])
        b = np.concatenate([t, [np.inf]])
        pa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
        pb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
        y = (pa - pb) / (_Phi(b) - _Phi(a))
    t = 0.5 * (y[1:] + y[:-1])
    return y, t, gaussian_quantizer_mse(y, t)


def gaussian_quantizer_mse(y, t) -> float:
    """E[(X - q(X))^2] for a unit Gaussian X, q mapping cell (t_{k-1}, t_k) to
    y_k, in closed form: E[X^2 1_cell] - 2 y E[X 1_cell] + y^2 P(cell)."""
    y = np.asarray(y, np.float64)
    a = np.concatenate([[-np.inf], np.asarray(t, np.float64)])
    b = np.concatenate([np.asarray(t, np.float64), [np.inf]])
    fa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
    fb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
    P = _Phi(b) - _Phi(a)
    m1 = fa - fb                                   # E[X 1_cell]
    az = np.where(np.isinf(a), 0.0, a)
    bz = np.where(np.isinf(b), 0.0, b)
    m2 = P + az * fa - bz * fb                     # E[X^2 1_cell]
    return float(np.sum(m2 - 2.0 * y * m1 + y * y * P))


def tree_sum_f32(a: np.ndarray) -> np.ndarray:
    """Sum over the last axis (a power of two) in float32, pairwise in a fixed
    order: first element i with element i + n/2, then the halves again, down
    to one value (one rounding per add)."""
    a = np.asarray(a, np.float32)
    while a.shape[-1] > 1:
        h = a.shape[-1] // 2
        a = (a[..., :h] + a[..., h:]).astype(np.float32)
    return a[..., 0]


def quantize_rows_lloyd_max(x32: np.ndarray, group: int, ratio: float) -> QuantizedRows:
    """Lloyd-Max INT2 quantization of fp32 rows, per group of G values, in IEEE
    fp32 with one rounding per operation:
        mu  = tree_sum(x) * (1/G)                 (G a power of two: exact scaling)
        var = tree_sum((x - mu) * (x - mu)) * (1/G)
        sd  = sqrt(var)                           (correctly rounded)
        s   = r * sd, r = LM_RATIO as fp32;  s16, z16 = fp16(s), fp16(mu)
        u   = (x - z) / s with z, s the stored fp16 values
        c   = [u >= -tau] + [u >= 0] + [u >= tau], tau = fp32(0.9816)
              (the nearest of the levels z + s l_k, l = LLOYD_MAX_LEVELS, ties
              to the higher level); c = 0 everywhere if s16 == 0.
    Pinned by: nearest-level brute force, the statistics against float64
    mean and deviation, a hand-worked example in tests/golden, and the
    levels against Lloyd's iteration.
    """
    x32 = canonical_zero(np.asarray(x32, dtype=np.float32))
    rows, D = x32.shape
    assert D % group == 0 and group & (group - 1) == 0
    assert np.all(np.isfinite(x32)), "non-finite quantizer input is out of contract"
    g = x32.reshape(rows, D // group, group)
    inv_g = np.float32(1.0 / group)
    mu = (tree_sum_f32(g) * inv_g).astype(np.float32)
    d = (g - mu[..., None]).astype(np.float32)
    var = (tree_sum_f32((d * d).astype(np.float32)) * inv_g).astype(np.float32)
    sd = np.sqrt(var).astype(np.float32)
    s = (np.float32(ratio) * sd).astype(np.float32)
    assert np.all(np.abs(s) <= FP16_MAX) and np.all(np.abs(mu) <= FP16_MAX), \
        "group statistics beyond fp16 metadata are out of contract"
    s16 = s.astype(np.float16)
    z16 = mu.astype(np.float16)
    sf = s16.astype(np.float32)[..., None]
    zf = z16.astype(np.float32)[..., None]
    tau = np.float32(LLOYD_MAX_THRESHOLD)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = ((g - zf).astype(np.float32) / sf).astype(np.float32)
        c = (u >= -tau).astype(np.uint8) + (u >= 0).astype(np.uint8) + (u >= tau).astype(np.uint8)
    c = np.where(sf == 0, 0, c)
    return QuantizedRows(codes=c.reshape(rows, D).astype(np.uint8), s16=s16, z16=z16)


def dequantize_rows_lloyd_max(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray, group: int) -> np.ndarray:
    """x_hat = z + s * l_c per group in float64, l_c the level of code c (the
    fp32 value of LLOYD_MAX_LEVELS[c], widened)."""
    codes = np.asarray(codes)
    rows, D = codes.shape
    lv = np.asarray(LLOYD_MAX_LEVELS, np.float32).astype(np.float64)
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    z = np.asarray(z16, dtype=np.float16).astype(np.float64)
    ell = lv[codes.astype(np.int64)].reshape(rows, D // group, group)
    return (ell * s[..., None] + z[..., None]).reshape(rows, D)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """4 codes per byte, little-endian 2-bit fields: code j -> byte j//4, bits 2*(j%4).

    Pinned by: hand examples in tests/golden and unpack(pack(c)) == c.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    *lead, D = codes.shape
    assert D % 4 == 0
    c = codes.reshape(*lead, D // 4, 4).astype(np.uint8)
    out = c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_codes: [..., D/4] bytes -> [..., D] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    parts = [(p >> np.uint8(2 * i)) & np.uint8(3) for i in range(4)]
    return np.stack(parts, axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 4)


# ----------------------------------------------------------------------------
# windows  ([Qwen3-4B card] "Run" table: the first and last tokens kept in
# high precision, 512 / 2048; [RotationZoo] "How to use" flags: prefix 64,
# recent 256; [Article] "What OSCAR compresses": BF16 sink + recent window)
# ----------------------------------------------------------------------------


def high_precision_mask(T: int, N: int, M: int) -> np.ndarray:
    """Boolean [T]: True for sink positions [0, min(N,T)) and recent positions
    [max(N, T-M), T); False for the INT2 positions [N, T-M).
    Pinned by: boundary cases T = N+M, N+M+1, N = 0, M = 0 and the brute-force
    attention loop.
    """
    t = np.arange(T)
    return (t < N) | (t >= max(N, T - M))


def ring_slot(t: int, M: int) -> int:
    """Recent-window storage slot of position t in a ring of M slots (layout reading)."""
    return t % M


# ----------------------------------------------------------------------------
# the cache, kept in logical per-token form
# ----------------------------------------------------------------------------

KV_INT2 = 0
KV_BF16 = 1


@dataclass
class OracleLayerPlanes:
    """Logical per-token planes of one of K or V for one layer, all sequences.

    x32:  float32 [B, Hkv, T, D] rotated quantizer input
    win:  uint16  [B, Hkv, T, D] bf16 bits of x32 (the high-precision value)
    codes:uint8   [B, Hkv, T, D] 2-bit codes (INT2 dtype only)
    s16, z16: float16 [B, Hkv, T, D/G]
    """
    x32: np.ndarray
    win: np.ndarray
    codes: np.ndarray | None
    s16: np.ndarray | None
    z16: np.ndarray | None
    codebook: int = CODEBOOK_UNIFORM     # how codes map to values


@dataclass
class OracleConfig:
    num_layers: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    sink_tokens: int
    recent_tokens: int
    group_size: int = 128
    k_clip: float = 0.96
    v_clip: float = 0.92
    k_dtype: int = KV_INT2
    v_dtype: int = KV_INT2
    codebook: int = CODEBOOK_UNIFORM
    lm_ratio: float = 1.16


def append_planes(x_bits: np.ndarray, R32: np.ndarray, group: int, clip: float,
                  dtype: int, codebook: int = CODEBOOK_UNIFORM, lm_ratio: float = 1.16) -> OracleLayerPlanes:
    """Append step for a block of new tokens, bf16 bits [B, n, Hkv, D]:
    rotate (fp64), round to fp32 (quantizer input), bf16 window value, and,
    for INT2, codes + fp16 scale/zero per group (min/max quantizer with the
    clip ratio, or the Lloyd-Max codebook with LM_RATIO).  Returned in
    [B, Hkv, n, ...].
    """
    x32 = rotated_fp32(x_bits, R32)                      # [B, n, Hkv, D]
    x32 = np.ascontiguousarray(np.transpose(x32, (0, 2, 1, 3)))
    B, H, n, D = x32.shape
    win = f32_to_bf16_bits(x32)
    if dtype == KV_BF16:
        return OracleLayerPlanes(x32, win, None, None, None)
    if codebook == CODEBOOK_LLOYD_MAX:
        q = quantize_rows_lloyd_max(x32.reshape(-1, D), group, lm_ratio)
    else:
        q = quantize_rows(x32.reshape(-1, D), group, clip)
    return OracleLayerPlanes(
        x32, win,
        q.codes.reshape(B, H, n, D),
        q.s16.reshape(B, H, n, D // group),
        q.z16.reshape(B, H, n, D // group), codebook)


def _cat(a, b, axis=2):
    if a is None:
        return b
    return np.concatenate([a, b], axis=axis)


class OracleKVCache:
    """Reference cache: every appended token is kept with its fp32 rotated value,
    bf16 window value and INT2 codes/metadata; attention selects the precision
    per token from the window rule at call time."""

    def __init__(self, cfg: OracleConfig, rot_k: np.ndarray | None, rot_v: np.ndarray | None):
        self.cfg = cfg
        D = cfg.head_dim
        eye = np.eye(D, dtype=np.float32)
        self.rot_k = [np.asarray(rot_k[l], np.float32) if rot_k is not None else eye
                      for l in range(cfg.num_layers)]
        self.rot_v = [np.asarray(rot_v[l], np.float32) if rot_v is not None else eye
                      for l in range(cfg.num_layers)]
        self.k: list[OracleLayerPlanes | None] = [None] * cfg.num_layers
        self.v: list[OracleLayerPlanes | None] = [None] * cfg.num_layers

    def length(self, layer: int) -> int:
        p = self.k[layer]
        return 0 if p is None else p.x32.shape[2]

    def append(self, layer: int, k_bits: np.ndarray, v_bits: np.ndarray) -> None:
        c = self.cfg
        nk = append_planes(k_bits, self.rot_k[layer], c.group_size, c.k_clip, c.k_dtype, c.codebook, c.lm_ratio)
        nv = append_planes(v_bits, self.rot_v[layer], c.group_size, c.v_clip, c.v_dtype, c.codebook, c.lm_ratio)
        self.k[layer] = nk if self.k[layer] is None else _join(self.k[layer], nk)
        self.v[layer] = nv if self.v[layer] is None else _join(self.v[layer], nv)

    def attend(self, layer: int, q_bits: np.ndarray, scale: float | None = None) -> np.ndarray:
        c = self.cfg
        return decode_attention(q_bits, self.k[layer], self.v[layer], self.rot_k[layer],
                                self.rot_v[layer], c.num_kv_heads, c.sink_tokens,
                                c.recent_tokens, c.group_size, c.k_dtype, c.v_dtype, scale)


class OracleRaggedCache:
    """A batch whose sequences hold different numbers of tokens (serving: each
    request at its own length, "OSCAR-RotationZoo", "How to use" step 2, the
    sglang server).  Each sequence is its own one-sequence cache: appends
    address one sequence or every sequence of a batch, each at its own length,
    and attention of sequence b reads its own T_b tokens with its own sink and
    recent windows.  The result for a batch is, row by row, the one-sequence
    result (there is no cross-sequence term in the method).
    Pinned by: equal lengths give the batched cache's result bit for bit;
    brute-force loops per sequence at lengths below, at and above N + M; a
    code change in one sequence's only INT2 token moves that sequence alone."""

    def __init__(self, cfg: OracleConfig, rot_k: np.ndarray | None, rot_v: np.ndarray | None):
        self.cfg = cfg
        one = OracleConfig(**{**cfg.__dict__, "batch": 1})
        self.seqs = [OracleKVCache(one, rot_k, rot_v) for _ in range(cfg.batch)]

    def length(self, layer: int, seq: int) -> int:
        return self.seqs[seq].length(layer)

    def append_seq(self, layer: int, seq: int, k_bits: np.ndarray, v_bits: np.ndarray) -> None:
        """k_bits, v_bits: [n_new, Hkv, D] of sequence seq."""
        self.seqs[seq].append(layer, k_bits[None], v_bits[None])

    def append(self, layer: int, k_bits: np.ndarray, v_bits: np.ndarray) -> None:
        """k_bits, v_bits: [batch, n_new, Hkv, D], sequence b at its own length."""
        for b in range(k_bits.shape[0]):
            self.append_seq(layer, b, k_bits[b], v_bits[b])

    def reset_seq(self, seq: int) -> None:
        c = self.seqs[seq]
        c.k = [None] * len(c.k)
        c.v = [None] * len(c.v)

    def attend(self, layer: int, q_bits: np.ndarray, scale: float | None = None) -> np.ndarray:
        """q_bits [batch, Hq, D] -> [batch, Hq, D]; every sequence of the batch
        must hold at least one token."""
        return np.concatenate([self.seqs[b].attend(layer, q_bits[b:b + 1], scale)
                               for b in range(q_bits.shape[0])])


def _join(a: OracleLayerPlanes, b: OracleLayerPlanes) -> OracleLayerPlanes:
    return OracleLayerPlanes(_cat(a.x32, b.x32), _cat(a.win, b.win), _cat(a.codes, b.codes),
                             _cat(a.s16, b.s16), _cat(a.z16, b.z16), a.codebook)


# ----------------------------------------------------------------------------
# attention  ([Qwen3-4B card] "Run" table: fused INT2 + f16 flash attention;
# [Article] "How the offline rotation is fit": attention reads the mixed layout
# directly; V rotation undone on the output: [RotationZoo] "How to use" flag
# that absorbs the V rotation into the output projection)
# ----------------------------------------------------------------------------


def mixed_values(planes: OracleLayerPlanes, b: int, h: int, T: int, N: int, M: int,
                 group: int, dtype: int) -> np.ndarray:
    """float64 [T, D] values attention reads for one (sequence, kv head):
    bf16 window value on sink/recent positions (and everywhere for BF16 dtype),
    s*c + z elsewhere."""
    win = bf16_bits_to_f64(planes.win[b, h, :T])
    if dtype == KV_BF16:
        return win
    hp = high_precision_mask(T, N, M)
    deq_fn = dequantize_rows_lloyd_max if planes.codebook == CODEBOOK_LLOYD_MAX else dequantize_rows
    deq = deq_fn(planes.codes[b, h, :T], planes.s16[b, h, :T], planes.z16[b, h, :T], group)
    return np.where(hp[:, None], win, deq)


def softmax_attention_f64(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Exact softmax attention for one query row q [D] over K, V [T, D] (float64)."""
    s = (K @ q) * scale
    s = s - s.max()
    p = np.exp(s)
    p /= p.sum()
    return p @ V


def decode_attention(q_bits: np.ndarray, kp: OracleLayerPlanes, vp: OracleLayerPlanes,
                     rot_k: np.ndarray, rot_v: np.ndarray, num_kv_heads: int, N: int, M: int,
                     group: int, k_dtype: int, v_dtype: int,
                     scale: float | None = None, absorb_v: bool = False) -> np.ndarray:
    """One decode step for every sequence: q bf16 bits [B, Hq, D] (post-RoPE,
    un-rotated) -> output float64 [B, Hq, D] (un-rotated).

        q_rot = q @ R_K                      (fp64)
        o'_j  = softmax(scale * K_hat q_rot_j) V_hat   over all T cached tokens,
                with query head j reading kv head j // (Hq/Hkv)
        o_j   = o'_j @ R_V^T
    absorb_v: return o' itself, the output still in the V-rotated basis, for a
    caller that folds R_V^T into its output projection (RotationZoo "How to
    use", the sglang flag that absorbs the V rotation).
    Pinned by: all-window equality with a library attention routine, rotation
    invariance with quantization off, GQA == replicated MHA, brute-force loops.
    """
    B, Hq, D = q_bits.shape
    Gq = Hq // num_kv_heads
    assert Gq * num_kv_heads == Hq
    T = kp.x32.shape[2]
    assert T > 0, "attention over an empty cache is undefined"
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    qr = rotate_f64(q_bits, rot_k)                       # [B, Hq, D]
    Rv = np.asarray(rot_v, np.float32).astype(np.float64)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for h in range(num_kv_heads):
            Kh = mixed_values(kp, b, h, T, N, M, group, k_dtype)
            Vh = mixed_values(vp, b, h, T, N, M, group, v_dtype)
            for j in range(h * Gq, (h + 1) * Gq):
                out[b, j] = softmax_attention_f64(qr[b, j], Kh, Vh, scale)
    return out if absorb_v else out @ Rv.T


def prefill_attention(q_bits: np.ndarray, kp: OracleLayerPlanes, vp: OracleLayerPlanes,
                      rot_k: np.ndarray, rot_v: np.ndarray, num_kv_heads: int, N: int, M: int,
                      group: int, k_dtype: int, v_dtype: int,
                      scale: float | None = None, absorb_v: bool = False,
                      query_ids=None) -> np.ndarray:
    """Chunked-prefill attention over the mixed cache ([RotationZoo] "How to
    use": the serving host runs a separate prefill backend beside the decode
    one).  q bf16 bits [B, n, Hq, D] are the queries of the last n cached
    positions T - n .. T - 1 (post-RoPE, un-rotated).  Query i, at position
    p = T - n + i, attends causally over positions [0, p] of the cache as it
    stands after the chunk was appended: the sink and recent windows of the
    current length T read their bf16 values, every other position its INT2
    dequantization.  Each query is the decode step's arithmetic over its
    causal prefix:

        q_rot = q @ R_K                      (fp64)
        o'    = softmax(scale * K_hat[:p+1] q_rot) V_hat[:p+1]
        o     = o' @ R_V^T                   (o' itself with absorb_v)

    Returns float64 [B, n, Hq, D], or [B, len(query_ids), Hq, D] for the listed
    query indices only (the same arithmetic for each listed query).
    Pinned by: n = 1 equal to decode_attention, an all-window cache with
    R = I equal to a library attention routine under an explicit causal mask,
    and brute-force loops on tiny shapes.
    """
    B, n, Hq, D = q_bits.shape
    Gq = Hq // num_kv_heads
    assert Gq * num_kv_heads == Hq
    T = kp.x32.shape[2]
    assert 0 < n <= T, "the queries are the last n of the T cached positions"
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    ids = list(range(n)) if query_ids is None else [int(i) for i in query_ids]
    assert all(0 <= i < n for i in ids)
    qr = rotate_f64(q_bits[:, ids], rot_k)               # [B, len(ids), Hq, D]
    Rv = np.asarray(rot_v, np.float32).astype(np.float64)
    out = np.zeros((B, len(ids), Hq, D), dtype=np.float64)
    for b in range(B):
        for h in range(num_kv_heads):
            Kh = mixed_values(kp, b, h, T, N, M, group, k_dtype)
            Vh = mixed_values(vp, b, h, T, N, M, group, v_dtype)
            for r, i in enumerate(ids):
                p = T - n + i
                for j in range(h * Gq, (h + 1) * Gq):
                    out[b, r, j] = softmax_attention_f64(qr[b, r, j], Kh[:p + 1], Vh[:p + 1], scale)
    return out if absorb_v else out @ Rv.T


# ----------------------------------------------------------------------------
# importing a cache held in storage layout (sink array + recent ring)
# ----------------------------------------------------------------------------


def planes_from_storage(packed_codes: np.ndarray | None, meta_s16: np.ndarray | None,
                        meta_z16: np.ndarray | None, sink_bits: np.ndarray,
                        ring_bits: np.ndarray, T: int, N: int, M: int,
                        full_bits: np.ndarray | None = None,
                        codebook: int = CODEBOOK_UNIFORM) -> OracleLayerPlanes:
    """Build logical planes from a cache held as: packed codes [B, H, T, D/4],
    fp16 scale/zero [B, H, T, D/G], sink bf16 [B, H, N, D], recent ring bf16
    [B, H, M, D] (position t in slot t % M); or, for a BF16 plane, full bf16
    values [B, H, T, D].  Window values of INT2 positions are left zero (never
    read); x32 is not known and is left zero."""
    if full_bits is not None:
        B, H, _, D = full_bits.shape
        win = np.ascontiguousarray(full_bits[:, :, :T]).astype(np.uint16)
        return OracleLayerPlanes(np.zeros(win.shape, np.float32), win, None, None, None)
    codes = unpack_codes(packed_codes[:, :, :T])
    B, H, _, D = codes.shape
    win = np.zeros((B, H, T, D), dtype=np.uint16)
    for t in range(min(N, T)):
        win[:, :, t] = sink_bits[:, :, t]
    if M > 0:
        for t in range(max(N, T - M), T):
            win[:, :, t] = ring_bits[:, :, ring_slot(t, M)]
    return OracleLayerPlanes(np.zeros((B, H, T, D), np.float32), win, codes,
                             np.asarray(meta_s16[:, :, :T], np.float16),
                             np.asarray(meta_z16[:, :, :T], np.float16), codebook)


# ----------------------------------------------------------------------------
# exact rotations used as bit-exact special cases
# ----------------------------------------------------------------------------


def bit_reversal_permutation(D: int) -> np.ndarray:
    """The bit-reversal permutation matrix on log2(D) bits ([RotationZoo] "File
    format": the K rotation ends with a bit-reversal permutation).  P[e, rev(e)] = 1
    so x @ P moves element e to position rev(e)."""
    nbits = int(round(math.log2(D)))
    assert 1 << nbits == D
    P = np.zeros((D, D), dtype=np.float32)
    for e in range(D):
        r = int(format(e, f"0{nbits}b")[::-1], 2)
        P[e, r] = 1.0
    return P


def block_hadamard(D: int, order: int = 128) -> np.ndarray:
    """The orthonormal Walsh-Hadamard matrix of the given order in Sylvester's
    construction, entry (i, j) = (-1)^popcount(i & j) / sqrt(order), placed
    D / order times along the diagonal (float64 [D, D]).

    The in-quant Hadamard: the llama.cpp fork's quantizer applies a Hadamard
    transform unless the rotation already sits in the graph ([Qwen3-4B card]
    "Run", env-var table), the sglang launch sets its order to 128
    ([RotationZoo] "How to use", step 2), and the shipped rotations themselves
    contain a head-dim Hadamard factor ([RotationZoo] "File format").
    Pinned by: equality with scipy's Sylvester Hadamard, orthogonality, the
    two-block recursion and the transform of a unit vector.
    """
    assert order > 0 and order & (order - 1) == 0 and D % order == 0
    i = np.arange(order)
    bits = np.bitwise_and.outer(i, i)
    pop = np.zeros_like(bits)
    while bits.any():
        pop += bits & 1
        bits >>= 1
    H = np.where(pop % 2 == 0, 1.0, -1.0) / math.sqrt(order)
    return np.kron(np.eye(D // order), H)


def with_in_quant_hadamard(R32: np.ndarray, order: int = 128) -> np.ndarray:
    """Rotations followed by the in-quant Hadamard: fp32(R @ H) per layer, the
    product taken in fp64 and rounded once (R32: fp32 [..., D, D]).  The
    quantizer input becomes fp32(x @ R @ H) up to that one rounding of the
    matrix, q is rotated by the same product and the output un-rotated by its
    transpose, so every other step is unchanged.
    Pinned by: the identity rotation giving the Hadamard itself, orthogonality
    of the product, and equality of the product applied to a vector with the
    rotation followed by an explicit fast Walsh-Hadamard transform.
    """
    R = np.asarray(R32, np.float32).astype(np.float64)
    H = block_hadamard(R.shape[-1], order)
    return (R @ H).astype(np.float32)


def compressed_bytes_per_token_head(D: int, group: int) -> int:
    """INT2 storage per token and head for one of K or V: D/4 code bytes plus an
    fp16 scale and an fp16 zero per group."""
    return D // 4 + 4 * (D // group)
