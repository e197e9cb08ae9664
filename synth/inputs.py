"""Seeded synthetic Q/K/V and rotations shaped like the pages' serving setups.

Recipe (also stated in the design notes):
  * seeds: numpy.random.default_rng([seed0, layer, role, *extra]);
  * values: N(0, 1) per element, with outlier channels multiplied by 8 (or
    another factor where a test sweeps the value range); the
    outlier channels are drawn per layer (and per kv head in the "percent"
    mode) and shared by Q (through q head -> kv head), K and V;  heavy-tailed
    variant: Student-t with 3 degrees of freedom, unscaled;
  * bf16 inputs are the float32 draws rounded by torch's bfloat16 conversion;
  * rotations: QR of a seeded float64 Gaussian D x D matrix, signs fixed so
    the triangular factor has a positive diagonal (Haar measure), stored fp32.
Large device-side fills use torch generators seeded from the same tuple.
"""
from __future__ import annotations

import numpy as np

ROLE = {"q": 0, "k": 1, "v": 2, "rot_k": 3, "rot_v": 4, "step": 5, "outlier": 6}


def rng(seed0: int, layer: int, role: str, *extra: int) -> np.random.Generator:
    return np.random.default_rng([int(seed0), int(layer), ROLE[role], *[int(e) for e in extra]])


def haar_rotation(D: int, seed0: int, layer: int, role: str) -> np.ndarray:
    g = rng(seed0, layer, role).standard_normal((D, D))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


def rotations(num_layers: int, D: int, seed0: int, role: str) -> np.ndarray:
    return np.stack([haar_rotation(D, seed0, l, role) for l in range(num_layers)])


def outlier_mask(D: int, num_kv_heads: int, seed0: int, layer: int, mode: str,
                 count: int = 4) -> np.ndarray:
    """bool [Hkv, D].  mode 'fixed': `count` channels per layer shared by all kv
    heads; 'percent': max(1, round(0.01 D)) channels per kv head; 'none'."""
    m = np.zeros((num_kv_heads, D), dtype=bool)
    g = rng(seed0, layer, "outlier")
    if mode == "fixed":
        m[:, g.choice(D, size=count, replace=False)] = True
    elif mode == "percent":
        n = max(1, int(round(0.01 * D)))
        for h in range(num_kv_heads):
            m[h, g.choice(D, size=n, replace=False)] = True
    elif mode != "none":
        raise ValueError(mode)
    return m


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns (uint16) using torch's float32 -> bfloat16 conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw(shape, seed0: int, layer: int, role: str, dist: str = "normal", *extra: int) -> np.ndarray:
    g = rng(seed0, layer, role, *extra)
    if dist == "normal":
        return g.standard_normal(shape)
    if dist == "student_t3":
        return g.standard_t(3, size=shape)
    raise ValueError(dist)


def kv_bits(batch: int, n: int, num_kv_heads: int, D: int, seed0: int, layer: int, role: str,
            mask: np.ndarray, dist: str = "normal", chunk: int = 0, outlier_scale: float = 8.0) -> np.ndarray:
    """bf16 bits [batch, n, Hkv, D] for K (role 'k') or V (role 'v')."""
    x = draw((batch, n, num_kv_heads, D), seed0, layer, role, dist, chunk)
    x = np.where(mask[None, None], x * outlier_scale, x)
    return to_bf16_bits(x)


def q_bits(batch: int, num_q_heads: int, num_kv_heads: int, D: int, seed0: int, layer: int,
           mask: np.ndarray, dist: str = "normal", step: int = 0, outlier_scale: float = 8.0) -> np.ndarray:
    """bf16 bits [batch, Hq, D]; query head j shares kv head j // (Hq/Hkv)'s outliers."""
    x = draw((batch, num_q_heads, D), seed0, layer, "q", dist, step)
    gq = num_q_heads // num_kv_heads
    qmask = np.repeat(mask, gq, axis=0)
    x = np.where(qmask[None], x * outlier_scale, x)
    return to_bf16_bits(x)


def bits_to_torch_bf16(bits: np.ndarray, device=None):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor (optionally on a device)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t


def device_kv_fill(shape, seed: int, device, mask_t, dist: str = "normal"):
    """Device-side bf16 draw for large cache fills: shape [B, n, Hkv, D];
    mask_t bool [Hkv, D] on the device marks outlier channels (x8)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    if dist == "normal":
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    elif dist == "student_t3":
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        c = torch.randn((3,) + tuple(shape), generator=g, device=device, dtype=torch.float32)
        x = z / torch.sqrt((c * c).sum(0) / 3.0)
    else:
        raise ValueError(dist)
    x = torch.where(mask_t[None, None], x * 8.0, x)
    return x.to(torch.bfloat16)


def seed_of(seed0: int, layer: int, role: str, *extra: int) -> int:
    """A 63-bit integer seed derived from the same tuple as `rng`."""
    return int(rng(seed0, layer, role, *extra).integers(0, 2**63 - 1))
