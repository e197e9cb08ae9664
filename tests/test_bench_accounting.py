"""Host-side accounting of the benchmark, checked on the CPU: the algorithmic
bytes of a decode-attention call, counted position by position from the cache
layout, the causal key count of a prefill chunk, and the one-GPU guard."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle as orc  # noqa: E402


def _bytes_by_position(B, Hkv, D, T, N, M, v_bf16):
    """Every position read once per (sequence, kv head): a window position as
    bf16 K and V (2 D bytes each), any other as its INT2 codes and per-group
    fp16 scale and zero (or bf16 V)."""
    hp = orc.high_precision_mask(T, N, M)
    int2 = orc.compressed_bytes_per_token_head(D, 128)
    per_pos = np.where(hp, 2 * D + 2 * D, int2 + (2 * D if v_bf16 else int2))
    return B * Hkv * int(per_pos.sum())


@pytest.mark.parametrize("B,Hkv,D,T,N,M,vb", [
    (16, 8, 128, 32769, 64, 256, False),      # 32k shape
    (8, 8, 128, 131073, 64, 256, False),      # 128k shape
    (4, 8, 512, 65537, 512, 2048, False),     # wide head
    (4, 8, 512, 65537, 512, 2048, True),      # wide head, bf16 V
    (1, 8, 128, 16385, 512, 2048, False),     # 16k batch 1
    (1, 1, 128, 100, 64, 256, False),         # all window
    (1, 1, 128, 321, 64, 256, False),         # one INT2 position
])
def test_algorithmic_bytes_match_position_count(B, Hkv, D, T, N, M, vb):
    assert bench.algorithmic_kv_bytes(B, Hkv, D, T, N, M, vb) == _bytes_by_position(B, Hkv, D, T, N, M, vb)


def test_headline_bytes_per_call():
    """36 B per INT2 token-head for K or V at head_dim 128, 256 B per bf16 row:
    320.0 MB per call at 32768 tokens (B=16, Hkv=8, sink 64, recent 256)."""
    got = bench.algorithmic_kv_bytes(16, 8, 128, 32768, 64, 256, False)
    assert got == 16 * 8 * ((32768 - 320) * 72 + 320 * 512)
    assert abs(got / 1e6 - 320.0) < 0.05


@pytest.mark.parametrize("T,n", [(16384, 4096), (100, 100), (50, 1), (7, 3)])
def test_prefill_key_count(T, n):
    """The bench's count of the causal keys of a chunk of n queries at the end
    of T positions, against counting them one query at a time."""
    keys = sum(T - n + i + 1 for i in range(n))
    assert bench.prefill_attention_keys(T, n) == keys


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stdout
