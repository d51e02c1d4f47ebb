"""The benchmark's contract and its algorithmic work counts (CPU only).

The roofline fractions bench.py reports divide these counts by measured time, so they are pinned
here against closed forms for the workload shapes and against a brute-force count over an
explicit causal/window mask.
"""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _shape(seqlens, qlens, window, hq, hkv, d, q_dtype="e4m3"):
    return SimpleNamespace(seqlens_k_host=list(seqlens), q_lens_host=list(qlens), window=window,
                           num_q_heads=hq, num_kv_heads=hkv, head_dim=d, q_dtype=q_dtype,
                           total_q=int(sum(qlens)))


def _brute_pairs(seqlens, qlens, window):
    """Visible (query, key) pairs per q head from an explicit mask: query i of a sequence of
    length L with q_len new tokens sits at L - q_len + i and sees keys j <= p, j > p - window."""
    total = 0
    for L, ql in zip(seqlens, qlens):
        p = np.arange(L - ql, L)[:, None]
        j = np.arange(L)[None, :]
        vis = j <= p
        if window >= 1:
            vis &= j > p - window
        total += int(vis.sum())
    return total


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("seqlens,qlens,window", [
    ([128], [16], -1),
    ([300, 37, 513], [300, 20, 257], 100),
    ([1, 65, 64], [1, 3, 64], 1),
    ([700, 2048], [4, 2048], 1024),
])
def test_visible_pairs_match_brute_force(seqlens, qlens, window):
    w = _shape(seqlens, qlens, window, 4, 2, 64)
    assert bench.visible_pairs(w) == _brute_pairs(seqlens, qlens, window)


def test_sliding_window_prefill_flops_closed_form():
    # 8 sequences of 8192 new tokens, window 1024: per (sequence, q head) the first 1024 rows
    # see 1..1024 keys (524,800 pairs) and the other 7,168 rows 1,024 each
    w = _shape([8192] * 8, [8192] * 8, 1024, 32, 16, 256)
    per_seq = 1024 * 1025 // 2 + 7168 * 1024
    assert per_seq == 523776 + 7169 * 1024
    assert bench.visible_pairs(w) == 8 * per_seq
    assert bench.algo_flops(w) == 4.0 * 256 * 8 * per_seq * 32      # 2.0616 TFLOP
    assert abs(bench.algo_flops(w) / 1e12 - 2.0616) < 1e-3


def test_sliding_window_decode_bytes_closed_form():
    # every length is at least the window, so each sequence reads 1,024 keys per kv head
    rng = np.random.default_rng(2)
    seqlens = rng.integers(1024, 8193, size=32)
    w = _shape(seqlens, [1] * 32, 1024, 32, 16, 256)
    total, kv = bench.algo_bytes(w, fused=True)
    assert kv == 32 * 1024 * 16 * 256 * 2
    assert total == kv + 32 * 32 * 256 * 2 + 32 * 32 * 256 * 2 == 269_484_032
    # E4M3 codes quantized by a separate call: Q is read as 1-byte codes
    total_codes, _ = bench.algo_bytes(w, fused=False)
    assert total_codes == kv + 32 * 32 * 256 + 32 * 32 * 256 * 2 == 269_221_888


def test_full_attention_bytes_scale_with_lengths():
    # causal, no window: every key of every sequence is read once per kv head
    seqlens = [8192, 20000, 32768]
    w = _shape(seqlens, [1, 1, 1], -1, 32, 4, 512, q_dtype="bf16")
    _, kv = bench.algo_bytes(w)
    assert kv == sum(seqlens) * 4 * 512 * 2


def test_unique_kv_bytes_spec_verify_closed_form():
    """The cache-aware bound of the spec-verify workload reads each distinct page once: 400 prefix
    pages shared by all 64 sequences plus 48 unique pages each = 3,472 pages of 64 tokens x 4 kv
    heads x 512 bytes, K and V: 910,163,968 bytes."""
    import torch
    B, prefix, own = 64, 400, 48
    table = np.zeros((B, prefix + own), dtype=np.int64)
    nxt = prefix
    for b in range(B):
        table[b, :prefix] = np.arange(prefix)
        table[b, prefix:] = np.arange(nxt, nxt + own)
        nxt += own
    w = _shape([(prefix + own) * 64] * B, [4] * B, -1, 32, 4, 512, "bf16")
    w.k_pool = SimpleNamespace(shape=(nxt, 64, 4, 512))
    w.block_table = torch.from_numpy(table)
    assert bench.unique_kv_bytes(w) == 3472 * 64 * 4 * 512 * 2 == 910_163_968
    # with a window, only the pages of the visible keys count
    w2 = _shape([1000], [1], 100, 2, 1, 64)
    w2.k_pool = SimpleNamespace(shape=(16, 64, 1, 64))
    w2.block_table = torch.arange(16).reshape(1, 16)
    # keys 900..999 sit in pages 14 and 15
    assert bench.unique_kv_bytes(w2) == 2 * 64 * 64 * 2
