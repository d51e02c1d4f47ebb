"""GPU parity of the decode over 32-row query tiles at head dim 512 (the verify kernel: each K/V tile
loaded once for 32 rows; per-tile softmax references brought to a common one by the FP8 MFMA's E8M0
operand scales with split Q, by exact power-of-two scaling of P with BF16 Q), through the C-ABI,
against the fp64 CPU oracle on every row, in both modes, and the two modes against each other:

* GQA 8 x 4 tokens (32 rows, the speculative-decode verify shape), with and without splits;
* partial tiles (24 and 20 rows), two row tiles (48 rows), GQA 6, 128-token blocks;
* sliding windows, sequences shorter than one 32-key tile and lengths off the tile grid;
* K/V descales per (sequence, kv head); pool slots past a sequence's end holding NaN codes.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from helpers import compare, gpu_run, log, oracle_run, with_nan_tails, with_page_size
from test_gpu_coverage import _per_bh_descales

pytestmark = pytest.mark.gpu

VERIFY_CASES = {
    # name: (hq, hkv, window, seqlens, qlens, page, splits)
    "g8x4": (32, 4, -1, [2000, 700, 333, 1024], [4, 4, 4, 4], 64, 0),
    "g8x4_3_splits": (32, 4, -1, [2000, 700, 333, 1024], [4, 4, 4, 4], 64, 3),
    "g8x3_page128": (32, 4, -1, [2000, 701], [3, 4], 128, 0),
    "g4x5_window_short": (16, 4, 300, [1500, 95, 40], [5, 5, 5], 64, 0),
    "g8x6_two_tiles_7_splits": (16, 2, -1, [900, 48], [6, 5], 64, 7),
    "g6x4_window_2_splits": (24, 4, 500, [1300, 777], [4, 2], 64, 2),
    "g8x4_tiny_lengths": (16, 2, -1, [4, 31, 33, 64, 65], [4, 4, 4, 4, 4], 64, 0),
}


@pytest.mark.parametrize("name", sorted(VERIFY_CASES))
def test_verify_kernel_cases(name):
    hq, hkv, window, seqlens, qlens, page, splits = VERIFY_CASES[name]
    w = wl.custom("bf16", 512, hq, hkv, window, seqlens, qlens, seed=91 + hq + len(seqlens))
    if page != 64:
        w = with_page_size(w, page)
    log(f"[case] verify {name}: G={hq // hkv} W={window} L={seqlens} q={qlens} page={page} splits={splits}")
    o_ref, l_ref, _ = oracle_run(w)
    o, l, _, s = gpu_run(w, "decode", num_splits=splits, split_q=True)
    compare(o, o_ref, l, l_ref, label=f"verify split Q {name} S={s}")
    o_b, l_b, _, s_b = gpu_run(w, "decode", num_splits=splits)
    compare(o_b, o_ref, l_b, l_ref, label=f"verify bf16 Q {name} S={s_b}")
    # the two modes: the same exact Q values and P kept to 8 bits in both, rounded differently
    assert s_b == s
    assert np.max(np.abs(o - o_b)) <= 1.6e-2 and np.max(np.abs(l - l_b)) <= 1e-4, \
        (np.max(np.abs(o - o_b)), np.max(np.abs(l - l_b)))


@pytest.mark.parametrize("split", [True, False], ids=["split", "bf16"])
@pytest.mark.parametrize("splits", [0, 2])
def test_verify_kernel_per_sequence_head_descales(splits, split):
    w = _per_bh_descales(wl.custom("bf16", 512, 32, 4, -1, [1200, 300, 77], [4, 4, 3], seed=97), seed=512)
    log(f"[case] verify (b,h) descales splits={splits} split_q={split}")
    o_ref, l_ref, _ = oracle_run(w)
    o, l, _, s = gpu_run(w, "decode", num_splits=splits, split_q=split)
    compare(o, o_ref, l, l_ref, label=f"verify (b,h) descales S={s} split_q={split}")


@pytest.mark.parametrize("split", [True, False], ids=["split", "bf16"])
@pytest.mark.parametrize("page", [64, 128])
def test_verify_kernel_nan_codes_past_sequence_end(page, split):
    w = wl.custom("bf16", 512, 32, 4, -1, [701, 77, 1501], [4, 4, 4], seed=98)
    if page != 64:
        w = with_page_size(w, page)
    wn = with_nan_tails(w)
    assert not torch.equal(wn.v_pool, w.v_pool)
    log(f"[case] verify NaN tails page={page} split_q={split}")
    o, l, _, s = gpu_run(w, "decode", split_q=split)
    o2, l2, _, s2 = gpu_run(wn, "decode", split_q=split)
    assert s2 == s
    assert np.isfinite(o2).all(), "a NaN past the sequence end reached the output"
    assert np.array_equal(o2, o) and np.array_equal(l2, l)
