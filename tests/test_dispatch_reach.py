"""The FP8 prefill runs each q block of 256 (token, q head) rows in one of two kernel instances: a
block whose first row sees fewer than 512 keys (min(position + 1, window)) takes the split-P
instance, every other block the single-P one.  These CPU checks apply that rule to the GPU parity
cases and show which instance each case reaches, so that a case meant for the single-P instance
cannot silently drift to the other one (no GPU needed)."""
import types

import pytest

from helpers import prefill_split_p_blocks
from test_gpu_coverage import SINGLE_P_CASES


@pytest.mark.parametrize("name", sorted(SINGLE_P_CASES))
def test_single_p_cases_reach_single_p(name):
    single, split = prefill_split_p_blocks(SINGLE_P_CASES[name]())
    assert single > 0, (name, single, split)


def _shape(hq, hkv, window, seqlens, qlens):
    return types.SimpleNamespace(num_q_heads=hq, num_kv_heads=hkv, window=window, seqlens_k_host=seqlens,
                                 q_lens_host=qlens)


def test_sliding_window_prefill_block_mix():
    # 8 x 8192 new tokens, 32/16 heads, W1024: per (sequence, kv head), 64 q blocks of 128 tokens;
    # blocks 0-3 start below token 512 and run split P, the other 60 single P
    single, split = prefill_split_p_blocks(_shape(32, 16, 1024, [8192] * 8, [8192] * 8))
    assert (single, split) == (60 * 16 * 8, 4 * 16 * 8)


def test_reduced_workload_with_short_window_is_split_p_only():
    # the reduced sliding-window prefill of the workload tests (scale 1/32: W = 32) never runs
    # single P, which is why the single-P cases above exist
    single, split = prefill_split_p_blocks(_shape(32, 16, 32, [256], [256]))
    assert single == 0 and split > 0


def test_rule_boundaries():
    # one sequence, G = 2: block qb's first token is 128 qb; it sees 128 qb + 1 keys with no window
    single, split = prefill_split_p_blocks(_shape(2, 1, -1, [1024], [1024]))
    assert (single, split) == (4, 4)      # tokens 0, 128, 256, 384 < 511 <= 512, 640, 768, 896
    # a window shorter than 512 keys puts every block in split P
    single, split = prefill_split_p_blocks(_shape(2, 1, 511, [4096], [4096]))
    assert single == 0
    # a window of exactly 512 keys: blocks whose first row sits at position >= 511 run single P
    single, split = prefill_split_p_blocks(_shape(2, 1, 512, [4096], [4096]))
    assert single == 28 and split == 4
