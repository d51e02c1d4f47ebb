"""fp8attn_decode_paged_noalloc: the decode call for callers that cannot allocate, with its split-KV
partials in the library's static device scratch.  Through the C-ABI it must give the workspace
call's outputs bit for bit (same plan, same kernels) and meet the oracle bar, on two calls in a row
whose second input is smaller (the scratch keeps the first call's contents), and it must refuse a
plan larger than its scratch before launching anything."""
import numpy as np
import pytest
import torch

import workloads as wl
from helpers import compare, log, oracle_run


def _fa():
    import fp8_kv_cache_e4m3_amd as fa
    return fa


def _calls(w, num_splits):
    fa = _fa()
    wd = w.to("cuda")
    args = (wd.q, wd.k_pool, wd.v_pool, wd.block_table, wd.cu_seqlens_q, wd.seqlens_k, w.max_seqlen_q,
            w.max_seqlen_k, None, wd.k_descale, wd.v_descale)
    o1, l1, s1 = fa.fp8attn_decode_paged(*args, window=w.window, num_splits=num_splits)
    o2, l2, s2 = fa.fp8attn_decode_paged_noalloc(*args, window=w.window, num_splits=num_splits)
    torch.cuda.synchronize()
    return (o1, l1, s1), (o2, l2, s2)


@pytest.mark.gpu
@pytest.mark.parametrize("num_splits", [-64, 0, 3])
def test_noalloc_decode_equals_workspace_decode_twice(num_splits):
    # first a larger input, then a smaller one: the scratch still holds the first call's partials
    big = wl.custom("bf16", 512, 16, 2, -1, [5000, 300, 4100, 17, 2000, 64], [1, 2, 1, 3, 1, 16], seed=91)
    small = wl.custom("bf16", 512, 16, 2, -1, [700, 1500], [1, 4], seed=92)
    for w in (big, small):
        (o1, l1, s1), (o2, l2, s2) = _calls(w, num_splits)
        log(f"[case] noalloc decode B={w.batch} splits requested={num_splits} used={s2}")
        assert s1 == s2 and (num_splits == 0 or s2 == num_splits or (num_splits > 0 and 1 <= s2 <= num_splits))
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "noalloc decode differs from the workspace call"
        o_ref, l_ref, _ = oracle_run(w)
        compare(o2.float().cpu().numpy().astype(np.float64), o_ref, l2.cpu().numpy().astype(np.float64), l_ref,
                label=f"noalloc decode S={s2}")


@pytest.mark.gpu
def test_noalloc_decode_fp8_windowed_balanced():
    w = wl.custom("e4m3", 256, 32, 16, 1024, [5000, 1030, 17, 3000], [1, 1, 1, 1], seed=93)
    fa = _fa()
    wd = w.to("cuda")
    q = fa.fp8attn_quantize_q(wd.q, wd.q_descale)
    args = (q, wd.k_pool, wd.v_pool, wd.block_table, wd.cu_seqlens_q, wd.seqlens_k, w.max_seqlen_q,
            w.max_seqlen_k, wd.q_descale, wd.k_descale, wd.v_descale)
    o1, l1, s1 = fa.fp8attn_decode_paged(*args, window=w.window, num_splits=-37)
    o2, l2, s2 = fa.fp8attn_decode_paged_noalloc(*args, window=w.window, num_splits=-37)
    torch.cuda.synchronize()
    assert s1 == s2 == -37 and torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_decode_refuses_plans_beyond_its_scratch():
    """A plan whose partials exceed the static scratch is refused with FP8ATTN_ERR_WORKSPACE before
    any HIP call (host tensors: validation and planning read host values only)."""
    fa = _fa()
    T, Hq, d = 64, 64, 512
    q = torch.zeros((T, Hq, d), dtype=torch.bfloat16)
    k = torch.zeros((4, 64, 8, d), dtype=torch.uint8)
    bt = torch.zeros((T, 512), dtype=torch.int32)
    cu = torch.arange(T + 1, dtype=torch.int32)
    sk = torch.full((T,), 32768, dtype=torch.int32)
    out = torch.zeros((T, Hq, d), dtype=torch.bfloat16)
    a = fa.make_args(q, k, k, bt, cu, sk, 1, 32768, out=out)
    import ctypes
    used = ctypes.c_int32(0)
    # 64 splits x 4096 rows x 512 x 4 bytes = 512 MiB of partials
    st = fa.LIB.fp8attn_decode_paged_noalloc(ctypes.byref(a), 64, ctypes.byref(used), None)
    assert st == fa.ERR_WORKSPACE, (st, fa.fp8attn_last_error())
    msg = fa.fp8attn_last_error()
    assert "static scratch" in msg and "fp8attn_decode_paged" in msg, msg
    assert 1 < used.value <= 64
