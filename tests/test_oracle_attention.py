"""Pins of the oracle's paged attention and split combine (CPU only).

Independent anchors: the pure-Python brute force (oracle/brute.py, written
separately with math.exp/math.fsum and an explicit dense mask), closed forms
(one visible key, Q = 0, window 1, constant V) and invariants (page
permutation, GQA replication, window >= length equals causal, split + combine
equals the unsplit result, scale folding).  A dropped descale, a wrong mask
bound, a transposed page/slot or a wrong GQA map each fails at least one test.
"""
import math

import numpy as np
import pytest

import workloads
from oracle import brute
from oracle.attention import (combine_splits, default_scale, gather_pages, paged_attention,
                              query_values, split_attention, visible_mask)
from oracle.e4m3 import E4M3_TABLE


def _run(w, scale=None, window=None, **kw):
    qv, _ = query_values(w.q, w.q_dtype, w.q_descale)
    return paged_attention(qv, w.k_pool, w.v_pool, w.block_table, w.cu_seqlens_q, w.seqlens_k,
                           w.num_kv_heads, default_scale(w.head_dim) if scale is None else scale,
                           w.window if window is None else window, w.k_descale, w.v_descale, **kw)


def _brute(w, page_size=64):
    qv, _ = query_values(w.q, w.q_dtype, w.q_descale)
    o, l = brute.brute_attention(qv.tolist(), w.k_pool.numpy().tolist(), w.v_pool.numpy().tolist(),
                                 w.block_table.numpy().tolist(), w.cu_seqlens_q.numpy().tolist(),
                                 w.seqlens_k.numpy().tolist(), w.num_kv_heads, default_scale(w.head_dim),
                                 w.window, float(w.k_descale[0]), float(w.v_descale[0]), page_size)
    return np.array(o), np.array(l)


def _small(q_dtype, d=8, hq=4, hkv=2, window=-1, seqlens=(70, 3, 130), qlens=(5, 3, 2), seed=1):
    return workloads.custom(q_dtype, d, hq, hkv, window, list(seqlens), list(qlens), seed=seed)


@pytest.mark.parametrize("q_dtype", ["bf16", "e4m3"])
@pytest.mark.parametrize("window", [-1, 1, 17, 64])
def test_matches_brute_force(q_dtype, window):
    w = _small(q_dtype, window=window)
    o, l = _run(w)
    ob, lb = _brute(w)
    assert np.max(np.abs(o - ob)) < 1e-12
    assert np.max(np.abs(l - lb)) < 1e-12


def test_tiny_workload_matches_brute_force():
    for qd in ("bf16", "e4m3"):
        w = workloads.tiny(qd)
        assert w.block_table.tolist() == [[1, 0]]
        o, l = _run(w)
        ob, lb = _brute(w)
        assert np.max(np.abs(o - ob)) < 1e-12 and np.max(np.abs(l - lb)) < 1e-12


def test_page_size_128_matches_brute_force():
    # framework blocks of 128 tokens (a multiple of the 64-token kernel page)
    w = _small("bf16", seqlens=(200, 129), qlens=(4, 1))
    # re-pack the 64-token pool into 128-token blocks with a fresh permuted table
    bt = w.block_table.numpy()
    k = w.k_pool.numpy()
    v = w.v_pool.numpy()
    nblk = [math.ceil(L / 128) for L in w.seqlens_k_host]
    perm = np.random.default_rng(3).permutation(sum(nblk))
    k2 = np.zeros((sum(nblk), 128) + k.shape[2:], np.uint8)
    v2 = np.zeros_like(k2)
    table = np.zeros((len(nblk), max(nblk)), np.int64)
    nxt = 0
    for b, L in enumerate(w.seqlens_k_host):
        for n in range(nblk[b]):
            table[b, n] = perm[nxt]
            nxt += 1
        for j in range(L):
            k2[table[b, j // 128], j % 128] = k[bt[b, j // 64], j % 64]
            v2[table[b, j // 128], j % 128] = v[bt[b, j // 64], j % 64]
    qv, _ = query_values(w.q, "bf16")
    sc = default_scale(w.head_dim)
    o1, l1 = paged_attention(qv, k2, v2, table, w.cu_seqlens_q, w.seqlens_k, 2, sc, -1,
                             w.k_descale, w.v_descale, page_size=128)
    o0, l0 = _run(w)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)
    ob, lb = brute.brute_attention(qv.tolist(), k2.tolist(), v2.tolist(), table.tolist(),
                                   w.cu_seqlens_q.numpy().tolist(), w.seqlens_k.numpy().tolist(), 2,
                                   sc, -1, float(w.k_descale[0]), float(w.v_descale[0]), 128)
    assert np.max(np.abs(o1 - np.array(ob))) < 1e-12


def test_constant_v_gives_constant_and_rows_sum_to_one():
    w = _small("bf16", window=9)
    w.v_pool[:] = 0x38  # every V value is 1.0
    o, _ = _run(w)
    # o = sum_j p_j * 1.0 * v_descale, so o / v_descale is the row sum of the softmax
    assert np.max(np.abs(o / float(w.v_descale[0]) - 1.0)) < 1e-12


def test_zero_query_is_mean_of_visible_values():
    w = _small("bf16", window=5)
    w.q[:] = 0
    o, l = _run(w)
    cu, sk = w.cu_seqlens_q.numpy(), w.seqlens_k.numpy()
    vd = float(w.v_descale[0])
    for b in range(w.batch):
        L, ql = int(sk[b]), int(cu[b + 1] - cu[b])
        for i in range(ql):
            p = L - ql + i
            keys = [j for j in range(L) if j <= p and j > p - 5]
            codes = gather_pages(w.v_pool, w.block_table[b], keys, 64)   # [n, Hkv, d]
            mean = E4M3_TABLE[codes].mean(axis=0) * vd                   # [Hkv, d]
            for h in range(w.num_q_heads):
                t = int(cu[b]) + i
                assert np.max(np.abs(o[t, h] - mean[h // 2])) < 1e-12
                assert abs(l[t, h] - math.log(len(keys))) < 1e-12


def test_window_one_returns_own_value_row():
    w = _small("e4m3", window=1)
    o, l = _run(w)
    cu, sk = w.cu_seqlens_q.numpy(), w.seqlens_k.numpy()
    qv, _ = query_values(w.q, "e4m3", w.q_descale)
    for b in range(w.batch):
        L, ql = int(sk[b]), int(cu[b + 1] - cu[b])
        for i in range(ql):
            p, t = L - ql + i, int(cu[b]) + i
            vrow = E4M3_TABLE[gather_pages(w.v_pool, w.block_table[b], [p], 64)[0]] * float(w.v_descale[0])
            krow = E4M3_TABLE[gather_pages(w.k_pool, w.block_table[b], [p], 64)[0]] * float(w.k_descale[0])
            for h in range(w.num_q_heads):
                assert np.array_equal(o[t, h], vrow[h // 2])
                s = default_scale(w.head_dim) * float(np.dot(qv[t, h], krow[h // 2]))
                assert abs(l[t, h] - s) < 1e-12


def test_long_window_equals_causal():
    w = _small("bf16", window=-1)
    o0, l0 = _run(w)
    o1, l1 = _run(w, window=max(w.seqlens_k_host))
    o2, l2 = _run(w, window=10 ** 6)
    assert np.array_equal(o0, o1) and np.array_equal(o0, o2)
    assert np.array_equal(l0, l1)


def test_window_is_w_keys_including_self():
    m = visible_mask([10], np.arange(12), 4)
    assert list(np.nonzero(m[0])[0]) == [7, 8, 9, 10]
    m = visible_mask([2], np.arange(12), -1)
    assert list(np.nonzero(m[0])[0]) == [0, 1, 2]


def test_page_permutation_invariance():
    w = _small("bf16", window=33)
    o0, l0 = _run(w)
    npg = w.k_pool.shape[0]
    perm = np.random.default_rng(9).permutation(npg)      # new physical id of old page p is perm[p]
    k2 = np.empty_like(w.k_pool.numpy())
    v2 = np.empty_like(k2)
    k2[perm] = w.k_pool.numpy()
    v2[perm] = w.v_pool.numpy()
    bt2 = perm[w.block_table.numpy()]
    qv, _ = query_values(w.q, "bf16")
    o1, l1 = paged_attention(qv, k2, v2, bt2, w.cu_seqlens_q, w.seqlens_k, 2,
                             default_scale(w.head_dim), 33, w.k_descale, w.v_descale)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_gqa_equals_replicated_mha():
    w = _small("bf16", hq=6, hkv=2, window=20)
    o0, l0 = _run(w)
    k = w.k_pool.numpy()
    v = w.v_pool.numpy()
    krep = np.repeat(k, 3, axis=2)   # kv head h -> q heads 3h..3h+2
    vrep = np.repeat(v, 3, axis=2)
    qv, _ = query_values(w.q, "bf16")
    o1, l1 = paged_attention(qv, krep, vrep, w.block_table, w.cu_seqlens_q, w.seqlens_k, 6,
                             default_scale(w.head_dim), 20, w.k_descale, w.v_descale)
    assert np.max(np.abs(o0 - o1)) < 1e-13 and np.max(np.abs(l0 - l1)) < 1e-13


def test_split_then_combine_equals_full():
    w = _small("e4m3", window=-1, seqlens=(70, 3, 130), qlens=(5, 3, 2))
    o0, l0 = _run(w)
    qv, _ = query_values(w.q, "e4m3", w.q_descale)
    for bounds in ([64], [1, 2, 64, 128], [13, 77]):
        o1, l1 = split_attention(qv, w.k_pool, w.v_pool, w.block_table, w.cu_seqlens_q, w.seqlens_k,
                                 2, default_scale(w.head_dim), -1, w.k_descale, w.v_descale, 64, bounds)
        assert np.max(np.abs(o0 - o1)) < 1e-12 and np.max(np.abs(l0 - l1)) < 1e-12


def test_combine_closed_forms():
    rng = np.random.default_rng(4)
    o = rng.standard_normal((3, 5, 7))
    l = rng.standard_normal((3, 5))
    # one split: identity
    oc, lc = combine_splits(o[:1], l[:1])
    assert np.array_equal(oc, o[0]) and np.array_equal(lc, l[0])
    # a -inf split is ignored, even if its o holds NaN
    o2 = o.copy()
    o2[1] = np.nan
    l2 = l.copy()
    l2[1] = -np.inf
    oc, lc = combine_splits(o2, l2)
    oe, le = combine_splits(o[[0, 2]], l[[0, 2]])
    assert np.max(np.abs(oc - oe)) < 1e-14 and np.max(np.abs(lc - le)) < 1e-14
    # a row no split saw: o = 0, lse = -inf
    l3 = l.copy()
    l3[:, 2] = -np.inf
    oc, lc = combine_splits(o, l3)
    assert np.all(oc[2] == 0) and np.isneginf(lc[2]) and np.isfinite(oc).all()
    # equal lse: plain mean, lse + ln S
    oc, lc = combine_splits(o, np.zeros((3, 5)))
    assert np.max(np.abs(oc - o.mean(axis=0))) < 1e-14 and np.max(np.abs(lc - math.log(3))) < 1e-14


def test_one_hot_logit_returns_value_row_exactly():
    # Q aligned with one key and a huge scale: all other weights underflow to exactly 0
    w = _small("bf16", d=8, hq=2, hkv=1, window=-1, seqlens=(100,), qlens=(1,))
    L = 100
    target = 37
    kcodes = gather_pages(w.k_pool, w.block_table[0], [target], 64)[0, 0]
    w.q[0, :, :] = 0
    w.q[0, :, :] = __import__("torch").from_numpy(E4M3_TABLE[kcodes].astype(np.float32)).to(w.q.dtype)
    o, _ = _run(w, scale=1e4)
    kall = E4M3_TABLE[gather_pages(w.k_pool, w.block_table[0], np.arange(L), 64)[:, 0]]
    s = kall @ E4M3_TABLE[kcodes]
    assert int(np.argmax(s)) == target and np.sort(s)[-1] - np.sort(s)[-2] > 0.1
    vrow = E4M3_TABLE[gather_pages(w.v_pool, w.block_table[0], [target], 64)[0, 0]] * float(w.v_descale[0])
    assert np.array_equal(o[0, 0], vrow) and np.array_equal(o[0, 1], vrow)


def test_scale_folding():
    # doubling k_descale while halving softmax_scale leaves the logits unchanged
    w = _small("e4m3", window=12)
    o0, l0 = _run(w, scale=0.3)
    w2 = workloads.Workload(**{**w.__dict__})
    w2.k_descale = w.k_descale * 2
    o1, l1 = _run(w2, scale=0.15)
    assert np.max(np.abs(o0 - o1)) < 1e-12 and np.max(np.abs(l0 - l1)) < 1e-12


def test_query_quantization_uses_codes():
    w = _small("e4m3")
    qv, codes = query_values(w.q, "e4m3", w.q_descale)
    assert codes.dtype == np.uint8 and codes.shape == tuple(w.q.shape)
    assert np.array_equal(qv, E4M3_TABLE[codes] * float(w.q_descale[0]))
    # the amax element maps to +-448 exactly
    qf = w.q.float().numpy()
    i = np.unravel_index(np.argmax(np.abs(qf)), qf.shape)
    assert codes[i] in (0x7E, 0xFE)


def test_token_subset_equals_full_rows():
    w = _small("bf16", window=-1)
    o0, l0 = _run(w)
    o1, l1 = _run(w, tokens=[1, 6, 9], chunk=2)
    for t in [1, 6, 9]:
        assert np.array_equal(o0[t], o1[t]) and np.array_equal(l0[t], l1[t])
    assert np.isnan(o1[0]).all()


def test_default_scale_closed_form():
    """The softmax scale the pages leave open is read as 1/sqrt(head_dim): exact powers of two at
    the even-power head dims, 2^-4.5 at 512 and a value whose square is 1/96 at 96."""
    assert default_scale(256) == 0.0625
    assert default_scale(64) == 0.125
    assert default_scale(16) == 0.25
    assert abs(default_scale(512) - 2.0 ** -4.5) < 1e-17          # 1/sqrt(512) = 2^-4.5
    assert abs(default_scale(96) * default_scale(96) * 96 - 1.0) < 1e-15


def test_per_sequence_head_descales_match_brute_force():
    """K/V descales laid out per (sequence, kv head): the oracle's lookup against the brute force,
    which reads its own nested lists [B][Hkv]."""
    w = _small("bf16", hq=4, hkv=2, seqlens=(70, 3, 130), qlens=(5, 3, 2), seed=4)
    kd = np.array([[0.5, 2.0], [1.25, 0.75], [3.0, 0.125]], dtype=np.float32) * float(w.k_descale[0])
    vd = np.array([[1.5, 0.25], [2.0, 1.0], [0.5, 4.0]], dtype=np.float32) * float(w.v_descale[0])
    qv, _ = query_values(w.q, "bf16")
    o, l = paged_attention(qv, w.k_pool, w.v_pool, w.block_table, w.cu_seqlens_q, w.seqlens_k, 2,
                           default_scale(w.head_dim), -1, kd, vd)
    ob, lb = brute.brute_attention(qv.tolist(), w.k_pool.numpy().tolist(), w.v_pool.numpy().tolist(),
                                   w.block_table.numpy().tolist(), w.cu_seqlens_q.numpy().tolist(),
                                   w.seqlens_k.numpy().tolist(), 2, default_scale(w.head_dim), -1,
                                   kd.astype(np.float64).tolist(), vd.astype(np.float64).tolist(), 64)
    assert np.max(np.abs(o - np.array(ob))) < 1e-12 and np.max(np.abs(l - np.array(lb))) < 1e-12
    # and the per-tensor case is the (b, h) case with every entry equal
    o1, l1 = _run(w)
    full = np.full((3, 2), np.float32(w.k_descale[0])), np.full((3, 2), np.float32(w.v_descale[0]))
    o2, l2 = paged_attention(qv, w.k_pool, w.v_pool, w.block_table, w.cu_seqlens_q, w.seqlens_k, 2,
                             default_scale(w.head_dim), -1, *full)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
