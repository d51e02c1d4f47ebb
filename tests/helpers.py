"""Shared test plumbing: run a workload through the HIP library and through the oracle.

The oracle side receives only generator outputs (copied to host memory); nothing the HIP
path computed is ever fed to it.  The GPU side receives the same generator tensors on the
device.  For E4M3 queries each side quantizes on its own, and the tests compare the two code
arrays bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as wl
from oracle.attention import default_scale, paged_attention, query_values

TOL_MAX_ABS = 3e-2    # the stated bar for attention outputs on N(0,1) inputs
TOL_MEAN_ABS = 3e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host_pool_for(w: wl.Workload, pool: torch.Tensor, tokens=None):
    """Host copy of the pool pages that the selected query tokens can see.  The pool keeps its
    physical layout (pages not needed stay zero), so the oracle performs the real paged gather."""
    if pool.device.type == "cpu":
        return pool.numpy()
    bt = w.block_table.cpu().numpy()
    cu = w.cu_seqlens_q.cpu().numpy()
    sk = w.seqlens_k.cpu().numpy()
    ps = pool.shape[1]
    sel = None if tokens is None else set(int(t) for t in tokens)
    need = set()
    for b in range(len(sk)):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        toks = [t for t in range(t0, t1) if sel is None or t in sel]
        if not toks:
            continue
        L, ql = int(sk[b]), t1 - t0
        pmin, pmax = L - ql + (min(toks) - t0), L - ql + (max(toks) - t0)
        lo = 0 if w.window < 1 else max(0, pmin - w.window + 1)
        for n in range(lo // ps, pmax // ps + 1):
            need.add(int(bt[b, n]))
    host = np.zeros(tuple(pool.shape), dtype=np.uint8)
    if need:
        ids = torch.tensor(sorted(need), dtype=torch.long, device=pool.device)
        host[ids.cpu().numpy()] = pool.index_select(0, ids).cpu().numpy()
    return host


def oracle_run(w: wl.Workload, tokens=None, window=None, softmax_scale=None):
    """fp64 oracle outputs (o [T, Hq, d], lse [T, Hq]) plus the oracle's own Q codes (e4m3 only)."""
    qv, codes = query_values(w.q.cpu(), w.q_dtype, None if w.q_descale is None else w.q_descale.cpu())
    win = w.window if window is None else window
    sc = default_scale(w.head_dim) if softmax_scale is None else softmax_scale
    k = host_pool_for(w, w.k_pool, tokens)
    v = host_pool_for(w, w.v_pool, tokens)
    o, lse = paged_attention(qv, k, v, w.block_table.cpu(), w.cu_seqlens_q.cpu(), w.seqlens_k.cpu(),
                             w.num_kv_heads, sc, win, w.k_descale.cpu(), w.v_descale.cpu(),
                             page_size=w.k_pool.shape[1], tokens=tokens)
    return o, lse, codes


def gpu_run(w: wl.Workload, entry="decode", num_splits=0, window=None, softmax_scale=0.0, want_lse=True,
            out=None, q_codes=None, fused_q=False, split_q=False):
    """Run the HIP path.  Returns (o float64 [T,Hq,d], lse [T,Hq] or None, q codes (uint8 numpy) or
    None, splits used).  With fused_q an e4m3 workload hands bf16 Q to the attention call, which
    quantizes it itself (no codes are returned then).  With split_q a bf16 workload runs QK^T on
    the FP8 MFMA with Q split into two E4M3 terms (q_dtype BF16_SPLIT)."""
    import fp8_kv_cache_e4m3_amd as fa
    dev = torch.device("cuda")
    wd = w.to(dev)
    codes = None
    if w.q_dtype == "e4m3" and fused_q:
        q, qd = wd.q, wd.q_descale
    elif w.q_dtype == "e4m3":
        q = fa.fp8attn_quantize_q(wd.q, wd.q_descale) if q_codes is None else q_codes
        codes = q.cpu().numpy()
        qd = wd.q_descale
    else:
        q, qd = wd.q, None
    win = w.window if window is None else window
    assert not split_q or w.q_dtype == "bf16", "split Q takes bf16 queries"
    # K/V descales: one per-tensor value, or [B, Hkv] per (sequence, kv head)
    ds_strides = (0, 0) if wd.k_descale.numel() == 1 else (wd.k_descale.stride(0), wd.k_descale.stride(1))
    assert wd.v_descale.numel() == wd.k_descale.numel(), "K and V descales share one layout"
    kw = dict(q_descale=qd, k_descale=wd.k_descale, v_descale=wd.v_descale, softmax_scale=softmax_scale,
              window=win, want_lse=want_lse, out=out, quantize_q=fused_q, split_q=split_q,
              descale_strides=ds_strides)
    args = (q, wd.k_pool, wd.v_pool, wd.block_table, wd.cu_seqlens_q, wd.seqlens_k, w.max_seqlen_q,
            w.max_seqlen_k)
    splits = 1
    if entry == "decode":
        o, lse, splits = fa.fp8attn_decode_paged(*args, num_splits=num_splits, **kw)
    else:
        o, lse = fa.fp8attn_prefill_varlen(*args, **kw)
    torch.cuda.synchronize()
    o64 = o.float().cpu().numpy().astype(np.float64)
    l64 = None if lse is None else lse.cpu().numpy().astype(np.float64)
    return o64, l64, codes, splits


def compare(o_gpu, o_ref, lse_gpu=None, lse_ref=None, rows=None, tol_max=TOL_MAX_ABS, tol_mean=TOL_MEAN_ABS,
            label=""):
    """Element-wise comparison on the selected token rows.  Returns a stats dict; asserts the bar."""
    if rows is not None:
        o_gpu, o_ref = o_gpu[rows], o_ref[rows]
        if lse_gpu is not None:
            lse_gpu, lse_ref = lse_gpu[rows], lse_ref[rows]
    assert np.isfinite(o_gpu).all(), f"{label}: non-finite GPU output"
    d = np.abs(o_gpu - o_ref)
    st = {"max_abs": float(d.max()), "mean_abs": float(d.mean()),
          "rel_l2": float(np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30))}
    if lse_gpu is not None:
        st["lse_max_abs"] = float(np.abs(lse_gpu - lse_ref).max())
    log(f"[parity] {label} {st}")
    assert st["max_abs"] <= tol_max, (label, st)
    assert st["mean_abs"] <= tol_mean, (label, st)
    if lse_gpu is not None:
        assert st["lse_max_abs"] <= 1e-2, (label, st)
    return st


def sample_tokens(w: wl.Workload, n: int, seed: int = 0):
    """A seeded sample of query tokens plus the first and last token of the batch."""
    rng = np.random.default_rng(seed)
    cu = w.cu_seqlens_q.cpu().numpy()
    picks = {0, int(cu[-1]) - 1}
    extra = rng.choice(int(cu[-1]), size=min(n, int(cu[-1])), replace=False)
    picks.update(int(x) for x in extra)
    return sorted(picks)


def with_page_size(w: wl.Workload, page_size: int, seed: int = 4) -> wl.Workload:
    """The same logical K/V rows re-packed into framework blocks of page_size tokens (a multiple of
    64), placed in a fresh seeded random order.  Slots past a sequence's length stay zero."""
    import math as _m
    k, v, bt = w.k_pool, w.v_pool, w.block_table
    nblk = [_m.ceil(L / page_size) for L in w.seqlens_k_host]
    perm = np.random.default_rng(seed).permutation(sum(nblk))
    k2 = torch.zeros((sum(nblk), page_size) + tuple(k.shape[2:]), dtype=torch.uint8)
    v2 = torch.zeros_like(k2)
    table = torch.zeros((len(nblk), max(nblk)), dtype=torch.int32)
    nxt = 0
    for b, L in enumerate(w.seqlens_k_host):
        for n in range(nblk[b]):
            table[b, n] = int(perm[nxt])
            nxt += 1
        j = torch.arange(L)
        src_pages = bt[b, j // 64].long()
        dst_pages = table[b, j // page_size].long()
        k2[dst_pages, j % page_size] = k[src_pages, j % 64]
        v2[dst_pages, j % page_size] = v[src_pages, j % 64]
    w2 = wl.Workload(**{**w.__dict__})
    w2.k_pool, w2.v_pool, w2.block_table = k2, v2, table
    return w2


def with_nan_tails(w: wl.Workload) -> wl.Workload:
    """A copy whose pool slots past each sequence's length, in its last page, hold the E4M3 NaN
    codes (0x7F in K, 0xFF in V).  Those slots are never written for the sequence; no key there is
    visible, so the outputs must not change."""
    k, v = w.k_pool.clone(), w.v_pool.clone()
    ps = k.shape[1]
    for b, L in enumerate(w.seqlens_k_host):
        last = (L - 1) // ps
        page = int(w.block_table[b, last])
        s0 = L - last * ps
        if s0 < ps:
            k[page, s0:] = 0x7F
            v[page, s0:] = 0xFF
    w2 = wl.Workload(**{**w.__dict__})
    w2.k_pool, w2.v_pool = k, v
    return w2


def prefill_split_p_blocks(w: wl.Workload, rows_per_block: int = 256, split_p_keys: int = 512):
    """Which q blocks of the FP8 prefill run the single-P instance and which the split-P one, from
    the kernel's dispatch rule: a block of rows_per_block (token, q head) rows whose first row sees
    fewer than split_p_keys keys, min(position + 1, window), takes split P.  Returns the counts
    (single_p, split_p) over every (sequence, kv head, q block) that holds rows."""
    G = w.num_q_heads // w.num_kv_heads
    single = split = 0
    for L, ql in zip(w.seqlens_k_host, w.q_lens_host):
        for qb in range((ql * G + rows_per_block - 1) // rows_per_block):
            pf = L - ql + (qb * rows_per_block) // G
            keys = pf + 1 if w.window < 1 else min(pf + 1, w.window)
            if keys < split_p_keys:
                split += w.num_kv_heads
            else:
                single += w.num_kv_heads
    return single, split
