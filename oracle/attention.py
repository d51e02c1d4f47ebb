"""Masked softmax attention over a paged E4M3 KV cache, in fp64 (TEST INFRASTRUCTURE).

What the path computes, stated plainly:

* Paged cache (vLLM PR #60372 review thread and prhub digest of vLLM PR
  #48666, Implementation item 2).  The cache is split into pages whose token
  count is a multiple of 64.  ``block_table[b, n]`` is the physical page that
  holds tokens ``n*page_size .. (n+1)*page_size-1`` of sequence b.  Pools are
  laid out ``[pages, page_size, Hkv, d]``, with K and V in separate pools.
* Descales (vLLM PR #60372, Claims; prhub digest of vLLM PR #48666, Key code).
  K/V/Q descales are per-tensor fp32 values that the kernel folds in.  The
  dequantized value is ``code_value * descale``.
* Queries (vLLM PR #63139, Overview).  In the native-FP8 variant Q is E4M3
  (quantized with q_descale).  In the dequant variant Q stays BF16.
* Mask (vLLM PR #60372 review thread: causal and local masks only).  Query i of
  a sequence with KV length L and q_len new tokens sits at position
  ``p = L - q_len + i``, i.e. the new tokens are the last positions.  Key j is
  visible iff ``j <= p`` and, with a window W >= 1, ``j > p - W``.  W = -1
  means no window.  GQA maps q head hq to kv head ``hq // (Hq / Hkv)``.
* Output.  ``s_j = scale * <q, k_j>``, ``o = sum_j softmax(s)_j v_j``, and
  ``lse = max(s) + ln(sum_j exp(s_j - max(s)))``, the natural log, as the
  second output the kernel call returns (prhub digest of vLLM PR #48666, Key
  code: ``out, softmax_lse``).
* Split-KV (vLLM PR #60372, Claims: the split count is picked automatically).
  Attention over disjoint key subsets is merged by log-sum-exp weights.

Everything is fp64.  Only the visible key range of each query is gathered.
Masked keys carry zero weight, so this is the definition itself, not an
approximation.
"""
from __future__ import annotations

import math

import numpy as np

from .e4m3 import E4M3_TABLE, quantize_e4m3


def _np(x):
    if hasattr(x, "detach"):          # torch tensor -> numpy (tests pass either)
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.float()
        x = x.numpy()
    return np.asarray(x)


def query_values(q, q_dtype: str, q_descale=None):
    """Query values the attention sees, plus the E4M3 codes for the native-FP8 variant.

    bf16 Q: the bf16 values, exactly, in fp64; the codes are None.
    e4m3 Q: codes = quantize_e4m3(q, q_descale); values = code value * q_descale.
    The native FP8 forward runs on the quantized Q (vLLM PR #63139, Overview)."""
    qf = _np(q).astype(np.float32)
    if q_dtype == "bf16":
        return qf.astype(np.float64), None
    ds = 1.0 if q_descale is None else float(_np(q_descale).reshape(-1)[0])
    codes = quantize_e4m3(qf, ds)
    return E4M3_TABLE[codes] * float(np.float32(ds)), codes


def gather_pages(pool, block_table_row, positions, page_size: int):
    """Codes of the given logical token positions of one sequence: ``pool[page, slot]``.

    ``page = block_table_row[j // page_size]`` and ``slot = j % page_size``."""
    pool = _np(pool)
    positions = np.asarray(positions, dtype=np.int64)
    pages = np.asarray(_np(block_table_row), dtype=np.int64)[positions // page_size]
    return pool[pages, positions % page_size]


def visible_mask(q_positions, key_positions, window: int):
    """Boolean [nq, nk]: key j is visible from query position p iff j <= p and (W < 1 or j > p - W)."""
    p = np.asarray(q_positions, dtype=np.int64)[:, None]
    j = np.asarray(key_positions, dtype=np.int64)[None, :]
    m = j <= p
    if window is not None and window >= 1:
        m &= j > p - window
    return m


def descale_at(x, b: int, h: int) -> float:
    """The fp32 descale of sequence b and kv head h.  ``x`` is None (1.0), one per-tensor value
    (a scalar or one-element array), or a [B, Hkv] array of per-(sequence, kv head) values, the
    layout the pages forward to the kernel (prhub digest of vLLM PR #48666, Key code: descales
    expanded to (batch, num_kv_heads))."""
    if x is None:
        return 1.0
    a = _np(x)
    if a.size == 1:
        return float(np.float32(a.reshape(-1)[0]))
    assert a.ndim == 2, "per-(sequence, kv head) descales are a [B, Hkv] array"
    return float(np.float32(a[b, h]))


def paged_attention(q_vals, k_pool, v_pool, block_table, cu_seqlens_q, seqlens_k,
                    num_kv_heads: int, softmax_scale: float, window: int = -1,
                    k_descale=None, v_descale=None, page_size: int = 64,
                    tokens=None, key_ranges=None, chunk: int = 256):
    """Exact masked softmax attention in fp64.

    q_vals   : float [total_q, Hq, d], the query values (see query_values)
    k_pool   : uint8 [pages, page_size, Hkv, d] E4M3 codes; v_pool likewise
    returns  : (o [total_q, Hq, d], lse [total_q, Hq]), both fp64.  Rows not
               selected by ``tokens`` (an optional list of global query-token
               indices) are NaN.
    k_descale, v_descale: None (1.0), one per-tensor value, or [B, Hkv] arrays of
               per-(sequence, kv head) values (see descale_at).
    key_ranges: optional [B] list of (k_lo, k_hi) that further limits the keys
               to lo <= j < hi.  This is the attention of one KV split.  A row
               with no visible key then gets o = 0 and lse = -inf, which is the
               neutral element of the combine.
    """
    q_vals = np.asarray(_np(q_vals), dtype=np.float64)
    k_pool = _np(k_pool)
    v_pool = _np(v_pool)
    bt = _np(block_table).astype(np.int64)
    cu = _np(cu_seqlens_q).astype(np.int64)
    sk = _np(seqlens_k).astype(np.int64)
    total_q, hq, d = q_vals.shape
    hkv = num_kv_heads
    assert hq % hkv == 0
    g = hq // hkv
    out = np.full((total_q, hq, d), np.nan)
    lse = np.full((total_q, hq), np.nan)
    sel = None if tokens is None else set(int(t) for t in tokens)
    for b in range(len(sk)):
        L = int(sk[b])
        t0, t1 = int(cu[b]), int(cu[b + 1])
        ql = t1 - t0
        toks = [t for t in range(t0, t1) if sel is None or t in sel]
        for c0 in range(0, len(toks), chunk):
            ct = np.array(toks[c0:c0 + chunk], dtype=np.int64)
            pos = L - ql + (ct - t0)
            lo = 0 if window is None or window < 1 else max(0, int(pos.min()) - window + 1)
            hi = int(pos.max()) + 1
            if key_ranges is not None:
                lo, hi = max(lo, key_ranges[b][0]), min(hi, key_ranges[b][1])
            if hi <= lo:
                out[ct] = 0.0
                lse[ct] = -np.inf
                continue
            keys = np.arange(lo, hi)
            mask = visible_mask(pos, keys, window)            # [n, nk]
            kc = gather_pages(k_pool, bt[b], keys, page_size)  # [nk, Hkv, d]
            vc = gather_pages(v_pool, bt[b], keys, page_size)
            for h in range(hkv):
                kd, vd = descale_at(k_descale, b, h), descale_at(v_descale, b, h)
                K = E4M3_TABLE[kc[:, h, :]] * kd              # [nk, d] fp64
                V = E4M3_TABLE[vc[:, h, :]] * vd
                Q = q_vals[ct, h * g:(h + 1) * g, :]           # [n, g, d]
                S = softmax_scale * (Q @ K.T)                  # [n, g, nk]
                S = np.where(mask[:, None, :], S, -np.inf)
                m = S.max(axis=-1, keepdims=True)
                empty = ~np.isfinite(m)
                m_safe = np.where(empty, 0.0, m)
                E = np.exp(S - m_safe)
                l = E.sum(axis=-1, keepdims=True)
                o = (E @ V) / np.where(empty, 1.0, l)
                o = np.where(empty, 0.0, o)
                out[ct, h * g:(h + 1) * g, :] = o
                lse[ct, h * g:(h + 1) * g] = np.where(empty[..., 0], -np.inf, (m_safe + np.log(np.where(empty, 1.0, l)))[..., 0])
    return out, lse


def combine_splits(partial_o, partial_lse):
    """Log-sum-exp merge of split partials.

    partial_o [S, n, d] holds each split's normalized output, partial_lse [S, n]
    its LSE (-inf for a split that saw no key).  M = max_s lse_s,
    w_s = exp(lse_s - M), o = sum_s w_s o_s / sum_s w_s and lse = M + ln sum_s w_s.
    A split with lse = -inf has weight 0 and its o is never read.  A row where every split is
    -inf (no visible key at all) has no softmax: it gets o = 0 and lse = -inf."""
    po = np.asarray(_np(partial_o), dtype=np.float64)
    pl = np.asarray(_np(partial_lse), dtype=np.float64)
    M = pl.max(axis=0)                                   # [n]
    fin = np.isfinite(pl)
    w = np.where(fin, np.exp(np.where(fin, pl, 0.0) - np.where(np.isfinite(M), M, 0.0)), 0.0)
    wsum = w.sum(axis=0)
    num = np.einsum("sn,snd->nd", w, np.where(fin[..., None], po, 0.0))
    seen = wsum > 0
    # a row that no split saw has no softmax; it gets o = 0 and lse = -inf
    o = np.where(seen[:, None], num / np.where(seen, wsum, 1.0)[:, None], 0.0)
    return o, np.where(seen, M + np.log(np.where(seen, wsum, 1.0)), -np.inf)


def split_attention(q_vals, k_pool, v_pool, block_table, cu_seqlens_q, seqlens_k,
                    num_kv_heads, softmax_scale, window, k_descale, v_descale, page_size,
                    boundaries):
    """Attention computed on key ranges cut at ``boundaries`` (a sorted list of key
    positions, shared by all sequences), then merged with combine_splits."""
    sk = _np(seqlens_k).astype(np.int64)
    edges = [0] + list(boundaries) + [int(sk.max()) + 1]
    parts_o, parts_l = [], []
    for a, b in zip(edges[:-1], edges[1:]):
        o, l = paged_attention(q_vals, k_pool, v_pool, block_table, cu_seqlens_q, seqlens_k,
                               num_kv_heads, softmax_scale, window, k_descale, v_descale,
                               page_size, key_ranges=[(a, b)] * len(sk))
        parts_o.append(o)
        parts_l.append(l)
    po = np.stack(parts_o)
    pl = np.stack(parts_l)
    s, n, hq, d = po.shape
    o, l = combine_splits(po.reshape(s, n * hq, d), pl.reshape(s, n * hq))
    return o.reshape(n, hq, d), l.reshape(n, hq)


def default_scale(head_dim: int) -> float:
    """The pages never state the softmax scale; the plain reading is 1/sqrt(head_dim)."""
    return 1.0 / math.sqrt(head_dim)
