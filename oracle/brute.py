"""Brute-force attention with pure-Python loops, for tiny inputs only (TEST INFRASTRUCTURE).

This is written independently of ``attention.py`` so that the two can pin each
other.  It uses no numpy arithmetic: E4M3 values are decoded bit by bit,
``math.exp`` and ``math.fsum`` do the arithmetic, and an explicit dense mask
is built as nested lists.  It implements the same definition: paged gather,
causal + window mask with the query tokens at the end of each sequence, GQA
map ``hq // G``, softmax attention and natural-log LSE.
"""
from __future__ import annotations

import math


def _decode(code: int) -> float:
    # independent restatement of OCP E4M3: value = (-1)^s * 2^(E-7) * (1 + M/8), subnormal for E == 0
    sign = -1.0 if (code >> 7) & 1 else 1.0
    E = (code >> 3) & 15
    M = code & 7
    if E == 15 and M == 7:
        return float("nan")
    if E == 0:
        return sign * math.ldexp(M, -9)
    return sign * math.ldexp(8 + M, E - 10)


def brute_attention(q_vals, k_pool, v_pool, block_table, cu_seqlens_q, seqlens_k,
                    num_kv_heads, softmax_scale, window, k_descale, v_descale, page_size):
    """q_vals: nested lists [total_q][Hq][d] of floats; pools: nested lists [pages][page_size][Hkv][d]
    of ints (codes); k_descale / v_descale: one float, or nested lists [B][Hkv] (one value per
    sequence and kv head); returns (o, lse) as nested lists."""
    total_q = len(q_vals)
    hq = len(q_vals[0])
    d = len(q_vals[0][0])
    g = hq // num_kv_heads
    o = [[[0.0] * d for _ in range(hq)] for _ in range(total_q)]
    lse = [[0.0] * hq for _ in range(total_q)]
    B = len(seqlens_k)
    for b in range(B):
        L = int(seqlens_k[b])
        t0, t1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        ql = t1 - t0
        # dense mask [ql][L]
        mask = [[False] * L for _ in range(ql)]
        for i in range(ql):
            p = L - ql + i
            for j in range(L):
                ok = j <= p
                if window >= 1 and not (j > p - window):
                    ok = False
                mask[i][j] = ok
        for i in range(ql):
            t = t0 + i
            for h in range(hq):
                kvh = h // g
                kds = k_descale[b][kvh] if isinstance(k_descale, (list, tuple)) else k_descale
                vds = v_descale[b][kvh] if isinstance(v_descale, (list, tuple)) else v_descale
                scores = []
                for j in range(L):
                    if not mask[i][j]:
                        continue
                    page = int(block_table[b][j // page_size])
                    slot = j % page_size
                    kr = [_decode(int(c)) * kds for c in k_pool[page][slot][kvh]]
                    s = softmax_scale * math.fsum(q_vals[t][h][x] * kr[x] for x in range(d))
                    scores.append((j, s))
                m = max(s for _, s in scores)
                w = [(j, math.exp(s - m)) for j, s in scores]
                l = math.fsum(e for _, e in w)
                for x in range(d):
                    acc = []
                    for j, e in w:
                        page = int(block_table[b][j // page_size])
                        slot = j % page_size
                        acc.append(e * _decode(int(v_pool[page][slot][kvh][x])) * vds)
                    o[t][h][x] = math.fsum(acc) / l
                lse[t][h] = m + math.log(l)
    return o, lse

