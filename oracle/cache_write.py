"""Paged KV-cache write: quantize new keys/values to E4M3 and scatter them into pages
(TEST INFRASTRUCTURE).

What it computes, stated plainly:

* The step (vLLM PR #60372, Details, "Why FP8 is slower than BF16", the KV-cache write rows
  of both profile tables and the note under the first one).  The kernels in this category
  reshape the newly produced keys and values and store them into the paged cache, and with an
  FP8 cache they also convert them to FP8.
* Quantization.  The cache holds ``float8_e4m3fn`` codes with a per-tensor descale (prhub
  digest of vLLM PR #48666, Key code).  The reading adopted for K and V is the one this oracle
  already uses for Q: fp32 division by the descale, round to nearest even, saturation at +-448,
  NaN kept with its sign (``oracle.e4m3.quantize_e4m3``).
* Addressing.  The pages do not print the slot numbering.  Plainest reading, consistent with the
  page table of the attention call: token t goes to ``slot = slot_mapping[t]``, i.e. page
  ``slot // page_size`` and position ``slot % page_size`` inside it; a slot outside
  ``[0, num_pages * page_size)`` (padding tokens use -1) writes nothing.  Pools are
  ``[pages, page_size, Hkv, d]`` as in ``oracle.attention``.
* Slots are distinct; with a repeated slot the result is whichever write lands last, so the
  oracle takes the last token in order and the tests use distinct slots.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import quantize_e4m3


def cache_write(k_new, v_new, slot_mapping, k_cache, v_cache, k_descale=1.0, v_descale=1.0):
    """Return copies of the two caches with the new tokens written.

    k_new, v_new: [T, Hkv, d] real values (bf16 or fp32 inputs, read as float32).
    slot_mapping: [T] integers.  k_cache, v_cache: uint8 codes [pages, page_size, Hkv, d].
    """
    k_new = np.asarray(k_new, dtype=np.float32)
    v_new = np.asarray(v_new, dtype=np.float32)
    kc = np.array(k_cache, dtype=np.uint8, copy=True)
    vc = np.array(v_cache, dtype=np.uint8, copy=True)
    pages, page_size = kc.shape[0], kc.shape[1]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64).tolist()):
        if slot < 0 or slot >= pages * page_size:
            continue
        page, pos = divmod(slot, page_size)
        kc[page, pos] = quantize_e4m3(k_new[t], k_descale)
        vc[page, pos] = quantize_e4m3(v_new[t], v_descale)
    return kc, vc


def slots_for_new_tokens(block_table, seqlens_k, q_lens, page_size: int):
    """Slot of every new token: the new tokens of sequence b are its last q_len positions
    ``L - q_len .. L - 1`` (the same placement the attention oracle uses for queries), and
    position j lives in page ``block_table[b, j // page_size]`` at ``j % page_size``."""
    out = []
    for b, (L, ql) in enumerate(zip(np.asarray(seqlens_k).tolist(), np.asarray(q_lens).tolist())):
        for j in range(L - ql, L):
            out.append(int(block_table[b][j // page_size]) * page_size + j % page_size)
    return np.asarray(out, dtype=np.int64)
