"""Seeded random sweep of the GPU path against the fp64 CPU oracle, through the C-ABI.

Each case draws its own configuration from a fixed seed, so the set is the same on every run:
Q mode (E4M3 codes, bf16 quantized in the kernel, bf16, bf16 split into two E4M3 terms), head
dim (the ones each mode supports), GQA group 1-16 (3, 5 and 6 included, whose rows straddle the
16- and 32-row tiles and the 256-row prefill blocks), one or two kv heads, batch 1-3, ragged
query and context lengths (a context as short as the query, lengths off the 16/64-key grids),
causal with or without a window (as small as 1), 64- or 128-token pages, per-tensor or
per-(sequence, kv head) K/V descales, E4M3 NaN codes in the pool slots past a sequence's end, and
the entry point: decode (up to 16 query tokens; the
automatic plan, one split, three splits or a balanced partition) or prefill.  Every output row
is compared with the oracle to the stated bar; E4M3 codes bit for bit.
"""
import numpy as np
import pytest

import workloads as wl
from helpers import compare, gpu_run, log, oracle_run, with_nan_tails, with_page_size
from test_gpu_coverage import _per_bh_descales

pytestmark = pytest.mark.gpu

N_CASES = 64


def _draw(i):
    rng = np.random.default_rng(9100 + i)
    mode = str(rng.choice(["e4m3", "e4m3_fused", "bf16", "bf16_split"]))
    dims = [64, 96, 128, 192, 256] + ([] if mode.startswith("e4m3") else [512])
    d = int(rng.choice(dims))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16]))
    hkv = int(rng.choice([1, 2])) if G <= 8 else 1
    entry = str(rng.choice(["decode", "prefill"]))
    B = int(rng.integers(1, 4))
    qmax = 16 if entry == "decode" else 400
    qlens = [int(x) for x in rng.integers(1, qmax + 1, B)]
    ctx = [int(x) for x in rng.integers(0, 2000, B)]
    if rng.random() < 0.3:
        ctx[int(rng.integers(0, B))] = 0                       # no cached context: pure prefill
    seqlens = [q + c for q, c in zip(qlens, ctx)]
    r = rng.random()
    window = -1 if r < 0.4 else 1 if r < 0.5 else int(rng.integers(2, 1200))
    page = 128 if rng.random() < 0.3 else 64
    per_bh = bool(rng.random() < 0.25)
    nan_tails = bool(rng.random() < 0.25)
    splits = int(rng.choice([0, 1, 3, -7])) if entry == "decode" else 0
    return dict(mode=mode, d=d, G=G, hkv=hkv, entry=entry, qlens=qlens, seqlens=seqlens, window=window,
                page=page, per_bh=per_bh, nan_tails=nan_tails, splits=splits)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = _draw(i)
    log(f"[case] sweep {i}: {c}")
    q_dtype = "e4m3" if c["mode"].startswith("e4m3") else "bf16"
    w = wl.custom(q_dtype, c["d"], c["G"] * c["hkv"], c["hkv"], c["window"], c["seqlens"], c["qlens"], seed=9200 + i)
    if c["per_bh"]:
        w = _per_bh_descales(w, seed=9300 + i)
    if c["page"] != 64:
        w = with_page_size(w, c["page"])
    if c["nan_tails"]:
        w = with_nan_tails(w)
    o_ref, l_ref, codes_ref = oracle_run(w)
    o, l, codes, used = gpu_run(w, c["entry"], num_splits=c["splits"], fused_q=c["mode"] == "e4m3_fused",
                                split_q=c["mode"] == "bf16_split")
    if codes is not None:
        assert np.array_equal(codes.reshape(-1), np.asarray(codes_ref).reshape(-1)), "Q codes differ"
    compare(o, o_ref, l, l_ref, label=f"sweep {i} {c['mode']} d{c['d']} G{c['G']} {c['entry']} S={used}")
