"""GPU parity: the HIP path (through the C-ABI) against the fp64 CPU oracle.

Bars: Q quantization and the page gather are bit-exact; attention outputs are within
max-abs 3e-2 and mean-abs 3e-3 of the oracle on N(0,1) inputs; LSE within 1e-2.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from helpers import compare, gpu_run, log, oracle_run, sample_tokens
from oracle.e4m3 import E4M3_TABLE, quantize_e4m3

pytestmark = pytest.mark.gpu


def _fa():
    import fp8_kv_cache_e4m3_amd as fa
    return fa


# ------------------------------------------------------------------------------------------
# Q quantization: bit-exact over every bf16 pattern
# ------------------------------------------------------------------------------------------
def test_quantize_q_exhaustive_bit_exact():
    fa = _fa()
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)  # all patterns
    q = bits.reshape(64, 4, 256).cuda()
    rng = np.random.default_rng(1)
    # 0.0: the descale of an all-zero tensor (amax / 448); 0 / 0 is a NaN quotient -> 0x7F | sign
    descales = [1.0, 2.0 ** -6, 1.0 / 448, 0.0100097656, 4.5 / 448, 3.0, 0.0] + list(rng.uniform(1e-3, 8.0, 24))
    xf = bits.float().numpy()
    for ds in descales:
        ds32 = np.float32(ds)
        dt = torch.tensor([ds32], dtype=torch.float32, device="cuda")
        got = fa.fp8attn_quantize_q(q, dt).cpu().numpy().reshape(-1)
        ref = quantize_e4m3(xf, ds32)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, f"descale {ds32!r}: {bad.size} codes differ; first x={xf[bad[0]]!r} " \
                              f"gpu={got[bad[0]]:#x} oracle={ref[bad[0]]:#x}"
    # NULL descale means 1.0
    got = fa.fp8attn_quantize_q(q, None).cpu().numpy().reshape(-1)
    assert np.array_equal(got, quantize_e4m3(xf, 1.0))


def test_quantize_q_strided_input():
    fa = _fa()
    base = torch.randn(37, 6, 320, dtype=torch.float32).to(torch.bfloat16).cuda()
    q = base[:, 1:5, 32:288]                    # head stride 320, token stride 1920, 256 wide
    ds = torch.tensor([0.0123], dtype=torch.float32, device="cuda")
    got = fa.fp8attn_quantize_q(q, ds).cpu().numpy()
    ref = quantize_e4m3(q.float().cpu().numpy(), np.float32(0.0123))
    assert np.array_equal(got, ref)


def test_quantize_q_large_ragged():
    """A 1 GB-class Q whose vector count leaves the last block ragged: 16,411 tokens x 31 heads x
    256 are 16,279,712 16-byte vectors, not a multiple of the 512 a block takes.  Sampled
    positions and the last 300,000 elements (the ragged block and the full blocks before it) are
    compared bit for bit with the oracle."""
    fa = _fa()
    g = torch.Generator(device="cuda").manual_seed(21)
    q = torch.randn((16411, 31, 256), generator=g, device="cuda").to(torch.bfloat16)
    ds32 = np.float32(q.float().abs().max().item() / 448.0)
    ds = torch.tensor([ds32], dtype=torch.float32, device="cuda")
    got = fa.fp8attn_quantize_q(q, ds).reshape(-1)
    n = got.numel()
    idx = torch.from_numpy(np.random.default_rng(3).choice(n, 1 << 21, replace=False)).cuda()
    tail = torch.arange(n - 300_000, n, device="cuda")
    for sel in (idx, tail):
        x = q.reshape(-1)[sel].float().cpu().numpy()
        ref = quantize_e4m3(x, ds32)
        assert np.array_equal(got[sel].cpu().numpy(), ref)


# ------------------------------------------------------------------------------------------
# the tiny workload through both entry points and both query dtypes
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("q_dtype", ["bf16", "e4m3"])
@pytest.mark.parametrize("entry", ["prefill", "decode"])
def test_tiny_case(q_dtype, entry):
    w = wl.tiny(q_dtype)
    log(f"[case] tiny {q_dtype} {entry}")
    o_ref, l_ref, codes_ref = oracle_run(w)
    o, l, codes, splits = gpu_run(w, entry)
    if q_dtype == "e4m3":
        assert np.array_equal(codes, codes_ref)
    compare(o, o_ref, l, l_ref, label=f"tiny {q_dtype} {entry} S={splits}")


# ------------------------------------------------------------------------------------------
# the performance workloads: reduced sizes element by element, full sizes on samples
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,scale,entry,split_q", [
    ("swa_decode", 0.25, "decode", False),
    ("full_decode", 0.125, "decode", False),
    ("spec_verify", 0.0625, "decode", False),
    ("spec_verify", 0.0625, "decode", True),
    ("swa_prefill", 1 / 32, "prefill", False),
    ("full_prefill", 1 / 8, "prefill", False),
    ("full_prefill", 1 / 8, "prefill", True),
])
def test_workload_reduced_all_rows(name, scale, entry, split_q):
    w = wl.BY_NAME[name](device="cpu", scale=scale)
    log(f"[case] {w.name} entry={entry} split_q={split_q} B={w.batch} total_q={w.total_q} maxL={w.max_seqlen_k}")
    o_ref, l_ref, codes_ref = oracle_run(w)
    o, l, codes, splits = gpu_run(w, entry, split_q=split_q)
    if codes is not None:
        assert np.array_equal(codes, codes_ref)
    compare(o, o_ref, l, l_ref, label=f"{w.name} S={splits}")


@pytest.mark.parametrize("name,entry,nsample,split_q", [
    ("swa_decode", "decode", 32, False),
    ("full_decode", "decode", 8, False),
    ("spec_verify", "decode", 8, False),
    # (the sliding-window prefill at full size: test_gpu_coverage.py, whole q blocks)
    ("full_decode", "decode", 8, True),      # bf16 Q on the FP8 MFMA (split Q)
    ("spec_verify", "decode", 8, True),
    ("full_prefill", "prefill", 16, False),
    ("full_prefill", "prefill", 16, True),
])
def test_workload_full_size_sampled(name, entry, nsample, split_q):
    w = wl.BY_NAME[name](device="cuda")
    log(f"[case] full-size {w.name} entry={entry} split_q={split_q} B={w.batch} total_q={w.total_q} "
        f"pool={tuple(w.k_pool.shape)}")
    o, l, codes, splits = gpu_run(w, entry, split_q=split_q)
    if codes is not None:   # bit-exact quantization over the whole Q tensor
        _, codes_ref = __import__("oracle").attention.query_values(w.q.cpu(), "e4m3", w.q_descale.cpu())
        assert np.array_equal(codes, codes_ref)
    toks = sample_tokens(w, nsample, seed=11)
    o_ref, l_ref, _ = oracle_run(w, tokens=toks)
    compare(o, o_ref, l, l_ref, rows=toks, label=f"full-size {w.name} S={splits} rows={len(toks)}")


# ------------------------------------------------------------------------------------------
# bf16 Q quantized inside the attention kernels: the same codes as the separate quantize
# call, so the outputs equal the two-call path bit for bit (and meet the oracle bar)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("name,scale,entry,splits", [
    ("tiny", None, "prefill", 0),
    ("tiny", None, "decode", 0),
    ("swa_decode", 0.25, "decode", 0),
    ("swa_decode", 0.25, "decode", 3),
    ("multi_token_d256", None, "decode", 0),
    ("multi_token_d64", None, "decode", 2),
    ("swa_prefill", 1 / 32, "prefill", 0),
    ("ragged_d64", None, "prefill", 0),
])
def test_fused_q_quantization(name, scale, entry, splits):
    if name == "tiny":
        w = wl.tiny("e4m3")
    elif name == "multi_token_d256":     # several query tokens per sequence, GQA 8:1, window
        w = wl.custom("e4m3", 256, 16, 2, 300, [700, 65, 1500], [4, 16, 1], seed=21)
    elif name == "multi_token_d64":
        w = wl.custom("e4m3", 64, 8, 1, -1, [129, 64, 999], [3, 7, 16], seed=22)
    elif name == "ragged_d64":           # prefill with ragged query lengths and tails
        w = wl.custom("e4m3", 64, 4, 2, 100, [300, 37, 513], [300, 20, 257], seed=23)
    else:
        w = wl.BY_NAME[name](device="cpu", scale=scale)
    assert w.q_dtype == "e4m3"
    log(f"[case] fused-q {w.name} entry={entry} splits={splits}")
    o2, l2, _, s2 = gpu_run(w, entry, num_splits=splits)
    o1, l1, codes, s1 = gpu_run(w, entry, num_splits=splits, fused_q=True)
    assert codes is None and s1 == s2
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o_ref, l_ref, _ = oracle_run(w)
    compare(o1, o_ref, l1, l_ref, label=f"fused-q {w.name} S={s1}")


def test_fused_q_full_size_swa_decode():
    w = wl.BY_NAME["swa_decode"](device="cuda")
    log(f"[case] fused-q full-size {w.name}")
    o2, l2, _, _ = gpu_run(w, "decode")
    o1, l1, _, _ = gpu_run(w, "decode", fused_q=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------------------------------------
# split-KV: every split count meets the bar; one split needs no workspace
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 0, 1000, -1, -2, -7, -64, -1000])
def test_split_counts(splits):
    # negative: the balanced partition into -splits parts (more parts than units included)
    w = wl.custom("bf16", 512, 8, 2, -1, [700, 64, 1500, 3], [1, 2, 1, 3], seed=21)
    o_ref, l_ref, _ = oracle_run(w)
    o, l, _, used = gpu_run(w, "decode", num_splits=splits)
    log(f"[case] splits requested={splits} used={used}")
    if splits > 0:
        assert 1 <= used <= splits
    elif splits < 0:
        assert used == splits
    compare(o, o_ref, l, l_ref, label=f"splits={splits}->{used}")


# ------------------------------------------------------------------------------------------
# balanced partition: the batch's units split evenly over the blocks, tiles cut by block
# boundaries merged by the partition's combine
# ------------------------------------------------------------------------------------------
_R25 = [int(x) for x in np.random.default_rng(9).integers(16, 3000, 25)]


@pytest.mark.parametrize("q_dtype,d,hq,hkv,window,seqlens,qlens,parts,fused", [
    ("bf16", 512, 32, 4, -1, [9000, 300, 4100, 17, 2000], [1, 1, 1, 1, 1], 0, False),   # automatic pick
    ("bf16", 512, 8, 2, -1, [700, 64, 1500, 16, 999], [1, 2, 1, 3, 16], -5, False),      # ragged q_len
    ("e4m3", 256, 32, 16, 1024, [5000, 1030, 17, 3000], [1, 1, 1, 1], -37, True),      # window, fused Q
    ("e4m3", 64, 16, 1, -1, [2000] * 70, [1] * 70, -100, True),                       # 70 tiles: two chunks
    ("bf16", 128, 8, 1, 77, [400, 90, 1300], [16, 3, 9], -3, False),                   # 8 row tiles, window
    ("bf16", 64, 16, 2, -1, _R25, [16] * 25, -50, False),                              # 200 tiles per kv head
])
def test_balanced_partition(q_dtype, d, hq, hkv, window, seqlens, qlens, parts, fused):
    w = wl.custom(q_dtype, d, hq, hkv, window, seqlens, qlens, seed=71)
    log(f"[case] balanced {q_dtype} d{d} {hq}/{hkv} W{window} B{len(seqlens)} parts={parts}")
    o_ref, l_ref, _ = oracle_run(w)
    o, l, _, used = gpu_run(w, "decode", num_splits=parts, fused_q=fused)
    assert used < 0 and (parts == 0 or used == parts), used
    compare(o, o_ref, l, l_ref, label=f"balanced parts={-used}")
    o2, l2, _, _ = gpu_run(w, "decode", num_splits=parts, fused_q=fused)
    assert np.array_equal(o, o2) and np.array_equal(l, l2), "two identical runs differ"


def test_combine_entry_point():
    fa = _fa()
    rng = np.random.default_rng(3)
    S, T, H, d = 5, 7, 3, 256
    po = rng.standard_normal((S, T, H, d)).astype(np.float32)
    pl = rng.standard_normal((S, T, H)).astype(np.float32) * 3
    pl[1, 2, :] = -np.inf          # a split that saw nothing for one token
    po[1, 2, :, :] = np.nan        # ... whose partial must not be read
    pl[:, 4, 1] = -np.inf          # a row no split saw
    from oracle.attention import combine_splits
    o_ref, l_ref = combine_splits(po.reshape(S, T * H, d), pl.reshape(S, T * H))
    o_ref = o_ref.reshape(T, H, d)
    out = torch.empty((T, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    fa.fp8attn_splitkv_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda(), out, lse)
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    assert np.max(np.abs(o - o_ref)) < 1e-2
    lg = lse.cpu().numpy().reshape(-1)
    fin = np.isfinite(l_ref)
    assert np.max(np.abs(lg[fin] - l_ref[fin])) < 1e-5
    assert np.all(np.isneginf(lg[~fin])) and np.all(o[4, 1] == 0)


# ------------------------------------------------------------------------------------------
# gather: bit-exact (one-hot logits), page permutation invariance, determinism
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("q_dtype,d", [("bf16", 512), ("e4m3", 256), ("bf16", 64), ("e4m3", 64),
                                       ("e4m3", 192), ("bf16", 128), ("e4m3", 96), ("bf16", 96)])
def test_one_hot_gather_bit_exact(q_dtype, d):
    """Q equal to one key's row with a huge softmax scale: every other weight is exactly 0 in
    fp32, so O must equal that key's dequantized V row bit for bit (v_descale a power of two)."""
    fa = _fa()
    w = wl.custom(q_dtype, d, 2, 1, -1, [300, 129], [1, 1], seed=5)
    w.v_descale = torch.tensor([0.25], dtype=torch.float32)
    targets = [173, 64]
    for b, j in enumerate(targets):
        page = int(w.block_table[b, j // 64])
        kcode = w.k_pool[page, j % 64, 0].numpy()
        qrow = torch.from_numpy(E4M3_TABLE[kcode].astype(np.float32))
        w.q[b, :, :] = qrow.to(torch.bfloat16)
    if q_dtype == "e4m3":
        w.q_descale = torch.tensor([1.0], dtype=torch.float32)
    o, _, _, _ = gpu_run(w, "decode", num_splits=3, softmax_scale=1e3, want_lse=False)
    for b, j in enumerate(targets):
        page = int(w.block_table[b, j // 64])
        vrow = E4M3_TABLE[w.v_pool[page, j % 64, 0].numpy()] * 0.25
        assert np.array_equal(o[b, 0], vrow) and np.array_equal(o[b, 1], vrow), (b, j)


def test_page_permutation_and_determinism():
    w = wl.custom("bf16", 512, 16, 2, -1, [1000, 300, 77], [1, 4, 2], seed=8)
    o1, l1, _, _ = gpu_run(w, "decode", num_splits=4)
    o2, l2, _, _ = gpu_run(w, "decode", num_splits=4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "two identical runs differ"
    npg = w.k_pool.shape[0]
    perm = torch.from_numpy(np.random.default_rng(2).permutation(npg))
    w2 = wl.Workload(**{**w.__dict__})
    w2.k_pool = torch.empty_like(w.k_pool)
    w2.v_pool = torch.empty_like(w.v_pool)
    w2.k_pool[perm] = w.k_pool
    w2.v_pool[perm] = w.v_pool
    w2.block_table = perm[w.block_table.long()].to(torch.int32)
    o3, l3, _, _ = gpu_run(w2, "decode", num_splits=4)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3), "page permutation changed the output"


# ------------------------------------------------------------------------------------------
# edge cases
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("q_dtype,d,hq,hkv,window,seqlens,qlens,entry", [
    ("bf16", 512, 32, 4, -1, [1], [1], "decode"),                          # a single key
    ("e4m3", 256, 32, 16, 1, [5000, 17], [1, 1], "decode"),                # window of one key
    ("e4m3", 256, 32, 16, 100000, [3000, 65], [1, 1], "decode"),           # window longer than the sequence
    ("bf16", 512, 32, 4, -1, [16, 33, 64, 65, 127], [16, 1, 9, 2, 5], "decode"),  # q_len up to 16, ragged
    ("e4m3", 64, 4, 4, 37, [400, 90], [90, 90], "prefill"),                # no prior cache, window
    ("bf16", 64, 6, 3, -1, [129, 2], [129, 2], "prefill"),                 # prefill of whole sequences
    ("e4m3", 256, 8, 1, 300, [2048, 700], [40, 3], "prefill"),             # GQA 8, chunked prefill
    ("bf16", 512, 8, 8, -1, [900], [5], "decode"),                         # MHA
])
def test_edge_cases(q_dtype, d, hq, hkv, window, seqlens, qlens, entry):
    w = wl.custom(q_dtype, d, hq, hkv, window, seqlens, qlens, seed=13)
    log(f"[case] edge {q_dtype} d{d} {hq}/{hkv} W{window} L={seqlens} q={qlens} {entry}")
    o_ref, l_ref, codes_ref = oracle_run(w)
    o, l, codes, splits = gpu_run(w, entry)
    if codes is not None:
        assert np.array_equal(codes, codes_ref)
    compare(o, o_ref, l, l_ref, label=f"edge {entry} S={splits}")


# ------------------------------------------------------------------------------------------
# head dims 96, 128 and 192, both variants, both entry points (96 also through the balanced
# partition); the in-kernel Q quantization gives the two-call path's outputs bit for bit
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("d", [96, 128, 192])
@pytest.mark.parametrize("q_dtype,entry,splits", [
    ("e4m3", "decode", 0), ("e4m3", "decode", 3), ("e4m3", "prefill", 0), ("e4m3", "decode", -6),
    ("bf16", "decode", 0), ("bf16", "decode", 2), ("bf16", "prefill", 0), ("bf16", "decode", -6),
])
def test_head_dims(d, q_dtype, entry, splits):
    window = 300 if q_dtype == "e4m3" else -1
    if entry == "decode":     # GQA 8:1, q_len 1..16, ragged lengths
        w = wl.custom(q_dtype, d, 16, 2, window, [700, 65, 1500], [4, 16, 1], seed=d + 1)
    else:                     # several 256-row q blocks, ragged tails, chunked prefill
        w = wl.custom(q_dtype, d, 8, 2, window, [600, 90, 1300], [300, 90, 41], seed=d + 2)
    log(f"[case] head dim {d} {q_dtype} {entry} splits={splits}")
    o_ref, l_ref, codes_ref = oracle_run(w)
    o, l, codes, s = gpu_run(w, entry, num_splits=splits)
    if codes is not None:
        assert np.array_equal(codes, codes_ref)
    compare(o, o_ref, l, l_ref, label=f"d{d} {q_dtype} {entry} S={s}")
    if q_dtype == "e4m3":
        o1, l1, _, s1 = gpu_run(w, entry, num_splits=splits, fused_q=True)
        assert s1 == s and np.array_equal(o1, o) and np.array_equal(l1, l)


# ------------------------------------------------------------------------------------------
# split Q (q_dtype BF16_SPLIT): QK^T on the FP8 MFMA with Q as hi + lo/16 (exact for bf16) and
# PV on the FP8 MFMA with P as 16 hi + lo (8 significant bits, like bf16 P), every head dim and
# plan; against the oracle and against the BF16-MFMA path: the same exact Q values and P kept
# to 8 bits in both, rounded differently, so outputs agree to two bf16 ulps and the LSE (which
# takes fp32 P in both) to the order of fp32 sums
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 96, 128, 192, 256, 512])
@pytest.mark.parametrize("entry,splits", [("decode", 0), ("decode", 3), ("decode", -5), ("prefill", 0)])
def test_split_q(d, entry, splits):
    window = -1 if d in (96, 512) else 200
    if entry == "decode":
        w = wl.custom("bf16", d, 16, 2, window, [700, 65, 1500], [4, 16, 1], seed=d + 5)
    else:
        w = wl.custom("bf16", d, 8, 2, window, [600, 90, 700], [300, 90, 41], seed=d + 6)
    log(f"[case] split-q d{d} {entry} splits={splits}")
    o_ref, l_ref, _ = oracle_run(w)
    o, l, _, s = gpu_run(w, entry, num_splits=splits, split_q=True)
    compare(o, o_ref, l, l_ref, label=f"split-q d{d} {entry} S={s}")
    o_b, l_b, _, s_b = gpu_run(w, entry, num_splits=splits)
    assert s_b == s
    assert np.max(np.abs(o - o_b)) <= 1.6e-2 and np.max(np.abs(l - l_b)) <= 1e-4, \
        (np.max(np.abs(o - o_b)), np.max(np.abs(l - l_b)))


def test_split_q_row_scales():
    """Per-row power-of-two scales: query rows of magnitude 0, 1e-30, 1e-3, 1, 1e3 and 1e30 (the
    large ones give one-hot softmax rows, the tiny ones near-uniform rows)."""
    w = wl.custom("bf16", 512, 8, 2, -1, [900, 300, 77], [2, 2, 2], seed=33)
    mags = [0.0, 1e-30, 1e-3, 1.0, 1e3, 1e30]
    q = w.q.float()
    for t in range(q.shape[0]):
        q[t] *= mags[t % len(mags)]
    w.q = q.to(torch.bfloat16)
    o_ref, l_ref, _ = oracle_run(w)
    o, l, _, _ = gpu_run(w, "decode", split_q=True)
    compare(o, o_ref, label="split-q row scales")
    # The LSE of the 1e30 rows is their largest logit, about 1e32: an fp32 sum of 512 products
    # with cancellation, so its error is relative (measured 1.4e-5), bounded here by 1e-4
    assert np.all(np.abs(l - l_ref) <= 1e-2 + 1e-4 * np.abs(l_ref)), np.max(np.abs(l - l_ref) / (1 + np.abs(l_ref)))


@pytest.mark.parametrize("d,q_dtype,fused", [(64, "e4m3", False), (256, "e4m3", False), (256, "e4m3", True)])
def test_prefill_short_window_long_sequence(d, q_dtype, fused):
    """FP8 prefill with a window shorter than the split-P threshold over a sequence long enough
    that most q blocks lie past the first few: every block belongs to the split-P instance, whose
    grid must then cover all of them (every row of the output is compared)."""
    w = wl.custom(q_dtype, d, 4, 2, 100, [1500, 700], [1500, 300], seed=31)
    log(f"[case] short window prefill d{d} fused={fused} W=100 lens={w.seqlens_k_host} q={w.q_lens_host}")
    o_ref, l_ref, codes_ref = oracle_run(w)
    o, l, codes, _ = gpu_run(w, "prefill", fused_q=fused)
    if codes is not None:
        assert np.array_equal(codes, codes_ref)
    compare(o, o_ref, l, l_ref, label=f"short window prefill d{d} fused={fused}")


def test_page_size_128_and_strided_output():
    """Framework blocks of 128 tokens (two kernel pages) and an output with padded strides."""
    fa = _fa()
    w = wl.custom("bf16", 512, 8, 2, -1, [300, 129], [2, 1], seed=17)
    # re-pack 64-token pages into 128-token blocks with a fresh random placement
    k, v, bt = w.k_pool, w.v_pool, w.block_table
    nblk = [math.ceil(L / 128) for L in w.seqlens_k_host]
    perm = np.random.default_rng(4).permutation(sum(nblk))
    k2 = torch.zeros((sum(nblk), 128) + tuple(k.shape[2:]), dtype=torch.uint8)
    v2 = torch.zeros_like(k2)
    table = torch.zeros((len(nblk), max(nblk)), dtype=torch.int32)
    nxt = 0
    for b, L in enumerate(w.seqlens_k_host):
        for n in range(nblk[b]):
            table[b, n] = int(perm[nxt])
            nxt += 1
        for j in range(L):
            k2[table[b, j // 128], j % 128] = k[bt[b, j // 64], j % 64]
            v2[table[b, j // 128], j % 128] = v[bt[b, j // 64], j % 64]
    o_ref, l_ref, _ = oracle_run(w)
    w2 = wl.Workload(**{**w.__dict__})
    w2.k_pool, w2.v_pool, w2.block_table = k2, v2, table
    for splits in (2, -5):   # split grid and balanced partition
        big = torch.zeros((w.total_q, 8, 640), dtype=torch.bfloat16, device="cuda")
        out = big[:, :, 64:576]
        o, l, _, _ = gpu_run(w2, "decode", num_splits=splits, out=out)
        compare(o, o_ref, l, l_ref, label=f"page 128 + strided out, splits {splits}")
        assert torch.all(big[:, :, :64] == 0) and torch.all(big[:, :, 576:] == 0), "wrote outside the output view"


def test_per_sequence_head_descales():
    """K/V descales laid out (batch, kv heads) via strides, as the pages forward them."""
    fa = _fa()
    w = wl.custom("bf16", 512, 8, 2, -1, [500, 200], [1, 1], seed=19)
    # per-(sequence, head) factors around the per-tensor recipe, so outputs stay O(1) as on N(0,1) data
    kd = w.k_descale * torch.tensor([[1.0, 2.0], [0.5, 1.5]], dtype=torch.float32)
    vd = w.v_descale * torch.tensor([[1.0, 0.5], [2.0, 0.25]], dtype=torch.float32)
    from oracle.attention import paged_attention, default_scale, query_values
    qv, _ = query_values(w.q, "bf16")
    o_ref = np.zeros((w.total_q, 8, 512))
    l_ref = np.zeros((w.total_q, 8))
    for b in range(2):
        for h in range(2):
            sel = slice(b, b + 1)
            o_b, l_b = paged_attention(qv[sel], w.k_pool, w.v_pool, w.block_table[sel], torch.tensor([0, 1]),
                                       w.seqlens_k[sel], 2, default_scale(512), -1, kd[b, h], vd[b, h])
            o_ref[b, 4 * h:4 * h + 4] = o_b[0, 4 * h:4 * h + 4]
            l_ref[b, 4 * h:4 * h + 4] = l_b[0, 4 * h:4 * h + 4]
    wd = w.to("cuda")
    for splits in (1, 2):
        o, l, _ = fa.fp8attn_decode_paged(wd.q, wd.k_pool, wd.v_pool, wd.block_table, wd.cu_seqlens_q,
                                          wd.seqlens_k, 1, 500, None, kd.cuda(), vd.cuda(), num_splits=splits,
                                          descale_strides=(2, 1))
        torch.cuda.synchronize()
        compare(o.float().cpu().numpy(), o_ref, l.cpu().numpy(), l_ref, label=f"per (b,h) descales S={splits}")


def test_null_descales_and_no_lse():
    w = wl.custom("bf16", 512, 8, 2, -1, [333], [1], seed=23)
    # unit descales: the codes themselves are N(0,1) values
    g = torch.Generator().manual_seed(23)
    w.k_pool = torch.randn(w.k_pool.shape, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    w.v_pool = torch.randn(w.v_pool.shape, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    w.k_descale = torch.tensor([1.0])
    w.v_descale = torch.tensor([1.0])
    o_ref, l_ref, _ = oracle_run(w)
    fa = _fa()
    wd = w.to("cuda")
    o, l, _ = fa.fp8attn_decode_paged(wd.q, wd.k_pool, wd.v_pool, wd.block_table, wd.cu_seqlens_q, wd.seqlens_k,
                                      1, 333, None, None, None, want_lse=False)
    assert l is None
    torch.cuda.synchronize()
    compare(o.float().cpu().numpy(), o_ref, label="NULL descales")


def test_empty_batch():
    fa = _fa()
    q = torch.empty((0, 8, 512), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 64, 2, 512), dtype=torch.uint8, device="cuda")
    bt = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    cu = torch.zeros((1,), dtype=torch.int32, device="cuda")
    sk = torch.zeros((0,), dtype=torch.int32, device="cuda")
    o, l, s = fa.fp8attn_decode_paged(q, k, k, bt, cu, sk, 0, 0)
    assert o.shape == (0, 8, 512)
    o, l = fa.fp8attn_prefill_varlen(q, k, k, bt, cu, sk, 0, 0)
    assert o.shape == (0, 8, 512)
