#!/usr/bin/env python3
"""Benchmark of the paged FP8-KV attention path on one MI355X.

Main line: the sliding-window decode workload (batch 32, one query token each, KV lengths
uniform in [1024, 8192], 32 q / 16 kv heads, head dim 256, window 1024, E4M3 Q/K/V).  One step
is the whole hot path over one batch: quantize Q to E4M3, then split-KV paged attention (plus
the LSE combine when more than one split is chosen).  ``value`` is the algorithmic KV-read rate:
bytes of the visible keys and values plus Q read and O written, divided by the step time.
Four independently drawn input sets rotate so that the working set exceeds the 256 MiB MALL.

``roofline`` covers the attention kernel alone, timed with HIP events on the stream it runs on.
``cpu_baseline`` times the CPU oracle on a bounded sample of the same workload (and, with one BLAS
thread, on one pass and on the tiny workload).  ``extra`` reports the other workload shapes
(full-attention decode, spec-verify with a shared prefix, sliding-window prefill, d512 prefill),
each with its own ``roofline`` object (HBM GB/s or MFMA TFLOP/s against the MI355X peak), and the
spec-verify lines with the cache-aware bound (each distinct page read once, or its MFMA work).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--profile-pass]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV-read GB/s + prefill attention TFLOP/s, % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0       # dense FP8 MFMA
BF16_PEAK_TFLOPS = 2500.0      # dense BF16 MFMA
# sources each measured kernel is built from: a recorded traffic figure is used only while they
# are unchanged
KERNEL_SOURCES = {
    "cache_write": ["fp8_kv_cache_e4m3_amd/csrc/cache_write.hip", "fp8_kv_cache_e4m3_amd/csrc/device.h",
                    "fp8_kv_cache_e4m3_amd/csrc/params.h"],
    "decode": ["fp8_kv_cache_e4m3_amd/csrc/decode.hip", "fp8_kv_cache_e4m3_amd/csrc/device.h",
               "fp8_kv_cache_e4m3_amd/csrc/params.h"],
    "prefill": ["fp8_kv_cache_e4m3_amd/csrc/prefill.hip", "fp8_kv_cache_e4m3_amd/csrc/device.h",
                "fp8_kv_cache_e4m3_amd/csrc/params.h"],
    "prefill_wide": ["fp8_kv_cache_e4m3_amd/csrc/prefill_wide.hip", "fp8_kv_cache_e4m3_amd/csrc/device.h",
                     "fp8_kv_cache_e4m3_amd/csrc/params.h"],
    "combine": ["fp8_kv_cache_e4m3_amd/csrc/combine.hip", "fp8_kv_cache_e4m3_amd/csrc/device.h",
                "fp8_kv_cache_e4m3_amd/csrc/params.h"],
    "verify": ["fp8_kv_cache_e4m3_amd/csrc/verify.hip", "fp8_kv_cache_e4m3_amd/csrc/device.h",
               "fp8_kv_cache_e4m3_amd/csrc/params.h"],
}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        fp = os.path.join(ROOT, p)
        if os.path.exists(fp):
            h.update(open(fp, "rb").read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------------------------------
# algorithmic work of a workload (visible keys only)
# ------------------------------------------------------------------------------------------
def visible_pairs(w):
    """Number of visible (query token, key) pairs per q head, summed over the batch."""
    total = 0
    for L, ql in zip(w.seqlens_k_host, w.q_lens_host):
        for i in range(ql):
            p = L - ql + i
            n = p + 1 if w.window < 1 else min(p + 1, w.window)
            total += n
    return total


def visible_keys(w):
    """Keys that at least one query of each sequence sees (the KV bytes any kernel must read)."""
    total = 0
    for L, ql in zip(w.seqlens_k_host, w.q_lens_host):
        lo = 0 if w.window < 1 else max(0, L - ql - w.window + 1)
        total += L - lo
    return total


def algo_bytes(w, fused=True):
    """Bytes the attention call must move: visible K/V (1 byte each), Q (bf16 when the call
    quantizes it or takes it unquantized, E4M3 codes when quantized beforehand) and bf16 out."""
    kv = visible_keys(w) * w.num_kv_heads * w.head_dim * 2          # K and V, 1 byte each
    qb = w.total_q * w.num_q_heads * w.head_dim * (1 if (w.q_dtype == "e4m3" and not fused) else 2)
    ob = w.total_q * w.num_q_heads * w.head_dim * 2
    return kv + qb + ob, kv


def unique_kv_bytes(w):
    """Bytes of the distinct pages that hold visible keys, K and V (shared-prefix pages once): what a
    kernel that kept every shared page on chip after its first read would fetch from HBM."""
    ps = w.k_pool.shape[1]
    bt = w.block_table.cpu().numpy()
    pages = set()
    for b, (L, ql) in enumerate(zip(w.seqlens_k_host, w.q_lens_host)):
        lo = 0 if w.window < 1 else max(0, L - ql - w.window + 1)
        pages.update(int(x) for x in bt[b, lo // ps:(L - 1) // ps + 1])
    return len(pages) * ps * w.num_kv_heads * w.head_dim * 2


def algo_flops(w):
    return 4.0 * w.head_dim * visible_pairs(w) * w.num_q_heads


# ------------------------------------------------------------------------------------------
# GPU steps
# ------------------------------------------------------------------------------------------
class Runner:
    """One input set.  For E4M3 workloads the step takes bf16 Q: by default the attention call
    quantizes it in-kernel (one launch); with fused=False a separate quantize call writes the
    codes first (two launches)."""
    def __init__(self, w, entry, fused=True, split=False):
        import torch
        import fp8_kv_cache_e4m3_amd as fa
        self.fa, self.torch, self.w, self.entry = fa, torch, w, entry
        self.out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((w.total_q, w.num_q_heads), dtype=torch.float32, device="cuda")
        self.qcodes = None
        if w.q_dtype == "e4m3" and not fused:
            self.qcodes = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.uint8, device="cuda")
        q = self.qcodes if self.qcodes is not None else w.q
        self.args = fa.make_args(q, w.k_pool, w.v_pool, w.block_table, w.cu_seqlens_q, w.seqlens_k,
                                 w.max_seqlen_q, w.max_seqlen_k,
                                 w.q_descale if w.q_dtype == "e4m3" else None, w.k_descale, w.v_descale,
                                 0.0, w.window, True, self.out, self.lse,
                                 quantize_q=(w.q_dtype == "e4m3" and fused), split_q=split)
        self.ws = None
        self.splits = 1
        if entry == "decode":
            need, self.splits = fa.decode_workspace_size(self.args, 0)
            if need:
                self.ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def quantize(self, stream):
        w = self.w
        if self.qcodes is not None:
            st = self.fa.LIB.fp8attn_quantize_q(w.q.data_ptr(), w.total_q, w.num_q_heads, w.head_dim,
                                                w.q.stride(0), w.q.stride(1), w.q_descale.data_ptr(),
                                                self.qcodes.data_ptr(), stream)
            assert st == 0, self.fa.fp8attn_last_error()

    def attend(self, stream):
        import ctypes
        fa = self.fa
        if self.entry == "decode":
            ws = self.ws
            st = fa.LIB.fp8attn_decode_paged(ctypes.byref(self.args), 0, None if ws is None else ws.data_ptr(),
                                             0 if ws is None else ws.numel(), None, None, stream)
        else:
            st = fa.LIB.fp8attn_prefill_varlen(ctypes.byref(self.args), stream)
        assert st == 0, fa.fp8attn_last_error()


def time_workload(make, entry, nsets, steps, warmup, label, fused=True, split=False):
    """Returns dict with ms_per_step (whole step) and kernel_ms (attention call only, HIP events).
    split: bf16 Q runs on the FP8 MFMA as two E4M3 terms (q_dtype BF16_SPLIT)."""
    import torch
    t0 = time.time()
    runners = [Runner(make(seed), entry, fused, split) for seed in range(nsets)]
    torch.cuda.synchronize()
    log(f"[bench] {label}: {nsets} input sets ready in {time.time() - t0:.1f}s; splits={runners[0].splits}")
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    for i in range(warmup):
        r = runners[i % nsets]
        r.quantize(sh)
        r.attend(sh)
    torch.cuda.synchronize()
    # whole-step timing
    t0 = time.perf_counter()
    for i in range(steps):
        r = runners[i % nsets]
        r.quantize(sh)
        r.attend(sh)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    # attention-call timing: HIP events on the launch stream around `steps` back-to-back calls
    # (Q codes already in place for the two-call form), averaged over the calls
    for i in range(nsets):
        runners[i].quantize(sh)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        runners[i % nsets].attend(sh)
    b.record(stream)
    torch.cuda.synchronize()
    kernel_ms = a.elapsed_time(b) / steps
    log(f"[bench] {label}: step {ms_step:.4f} ms, attention call {kernel_ms:.4f} ms")
    w = runners[0].w
    out = {"ms_per_step": ms_step, "kernel_ms": kernel_ms,
           "splits": runners[0].splits, "w": w}
    del runners
    torch.cuda.empty_cache()
    return out


def time_graph(make, entry, nsets, steps, label, fused=True):
    """The same steps captured in one HIP graph (one attention call per input set, the split-KV
    combine included) and replayed back to back: HIP events around the replays, per step."""
    import torch
    runners = [Runner(make(seed), entry, fused) for seed in range(nsets)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on a side stream, as capture requires
        for r in runners:
            r.quantize(side.cuda_stream)
            r.attend(side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for r in runners:
            r.quantize(cs)
            r.attend(cs)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // nsets)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / (reps * nsets)
    w = runners[0].w
    tb, _ = algo_bytes(w, fused)
    log(f"[bench] {label}: graph replay {ms:.4f} ms per step")
    out = {"workload": w.name, "graph_ms_per_step": round(ms, 4), "steps_per_graph": nsets,
           "splits": runners[0].splits, "kv_read_GBps": round(tb / (ms * 1e-3) / 1e9, 1),
           "hbm_frac": round(tb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del runners, g
    torch.cuda.empty_cache()
    return out


def time_cache_write(make, steps, label):
    """The KV-cache write of a workload's new tokens (bf16 K/V for every new token and kv head,
    stored at the tokens' slots in the workload's pools), timed with events around `steps`
    back-to-back calls that alternate between two input sets.  Algorithmic bytes: bf16 K and V
    read, E4M3 codes written, the slot ids read."""
    import numpy as np
    import torch
    import fp8_kv_cache_e4m3_amd as fa
    sets = []
    for seed in range(2):
        w = make(seed)
        T, H, d = w.total_q, w.num_kv_heads, w.head_dim
        ps = w.k_pool.shape[1]
        bt = w.block_table.cpu().numpy()
        slots = []
        for b, (L, ql) in enumerate(zip(w.seqlens_k_host, w.q_lens_host)):
            j = np.arange(L - ql, L)
            slots.append(bt[b][j // ps].astype(np.int64) * ps + j % ps)
        g = torch.Generator(device="cuda").manual_seed(seed)
        sets.append((torch.randn((T, H, d), generator=g, device="cuda").to(torch.bfloat16),
                     torch.randn((T, H, d), generator=g, device="cuda").to(torch.bfloat16),
                     torch.from_numpy(np.concatenate(slots)).cuda(), w.k_pool, w.v_pool, w.k_descale, w.v_descale))
    w = sets[0]
    T, H, d = w[0].shape
    nbytes = 2 * T * H * d * 2 + 2 * T * H * d + 8 * T
    for i in range(4):
        fa.fp8attn_cache_write(*sets[i % 2])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        fa.fp8attn_cache_write(*sets[i % 2])
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    log(f"[bench] {label}: {T} tokens x {H} kv heads x d{d}: {ms:.4f} ms")
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"KV-cache write, {T} new tokens x {H} kv heads x d{d}", "ms_per_call": round(ms, 4),
            "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes,
            "traffic": load_traffic(label) if label == "kv_write_swa_prefill" else None}


def time_quantize(shape, steps, label):
    """fp8attn_quantize_q on a bf16 Q of the given shape [tokens, heads, d] (values N(0,1),
    per-tensor descale amax/448), timed with events around `steps` back-to-back calls that
    alternate between two input sets.  Algorithmic bytes: bf16 in, E4M3 codes out."""
    import torch
    import fp8_kv_cache_e4m3_amd as fa
    sets = []
    for seed in range(2):
        g = torch.Generator(device="cuda").manual_seed(600 + seed)
        q = torch.randn(shape, generator=g, device="cuda").to(torch.bfloat16)
        ds = (q.float().abs().amax() / 448.0).reshape(1)
        out = torch.empty(shape, dtype=torch.uint8, device="cuda")
        sets.append((q, ds, out))
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def call(i):
        q, ds, out = sets[i % 2]
        st = fa.LIB.fp8attn_quantize_q(q.data_ptr(), q.shape[0], q.shape[1], q.shape[2], q.stride(0), q.stride(1),
                                       ds.data_ptr(), out.data_ptr(), sh)
        assert st == 0, fa.fp8attn_last_error()
    for i in range(4):
        call(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        call(i)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    n = sets[0][0].numel()
    nbytes = 3 * n
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] {label}: {tuple(shape)}: {ms:.4f} ms, {gbs:.0f} GB/s")
    del sets
    torch.cuda.empty_cache()
    return {"workload": f"quantize_q, bf16 Q {list(shape)}", "ms_per_call": round(ms, 4), "GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes}


def cpu_baseline(budget_s=15.0):
    """The CPU oracle, as is, on a bounded sample of the sliding-window decode workload: whole
    sequences (all 32 q heads) until the time budget is spent.  Rate = the same algorithmic bytes
    per second as the GPU value."""
    import numpy as np
    import threadpoolctl
    import workloads as wl
    from oracle.attention import default_scale, paged_attention, query_values
    import torch
    full = wl.swa_decode(device="cuda", seed=0)
    cores = 0
    for info in threadpoolctl.threadpool_info():
        cores = max(cores, int(info.get("num_threads", 0)))
    cores = cores or len(os.sched_getaffinity(0))
    qv, _ = query_values(full.q.cpu(), "e4m3", full.q_descale.cpu())
    bt = full.block_table.cpu().numpy()
    cu = full.cu_seqlens_q.cpu().numpy()
    sk = full.seqlens_k.cpu().numpy()
    hosts = []
    for b in range(full.batch):
        L = int(sk[b])
        lo = max(0, L - 1 - full.window + 1)
        pages = sorted(set(int(bt[b, n]) for n in range(lo // 64, (L - 1) // 64 + 1)))
        ids = torch.tensor(pages, dtype=torch.long, device="cuda")
        k = np.zeros(tuple(full.k_pool.shape), np.uint8)
        v = np.zeros(tuple(full.v_pool.shape), np.uint8)
        k[pages] = full.k_pool.index_select(0, ids).cpu().numpy()
        v[pages] = full.v_pool.index_select(0, ids).cpu().numpy()
        hosts.append((k, v, (L - lo) * full.num_kv_heads * 256 * 2 + 32 * 256 * 1 + 32 * 256 * 2))
    def run(budget):
        done, used, npass = 0, 0.0, 0
        while npass == 0 or used < budget:    # whole passes over the batch until the budget is spent
            for b in range(full.batch):
                k, v, nbytes = hosts[b]
                t0 = time.perf_counter()
                paged_attention(qv[cu[b]:cu[b + 1]], k, v, bt[b:b + 1], np.array([0, 1]), sk[b:b + 1],
                                full.num_kv_heads, default_scale(256), full.window, full.k_descale.cpu(),
                                full.v_descale.cpu())
                used += time.perf_counter() - t0
                done += nbytes
            npass += 1
        return done, used, npass

    done_bytes, t_used, passes = run(budget_s)
    # the same oracle with its BLAS held to one thread, on one pass over the batch, and on the tiny
    # workload (1 sequence, 1/1 heads, d64, 128 keys, 16 queries)
    with threadpoolctl.threadpool_limits(1):
        d1, t1, p1 = run(0.0)
        tiny = wl.tiny("e4m3")
        tq, _ = query_values(tiny.q, "e4m3", tiny.q_descale)
        tb = tiny.seqlens_k_host[0] * 64 * 2 + 16 * 64 * 3
        reps, t_tiny = 0, 0.0
        while reps == 0 or t_tiny < 1.0:
            t0 = time.perf_counter()
            paged_attention(tq, tiny.k_pool, tiny.v_pool, tiny.block_table, tiny.cu_seqlens_q, tiny.seqlens_k, 1,
                            default_scale(64), -1, tiny.k_descale, tiny.v_descale)
            t_tiny += time.perf_counter() - t0
            reps += 1
    del full
    torch.cuda.empty_cache()
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole sliding-window decode workload (32 sequences, all 32 q heads, 1024 "
                      f"visible keys each), {passes} passes, numpy fp64, {t_used:.1f} s",
            "one_thread": {"sliding_window_decode": {"value": d1 / t1 / 1e9, "unit": "GB/s", "seconds": round(t1, 2),
                                                     "sample": f"{p1} pass over the 32 sequences"},
                           "tiny": {"value": tb / (t_tiny / reps) / 1e9, "unit": "GB/s",
                                    "ms_per_call": round(t_tiny / reps * 1e3, 3),
                                    "sample": f"{reps} calls on the tiny d64 workload (128 keys, 16 queries)"}}}


def load_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel source; else None."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    try:
        d = json.load(open(COUNTERS_FILE))
    except Exception:
        return None
    ent = d.get("kernels", {}).get(kernel_key)
    if ent is None or ent.get("source") not in KERNEL_SOURCES:
        return None
    if ent.get("source_hash") != kernel_source_hash(ent["source"]):
        return None
    return ent.get("hbm_bytes_per_launch")


def decode_timeline(launches=5):
    """Phase stamps of the split-grid decode kernel on the sliding-window decode workload, from the
    timeline build of the library (python fp8_kv_cache_e4m3_amd/build.py --timeline): per block,
    its start, the first K/V unit computed by each wave, the end of each wave's stream, the merge
    and the output stores, in shader-clock ticks converted with the blocks' real-time clock
    (100 MHz).  Prints the distributions over the blocks of each measured launch as one JSON line."""
    import ctypes
    import numpy as np
    import torch
    import fp8_kv_cache_e4m3_amd as fa
    import workloads as wl

    path = os.path.join(os.path.dirname(fa.LIB_PATH), "libfp8attn_timeline.so")
    if not os.path.exists(path):
        sys.exit(f"{path} is missing: build it with python fp8_kv_cache_e4m3_amd/build.py --timeline")
    tl = ctypes.CDLL(path)
    tl.fp8attn_decode_paged.argtypes = fa.LIB.fp8attn_decode_paged.argtypes
    tl.fp8attn_decode_paged.restype = ctypes.c_int32
    tl.fp8attn_decode_timeline.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    tl.fp8attn_decode_timeline.restype = ctypes.c_int
    tl.fp8attn_decode_timeline_clear.restype = ctypes.c_int
    nblk, nslot = 4096, 16
    runners = [Runner(wl.swa_decode(device="cuda", seed=100 + s), "decode") for s in range(4)]
    w = runners[0].w
    assert runners[0].ws is None and runners[0].splits == 1
    grid = w.num_kv_heads * w.batch
    assert grid <= nblk
    sh = torch.cuda.current_stream().cuda_stream

    def launch(r):
        st = tl.fp8attn_decode_paged(ctypes.byref(r.args), 0, None, 0, None, None, sh)
        assert st == 0

    for i in range(20):
        launch(runners[i % 4])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(40):
        launch(runners[i % 4])
    b.record()
    torch.cuda.synchronize()
    ms_avg = a.elapsed_time(b) / 40
    buf = np.zeros(nblk * nslot, dtype=np.uint64)

    def q(x):
        return {k: round(float(np.percentile(x, p)), 2) for k, p in (("min", 0), ("p10", 10), ("p50", 50),
                                                                      ("p90", 90), ("max", 100))}
    res = []
    for i in range(launches):
        assert tl.fp8attn_decode_timeline_clear() == 0
        r = runners[i % 4]
        a.record()
        launch(r)
        b.record()
        torch.cuda.synchronize()
        assert tl.fp8attn_decode_timeline(buf.ctypes.data, buf.size) == 0
        t = buf.reshape(nblk, nslot)[:grid].astype(np.int64)
        assert (t[:, 0] > 0).all() and (t[:, 10] > 0).all(), "a block left no stamps"
        # s_memtime counts the shader clock of each XCD and is not aligned across XCDs; the 100 MHz
        # real-time clock is.  Absolute times: the block's real-time start plus its own shader-clock
        # offsets, converted with the ratio of the two clocks over the block.
        rt = (t[:, 14] - t[:, 13]).astype(np.float64) / 100.0            # us
        mt = (t[:, 10] - t[:, 0]).astype(np.float64)
        ok = rt > 0
        tick_per_us = float(np.median(mt[ok] / rt[ok]))
        start = (t[:, 13] - t[:, 13].min()) / 100.0
        at = start[:, None] + (t[:, :11] - t[:, :1]) / tick_per_us       # [blocks, 11] us
        first = at[:, 1:5].max(1)
        stream_end = at[:, 5:9].max(1)
        end = at[:, 10]
        xcc = (t[:, 12] & 0xF)
        span = float(end.max())
        # blocks streaming over time (between their first unit and the end of their stream)
        grid_us = np.arange(0.0, span, 0.5)
        active = ((first[None, :] <= grid_us[:, None]) & (stream_end[None, :] > grid_us[:, None])).sum(1)
        full = grid_us[active >= 0.9 * grid]
        res.append({
            "launch_ms_events": round(a.elapsed_time(b), 4),
            "span_us": round(span, 2),
            "shader_ticks_per_us": round(tick_per_us, 1),
            "block_start_us": q(start),
            "first_unit_done_us": q(first),
            "stream_end_us": q(stream_end),
            "block_end_us": q(end),
            "first_unit_after_start_us": q(first - start),
            "stream_us": q(stream_end - first),
            "wave_stream_end_spread_us": q(at[:, 5:9].max(1) - at[:, 5:9].min(1)),
            "merge_us": q(at[:, 9] - stream_end),
            "store_us": q(at[:, 10] - at[:, 9]),
            "ninety_pct_streaming_us": [round(float(full.min()), 1), round(float(full.max()), 1)] if len(full) else None,
            "blocks": int(grid),
            "blocks_per_xcc": {int(x): int((xcc == x).sum()) for x in np.unique(xcc)},
            "end_p50_by_xcc_us": {int(x): round(float(np.median(end[xcc == x])), 2) for x in np.unique(xcc)},
        })
    print(json.dumps({"workload": "sliding-window decode (B32, L U[1024, 8192], 32/16 heads, d256, W1024)",
                      "kernel": "decode_kernel (timeline build)", "avg_launch_ms_events": round(ms_avg, 4),
                      "launches": res}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="only the main workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--profile-pass", default=None,
                    choices=["swa_decode", "full_decode", "spec_verify", "swa_prefill", "full_prefill",
                             "kv_write_swa_prefill"],
                    help="short run for rocprofv3 counter passes: one workload plus a 1 GiB device copy")
    ap.add_argument("--split-q", action="store_true",
                    help="with --profile-pass on a bf16-Q workload: q_dtype BF16_SPLIT (QK^T and PV on the FP8 MFMA)")
    ap.add_argument("--separate-quantize", action="store_true",
                    help="quantize Q with its own call before attention (two launches per step) instead of "
                         "inside the attention kernel")
    ap.add_argument("--timeline", action="store_true",
                    help="phase stamps of the decode kernel per block (needs the timeline build of the library)")
    args = ap.parse_args()
    fused = not args.separate_quantize
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as wl
    import fp8_kv_cache_e4m3_amd  # noqa: F401  (fails loudly if the HIP library is missing)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.timeline:
        decode_timeline()
        return
    nsets = 4

    makers = {
        "swa_decode": (lambda s: wl.swa_decode(device="cuda", seed=100 + s), "decode"),
        "full_decode": (lambda s: wl.full_decode(device="cuda", seed=200 + s), "decode"),
        "spec_verify": (lambda s: wl.spec_verify(device="cuda", seed=300 + s), "decode"),
        "swa_prefill": (lambda s: wl.swa_prefill(device="cuda", seed=400 + s), "prefill"),
        "full_prefill": (lambda s: wl.full_prefill(device="cuda", seed=500 + s), "prefill"),
    }
    if args.profile_pass:
        # a plain copy of known size (1 GiB read + 1 GiB written) calibrates FETCH_SIZE / WRITE_SIZE
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        if args.profile_pass == "kv_write_swa_prefill":
            time_cache_write(lambda s: wl.swa_prefill(device="cuda", seed=400 + s), args.steps, "kv_write (profile pass)")
            return
        make, entry = makers[args.profile_pass]
        time_workload(make, entry, 2, args.steps, args.warmup, f"{args.profile_pass} (profile pass)", fused,
                      args.split_q)
        return

    main = time_workload(lambda s: wl.swa_decode(device="cuda", seed=100 + s), "decode", nsets, args.steps,
                         args.warmup, "sliding-window decode", fused)
    w = main["w"]
    total_b, kv_b = algo_bytes(w, fused)
    value = total_b / (main["ms_per_step"] * 1e-3) / 1e9
    achieved = total_b / (main["kernel_ms"] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic("decode_swa") if fused else None,
            "kernel": f"decode_kernel<{2 if fused else 1},256> (sliding-window decode, one split, "
                      f"{'bf16 Q quantized in-kernel' if fused else 'E4M3 Q codes'})",
            "algorithmic_bytes_per_launch": total_b}

    extra = {}
    if not args.no_extra:
        specs = [
            ("full_decode", lambda s: wl.full_decode(device="cuda", seed=200 + s), "decode", 4, "hbm", False),
            ("spec_verify", lambda s: wl.spec_verify(device="cuda", seed=300 + s), "decode", 2, "hbm", False),
            ("swa_prefill", lambda s: wl.swa_prefill(device="cuda", seed=400 + s), "prefill", 2, "mfma", False),
            # the same prefill on E4M3 codes quantized by a separate call: the attention kernel alone
            ("swa_prefill_codes", lambda s: wl.swa_prefill(device="cuda", seed=400 + s), "prefill", 2, "mfma", False),
            # the same bf16-Q workloads with QK^T on the FP8 MFMA (split Q)
            ("full_decode_split_q", lambda s: wl.full_decode(device="cuda", seed=200 + s), "decode", 4, "hbm", True),
            ("spec_verify_split_q", lambda s: wl.spec_verify(device="cuda", seed=300 + s), "decode", 2, "hbm", True),
            # d512 prefill (BF16 Q and split Q): the wide MFMA prefill kernel
            ("full_prefill", lambda s: wl.full_prefill(device="cuda", seed=500 + s), "prefill", 2, "mfma", False),
            ("full_prefill_split_q", lambda s: wl.full_prefill(device="cuda", seed=500 + s), "prefill", 2, "mfma",
             True),
        ]
        for name, make, entry, ns, bound, split in specs:
            fz = fused and not name.endswith("_codes")
            r = time_workload(make, entry, ns, max(5, args.steps // 5), 2, name, fz, split)
            ww = r["w"]
            tb, kvb = algo_bytes(ww, fz)
            fl = algo_flops(ww)
            e = {"workload": ww.name, "ms_per_step": round(r["ms_per_step"], 4),
                 "attention_ms": round(r["kernel_ms"], 4), "splits": r["splits"],
                 "kv_read_GBps": round(tb / (r["kernel_ms"] * 1e-3) / 1e9, 1),
                 "TFLOPs": round(fl / (r["kernel_ms"] * 1e-3) / 1e12, 2)}
            if not fz and ww.q_dtype == "e4m3":
                e["step"] = "quantize_q, then the attention call on E4M3 codes (attention_ms: that call alone)"
            # HBM bytes of the step's kernels (decode plus the partition's combine; both prefill instances)
            keys = {"full_decode": ["decode_full", "decode_full_combine"], "spec_verify": ["decode_spec"],
                    "spec_verify_split_q": ["decode_spec_split_q"],
                    "swa_prefill": ["prefill_swa", "prefill_swa_splitp"], "full_prefill": ["prefill_full"],
                    "full_prefill_split_q": ["prefill_full_split_q"]}.get(name)
            tr = [load_traffic(k) for k in keys] if keys else [None]
            e["traffic"] = sum(tr) if fz and all(t is not None for t in tr) else None
            mfma_peak = FP8_PEAK_TFLOPS if ww.q_dtype == "e4m3" or split else BF16_PEAK_TFLOPS
            if bound == "hbm":
                e["hbm_frac"] = round(e["kv_read_GBps"] / HBM_PEAK_GBS, 4)
                e["roofline"] = {"bound": "hbm", "achieved": e["kv_read_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": e["hbm_frac"], "traffic": e["traffic"], "algorithmic_bytes_per_launch": tb}
            else:
                e["mfma_frac"] = round(e["TFLOPs"] / mfma_peak, 4)
                e["roofline"] = {"bound": "mfma", "achieved": e["TFLOPs"], "peak": mfma_peak, "unit": "TFLOP/s",
                                 "frac": e["mfma_frac"], "traffic": e["traffic"], "algorithmic_flops_per_launch": fl}
            if name.startswith("spec_verify"):
                # the shared prefix need not come from HBM once per sequence: the bound of a kernel that
                # reads each distinct page once, or of its MFMA work, whichever is longer
                ub = unique_kv_bytes(ww)
                hbm_ms = ub / (HBM_PEAK_GBS * 1e9) * 1e3
                mfma_ms = fl / (mfma_peak * 1e12) * 1e3
                e["cache_aware"] = {"unique_kv_bytes": ub, "hbm_bound_ms": round(hbm_ms, 4),
                                    "mfma_bound_ms": round(mfma_ms, 4), "bound_ms": round(max(hbm_ms, mfma_ms), 4),
                                    "frac": round(max(hbm_ms, mfma_ms) / r["kernel_ms"], 4)}
            extra[name] = e
        for name, make, ns in [("swa_decode_graph", lambda s: wl.swa_decode(device="cuda", seed=100 + s), nsets),
                               ("full_decode_graph", lambda s: wl.full_decode(device="cuda", seed=200 + s), 4)]:
            extra[name] = time_graph(make, "decode", ns, max(8, args.steps), name, fused)
        for name, make in [("kv_write_swa_prefill", lambda s: wl.swa_prefill(device="cuda", seed=400 + s)),
                           ("kv_write_swa_decode", lambda s: wl.swa_decode(device="cuda", seed=100 + s))]:
            extra[name] = time_cache_write(make, max(5, args.steps // 5), name)
        # the stand-alone Q quantization (the steps above quantize inside the attention kernels)
        extra["quantize_q_swa_prefill"] = time_quantize((65536, 32, 256), max(5, args.steps // 5),
                                                        "quantize_q_swa_prefill")

    cpu = None
    if not args.no_cpu:
        try:
            cpu = cpu_baseline()
        except Exception as ex:  # the baseline must not hide the GPU result
            log(f"[bench] cpu baseline failed: {ex!r}")

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(main["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e4m3", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "window": w.window, "kv_len": "uniform[1024,8192]", "page": 64,
                   "input_sets": nsets, "splits": main["splits"],
                   "step": "decode_paged (bf16 Q quantized in-kernel)" if fused else "quantize_q + decode_paged"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
