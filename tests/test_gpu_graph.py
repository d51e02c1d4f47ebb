"""Decode captured once in a HIP graph and replayed with changing inputs.

The decode call plans its split count from host maxima only (batch, q_len bound, key-length
bound) and never reads device memory to plan, so a caller can capture it, together with the
split-KV combine, once and replay it while the sequence lengths, block tables and queries
change in place (vLLM PR #60372, Claims: an automatic split count that also holds under CUDA
graphs).  Every replay must equal an eager call with the same host maxima bit for bit, and
meet the oracle bar.  Eager work and synchronizations run between the replays.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from helpers import compare, log, oracle_run

pytestmark = pytest.mark.gpu


def _fa():
    import fp8_kv_cache_e4m3_amd as fa
    return fa


@pytest.mark.parametrize("q_dtype,d,hq,hkv,window,q_len,fused,cap", [
    ("e4m3", 256, 32, 16, 1024, 1, True, 3000),    # sliding-window layer, bf16 Q quantized in-kernel
    ("bf16", 512, 32, 4, -1, 1, False, 3000),      # full-attention layer, split plan
    ("bf16", 512, 32, 4, -1, 1, False, 6000),      # full-attention layer, balanced partition
    ("bf16", 512, 32, 4, -1, 4, False, 3000),      # spec-decode verify (4 query tokens)
])
def test_graph_replay_with_changing_lengths(q_dtype, d, hq, hkv, window, q_len, fused, cap):
    fa = _fa()
    B = 4                                    # cap: the key-length bound fixed at capture
    base = wl.custom(q_dtype, d, hq, hkv, window, [cap] * B, [q_len] * B, seed=61)
    dev = torch.device("cuda")
    wd = base.to(dev)
    if q_dtype == "e4m3" and not fused:
        raise AssertionError("e4m3 cases run with in-kernel quantization here")
    qd = wd.q_descale if q_dtype == "e4m3" else None
    q_s = wd.q.clone()
    sk_s = wd.seqlens_k.clone()
    bt_s = wd.block_table.clone()
    T = base.total_q
    out = torch.empty((T, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, hq), dtype=torch.float32, device=dev)

    def call(o, l, ws=None):
        return fa.fp8attn_decode_paged(q_s, wd.k_pool, wd.v_pool, bt_s, wd.cu_seqlens_q, sk_s, q_len, cap,
                                       q_descale=qd, k_descale=wd.k_descale, v_descale=wd.v_descale,
                                       window=window, out=o, lse=l, workspace=ws, quantize_q=fused)

    # workspace sized once, outside the capture
    a = fa.make_args(q_s, wd.k_pool, wd.v_pool, bt_s, wd.cu_seqlens_q, sk_s, q_len, cap, qd, wd.k_descale,
                     wd.v_descale, 0.0, window, True, out, lse, quantize_q=fused)
    need, splits = fa.decode_workspace_size(a, 0)
    assert splits != 1, "the case should exercise the combine inside the graph"
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):             # warm-up on the capture stream
        call(out, lse, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _, _, used = call(out, lse, ws)
    assert used == splits
    log(f"[case] graph {q_dtype} d{d} W{window} q_len {q_len}: {splits} splits captured")

    rng = np.random.default_rng(5)
    npages = base.k_pool.shape[0]
    max_pages = base.block_table.shape[1]
    for rep in range(4):
        # new lengths (one at the bound, one short), new page assignment, new queries
        lens = rng.integers(q_len, cap + 1, size=B)
        lens[0] = cap
        lens[1] = max(q_len, int(rng.integers(1, 80)))
        bt = rng.permutation(npages)[: B * max_pages].reshape(B, max_pages).astype(np.int32)
        gq = torch.Generator().manual_seed(100 + rep)
        qh = torch.randn(tuple(base.q.shape), generator=gq).to(torch.bfloat16)
        sk_s.copy_(torch.from_numpy(lens.astype(np.int32)))
        bt_s.copy_(torch.from_numpy(bt))
        q_s.copy_(qh)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = out.clone(), lse.clone()
        # eager call on the same inputs and the same host maxima
        o_e, l_e, s_e = call(torch.empty_like(out), torch.empty_like(lse))
        torch.cuda.synchronize()
        assert s_e == splits
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), f"replay {rep} differs from eager"
        # oracle on the host copies of the same inputs
        w2 = wl.Workload(**{**base.__dict__})
        w2.q = qh
        w2.block_table = torch.from_numpy(bt)
        w2.seqlens_k = torch.from_numpy(lens.astype(np.int32))
        w2.seqlens_k_host = [int(x) for x in lens]
        if q_dtype == "e4m3":   # the static q descale of the capture stays in force
            w2.q_descale = base.q_descale
        o_ref, l_ref, _ = oracle_run(w2)
        compare(o_g.float().cpu().numpy().astype(np.float64), o_ref,
                l_g.cpu().numpy().astype(np.float64), l_ref, label=f"graph replay {rep} lens={lens.tolist()}")
