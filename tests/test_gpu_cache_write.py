"""GPU parity of the paged KV-cache write (fp8attn_cache_write) against the CPU oracle.

Bar: bit-exact.  Every cache byte after the call equals the oracle's (written entries and the
untouched rest), on random bf16 inputs that include NaN, infinities, values far past the E4M3
range and values below its smallest subnormal, with padding (-1) and out-of-range slots.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from helpers import compare, gpu_run, log, oracle_run
from oracle.cache_write import cache_write, slots_for_new_tokens
from oracle.e4m3 import quantize_e4m3

pytestmark = pytest.mark.gpu


def _fa():
    import fp8_kv_cache_e4m3_amd as fa
    return fa


def _inputs(T, H, d, pages, ps, seed, fused_qkv=False):
    g = torch.Generator().manual_seed(seed)
    if fused_qkv:   # k and v as views of one [T, 3, H, d] tensor (token stride 3 H d)
        qkv = (torch.randn((T, 3, H, d), generator=g) * 3).to(torch.bfloat16)
        k, v = qkv[:, 1], qkv[:, 2]
    else:
        k = (torch.randn((T, H, d), generator=g) * 3).to(torch.bfloat16)
        v = (torch.randn((T, H, d), generator=g) * 0.01).to(torch.bfloat16)
    # special values in the first token's first head
    sp = torch.tensor([float("nan"), -float("nan"), float("inf"), -float("inf"), 1e30, -1e30, 1e-30, -0.0],
                      dtype=torch.bfloat16)
    k[0, 0, :8] = sp
    v[0, 0, 8:16] = sp
    kc = torch.randint(0, 256, (pages, ps, H, d), generator=g, dtype=torch.uint8)
    vc = torch.randint(0, 256, (pages, ps, H, d), generator=g, dtype=torch.uint8)
    nslots = pages * ps
    perm = torch.randperm(nslots, generator=g)[:T].to(torch.int64)
    perm[1 % T] = -1                      # padding token
    if T > 3:
        perm[3] = nslots + 5              # out of range: skipped
    return k, v, perm, kc, vc


@pytest.mark.parametrize("T,H,d,pages,ps,fused", [
    (37, 2, 64, 3, 64, False),
    (100, 16, 256, 4, 64, False),
    (20, 4, 512, 2, 128, True),
    (2, 1, 16, 1, 64, False),
])
def test_cache_write_bit_exact(T, H, d, pages, ps, fused):
    fa = _fa()
    log(f"[case] cache_write T={T} H={H} d={d} pages={pages} ps={ps} fused={fused}")
    k, v, slots, kc, vc = _inputs(T, H, d, pages, ps, seed=T * 31 + d, fused_qkv=fused)
    kd, vd = np.float32(0.0123), np.float32(0.0009765625)
    ref_k, ref_v = cache_write(k.float().numpy(), v.float().numpy(), slots.numpy(), kc.numpy(), vc.numpy(), kd, vd)
    kcg, vcg = kc.cuda(), vc.cuda()
    fa.fp8attn_cache_write(k.cuda(), v.cuda(), slots.cuda(), kcg, vcg,
                           torch.tensor([kd], device="cuda"), torch.tensor([vd], device="cuda"))
    torch.cuda.synchronize()
    gk, gv = kcg.cpu().numpy(), vcg.cpu().numpy()
    assert np.array_equal(gk, ref_k), f"K: {np.count_nonzero(gk != ref_k)} bytes differ"
    assert np.array_equal(gv, ref_v), f"V: {np.count_nonzero(gv != ref_v)} bytes differ"


def test_cache_write_zero_descale():
    """An all-zero K/V tensor gets descale amax / 448 = 0: every nonzero value saturates, +-0 and
    NaN give NaN quotients (0x7F | sign of x XOR sign of the descale); every byte as the oracle."""
    fa = _fa()
    T, H, d, pages, ps = 40, 2, 64, 2, 64
    k, v, slots, kc, vc = _inputs(T, H, d, pages, ps, seed=77)
    k[2] = 0.0
    k[4, 0, :16] = -0.0
    ref_k, ref_v = cache_write(k.float().numpy(), v.float().numpy(), slots.numpy(), kc.numpy(), vc.numpy(),
                               np.float32(0.0), np.float32(0.0))
    kcg, vcg = kc.cuda(), vc.cuda()
    zero = torch.zeros(1, device="cuda")
    fa.fp8attn_cache_write(k.cuda(), v.cuda(), slots.cuda(), kcg, vcg, zero, zero)
    torch.cuda.synchronize()
    gk, gv = kcg.cpu().numpy(), vcg.cpu().numpy()
    assert np.array_equal(gk, ref_k), f"K: {np.count_nonzero(gk != ref_k)} bytes differ"
    assert np.array_equal(gv, ref_v), f"V: {np.count_nonzero(gv != ref_v)} bytes differ"


def test_cache_write_strided_views_and_null_descales():
    fa = _fa()
    T, H, d, pages, ps = 50, 4, 256, 2, 64
    k, v, slots, kc, vc = _inputs(T, H, d, pages, ps, seed=5, fused_qkv=True)
    kg, vg = k.cuda(), v.cuda()        # keep the fused layout on the device
    base = torch.empty((T, 3, H, d), dtype=torch.bfloat16, device="cuda")
    base[:, 1] = kg
    base[:, 2] = vg
    kcg, vcg = kc.cuda(), vc.cuda()
    fa.fp8attn_cache_write(base[:, 1], base[:, 2], slots.cuda(), kcg, vcg)
    torch.cuda.synchronize()
    ref_k, ref_v = cache_write(k.float().numpy(), v.float().numpy(), slots.numpy(), kc.numpy(), vc.numpy())
    assert np.array_equal(kcg.cpu().numpy(), ref_k) and np.array_equal(vcg.cpu().numpy(), ref_v)


def test_cache_write_prefill_size_sampled():
    # the sliding-window prefill's new K/V (8 x 8192 tokens, 16 kv heads, d256) into its pool
    fa = _fa()
    w = wl.swa_prefill(device="cuda")
    T, H, d = w.total_q, w.num_kv_heads, w.head_dim
    ps = w.k_pool.shape[1]
    slots = torch.from_numpy(slots_for_new_tokens(w.block_table.cpu().numpy(), w.seqlens_k_host,
                                                  w.q_lens_host, ps)).cuda()
    g = torch.Generator(device="cuda").manual_seed(9)
    k = torch.randn((T, H, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((T, H, d), generator=g, device="cuda").to(torch.bfloat16)
    kd = torch.tensor([0.011], device="cuda")
    vd = torch.tensor([0.009], device="cuda")
    kc, vc = w.k_pool.view(torch.uint8).clone(), w.v_pool.view(torch.uint8).clone()
    log(f"[case] cache_write prefill-size T={T} pool={tuple(kc.shape)}")
    fa.fp8attn_cache_write(k, v, slots, kc, vc, kd, vd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    toks = rng.choice(T, size=64, replace=False)
    s_host = slots.cpu().numpy()
    for t in toks:
        page, pos = divmod(int(s_host[t]), ps)
        want_k = quantize_e4m3(k[t].float().cpu().numpy(), np.float32(0.011))
        want_v = quantize_e4m3(v[t].float().cpu().numpy(), np.float32(0.009))
        assert np.array_equal(kc[page, pos].cpu().numpy(), want_k), t
        assert np.array_equal(vc[page, pos].cpu().numpy(), want_v), t
    # a page no sequence uses is untouched
    used = set((s_host // ps).tolist())
    free = [p for p in range(kc.shape[0]) if p not in used]
    if free:
        assert torch.equal(kc[free[0]], w.k_pool.view(torch.uint8)[free[0]])


def test_write_then_decode_matches_oracle():
    # the step before the path: new tokens are written with the cache write, then attended to
    fa = _fa()
    w = wl.custom("e4m3", 256, 8, 2, 300, [700, 65, 1500], [4, 16, 1], seed=41)
    ps = w.k_pool.shape[1]
    slots = slots_for_new_tokens(w.block_table.numpy(), w.seqlens_k_host, w.q_lens_host, ps)
    g = torch.Generator().manual_seed(12)
    k = torch.randn((w.total_q, w.num_kv_heads, w.head_dim), generator=g).to(torch.bfloat16)
    v = torch.randn((w.total_q, w.num_kv_heads, w.head_dim), generator=g).to(torch.bfloat16)
    kd, vd = float(w.k_descale[0]), float(w.v_descale[0])
    ref_k, ref_v = cache_write(k.float().numpy(), v.float().numpy(), slots, w.k_pool.view(torch.uint8).numpy(),
                               w.v_pool.view(torch.uint8).numpy(), np.float32(kd), np.float32(vd))
    kcg = w.k_pool.view(torch.uint8).clone().cuda()
    vcg = w.v_pool.view(torch.uint8).clone().cuda()
    fa.fp8attn_cache_write(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), kcg, vcg,
                           w.k_descale.cuda(), w.v_descale.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(kcg.cpu().numpy(), ref_k) and np.array_equal(vcg.cpu().numpy(), ref_v)
    w2 = wl.Workload(**{**w.__dict__})
    w2.k_pool = torch.from_numpy(ref_k).view(w.k_pool.dtype)
    w2.v_pool = torch.from_numpy(ref_v).view(w.v_pool.dtype)
    o_ref, l_ref, _ = oracle_run(w2)
    o, l, _, s = gpu_run(w2, "decode", fused_q=True)
    compare(o, o_ref, l, l_ref, label=f"write+decode S={s}")
