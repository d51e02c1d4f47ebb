"""Pins of the oracle's paged KV-cache write (CPU only).

Independent anchors:
* the attention oracle's page gather (``oracle.attention.gather_pages``), a separate function
  that reads the cache the way the attention call does: what the write stores at a token's slot
  must come back at that token's position;
* the ``torch.float8_e4m3fn`` cast (the dtype the pages name for the cache, prhub digest of vLLM
  PR #48666, Key code), on in-range values where it agrees with the saturating rule;
* exact round trips of values that are E4M3 values times the descale.
"""
import numpy as np
import torch

from oracle.attention import gather_pages
from oracle.cache_write import cache_write, slots_for_new_tokens
from oracle.e4m3 import E4M3_TABLE, dequantize_e4m3


def _pools(rng, pages, ps, hkv, d):
    k = rng.integers(0, 256, size=(pages, ps, hkv, d), dtype=np.uint8)
    v = rng.integers(0, 256, size=(pages, ps, hkv, d), dtype=np.uint8)
    return k, v


def test_written_codes_match_torch_cast_and_nothing_else_changes():
    rng = np.random.default_rng(0)
    pages, ps, hkv, d = 5, 64, 2, 16
    kc, vc = _pools(rng, pages, ps, hkv, d)
    T = 7
    k_new = rng.normal(size=(T, hkv, d)).astype(np.float32) * 3
    v_new = rng.normal(size=(T, hkv, d)).astype(np.float32) * 3
    kd, vd = np.float32(0.0123), np.float32(0.5)
    slots = np.array([3, 64 + 5, 4 * 64 + 63, -1, 2 * 64, 5 * 64, 130], dtype=np.int64)   # -1 and 320 skip
    k2, v2 = cache_write(k_new, v_new, slots, kc, vc, kd, vd)
    def ref(x, ds):
        # torch's cast rounds to nearest even but does not saturate: out-of-range quotients are
        # checked against the saturated code instead
        y = torch.from_numpy(x) / torch.tensor(ds)
        c = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        big = (y.abs() >= 448).numpy()
        c[big] = np.where(np.signbit(y.numpy()[big]), 0xFE, 0x7E)
        return c
    ref_k, ref_v = ref(k_new, kd), ref(v_new, vd)
    assert (np.abs(k_new / kd) >= 448).any()   # the saturation branch is exercised
    touched = np.zeros((pages, ps), dtype=bool)
    for t, s in enumerate(slots):
        if 0 <= s < pages * ps:
            p, o = divmod(int(s), ps)
            assert np.array_equal(k2[p, o], ref_k[t]) and np.array_equal(v2[p, o], ref_v[t]), t
            touched[p, o] = True
    assert np.array_equal(k2[~touched], kc[~touched]) and np.array_equal(v2[~touched], vc[~touched])
    assert touched.sum() == 5


def test_round_trip_through_the_attention_gather():
    # new tokens of each sequence are its last q_len positions; the attention oracle's gather must
    # return the written codes at exactly those positions, for any page placement
    rng = np.random.default_rng(1)
    ps, hkv, d, pages = 64, 3, 32, 12
    seqlens, qlens = np.array([130, 64, 5]), np.array([3, 64, 5])
    bt = np.array(rng.permutation(pages)[:9].reshape(3, 3), dtype=np.int32)
    slots = slots_for_new_tokens(bt, seqlens, qlens, ps)
    assert len(slots) == qlens.sum() and len(set(slots.tolist())) == len(slots)
    # values that are E4M3 values times the descale survive the round trip exactly
    kd, vd = np.float32(0.25), np.float32(2.0)
    codes = rng.integers(0, 126, size=(len(slots), hkv, d))          # finite non-negative codes
    signs = np.where(rng.random(size=codes.shape) < 0.5, -1.0, 1.0)
    k_new = (E4M3_TABLE[codes] * signs * kd).astype(np.float32)
    v_new = (E4M3_TABLE[codes[::-1]] * signs * vd).astype(np.float32)
    kc, vc = _pools(rng, pages, ps, hkv, d)
    k2, v2 = cache_write(k_new, v_new, slots, kc, vc, kd, vd)
    t0 = 0
    for b in range(3):
        pos = np.arange(seqlens[b] - qlens[b], seqlens[b])
        gk = gather_pages(k2, bt[b], pos, ps)   # [n, hkv, d] codes
        gv = gather_pages(v2, bt[b], pos, ps)
        n = len(pos)
        np.testing.assert_array_equal(dequantize_e4m3(gk, kd), k_new[t0:t0 + n].astype(np.float64))
        np.testing.assert_array_equal(dequantize_e4m3(gv, vd), v_new[t0:t0 + n].astype(np.float64))
        t0 += n


def test_saturation_nan_and_last_write_wins():
    pages, ps, hkv, d = 2, 64, 1, 8
    kc = np.zeros((pages, ps, hkv, d), dtype=np.uint8)
    vc = np.zeros_like(kc)
    x = np.array([[[1e6, -1e6, np.inf, -np.inf, np.nan, -np.nan, 448.0, -0.0]]], dtype=np.float32)
    k2, v2 = cache_write(x, x, [65], kc, vc, 1.0, 1.0)
    assert k2[1, 1, 0].tolist() == [0x7E, 0xFE, 0x7E, 0xFE, 0x7F, 0xFF, 0x7E, 0x80]
    assert np.array_equal(v2, k2)
    # a repeated slot: the later token's values remain
    y = np.ones((2, hkv, d), dtype=np.float32)
    y[1] *= 2
    k3, _ = cache_write(y, y, [7, 7], kc, vc)
    assert np.all(k3[0, 7] == 0x40)    # 2.0 = 0x40 in E4M3
