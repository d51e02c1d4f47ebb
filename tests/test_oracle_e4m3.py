"""Pins of the oracle's E4M3 decode table and quantizer (CPU only).

Independent anchors:
* the OCP 8-bit floating point specification (E4M3 variant): max 448 at 0x7E,
  NaN at 0x7F/0xFF, no infinity, subnormals m/8 * 2^-6;
* the ``torch.float8_e4m3fn`` dtype the pages name for the cache (prhub digest
  of vLLM PR #48666, Key code).  Its cast rounds to nearest even but does not
  saturate, so it is compared on the in-range subset;
* hand-worked ties and saturation cases (tests/golden/e4m3_cases.txt).
"""
import os

import numpy as np
import pytest
import torch

from oracle.e4m3 import E4M3_TABLE, dequantize_e4m3, descale_from_amax, e4m3_decode, quantize_e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_table_matches_torch_float8_e4m3fn():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(t) & np.isnan(E4M3_TABLE)
    assert np.all(both_nan | (t == E4M3_TABLE))
    assert np.count_nonzero(np.isnan(E4M3_TABLE)) == 2


def test_table_spec_values():
    # OCP FP8 E4M3: bias 7, no infinities, 0x7E is the largest finite magnitude.
    assert e4m3_decode(0x7E) == 448.0
    assert e4m3_decode(0xFE) == -448.0
    assert e4m3_decode(0x38) == 1.0
    assert e4m3_decode(0x08) == 2.0 ** -6          # smallest normal
    assert e4m3_decode(0x01) == 2.0 ** -9          # smallest subnormal
    assert e4m3_decode(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert e4m3_decode(0x80) == 0.0 and np.signbit(e4m3_decode(0x80))
    assert np.isnan(e4m3_decode(0x7F)) and np.isnan(e4m3_decode(0xFF))
    pos = E4M3_TABLE[:127]
    assert np.all(np.diff(pos) > 0), "finite non-negative codes must be strictly increasing"
    assert np.array_equal(E4M3_TABLE[128:255], -E4M3_TABLE[0:127])


def _all_bf16_as_f32():
    u = np.arange(65536, dtype=np.uint32) << 16
    return u.view(np.float32)


@pytest.mark.parametrize("descale", [1.0, 2.0 ** -6, 0.0100097656, 0.3, 7.25, 1.0 / 448])
def test_quantizer_matches_torch_in_range(descale):
    x = _all_bf16_as_f32()
    codes = quantize_e4m3(x, descale)
    y = torch.from_numpy(x.copy()) / torch.tensor(descale, dtype=torch.float32)
    ok = torch.isfinite(y) & (y.abs() < 448)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    okn = ok.numpy()
    assert okn.sum() > 1000
    mism = np.nonzero(codes[okn] != ref[okn])[0]
    assert mism.size == 0, f"{mism.size} codes differ from torch, first input {x[okn][mism[0]]!r}"


def test_quantizer_random_descales_vs_torch():
    rng = np.random.default_rng(11)
    x = _all_bf16_as_f32()
    for ds in rng.uniform(1e-3, 4.0, size=12).astype(np.float32):
        codes = quantize_e4m3(x, ds)
        y = torch.from_numpy(x.copy()) / torch.tensor(float(ds), dtype=torch.float32)
        ok = (torch.isfinite(y) & (y.abs() < 448)).numpy()
        ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(codes[ok], ref[ok])


def test_quantizer_saturation_and_nan():
    x = np.array([448.0, 449.0, 464.0, 465.0, 480.0, 1e30, np.inf, -448.0, -500.0, -np.inf],
                 dtype=np.float32)
    assert list(quantize_e4m3(x, 1.0)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0xFE]
    nan = np.array([np.nan, -np.nan], dtype=np.float32)
    nan[1] = -np.abs(nan[1])
    assert list(quantize_e4m3(nan, 1.0)) == [0x7F, 0xFF]
    # descale pushes an in-range value out of range
    assert quantize_e4m3(np.float32(2.0), 1.0 / 256)[()] == 0x7E


def test_quantizer_golden_cases():
    path = os.path.join(GOLDEN, "e4m3_cases.txt")
    n = 0
    with open(path) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            xs, ds, code = line.split()
            got = int(quantize_e4m3(np.float32(float.fromhex(xs)), np.float32(float.fromhex(ds))))
            assert got == int(code, 16), (xs, ds, hex(got), code)
            n += 1
    assert n >= 20


def test_quantizer_round_trip_and_neg_zero():
    finite = [c for c in range(256) if not np.isnan(E4M3_TABLE[c])]
    vals = E4M3_TABLE[finite].astype(np.float32)
    assert list(quantize_e4m3(vals, 1.0)) == finite
    assert quantize_e4m3(np.float32(-0.0), 1.0)[()] == 0x80


def test_quantizer_divides_in_fp32():
    # y must be the fp32 quotient: 1/3 in fp32 is 0.3333333432674408, which must quantize as that value.
    x = np.float32(1.0)
    ds = np.float32(3.0)
    y32 = np.float32(x / ds)
    assert quantize_e4m3(x, ds)[()] == quantize_e4m3(y32, 1.0)[()]
    # a case where the fp32 quotient sits exactly on an E4M3 tie while the exact quotient does not:
    # find one by search and check the oracle follows the fp32 value (RNE to even)
    rng = np.random.default_rng(5)
    found = 0
    for _ in range(200000):
        code = int(rng.integers(8, 0x7D))
        mid = (E4M3_TABLE[code] + E4M3_TABLE[code + 1]) / 2  # exact tie value (representable in fp32)
        ds = np.float32(rng.uniform(0.01, 2.0))
        x = np.float32(mid * float(ds))
        if np.float32(x / ds) == np.float32(mid) and float(x) / float(ds) != mid:
            even = code if code % 2 == 0 else code + 1
            assert quantize_e4m3(x, ds)[()] == even
            found += 1
            if found > 20:
                break
    assert found > 0


def test_dequantize_and_descale_recipe():
    x = np.array([0.5, -3.0, 2.25], dtype=np.float32)
    ds = descale_from_amax(x)
    assert ds == np.float32(np.float32(3.0) / np.float32(448.0))
    codes = quantize_e4m3(x, ds)
    assert codes[1] == 0xFE                                # amax maps to -448
    assert dequantize_e4m3(codes[1:2], ds)[0] == -448.0 * float(ds)


def test_two_e4m3_terms_hold_every_bf16_value():
    """Why split Q (hi + lo/16 on the FP8 MFMA) gives the BF16 product: for every finite bf16
    value x and the power-of-two row scale 2^e that brings the row's largest magnitude into
    (224, 448], hi = E4M3(x 2^e) and lo = E4M3(16 (x 2^e - hi)) satisfy hi + lo/16 == x 2^e
    exactly whenever |x 2^e| >= 2^-6 (E4M3's smallest normal): x has 8 significant bits, hi
    keeps the top 4, the residual has at most 4.  Below that the error stays under 2^-13."""
    import torch
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    with np.errstate(invalid="ignore"):
        x = bits.float().numpy().astype(np.float64)
    x = x[np.isfinite(x) & (x != 0)]
    for amax_exp in (-100, -3, 0, 7, 60, 127):            # rows of very different magnitudes
        amax = 2.0 ** amax_exp * 1.7
        e = int(np.floor(np.log2(448.0 / amax)))
        row = x[np.abs(x) <= amax]
        xs = (row * 2.0 ** e).astype(np.float32)           # exact: a power-of-two scale
        hi = quantize_e4m3(xs)
        r = (xs.astype(np.float64) - dequantize_e4m3(hi)) * 16.0
        assert np.all(r.astype(np.float32) == r)           # the residual is an exact fp32 value
        lo = quantize_e4m3(r.astype(np.float32))
        back = dequantize_e4m3(hi) + dequantize_e4m3(lo) / 16.0
        normal = np.abs(xs) >= 2.0 ** -6
        assert np.all(back[normal] == xs[normal]), amax_exp
        assert np.max(np.abs(back - xs)) <= 2.0 ** -13
