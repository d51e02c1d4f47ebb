"""Planted mistakes in the CPU oracle, used to show that its pins catch them.

Each mutation is one textual edit of one oracle source file: a plausible slip (a mask bound off
by one, a dropped descale, a log2 in place of ln, ...).  ``make_mutated_oracle(name)`` copies the
``oracle`` package into a temporary directory with that edit applied and returns the directory,
which ``tests/conftest.py`` puts first on ``sys.path`` when ``FP8ATTN_ORACLE_MUTATION`` names a
mutation.  ``tests/test_oracle_mutations.py`` then runs the oracle's own pin tests against each
mutated copy in a subprocess and requires at least one of them to fail.  Mutations are applied on
the CPU only; nothing here touches the GPU library.
"""
from __future__ import annotations

import os
import shutil
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (file under oracle/, text to replace (must occur exactly once), replacement)
MUTATIONS = {
    "causal_bound": ("attention.py", "    m = j <= p\n", "    m = j < p\n"),
    "window_bound": ("attention.py", "        m &= j > p - window\n", "        m &= j >= p - window\n"),
    "gqa_map_interleaved": ("attention.py", "                Q = q_vals[ct, h * g:(h + 1) * g, :]",
                            "                Q = q_vals[ct, h::hkv, :]"),
    "k_descale_dropped": ("attention.py", "                K = E4M3_TABLE[kc[:, h, :]] * kd",
                          "                K = E4M3_TABLE[kc[:, h, :]] * 1.0"),
    "block_table_ignored": ("attention.py",
                            "    pages = np.asarray(_np(block_table_row), dtype=np.int64)[positions // page_size]",
                            "    pages = positions // page_size"),
    "lse_in_log2": ("attention.py", "(m_safe + np.log(np.where(empty, 1.0, l)))",
                    "(m_safe + np.log2(np.where(empty, 1.0, l)))"),
    "queries_at_sequence_start": ("attention.py", "            pos = L - ql + (ct - t0)",
                                  "            pos = (ct - t0)"),
    "combine_weight_sign": ("attention.py",
                            "np.exp(np.where(fin, pl, 0.0) - np.where(np.isfinite(M), M, 0.0))",
                            "np.exp(np.where(np.isfinite(M), M, 0.0) - np.where(fin, pl, 0.0))"),
    "ties_to_odd": ("e4m3.py", "((d_hi == d_lo) & (hi % 2 == 0))", "((d_hi == d_lo) & (hi % 2 == 1))"),
    # (dividing in fp64 and rounding the quotient to fp32 would be no mistake: for binary32
    # operands that is the correctly rounded fp32 quotient; the slip is to skip the rounding)
    "quotient_not_rounded_to_fp32": ("e4m3.py", "        y = (x32 / d32).astype(np.float32)",
                                     "        y = x32.astype(np.float64) / np.float64(d32)"),
    "subnormal_exponent": ("e4m3.py", "        return s * (m / 8.0) * 2.0 ** -6", "        return s * (m / 8.0) * 2.0 ** -7"),
    "saturation_to_nan": ("e4m3.py", "    mag = np.where(a_f >= E4M3_MAX, 0x7E, mag)",
                          "    mag = np.where(a_f >= E4M3_MAX, 0x7F, mag)"),
    "nan_sign_from_platform": ("e4m3.py", "np.signbit(x32) ^ np.signbit(d32)", "np.signbit(y)"),
    "default_scale_one_over_d": ("attention.py", "    return 1.0 / math.sqrt(head_dim)", "    return 1.0 / head_dim"),
    "descale_per_head_transposed": ("attention.py", "    return float(np.float32(a[b, h]))",
                                    "    return float(np.float32(a.reshape(-1)[h * a.shape[0] + b]))"),
    "cache_page_slot_swapped": ("cache_write.py", "        page, pos = divmod(slot, page_size)",
                                "        pos, page = divmod(slot, page_size)"),
    "cache_descale_swapped": ("cache_write.py", "        vc[page, pos] = quantize_e4m3(v_new[t], v_descale)",
                              "        vc[page, pos] = quantize_e4m3(v_new[t], k_descale)"),
}


def make_mutated_oracle(name: str) -> str:
    """Directory holding a copy of the oracle package with mutation ``name`` applied ("none":
    an unmodified copy, which checks the harness itself)."""
    dst = tempfile.mkdtemp(prefix="oracle_mut_")
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so", "*.o"))
    if name != "none":
        fname, old, new = MUTATIONS[name]
        path = os.path.join(dst, "oracle", fname)
        src = open(path).read()
        assert src.count(old) == 1, f"mutation {name}: the text to replace occurs {src.count(old)} times"
        open(path, "w").write(src.replace(old, new))
    return dst
