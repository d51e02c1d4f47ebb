"""C-ABI checks that need no GPU: the library loads, exports every function the header declares,
the ctypes mirror of fp8attn_attn_args matches the C layout, and every rejection path returns
its status and message before any HIP call (validation reads host values only)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import fp8_kv_cache_e4m3_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8attn.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8attn_[a-z_0-9]+)\s*\(", src)))


def test_header_symbols_exported():
    names = _declared()
    assert {"fp8attn_quantize_q", "fp8attn_prefill_varlen", "fp8attn_decode_paged",
            "fp8attn_splitkv_combine", "fp8attn_last_error"} <= set(names)
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert fa.fp8attn_version() >= 100


def test_struct_layout_matches_c(tmp_path):
    fields = [f for f, _ in fa.AttnArgs._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "fp8attn.h"', "int main(void){",
            'printf("%zu\\n", sizeof(fp8attn_attn_args));']
    for f in fields:
        prog.append(f'printf("%zu\\n", offsetof(fp8attn_attn_args, {f}));')
    prog.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.dirname(HEADER),
                        str(c), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(fa.AttnArgs)
    for f, off in zip(fields, vals[1:]):
        assert getattr(fa.AttnArgs, f).offset == off, f


def _valid_args(**kw):
    # host tensors: validation never dereferences them, and every case below fails validation
    q = torch.zeros((4, 8, 512), dtype=torch.bfloat16)
    k = torch.zeros((4, 64, 2, 512), dtype=torch.uint8)
    bt = torch.zeros((2, 4), dtype=torch.int32)
    cu = torch.tensor([0, 2, 4], dtype=torch.int32)
    sk = torch.tensor([100, 200], dtype=torch.int32)
    out = torch.zeros((4, 8, 512), dtype=torch.bfloat16)
    a = fa.make_args(q, k, k, bt, cu, sk, 2, 200, out=out)
    for n, v in kw.items():
        setattr(a, n, v)
    return a, (q, k, bt, cu, sk, out)


def _status(a, fn="prefill"):
    if fn == "prefill":
        return fa.LIB.fp8attn_prefill_varlen(ctypes.byref(a), None)
    need = ctypes.c_size_t(0)
    return fa.LIB.fp8attn_decode_paged(ctypes.byref(a), 0, None, 0, None, None, None)


@pytest.mark.parametrize("fn", ["prefill", "decode"])
@pytest.mark.parametrize("change,status,words", [
    ({"causal": 0}, fa.ERR_UNSUPPORTED, ["non-causal", "q=bf16", "head_size=512"]),
    ({"head_dim": 320}, fa.ERR_UNSUPPORTED, ["q=bf16", "k=e4m3", "v=e4m3", "head_size=320", "head_size_v=320"]),
    ({"q_dtype": fa.E4M3, "head_dim": 512}, fa.ERR_UNSUPPORTED, ["q=e4m3", "head_size=512"]),
    ({"q_dtype": fa.BF16_TO_E4M3, "head_dim": 512}, fa.ERR_UNSUPPORTED, ["q=bf16->e4m3", "head_size=512"]),
    ({"head_dim": 80}, fa.ERR_UNSUPPORTED, ["head_size=80"]),
    ({"q_dtype": fa.E4M3, "head_dim": 80}, fa.ERR_UNSUPPORTED, ["q=e4m3", "head_size=80"]),
    ({"page_size": 32}, fa.ERR_UNSUPPORTED, ["page_size 32", "multiple of 64"]),
    ({"page_size": 96}, fa.ERR_UNSUPPORTED, ["page_size 96"]),
    ({"window": 0}, fa.ERR_UNSUPPORTED, ["window 0", "q=bf16", "head_size=512"]),
    ({"window": -2}, fa.ERR_INVALID_ARG, ["window"]),
    ({"num_q_heads": 7}, fa.ERR_INVALID_ARG, ["multiple of num_kv_heads"]),
    ({"num_kv_heads": 0}, fa.ERR_INVALID_ARG, ["positive"]),
    ({"q_descale": 0x1000}, fa.ERR_UNSUPPORTED, ["q=bf16", "q_descale must be NULL"]),
    ({"max_seqlen_q": 300}, fa.ERR_INVALID_ARG, ["max_seqlen_q"]),
    ({"reserved0": 1}, fa.ERR_INVALID_ARG, ["reserved"]),
    ({"q": 0}, fa.ERR_INVALID_ARG, ["NULL"]),
    ({"out": 0}, fa.ERR_INVALID_ARG, ["NULL"]),
    ({"kv_stride_tok": 1000}, fa.ERR_UNSUPPORTED, ["16-byte"]),
    ({"kv_stride_tok": 1 << 26}, fa.ERR_UNSUPPORTED, ["kv_stride_tok", "2^32"]),
    ({"q_stride_head": 100}, fa.ERR_UNSUPPORTED, ["q must be 16-byte"]),
    ({"softmax_scale": float("nan")}, fa.ERR_INVALID_ARG, ["softmax_scale"]),
    ({"block_table_stride": 1}, fa.ERR_INVALID_ARG, ["block_table_stride"]),
    ({"q_dtype": 7}, fa.ERR_INVALID_ARG, ["q_dtype"]),
])
def test_rejections(fn, change, status, words):
    a, keep = _valid_args(**change)
    st = _status(a, fn)
    assert st == status, (st, fa.fp8attn_last_error())
    msg = fa.fp8attn_last_error()
    for w in words:
        assert w in msg, (w, msg)


@pytest.mark.parametrize("fn", ["prefill", "decode"])
@pytest.mark.parametrize("q_dtype", [fa.E4M3, fa.BF16_TO_E4M3])
@pytest.mark.parametrize("head_dim", [64, 96, 128, 192, 256])
def test_quantized_q_modes_pass_validation(fn, q_dtype, head_dim):
    # Both quantized-query modes are accepted at every native-FP8 head size, with or without a
    # q_descale; an empty batch then returns OK without touching the device.
    for qd in (0, 0x1000):
        a, keep = _valid_args(q_dtype=q_dtype, head_dim=head_dim, q_descale=qd, batch=0, total_q=0)
        st = _status(a, fn)
        assert st == fa.OK, (st, fa.fp8attn_last_error())


@pytest.mark.parametrize("fn", ["prefill", "decode"])
@pytest.mark.parametrize("head_dim", [64, 96, 128, 192, 256, 512])
def test_split_q_mode_validation(fn, head_dim):
    # split Q takes every head dim and unquantized queries: a q_descale is rejected
    a, keep = _valid_args(q_dtype=fa.BF16_SPLIT, head_dim=head_dim, batch=0, total_q=0)
    assert _status(a, fn) == fa.OK, fa.fp8attn_last_error()
    a, keep = _valid_args(q_dtype=fa.BF16_SPLIT, head_dim=head_dim, q_descale=0x1000)
    assert _status(a, fn) == fa.ERR_UNSUPPORTED
    assert "q=bf16-split" in fa.fp8attn_last_error() and "q_descale must be NULL" in fa.fp8attn_last_error()


def test_decode_rejects_long_query():
    a, keep = _valid_args(max_seqlen_q=17, max_seqlen_k=200)
    assert _status(a, "decode") == fa.ERR_UNSUPPORTED
    assert "max_seqlen_q 17 > 16" in fa.fp8attn_last_error()


def test_empty_batch_is_noop():
    a, keep = _valid_args(total_q=0)
    assert _status(a, "prefill") == fa.OK and fa.fp8attn_last_error() == ""
    a, keep = _valid_args(batch=0)
    assert _status(a, "decode") == fa.OK


def test_quantize_rejections():
    L = fa.LIB
    assert L.fp8attn_quantize_q(None, 4, 2, 12, 24, 12, None, None, None) == fa.ERR_UNSUPPORTED
    assert "multiple of 8" in fa.fp8attn_last_error()
    assert L.fp8attn_quantize_q(None, -1, 2, 16, 32, 16, None, None, None) == fa.ERR_INVALID_ARG
    assert L.fp8attn_quantize_q(None, 4, 2, 16, 32, 16, None, None, None) == fa.ERR_INVALID_ARG
    assert "non-NULL" in fa.fp8attn_last_error()
    assert L.fp8attn_quantize_q(None, 0, 2, 16, 32, 16, None, None, None) == fa.OK
    assert L.fp8attn_quantize_q(None, 4, 2, 16, 33, 16, None, None, None) == fa.ERR_UNSUPPORTED


def test_combine_rejections():
    L = fa.LIB
    assert L.fp8attn_splitkv_combine(None, None, 0, 1, 1, 64, None, 64, 64, None, None) == fa.ERR_INVALID_ARG
    assert L.fp8attn_splitkv_combine(None, None, 2, 1, 1, 80, None, 64, 64, None, None) == fa.ERR_UNSUPPORTED
    assert "head_dim 80" in fa.fp8attn_last_error()
    assert L.fp8attn_splitkv_combine(None, None, 2, 0, 1, 64, None, 64, 64, None, None) == fa.OK
    assert L.fp8attn_splitkv_combine(None, None, 2, 3, 1, 64, None, 64, 64, None, None) == fa.ERR_INVALID_ARG


def test_decode_workspace_query_needs_no_gpu_reads():
    # a size query validates and plans from host values only
    a, keep = _valid_args()
    need, used = ctypes.c_size_t(0), ctypes.c_int32(0)
    st = fa.LIB.fp8attn_decode_paged(ctypes.byref(a), 4, None, 0, ctypes.byref(need), ctypes.byref(used), None)
    assert st == fa.OK, fa.fp8attn_last_error()
    assert used.value == 4
    rows = 4 * 8
    assert need.value >= 4 * rows * 512 * 4 + 4 * rows * 4
    # one split: no workspace
    st = fa.LIB.fp8attn_decode_paged(ctypes.byref(a), 1, None, 0, ctypes.byref(need), ctypes.byref(used), None)
    assert st == fa.OK and need.value == 0 and used.value == 1
    # workspace too small for the chosen split count
    buf = torch.zeros(64, dtype=torch.uint8)
    st = fa.LIB.fp8attn_decode_paged(ctypes.byref(a), 4, buf.data_ptr(), 64, None, None, None)
    assert st == fa.ERR_WORKSPACE and "workspace" in fa.fp8attn_last_error()


def test_decode_balanced_partition_plan():
    # num_splits = -R asks for the balanced partition into R parts; automatic mode takes it for
    # long key ranges with one 16-row tile per sequence (planned from host values only)
    a, keep = _valid_args()
    need, used = ctypes.c_size_t(0), ctypes.c_int32(0)

    def query(n):
        st = fa.LIB.fp8attn_decode_paged(ctypes.byref(a), n, None, 0, ctypes.byref(need), ctypes.byref(used), None)
        assert st == fa.OK, fa.fp8attn_last_error()
        return used.value, need.value

    u, n = query(-5)
    items = 2 * 2 * 1                      # kv heads x sequences x row tiles
    slots = 5 + items
    assert u == -5 and n >= slots * 16 * 512 * 4 + slots * 16 * 4 + items * 8
    assert query(0)[0] > 0                 # 200 keys: the split plan
    a.max_seqlen_k = 8192
    a.block_table_stride = 128
    assert query(0)[0] < 0                 # 8192 keys, 8 rows per sequence: balanced
    a.max_seqlen_q = 5                     # 20 rows per sequence: two row tiles, split plan
    assert query(0)[0] > 0
    a.max_seqlen_q = 2
    st = fa.LIB.fp8attn_decode_paged(ctypes.byref(a), -(1 << 20) - 1, None, 0, ctypes.byref(need), None, None)
    assert st == fa.ERR_INVALID_ARG and "balanced" in fa.fp8attn_last_error()
    buf = torch.zeros(64, dtype=torch.uint8)
    st = fa.LIB.fp8attn_decode_paged(ctypes.byref(a), -5, buf.data_ptr(), 64, None, None, None)
    assert st == fa.ERR_WORKSPACE and "balanced" in fa.fp8attn_last_error()


def test_cache_write_rejections():
    L = fa.LIB
    args = lambda **kw: {**dict(k=None, v=None, T=4, H=2, d=32, kst=64, ksh=32, vst=64, vsh=32, slots=None,
                                kc=None, vc=None, pages=3, ps=64, sp=64 * 64, stt=64, sth=32, kd=None, vd=None), **kw}
    def call(a):
        return L.fp8attn_cache_write(a["k"], a["v"], a["T"], a["H"], a["d"], a["kst"], a["ksh"], a["vst"], a["vsh"],
                                     a["slots"], a["kc"], a["vc"], a["pages"], a["ps"], a["sp"], a["stt"], a["sth"],
                                     a["kd"], a["vd"], None)
    assert call(args(d=24)) == fa.ERR_UNSUPPORTED and "multiple of 16" in fa.fp8attn_last_error()
    assert call(args(H=0)) == fa.ERR_INVALID_ARG
    assert call(args(ps=0)) == fa.ERR_INVALID_ARG
    assert call(args(T=-1)) == fa.ERR_INVALID_ARG
    assert call(args(kst=60)) == fa.ERR_UNSUPPORTED and "strides" in fa.fp8attn_last_error()
    assert call(args(stt=40)) == fa.ERR_UNSUPPORTED and "cache strides" in fa.fp8attn_last_error()
    assert call(args()) == fa.ERR_INVALID_ARG and "non-NULL" in fa.fp8attn_last_error()
    assert call(args(T=0)) == fa.OK
    assert call(args(k=0x1008, v=0x2000, slots=0x3000, kc=0x4000, vc=0x5000)) == fa.ERR_UNSUPPORTED
    assert "aligned" in fa.fp8attn_last_error()


def test_last_error_is_per_thread():
    # each thread reads the message of its own last failed call, whatever the other thread did
    import threading
    results = {}

    def worker(name, change, word):
        a, keep = _valid_args(**change)
        for _ in range(200):
            st = _status(a, "prefill")
            msg = fa.fp8attn_last_error()
            if st == fa.OK or word not in msg:
                results[name] = (st, msg)
                return
        results[name] = "ok"

    t1 = threading.Thread(target=worker, args=("a", {"causal": 0}, "non-causal"))
    t2 = threading.Thread(target=worker, args=("b", {"window": -3}, "window must be"))
    t1.start(); t2.start(); t1.join(); t2.join()
    assert results == {"a": "ok", "b": "ok"}, results
