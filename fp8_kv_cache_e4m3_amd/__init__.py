"""Python binding of libfp8attn (paged attention over an FP8 E4M3 KV cache on MI355X).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libfp8attn.so``.  torch provides device memory and the current stream.  If the
library is missing, importing this package raises: there is no fallback path.

The functions carry the C names (see include/fp8attn.h):
  fp8attn_quantize_q, fp8attn_prefill_varlen, fp8attn_decode_paged,
  fp8attn_decode_paged_noalloc, fp8attn_splitkv_combine, fp8attn_cache_write,
  fp8attn_last_error, fp8attn_version
"""
from __future__ import annotations

import ctypes
import os

import torch  # must be imported before the library: the library reuses torch's HIP runtime

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8attn.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is not built; run `python fp8_kv_cache_e4m3_amd/build.py` "
                      "(there is no non-HIP fallback)")
_lib = ctypes.CDLL(_LIB_PATH)

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
BF16, E4M3, BF16_TO_E4M3, BF16_SPLIT = 0, 1, 2, 3
_STATUS = {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class AttnArgs(ctypes.Structure):
    """Mirror of fp8attn_attn_args (same field order; ctypes applies the C alignment rules)."""
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_dtype", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("kv_stride_page", ctypes.c_int64),
        ("kv_stride_tok", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("reserved1", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("block_table_stride", ctypes.c_int64),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("seqlens_k", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_descale", ctypes.c_void_p),
        ("k_descale", ctypes.c_void_p),
        ("v_descale", ctypes.c_void_p),
        ("descale_stride_b", ctypes.c_int64),
        ("descale_stride_h", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("out", ctypes.c_void_p),
        ("out_stride_tok", ctypes.c_int64),
        ("out_stride_head", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
    ]


_i32, _i64, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
_lib.fp8attn_quantize_q.argtypes = [_vp, _i64, _i32, _i32, _i64, _i64, _vp, _vp, _vp]
_lib.fp8attn_quantize_q.restype = _i32
_lib.fp8attn_prefill_varlen.argtypes = [ctypes.POINTER(AttnArgs), _vp]
_lib.fp8attn_prefill_varlen.restype = _i32
_lib.fp8attn_decode_paged.argtypes = [ctypes.POINTER(AttnArgs), _i32, _vp, _sz, ctypes.POINTER(_sz),
                                      ctypes.POINTER(_i32), _vp]
_lib.fp8attn_decode_paged.restype = _i32
_lib.fp8attn_decode_paged_noalloc.argtypes = [ctypes.POINTER(AttnArgs), _i32, ctypes.POINTER(_i32), _vp]
_lib.fp8attn_decode_paged_noalloc.restype = _i32
_lib.fp8attn_splitkv_combine.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _vp, _i64, _i64, _vp, _vp]
_lib.fp8attn_splitkv_combine.restype = _i32
_lib.fp8attn_cache_write.argtypes = [_vp, _vp, _i64, _i32, _i32, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _i32,
                                     _i64, _i64, _i64, _vp, _vp, _vp]
_lib.fp8attn_cache_write.restype = _i32
_lib.fp8attn_last_error.argtypes = []
_lib.fp8attn_last_error.restype = ctypes.c_char_p
_lib.fp8attn_version.argtypes = []
_lib.fp8attn_version.restype = _i32

LIB = _lib
LIB_PATH = _LIB_PATH


class Fp8AttnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with {_STATUS.get(status, status)}: {msg}")
        self.status = status


def fp8attn_last_error() -> str:
    return _lib.fp8attn_last_error().decode()


def fp8attn_version() -> int:
    return int(_lib.fp8attn_version())


def _check(fn, st):
    if st != OK:
        raise Fp8AttnError(fn, st, fp8attn_last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


def _bytes(t):
    """E4M3 tensors may arrive as torch.float8_e4m3fn or uint8; the library sees bytes."""
    if t is not None and t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8)
    return t


def fp8attn_cache_write(k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor, k_descale=None, v_descale=None,
                        stream=None) -> None:
    """Quantize bf16 k_new/v_new [T, Hkv, d] and store them at slot_mapping (int64 [T]) in the
    E4M3 caches [pages, page_size, Hkv, d] (uint8 or float8_e4m3fn, d contiguous), in place."""
    k_cache, v_cache = _bytes(k_cache), _bytes(v_cache)
    assert k_new.dtype == torch.bfloat16 and v_new.dtype == torch.bfloat16 and k_new.shape == v_new.shape
    assert k_new.stride(2) == 1 and v_new.stride(2) == 1 and k_cache.stride(3) == 1
    assert k_cache.shape == v_cache.shape and k_cache.stride() == v_cache.stride()
    assert slot_mapping.dtype == torch.int64 and slot_mapping.numel() == k_new.shape[0]
    T, H, d = k_new.shape
    st = _lib.fp8attn_cache_write(_ptr(k_new), _ptr(v_new), T, H, d, k_new.stride(0), k_new.stride(1),
                                  v_new.stride(0), v_new.stride(1), _ptr(slot_mapping), _ptr(k_cache),
                                  _ptr(v_cache), k_cache.shape[0], k_cache.shape[1], k_cache.stride(0),
                                  k_cache.stride(1), k_cache.stride(2), _ptr(k_descale), _ptr(v_descale),
                                  _stream(stream))
    _check("fp8attn_cache_write", st)


def fp8attn_quantize_q(q: torch.Tensor, q_descale=None, out=None, stream=None) -> torch.Tensor:
    """bf16 [T, H, d] (head_dim contiguous) -> E4M3 codes (uint8, contiguous [T, H, d])."""
    assert q.dtype == torch.bfloat16 and q.dim() == 3 and q.stride(2) == 1
    T, H, d = q.shape
    if out is None:
        out = torch.empty((T, H, d), dtype=torch.uint8, device=q.device)
    st = _lib.fp8attn_quantize_q(_ptr(q), T, H, d, q.stride(0), q.stride(1), _ptr(q_descale), _ptr(out),
                                 _stream(stream))
    _check("fp8attn_quantize_q", st)
    return out


def make_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k,
              q_descale=None, k_descale=None, v_descale=None, softmax_scale=0.0, window=-1, causal=True,
              out=None, lse=None, descale_strides=(0, 0), total_q=None, batch=None,
              quantize_q=False, split_q=False) -> AttnArgs:
    """Fill the C argument struct from tensors (shapes: q [T, Hq, d]; caches [pages, page, Hkv, d]).
    quantize_q: bf16 q is quantized to E4M3 inside the call (q_dtype BF16_TO_E4M3).
    split_q: bf16 q is split into two E4M3 terms inside the call (q_dtype BF16_SPLIT)."""
    k_cache, v_cache = _bytes(k_cache), _bytes(v_cache)
    a = AttnArgs()
    if q.dtype == torch.bfloat16:
        assert not (quantize_q and split_q), "quantize_q and split_q exclude each other"
        a.q_dtype = BF16_TO_E4M3 if quantize_q else BF16_SPLIT if split_q else BF16
    else:
        q = _bytes(q)
        assert q.dtype == torch.uint8, "q must be bf16 or E4M3 codes"
        a.q_dtype = E4M3
    T, Hq, d = q.shape
    a.q = _ptr(q)
    a.q_stride_tok, a.q_stride_head = q.stride(0), q.stride(1)
    a.k_cache, a.v_cache = _ptr(k_cache), _ptr(v_cache)
    assert k_cache.stride() == v_cache.stride(), "K and V pools must share one layout"
    a.kv_stride_page, a.kv_stride_tok, a.kv_stride_head = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    a.page_size = k_cache.shape[1]
    a.block_table = _ptr(block_table)
    a.block_table_stride = block_table.stride(0)
    a.cu_seqlens_q = _ptr(cu_seqlens_q)
    a.seqlens_k = _ptr(seqlens_k)
    a.batch = seqlens_k.shape[0] if batch is None else batch
    a.total_q = T if total_q is None else total_q
    a.max_seqlen_q, a.max_seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
    a.num_q_heads, a.num_kv_heads, a.head_dim = Hq, k_cache.shape[2], d
    a.q_descale, a.k_descale, a.v_descale = _ptr(q_descale), _ptr(k_descale), _ptr(v_descale)
    a.descale_stride_b, a.descale_stride_h = descale_strides
    a.softmax_scale = float(softmax_scale)
    a.causal = 1 if causal else 0
    a.window = int(window)
    a.out = _ptr(out)
    if out is not None:
        a.out_stride_tok, a.out_stride_head = out.stride(0), out.stride(1)
    a.lse = _ptr(lse)
    return a


def _alloc_out(q, out, lse, want_lse):
    T, Hq, d = q.shape
    if out is None:
        out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    return out, lse


def fp8attn_prefill_varlen(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, max_seqlen_q,
                           max_seqlen_k, q_descale=None, k_descale=None, v_descale=None, softmax_scale=0.0,
                           window=-1, causal=True, out=None, lse=None, want_lse=True, descale_strides=(0, 0),
                           quantize_q=False, split_q=False, stream=None):
    out, lse = _alloc_out(q, out, lse, want_lse)
    a = make_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k,
                  q_descale, k_descale, v_descale, softmax_scale, window, causal, out, lse, descale_strides,
                  quantize_q=quantize_q, split_q=split_q)
    _check("fp8attn_prefill_varlen", _lib.fp8attn_prefill_varlen(ctypes.byref(a), _stream(stream)))
    return out, lse


def decode_workspace_size(args: AttnArgs, num_splits: int = 0):
    need = _sz(0)
    used = _i32(0)
    st = _lib.fp8attn_decode_paged(ctypes.byref(args), num_splits, None, 0, ctypes.byref(need),
                                   ctypes.byref(used), None)
    _check("fp8attn_decode_paged", st)
    return need.value, used.value


def fp8attn_decode_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k,
                         q_descale=None, k_descale=None, v_descale=None, softmax_scale=0.0, window=-1,
                         causal=True, out=None, lse=None, want_lse=True, num_splits=0, workspace=None,
                         descale_strides=(0, 0), quantize_q=False, split_q=False, stream=None):
    """Returns (out, lse, splits_used).  num_splits: 0 automatic, N > 0 that many splits, -R the
    balanced partition into R parts (splits_used is then -R).  The workspace is sized by a query
    and allocated with torch if the caller passes none.  quantize_q: bf16 q is quantized to E4M3
    inside the call; split_q: bf16 q runs on the FP8 MFMA as two E4M3 terms (q_dtype BF16_SPLIT)."""
    out, lse = _alloc_out(q, out, lse, want_lse)
    a = make_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k,
                  q_descale, k_descale, v_descale, softmax_scale, window, causal, out, lse, descale_strides,
                  quantize_q=quantize_q, split_q=split_q)
    need, used = decode_workspace_size(a, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    used_c = _i32(0)
    st = _lib.fp8attn_decode_paged(ctypes.byref(a), num_splits, _ptr(workspace), ws_bytes, None,
                                   ctypes.byref(used_c), _stream(stream))
    _check("fp8attn_decode_paged", st)
    return out, lse, used_c.value


def fp8attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, max_seqlen_q,
                                 max_seqlen_k, q_descale=None, k_descale=None, v_descale=None, softmax_scale=0.0,
                                 window=-1, causal=True, out=None, lse=None, want_lse=True, num_splits=0,
                                 descale_strides=(0, 0), quantize_q=False, split_q=False, stream=None):
    """fp8attn_decode_paged with the split-KV partials in the library's static device scratch (no
    workspace; the call allocates nothing).  Returns (out, lse, splits_used); out and lse are
    allocated here only if the caller passes none."""
    out, lse = _alloc_out(q, out, lse, want_lse)
    a = make_args(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k,
                  q_descale, k_descale, v_descale, softmax_scale, window, causal, out, lse, descale_strides,
                  quantize_q=quantize_q, split_q=split_q)
    used = _i32(0)
    st = _lib.fp8attn_decode_paged_noalloc(ctypes.byref(a), num_splits, ctypes.byref(used), _stream(stream))
    _check("fp8attn_decode_paged_noalloc", st)
    return out, lse, used.value


def fp8attn_splitkv_combine(partial_o, partial_lse, out=None, lse=None, stream=None):
    """partial_o fp32 [S, T, Hq, d], partial_lse fp32 [S, T, Hq] -> (bf16 out [T, Hq, d], lse [T, Hq])."""
    S, T, Hq, d = partial_o.shape
    if out is None:
        out = torch.empty((T, Hq, d), dtype=torch.bfloat16, device=partial_o.device)
    st = _lib.fp8attn_splitkv_combine(_ptr(partial_o), _ptr(partial_lse), S, T, Hq, d, _ptr(out), out.stride(0),
                                      out.stride(1), _ptr(lse), _stream(stream))
    _check("fp8attn_splitkv_combine", st)
    return out, lse
