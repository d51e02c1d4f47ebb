"""Seeded synthetic inputs for paged FP8-KV attention.

This module only draws inputs.  It holds none of the attention arithmetic and
none of the Q quantization: both the CPU oracle (``oracle/``) and the GPU
library consume what it returns.  What it does produce:

* Q as bf16 values drawn from N(0, 1).
* K and V page pools already stored as OCP E4M3 bytes.  Each pool is drawn from
  N(0, 1) in fp32, divided by its per-tensor descale ``amax / 448`` and cast
  with ``torch.float8_e4m3fn`` (a library cast).  Because every scaled value
  lies within [-448, 448] that cast needs no saturation.  The KV cache is an
  input of the attention path: how a serving engine writes it is a separate
  step.
* Page tables that scatter each sequence's 64-token pages over a shared pool
  in a seeded random order.  In the spec-verify workload the prefix pages are
  the same physical pages in every sequence's table.
* Sequence lengths drawn as integers uniform over an inclusive range.

The workloads follow the shapes and structure of the serving runs the pages
profile (an 8k-in/1k-out random-token run on Gemma-4 with 64-token pages, and a
25K shared-prefix plus 3K unique-token MTP run).  Each one is named by what it
is.  ``scale`` shrinks lengths and batch for parity tests while keeping the
structure: several tiles, ragged tails, windows and permuted pages.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

PAGE = 64           # tokens per kernel page (the pages' 64-token block contract)
E4M3_MAX = 448.0    # largest finite OCP E4M3 magnitude


@dataclasses.dataclass
class Workload:
    """One batch of synthetic inputs.  Tensors live on ``device``."""
    name: str
    q_dtype: str                      # "bf16": the kernel takes bf16 Q; "e4m3": Q is quantized first
    head_dim: int
    num_q_heads: int
    num_kv_heads: int
    window: int                       # -1: no window; W >= 1: keys p-W < j <= p are visible
    q: torch.Tensor                   # bf16 [total_q, Hq, d]
    q_descale: Optional[torch.Tensor]  # f32 [1] (e4m3 Q only): amax|q| / 448
    k_pool: torch.Tensor              # uint8 [pages, 64, Hkv, d] (E4M3 codes)
    v_pool: torch.Tensor
    k_descale: torch.Tensor           # f32 [1]
    v_descale: torch.Tensor           # f32 [1]
    block_table: torch.Tensor         # int32 [B, max_pages]
    cu_seqlens_q: torch.Tensor        # int32 [B+1]
    seqlens_k: torch.Tensor           # int32 [B]
    seqlens_k_host: list              # python ints (the host knows its own batch)
    q_lens_host: list

    @property
    def batch(self) -> int:
        return len(self.seqlens_k_host)

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens_host))

    @property
    def max_seqlen_k(self) -> int:
        return int(max(self.seqlens_k_host))

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.q_lens_host))

    def to(self, device) -> "Workload":
        out = dataclasses.replace(self)
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                setattr(out, f.name, v.to(device))
        return out


# ----------------------------------------------------------------------------------------
# random sources: numpy on the host for small workloads, torch on a device for large ones
# ----------------------------------------------------------------------------------------
class _Rng:
    def __init__(self, seed: int, device):
        self.device = torch.device(device)
        if self.device.type == "cpu":
            self.np = np.random.default_rng(seed)
            self.gen = None
        else:
            self.np = np.random.default_rng(seed)           # integer draws (lengths, permutations)
            self.gen = torch.Generator(device=self.device)
            self.gen.manual_seed(seed)

    def normal(self, shape) -> torch.Tensor:
        """float32 N(0,1) tensor on the device."""
        if self.gen is None:
            return torch.from_numpy(self.np.standard_normal(size=shape, dtype=np.float32))
        return torch.randn(shape, generator=self.gen, device=self.device, dtype=torch.float32)

    def lengths(self, lo: int, hi: int, n: int) -> list:
        return [int(x) for x in self.np.integers(lo, hi, size=n, endpoint=True)]

    def permutation(self, n: int) -> np.ndarray:
        return self.np.permutation(n)


def _amax_descale(x: torch.Tensor) -> torch.Tensor:
    """Per-tensor descale amax|x| / 448 in fp32 (the static-scale recipe of the inputs)."""
    amax = x.abs().amax().to(torch.float32)
    return (amax / torch.tensor(E4M3_MAX, dtype=torch.float32, device=x.device)).reshape(1)


def _e4m3_pool(rng: _Rng, num_pages: int, num_kv_heads: int, d: int, chunk_pages: int = 2048,
               layout: str = "token_major"):
    """Draw a pool [pages, 64, Hkv, d] from N(0,1) and store it as E4M3 bytes.

    The descale is amax over the whole pool / 448.  Large pools are drawn in
    chunks so that the fp32 staging stays bounded: the chunk draws happen in a
    fixed order, so the result depends only on the seed."""
    dev = rng.device
    if layout == "head_major":
        # physical order [pages, Hkv, 64, d] (one contiguous tile per page and kv head), returned as a
        # [pages, 64, Hkv, d] view: the logical indexing is the same, only the strides differ
        return _e4m3_pool_hm(rng, num_pages, num_kv_heads, d, chunk_pages)
    shape_tail = (PAGE, num_kv_heads, d)
    if num_pages * PAGE * num_kv_heads * d <= (1 << 27):
        x = rng.normal((num_pages,) + shape_tail)
        ds = _amax_descale(x)
        codes = (x / ds).to(torch.float8_e4m3fn).view(torch.uint8)
        return codes.contiguous(), ds
    # two passes: first draw chunks and record amax, then redraw with the same seed state copy
    state_np = None
    amax = torch.zeros((), dtype=torch.float32, device=dev)
    gen_state = rng.gen.get_state() if rng.gen is not None else None
    if rng.gen is None:
        state_np = rng.np.bit_generator.state
    for p0 in range(0, num_pages, chunk_pages):
        n = min(chunk_pages, num_pages - p0)
        x = rng.normal((n,) + shape_tail)
        amax = torch.maximum(amax, x.abs().amax())
        del x
    ds = (amax / torch.tensor(E4M3_MAX, dtype=torch.float32, device=dev)).reshape(1)
    if rng.gen is not None:
        rng.gen.set_state(gen_state)
    else:
        rng.np.bit_generator.state = state_np
    out = torch.empty((num_pages,) + shape_tail, dtype=torch.uint8, device=dev)
    for p0 in range(0, num_pages, chunk_pages):
        n = min(chunk_pages, num_pages - p0)
        x = rng.normal((n,) + shape_tail)
        out[p0:p0 + n] = (x / ds).to(torch.float8_e4m3fn).view(torch.uint8)
        del x
    return out, ds


def _e4m3_pool_hm(rng: _Rng, num_pages: int, num_kv_heads: int, d: int, chunk_pages: int):
    """Head-major pool: drawn in physical order [pages, Hkv, 64, d], viewed as [pages, 64, Hkv, d]."""
    phys, ds = _e4m3_pool(rng, num_pages, 1, num_kv_heads * d, chunk_pages)   # [pages, 64, 1, Hkv*d] bytes
    phys = phys.reshape(num_pages, num_kv_heads, PAGE, d)                     # reinterpret the same bytes
    return phys.permute(0, 2, 1, 3), ds


def _assemble(name, rng: _Rng, q_dtype, d, hq, hkv, window, seqlens, qlens,
              shared_prefix_pages: int = 0, fixed_table=None, layout: str = "token_major") -> Workload:
    dev = rng.device
    B = len(seqlens)
    npages = [math.ceil(L / PAGE) for L in seqlens]
    max_pages = max(npages)
    if fixed_table is not None:
        table = np.asarray(fixed_table, dtype=np.int64).reshape(B, -1)
        pool_pages = int(table.max()) + 1
    else:
        own = [n - shared_prefix_pages for n in npages]
        pool_pages = shared_prefix_pages + sum(own)
        perm = rng.permutation(pool_pages)
        table = np.zeros((B, max_pages), dtype=np.int64)
        nxt = shared_prefix_pages
        for b in range(B):
            table[b, :shared_prefix_pages] = perm[:shared_prefix_pages]
            table[b, shared_prefix_pages:npages[b]] = perm[nxt:nxt + own[b]]
            nxt += own[b]
    total_q = int(sum(qlens))
    q = rng.normal((total_q, hq, d)).to(torch.bfloat16)
    q_descale = None
    if q_dtype == "e4m3":
        q_descale = _amax_descale(q.to(torch.float32))
    k_pool, k_ds = _e4m3_pool(rng, pool_pages, hkv, d, layout=layout)
    v_pool, v_ds = _e4m3_pool(rng, pool_pages, hkv, d, layout=layout)
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(qlens)
    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32)).to(dev)
    return Workload(name=name, q_dtype=q_dtype, head_dim=d, num_q_heads=hq, num_kv_heads=hkv,
                    window=window, q=q, q_descale=q_descale, k_pool=k_pool, v_pool=v_pool,
                    k_descale=k_ds, v_descale=v_ds, block_table=i32(table), cu_seqlens_q=i32(cu),
                    seqlens_k=i32(seqlens), seqlens_k_host=list(seqlens), q_lens_host=list(qlens))


# ----------------------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------------------
def tiny(q_dtype: str = "bf16", device="cpu", seed: int = 0) -> Workload:
    """One sequence, one q head / one kv head, d 64, 128 cached tokens in two pages with
    page table [1, 0], 16 causal query tokens at the end (positions 112..127)."""
    rng = _Rng(seed, device)
    return _assemble("tiny d64 2-page causal", rng, q_dtype, 64, 1, 1, -1, [128], [16],
                     fixed_table=[[1, 0]])


def swa_decode(device="cpu", layout: str = "token_major", seed: int = 2, scale: float = 1.0) -> Workload:
    """Sliding-window decode: batch 32, one query token each, KV lengths uniform in
    [1024, 8192], 32 q / 16 kv heads, d 256, window 1024, E4M3 Q/K/V."""
    rng = _Rng(seed, device)
    B = max(1, int(round(32 * scale)))
    lo, hi = max(1, int(1024 * scale)), max(2, int(8192 * scale))
    W = max(1, int(1024 * scale))
    seqlens = rng.lengths(lo, hi, B)
    return _assemble(f"sliding-window decode B{B} d256 W{W}", rng, "e4m3", 256, 32, 16, W,
                     seqlens, [1] * B, layout=layout)


def full_decode(device="cpu", layout: str = "token_major", seed: int = 3, scale: float = 1.0) -> Workload:
    """Full-attention decode: batch 64, one query token each, KV lengths uniform in
    [8192, 32768], 32 q / 4 kv heads (GQA 8), d 512, bf16 Q with E4M3 K/V, causal."""
    rng = _Rng(seed, device)
    B = max(1, int(round(64 * scale)))
    lo, hi = max(1, int(8192 * scale)), max(2, int(32768 * scale))
    seqlens = rng.lengths(lo, hi, B)
    return _assemble(f"full-attention decode B{B} d512", rng, "bf16", 512, 32, 4, -1,
                     seqlens, [1] * B, layout=layout)


def swa_prefill(device="cpu", layout: str = "token_major", seed: int = 4, scale: float = 1.0) -> Workload:
    """Chunked prefill, sliding-window layer: 8 sequences of 8192 new tokens each (no prior
    cache), 32 q / 16 kv heads, d 256, causal + window 1024, E4M3 Q/K/V."""
    rng = _Rng(seed, device)
    B = max(1, int(round(8 * scale)))
    L = max(1, int(8192 * scale))
    W = max(1, int(1024 * scale))
    return _assemble(f"sliding-window prefill B{B}x{L} d256 W{W}", rng, "e4m3", 256, 32, 16, W,
                     [L] * B, [L] * B, layout=layout)


def full_prefill(device="cpu", layout: str = "token_major", seed: int = 6, scale: float = 1.0) -> Workload:
    """Prefill of full-attention layers: 4 sequences of 2048 new tokens each (no prior cache),
    32 q / 4 kv heads (GQA 8), d 512, bf16 Q with E4M3 K/V, causal."""
    rng = _Rng(seed, device)
    B = max(1, int(round(4 * scale)))
    L = max(1, int(2048 * scale))
    return _assemble(f"full-attention prefill B{B}x{L} d512", rng, "bf16", 512, 32, 4, -1,
                     [L] * B, [L] * B, layout=layout)


def spec_verify(device="cpu", layout: str = "token_major", seed: int = 5, scale: float = 1.0) -> Workload:
    """Spec-decode verify with a shared prefix: 64 sequences, each a 25,600-token prefix whose
    pages every sequence shares, plus 3,072 unique tokens; 4 query tokens (1 + 3 speculative)
    at the end, causal among themselves; 32 q / 4 kv heads, d 512, bf16 Q, E4M3 K/V."""
    rng = _Rng(seed, device)
    B = max(1, int(round(64 * scale)))
    prefix_pages = max(1, int(round(400 * scale)))
    unique_pages = max(1, int(round(48 * scale)))
    L = (prefix_pages + unique_pages) * PAGE
    return _assemble(f"spec-verify shared prefix B{B} L{L} d512", rng, "bf16", 512, 32, 4, -1,
                     [L] * B, [4] * B, shared_prefix_pages=prefix_pages, layout=layout)


def custom(q_dtype: str, d: int, hq: int, hkv: int, window: int, seqlens, qlens,
           device="cpu", seed: int = 7, shared_prefix_pages: int = 0, layout: str = "token_major") -> Workload:
    """Any shape, same recipe (used by edge-case tests)."""
    rng = _Rng(seed, device)
    return _assemble(f"custom d{d} {hq}/{hkv} W{window}", rng, q_dtype, d, hq, hkv, window,
                     list(seqlens), list(qlens), shared_prefix_pages=shared_prefix_pages, layout=layout)


BY_NAME = {
    "tiny": tiny,
    "swa_decode": swa_decode,
    "full_decode": full_decode,
    "swa_prefill": swa_prefill,
    "spec_verify": spec_verify,
    "full_prefill": full_prefill,
}
