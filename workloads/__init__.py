"""Seeded synthetic inputs for the ring-attention step: shared by the HIP path's
tests and benchmark and by the CPU oracle's tests.

This module only draws random numbers and builds shapes; it holds none of the
attention arithmetic.  Every tensor is produced on the host by torch's CPU
generator (or numpy's PCG64 for document lengths) so that both sides see the
same bytes; callers copy to the GPU themselves.

Workloads (sizes follow the pages' two worked examples and three long-context
cases; token positions are global indices 0..T-1):

* ``p4_ring4_b8_d16``   -- Ultralytics "Ring Attention" page, section "Come
  funziona": seed 0, ``randn(3, 32, 16)`` unpacked to q, k, v; 4 blocks of 8;
  scale 1/sqrt(16); fp32; no mask.
* ``p2_1024tok_d2_16blk`` -- "Ring Attention simulation" gist: seed 1337, three
  ``randn(1024, 2)`` draws in the order q, k, v; 16 blocks of 64; unscaled;
  fp32; no mask.
* ``causal32k_h32_d128_8blk`` -- 32768 tokens, 32 heads, d=128, 8 contiguous
  blocks, causal, bf16 from N(0,1) (seed 3).
* ``gqa_striped64k_h32kv8_d128_16blk`` -- 65536 tokens, 32 query / 8 key-value
  heads, d=128, 16 striped blocks (token t in block t mod 16), causal, bf16
  (seed 4).
* ``varlen_packed128k_h32_d128_8blk_p4`` -- packed qkv [T, 3, 32, 128] with
  T=131072, documents of seeded lengths uniform on [1024, 16384] (last one cut
  to fill T), per-document causal, 8 contiguous blocks, 4 ring passes (seed 5;
  lengths drawn from an independent stream).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

MASK_NONE, MASK_CAUSAL, MASK_DOC_CAUSAL = 0, 1, 2
LAYOUT_CONTIGUOUS, LAYOUT_STRIPED = 0, 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    Hq: int
    Hkv: int
    d: int
    n_blocks: int
    mask: int
    layout: int
    max_ring_passes: int
    dtype: str            # "f32", "bf16" or "f16"
    scale: float
    seed: int
    packed: bool = False  # q, k, v are views into one [T, 3, H, d] tensor
    doc_len_range: Optional[tuple] = None

    @property
    def block(self) -> int:
        return self.T // self.n_blocks


WORKLOADS = {
    w.name: w
    for w in [
        Workload("p4_ring4_b8_d16", 32, 1, 1, 16, 4, MASK_NONE, LAYOUT_CONTIGUOUS, 4,
                 "f32", 1.0 / math.sqrt(16), 0),
        Workload("p2_1024tok_d2_16blk", 1024, 1, 1, 2, 16, MASK_NONE, LAYOUT_CONTIGUOUS, 16,
                 "f32", 1.0, 1337),
        Workload("causal32k_h32_d128_8blk", 32768, 32, 32, 128, 8, MASK_CAUSAL,
                 LAYOUT_CONTIGUOUS, 8, "bf16", 1.0 / math.sqrt(128), 3),
        Workload("gqa_striped64k_h32kv8_d128_16blk", 65536, 32, 8, 128, 16, MASK_CAUSAL,
                 LAYOUT_STRIPED, 16, "bf16", 1.0 / math.sqrt(128), 4),
        Workload("varlen_packed128k_h32_d128_8blk_p4", 131072, 32, 32, 128, 8,
                 MASK_DOC_CAUSAL, LAYOUT_CONTIGUOUS, 4, "bf16", 1.0 / math.sqrt(128), 5,
                 packed=True, doc_len_range=(1024, 16384)),
    ]
}
ORDER = list(WORKLOADS)


def doc_cu_seqlens(seed: int, T: int, lo: int, hi: int) -> np.ndarray:
    """Cumulative document boundaries [0, L1, L1+L2, ..., T] as int32.

    Lengths are integers uniform on [lo, hi] inclusive from numpy's PCG64
    seeded with ``seed``; drawing stops once the running sum reaches T and the
    last document is cut so that the total is exactly T.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = [0]
    while cu[-1] < T:
        cu.append(min(T, cu[-1] + int(rng.integers(lo, hi + 1))))
    return np.asarray(cu, dtype=np.int32)


def _to_dtype(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x.float()
    if dtype == "bf16":
        return x.to(torch.bfloat16)  # round to nearest even
    if dtype == "f16":
        return x.to(torch.float16)  # round to nearest even
    raise ValueError(dtype)


def make_inputs(w: Workload):
    """Host tensors for a workload: dict with q, k, v ([T, H, d] views), and
    for the packed workload ``qkv`` ([T, 3, H, d]) and ``cu_seqlens``."""
    if w.name == "p4_ring4_b8_d16":
        torch.manual_seed(w.seed)
        q, k, v = torch.randn(3, w.T, w.d)
        q, k, v = (x.reshape(w.T, 1, w.d).contiguous() for x in (q, k, v))
        return {"q": q, "k": k, "v": v}
    if w.name == "p2_1024tok_d2_16blk":
        torch.manual_seed(w.seed)
        q, k, v = torch.randn(w.T, w.d), torch.randn(w.T, w.d), torch.randn(w.T, w.d)
        q, k, v = (x.reshape(w.T, 1, w.d).contiguous() for x in (q, k, v))
        return {"q": q, "k": k, "v": v}
    g = torch.Generator().manual_seed(w.seed)
    if w.packed:
        assert w.Hq == w.Hkv
        qkv = _to_dtype(torch.randn(w.T, 3, w.Hq, w.d, generator=g), w.dtype)
        out = {"qkv": qkv, "q": qkv[:, 0], "k": qkv[:, 1], "v": qkv[:, 2]}
    else:
        q = _to_dtype(torch.randn(w.T, w.Hq, w.d, generator=g), w.dtype)
        k = _to_dtype(torch.randn(w.T, w.Hkv, w.d, generator=g), w.dtype)
        v = _to_dtype(torch.randn(w.T, w.Hkv, w.d, generator=g), w.dtype)
        out = {"q": q, "k": k, "v": v}
    if w.mask == MASK_DOC_CAUSAL:
        lo, hi = w.doc_len_range
        out["cu_seqlens"] = torch.from_numpy(doc_cu_seqlens(w.seed, w.T, lo, hi))
    return out


def random_qkv(T: int, Hq: int, Hkv: int, d: int, dtype: str, seed: int, packed: bool = False):
    """Small seeded N(0,1) inputs in [T, H, d] layout (or packed [T, 3, H, d])."""
    g = torch.Generator().manual_seed(seed)
    if packed:
        assert Hq == Hkv
        qkv = _to_dtype(torch.randn(T, 3, Hq, d, generator=g), dtype)
        return qkv[:, 0], qkv[:, 1], qkv[:, 2]
    q = _to_dtype(torch.randn(T, Hq, d, generator=g), dtype)
    k = _to_dtype(torch.randn(T, Hkv, d, generator=g), dtype)
    v = _to_dtype(torch.randn(T, Hkv, d, generator=g), dtype)
    return q, k, v


def random_dout(T: int, Hq: int, d: int, dtype: str, seed: int):
    """Seeded N(0,1) output gradient [T, Hq, d] (its own stream, seed + 7919)."""
    g = torch.Generator().manual_seed(seed + 7919)
    return _to_dtype(torch.randn(T, Hq, d, generator=g), dtype)


def random_key_valid(T: int, seed: int, frac: float = 0.3) -> torch.Tensor:
    """Seeded key-padding mask [T] (True = real key): each key padded with
    probability frac, plus one run of 150 padded keys (whole 64-key tiles
    with no real key), key 0 padded (under a causal mask row 0 keeps no
    key) and the last key kept."""
    g = torch.Generator().manual_seed(seed)
    kv = torch.rand(T, generator=g) >= frac
    start = int(torch.randint(0, max(T - 150, 1), (1,), generator=g))
    kv[start:start + 150] = False
    kv[0] = False
    kv[-1] = True
    return kv


def random_doc_cu_seqlens(T: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    return torch.from_numpy(doc_cu_seqlens(seed, T, lo, hi))
