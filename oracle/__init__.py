"""fp64 CPU oracle for the ring-attention step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP path and does not import it.

The arithmetic lives in ``ring_oracle.c`` (plain fp64 loops, OpenMP over
query rows); this module only marshals tensors and adds the two plain
definitions that need no loops over keys:

* ``finalize`` -- out = O / l and lse = m + ln l from a running state
  (Ultralytics glossary page "Ring Attention", section "Come funziona": the
  device divides the accumulated weighted values by the accumulated
  exponentiated scores at the end; the worked example's code divides
  numerator by denominator).
* ``merge`` -- the combination of two normalised partial results through
  their log-sum-exp (GitHub issue "A ring attention with flash attention
  kernel implementation": the returned lse is what lets blockwise attention
  results be combined).  Written as the plain weighted average with weights
  e^{lse_a}, e^{lse_b}, with the larger exponent factored out (Zhihu article
  "Attention的分块计算", local vs. global softmax: shift invariance).

Every function takes torch CPU tensors (float32 or bfloat16; bf16 decodes to
fp64 exactly) in [tokens, heads, dim] layout with any token/head strides and a
unit dim stride, and returns numpy float64 arrays.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ring_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libring_oracle.so")
# A test may point the oracle at another build of ring_oracle.c (for example a
# copy with a planted mistake, to show that the pins catch it).
_LIB_OVERRIDE = os.environ.get("RING_ORACLE_LIB")

MASK_NONE, MASK_CAUSAL, MASK_DOC_CAUSAL = 0, 1, 2
LAYOUT_CONTIGUOUS, LAYOUT_STRIPED = 0, 1
_F32, _BF16 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile ring_oracle.c into libring_oracle.so next to it."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB_PATH
        if not _LIB_OVERRIDE and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        i64, vp, dbl, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
        lib.ro_forward_rows.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64,
                                        i64, i64, i64, i64, i64, i64, dbl, ci, ci, i64, i64,
                                        vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.ro_forward_rows.restype = ci
        lib.ro_block_rows.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64,
                                      i64, i64, i64, i64, i64, i64, vp, vp, dbl, ci, vp, i64, i64,
                                      vp, vp, vp, vp, vp, vp]
        lib.ro_block_rows.restype = ci
        lib.ro_tile_tallies.argtypes = [i64, i64, ci, ci, i64, vp, i64, i64, i64, vp]
        lib.ro_tile_tallies.restype = ci
        lib.ro_allowed_pairs.argtypes = [i64, i64, ci, ci, i64, vp, i64, vp]
        lib.ro_allowed_pairs.restype = ci
        lib.ro_backward.argtypes = [vp, vp, vp, vp, ci, ci, i64, i64, i64, i64,
                                    i64, i64, i64, i64, i64, i64, i64, i64, dbl, ci, ci, i64, i64,
                                    vp, i64, vp, vp, vp, vp]
        lib.ro_backward.restype = ci
        lib.ro_backward_rows.argtypes = [vp, vp, vp, vp, ci, ci, i64, i64, i64, i64,
                                         i64, i64, i64, i64, i64, i64, i64, i64, dbl, ci, ci, i64, i64,
                                         vp, i64, vp, vp, vp, i64, vp, vp, vp]
        lib.ro_backward_rows.restype = ci
        _lib = lib
    return _lib


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return _F32
    if x.dtype == torch.bfloat16:
        return _BF16
    raise TypeError("oracle takes float32, bfloat16 or float16 tensors, got %s" % x.dtype)


def _widen(x: torch.Tensor) -> torch.Tensor:
    """fp16 inputs as fp32 tensors: every binary16 value is exactly a binary32
    value, so the fp64 decode downstream sees the same numbers."""
    return x.float() if isinstance(x, torch.Tensor) and x.dtype == torch.float16 else x


def _key_valid(key_valid, n: int):
    """A key-padding mask as a contiguous uint8 array of n entries (1 = key
    takes part), or None."""
    if key_valid is None:
        return None
    kv = np.ascontiguousarray(np.asarray(key_valid).reshape(-1) != 0, dtype=np.uint8)
    if kv.size != n:
        raise ValueError("key_valid must have %d entries" % n)
    return kv


def _check_view(x: torch.Tensor, name: str):
    if x.device.type != "cpu":
        raise ValueError("%s must be a CPU tensor" % name)
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("%s must be [tokens, heads, dim] with unit dim stride" % name)


def _ptr(a) -> Optional[int]:
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        return a.ctypes.data
    return a.data_ptr()


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None, 0
    cu = torch.as_tensor(cu_seqlens).to(torch.int32).contiguous().cpu()
    return cu, cu.numel() - 1


def forward(q, k, v, *, n_blocks: int, layout: int = LAYOUT_CONTIGUOUS, mask: int = MASK_NONE,
            max_ring_passes: Optional[int] = None, cu_seqlens=None, scale: Optional[float] = None,
            rows: Optional[Sequence] = None, key_valid=None):
    """Attention of every (or each listed) query row over the keys the ring lets
    it see.  Returns dict(out, lse, m, l, O) of float64 arrays.

    key_valid: optional [T] key-padding mask (nonzero = the key takes part).

    Without ``rows``: out/O are [T, Hq, d] and lse/m/l are [Hq, T].
    With ``rows`` = (heads, tokens) index arrays of equal length n: out/O are
    [n, d] and lse/m/l are [n].
    """
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    q, k, v = _widen(q), _widen(k), _widen(v)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_view(x, name)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (T, Hkv, d) or v.shape != (T, Hkv, d):
        raise ValueError("k, v must be [T, Hkv, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    P = n_blocks if max_ring_passes is None else int(max_ring_passes)
    cu, n_docs = _cu(cu_seqlens)
    kv = _key_valid(key_valid, T)
    full = rows is None
    if full:
        hh, tt = np.meshgrid(np.arange(Hq), np.arange(T), indexing="ij")
        row_head = np.ascontiguousarray(hh.reshape(-1), dtype=np.int64)
        row_tok = np.ascontiguousarray(tt.reshape(-1), dtype=np.int64)
    else:
        row_head = np.ascontiguousarray(np.asarray(rows[0]), dtype=np.int64)
        row_tok = np.ascontiguousarray(np.asarray(rows[1]), dtype=np.int64)
    n = row_head.size
    out = np.zeros((n, d))
    O = np.zeros((n, d))
    lse, m, l = np.zeros(n), np.zeros(n), np.zeros(n)
    rc = _load().ro_forward_rows(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), T, Hq, Hkv, d,
        q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
        float(scale), int(mask), int(layout), int(n_blocks), P, _ptr(cu), n_docs, _ptr(kv),
        n, _ptr(row_head), _ptr(row_tok), _ptr(out), _ptr(lse), _ptr(m), _ptr(l), _ptr(O))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    if full:
        return {"out": out.reshape(Hq, T, d).transpose(1, 0, 2), "O": O.reshape(Hq, T, d).transpose(1, 0, 2),
                "lse": lse.reshape(Hq, T), "m": m.reshape(Hq, T), "l": l.reshape(Hq, T)}
    return {"out": out, "O": O, "lse": lse, "m": m, "l": l}


def block(q_blk, k_blk, v_blk, q_pos, k_pos, *, mask: int = MASK_NONE, cu_seqlens=None,
          doc_T: Optional[int] = None, scale: Optional[float] = None, key_valid=None):
    """One query block against one key/value block at explicit global positions.
    Returns dict(out, O: [Hq, nq, d]; lse, m, l: [Hq, nq]).  key_valid:
    optional key-padding mask of the block's own key rows ([nk])."""
    q_blk, k_blk, v_blk = _widen(q_blk), _widen(k_blk), _widen(v_blk)
    for name, x in (("q_blk", q_blk), ("k_blk", k_blk), ("v_blk", v_blk)):
        _check_view(x, name)
    nq, Hq, d = q_blk.shape
    nk, Hkv = k_blk.shape[0], k_blk.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qp = np.ascontiguousarray(np.asarray(q_pos), dtype=np.int64)
    kp = np.ascontiguousarray(np.asarray(k_pos), dtype=np.int64)
    if qp.size != nq or kp.size != nk:
        raise ValueError("position arrays must match block lengths")
    cu, n_docs = _cu(cu_seqlens)
    if doc_T is None:
        doc_T = int(cu[-1]) if cu is not None else 0
    kv = _key_valid(key_valid, nk)  # kept alive across the call
    out = np.zeros((Hq, nq, d))
    O = np.zeros((Hq, nq, d))
    lse, m, l = np.zeros((Hq, nq)), np.zeros((Hq, nq)), np.zeros((Hq, nq))
    rc = _load().ro_block_rows(
        _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _dtype_code(q_blk), nq, nk, Hq, Hkv, d,
        q_blk.stride(0), q_blk.stride(1), k_blk.stride(0), k_blk.stride(1),
        v_blk.stride(0), v_blk.stride(1), _ptr(qp), _ptr(kp), float(scale), int(mask),
        _ptr(cu), n_docs, int(doc_T), _ptr(kv), _ptr(out), _ptr(lse), _ptr(m), _ptr(l), _ptr(O))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return {"out": out, "O": O, "lse": lse, "m": m, "l": l}


def tallies(T: int, n_blocks: int, *, layout: int = LAYOUT_CONTIGUOUS, mask: int = MASK_NONE,
            max_ring_passes: Optional[int] = None, cu_seqlens=None, tile_q: int, tile_k: int):
    """Block-pair and tile classification counts of the ring forward (dict)."""
    cu, n_docs = _cu(cu_seqlens)
    P = n_blocks if max_ring_passes is None else int(max_ring_passes)
    c = np.zeros(7, dtype=np.int64)
    rc = _load().ro_tile_tallies(int(T), int(n_blocks), int(layout), int(mask), P, _ptr(cu), n_docs,
                                 int(tile_q), int(tile_k), _ptr(c))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    keys = ("block_pairs_visited", "block_pairs_skipped", "block_pairs_full",
            "block_pairs_partial", "tiles_skipped", "tiles_full", "tiles_partial")
    return dict(zip(keys, (int(x) for x in c)))


def finalize(O, m, l):
    """out = O / l, lse = m + ln l; a row with l = 0 has out 0 and lse -inf."""
    O = np.asarray(O, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    empty = l == 0
    safe_l = np.where(empty, 1.0, l)
    out = np.where(empty[..., None], 0.0, O / safe_l[..., None])
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m + np.log(safe_l))
    return out, lse


def merge(out_a, lse_a, out_b, lse_b):
    """Combine two normalised partial results over disjoint key sets.

    out = (e^{lse_a} out_a + e^{lse_b} out_b) / (e^{lse_a} + e^{lse_b}) and
    lse = ln(e^{lse_a} + e^{lse_b}); the larger lse is factored out of both
    exponentials first.  A side with lse = -inf has weight 0; both -inf gives
    out 0 and lse -inf.  lse arrays have the shape of out without its last axis.
    """
    out_a = np.asarray(out_a, dtype=np.float64)
    out_b = np.asarray(out_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    big = np.maximum(lse_a, lse_b)
    both_empty = np.isneginf(big)
    ref = np.where(both_empty, 0.0, big)
    wa = np.exp(lse_a - ref)
    wb = np.exp(lse_b - ref)
    tot = wa + wb
    safe = np.where(both_empty, 1.0, tot)
    out = np.where(both_empty[..., None], 0.0, (wa[..., None] * out_a + wb[..., None] * out_b) / safe[..., None])
    with np.errstate(divide="ignore"):
        lse = np.where(both_empty, -np.inf, ref + np.log(safe))
    return out, lse


def allowed_pairs(T: int, n_blocks: int, *, layout: int = LAYOUT_CONTIGUOUS, mask: int = MASK_NONE,
                  max_ring_passes: Optional[int] = None, cu_seqlens=None) -> int:
    """Number of (query, key) pairs per head that the ring forward lets through
    (brute force over all T^2 pairs)."""
    cu, n_docs = _cu(cu_seqlens)
    P = n_blocks if max_ring_passes is None else int(max_ring_passes)
    out = np.zeros(1, dtype=np.int64)
    rc = _load().ro_allowed_pairs(int(T), int(n_blocks), int(layout), int(mask), P, _ptr(cu), n_docs,
                                  _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return int(out[0])


def backward(q, k, v, dout, *, n_blocks: int, layout: int = LAYOUT_CONTIGUOUS, mask: int = MASK_NONE,
             max_ring_passes: Optional[int] = None, cu_seqlens=None, scale: Optional[float] = None,
             rows: Optional[Sequence] = None, rows_dkdv: bool = False, key_valid=None):
    """Gradients (dq, dk, dv) of ``forward``'s output with respect to q, k, v
    for the output gradient ``dout`` ([T, Hq, d], float32, bfloat16 or float16), as
    float64 arrays [T, Hq, d], [T, Hkv, d], [T, Hkv, d].  The arithmetic is in
    ``ring_oracle.c`` (``ro_backward``).

    With ``rows`` = (heads, tokens) index arrays of equal length n (distinct
    pairs), only those query rows' terms are computed (``ro_backward_rows``):
    their dq as an [n, d] array (each equal to the matching row of the full
    dq), and with ``rows_dkdv`` also (dq_rows, dk, dv) where dk / dv sum those
    rows' terms only -- the full dk / dv whenever dout vanishes on every other
    row.  key_valid: optional [T] key-padding mask, as for ``forward``."""
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    q, k, v, dout = _widen(q), _widen(k), _widen(v), _widen(dout)
    for name, x in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check_view(x, name)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (T, Hkv, d) or v.shape != (T, Hkv, d) or dout.shape != (T, Hq, d):
        raise ValueError("k, v must be [T, Hkv, d] and dout [T, Hq, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    P = n_blocks if max_ring_passes is None else int(max_ring_passes)
    cu, n_docs = _cu(cu_seqlens)
    kv = _key_valid(key_valid, T)
    if rows is not None:
        row_head = np.ascontiguousarray(np.asarray(rows[0]), dtype=np.int64)
        row_tok = np.ascontiguousarray(np.asarray(rows[1]), dtype=np.int64)
        if row_head.shape != row_tok.shape or row_head.ndim != 1:
            raise ValueError("rows must be two index arrays of equal length")
        if len(set(zip(row_head.tolist(), row_tok.tolist()))) != row_head.size:
            raise ValueError("rows must be distinct (head, token) pairs")
        out = np.zeros((row_head.size, d))
        dk = np.zeros((T, Hkv, d)) if rows_dkdv else None
        dv = np.zeros((T, Hkv, d)) if rows_dkdv else None
        rc = _load().ro_backward_rows(
            _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _dtype_code(q), _dtype_code(dout), T, Hq, Hkv, d,
            q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
            dout.stride(0), dout.stride(1), float(scale), int(mask), int(layout), int(n_blocks), P,
            _ptr(cu), n_docs, _ptr(kv), _ptr(row_head), _ptr(row_tok), row_head.size, _ptr(out), _ptr(dk), _ptr(dv))
        if rc != 0:
            raise ValueError("oracle rejected the arguments (code %d)" % rc)
        return (out, dk, dv) if rows_dkdv else out
    dq = np.zeros((T, Hq, d))
    dk = np.zeros((T, Hkv, d))
    dv = np.zeros((T, Hkv, d))
    rc = _load().ro_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _dtype_code(q), _dtype_code(dout), T, Hq, Hkv, d,
        q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
        dout.stride(0), dout.stride(1), float(scale), int(mask), int(layout), int(n_blocks), P,
        _ptr(cu), n_docs, _ptr(kv), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle rejected the arguments (code %d)" % rc)
    return dq, dk, dv
