"""Python binding of libring_attn.so, the MI355X ring-attention step library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/ring_attn.h.  torch supplies
device memory and the current stream; tensors must live on the GPU, and a
missing library raises instead of falling back to anything else.

Entry points (same names as the C ABI):
  ring_attn_step, ring_attn_finalize, ring_attn_merge,
  ring_attn_forward_workspace_size, ring_attn_forward, ring_attn_plan,
  ring_attn_tile_shape, ring_attn_backward_workspace_size, ring_attn_backward
plus the conveniences ``forward``, ``forward_qkvpacked`` and ``backward`` that
allocate outputs, lse, gradients and workspace with torch.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch  # loaded first: the library then binds to torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libring_attn.so")

RA_OK, RA_E_ARG, RA_E_UNSUPPORTED, RA_E_HIP, RA_E_WORKSPACE, RA_E_TOO_LARGE = range(6)
RA_F32, RA_BF16, RA_F16 = 0, 1, 2
RA_MASK_NONE, RA_MASK_CAUSAL, RA_MASK_DOC_CAUSAL = 0, 1, 2
RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_STRIPED = 0, 1

_i64, _i32, _vp, _f32, _int, _sz = (ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float,
                                    ctypes.c_int, ctypes.c_size_t)


class RaTensor(ctypes.Structure):
    _fields_ = [("data", _vp), ("dtype", _int), ("n_tok", _i64), ("n_head", _i64), ("head_dim", _i64),
                ("stride_tok", _i64), ("stride_head", _i64)]


class RaStats(ctypes.Structure):
    _fields_ = [("block_pairs_visited", _i64), ("block_pairs_skipped", _i64), ("block_pairs_full", _i64),
                ("block_pairs_partial", _i64), ("tiles_skipped", _i64), ("tiles_full", _i64),
                ("tiles_partial", _i64), ("allowed_pairs", _i64), ("tile_q", _i32), ("tile_k", _i32)]

    def as_dict(self):
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class RingAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load libring_attn.so (built by ``python -m ring_attention_step_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libring_attn.so is not built (run: python -m ring_attention_step_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.ring_attn_step.argtypes = [P(RaTensor), P(RaTensor), P(RaTensor), _vp, _vp, _vp, _int, _f32, _int,
                                   _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp]
    lib.ring_attn_pack_key_mask.argtypes = [_vp, _i64, _i64, _vp, _vp]
    lib.ring_attn_finalize.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp, _int, _i64, _i64, _vp, _vp]
    lib.ring_attn_merge.argtypes = [_vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _vp]
    lib.ring_attn_forward_workspace_size.argtypes = [P(RaTensor), P(RaTensor), _i32, _i32, _int]
    lib.ring_attn_forward_workspace_size.restype = _sz
    lib.ring_attn_forward.argtypes = [P(RaTensor), P(RaTensor), P(RaTensor), _vp, _int, _vp, _i32, _int, _int,
                                      _i32, _vp, _i32, _vp, _f32, _int, _vp, _sz, P(RaStats), _vp]
    lib.ring_attn_forward_noalloc.argtypes = [P(RaTensor), P(RaTensor), P(RaTensor), _vp, _int, _vp, _i32, _int,
                                              _int, _i32, _vp, _i32, _vp, _f32, P(RaStats), _vp]
    lib.ring_attn_forward_noalloc_scratch_bytes.argtypes = []
    lib.ring_attn_forward_noalloc_scratch_bytes.restype = _sz
    lib.ring_attn_test_prefetch_delays.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    lib.ring_attn_test_prefetch_delays.restype = _int
    lib.ring_attn_backward_workspace_size.argtypes = [P(RaTensor), _i32, _i32]
    lib.ring_attn_backward_workspace_size.restype = _sz
    lib.ring_attn_backward.argtypes = [P(RaTensor), P(RaTensor), P(RaTensor), P(RaTensor), P(RaTensor), _vp, _vp,
                                       _vp, _vp, _int, _i32, _int, _int, _i32, _vp, _i32, _vp, _f32, _vp, _sz, _vp]
    lib.ring_attn_plan.argtypes = [_i64, _i32, _int, _int, _i32, _vp, _i32, _int, _i64, P(RaStats)]
    lib.ring_attn_tile_shape.argtypes = [_int, _i64, P(_i32), P(_i32)]
    lib.ring_attn_status_string.argtypes = [_int]
    lib.ring_attn_status_string.restype = ctypes.c_char_p
    for fn in ("ring_attn_step", "ring_attn_finalize", "ring_attn_merge", "ring_attn_forward", "ring_attn_forward_noalloc",
               "ring_attn_plan", "ring_attn_tile_shape", "ring_attn_backward", "ring_attn_pack_key_mask"):
        getattr(lib, fn).restype = _int
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != RA_OK:
        raise RingAttnError(fn, status, load_library().ring_attn_status_string(status).decode())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return RA_F32
    if dt == torch.bfloat16:
        return RA_BF16
    if dt == torch.float16:
        return RA_F16
    raise TypeError("ring attention takes float32, bfloat16 or float16 tensors, got %s" % dt)


def _gpu(x: torch.Tensor, name: str):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)


def _view3(x: torch.Tensor, name: str):
    if not isinstance(x, torch.Tensor) or x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("%s must be a [tokens, heads, head_dim] view with unit head_dim stride" % name)


def _f32_buffer(x, shape, name: str):
    """A contiguous float32 tensor of exactly this shape (the library writes all of it)."""
    if not isinstance(x, torch.Tensor) or tuple(x.shape) != tuple(shape) or x.dtype != torch.float32 \
            or not x.is_contiguous():
        raise ValueError("%s must be a contiguous float32 tensor of shape %s" % (name, list(shape)))


def _forward_operands(q, k, v, out, lse):
    """Shapes, dtypes and layouts of a forward's tensors, checked before any pointer is taken:
    q [T, Hq, d], k / v [T, Hkv, d] views of one dtype, out [T, Hq, d] contiguous (float32 or
    q's dtype), lse None or [Hq, T] float32 contiguous."""
    for x, name in ((q, "q"), (k, "k"), (v, "v")):
        _view3(x, name)
    T, Hq, d = q.shape
    if k.shape[0] != T or k.shape[2] != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [T, Hkv, d] views with q's T and d")
    if Hq % k.shape[1]:
        raise ValueError("q's head count must be a multiple of k's")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    if not isinstance(out, torch.Tensor) or tuple(out.shape) != (T, Hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T, Hq, d] tensor")
    if out.dtype not in (torch.float32, q.dtype):
        raise ValueError("out must be float32 or q's dtype")
    if lse is not None:
        _f32_buffer(lse, (Hq, T), "lse")


def _tensor(x: torch.Tensor, name: str) -> RaTensor:
    _view3(x, name)
    _gpu(x, name)
    return RaTensor(x.data_ptr(), _dtype_code(x.dtype), x.shape[0], x.shape[1], x.shape[2], x.stride(0),
                    x.stride(1))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(x: Optional[torch.Tensor]):
    return None if x is None else x.data_ptr()


def ring_attn_tile_shape(dtype: torch.dtype, head_dim: int):
    tq, tk = _i32(), _i32()
    _check("ring_attn_tile_shape", load_library().ring_attn_tile_shape(_dtype_code(dtype), head_dim,
                                                                        ctypes.byref(tq), ctypes.byref(tk)))
    return tq.value, tk.value


def ring_attn_step(q_blk, k_blk, v_blk, O, m, l, *, first_step: bool, scale: float, mask_mode: int = RA_MASK_NONE,
                   q_offset: int = 0, kv_offset: int = 0, pos_stride: int = 1, cu_seqlens=None,
                   key_bits: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None, stream=None):
    """One ring step on the GPU; O [Hq, Bq, d], m / l [Hq, Bq] fp32 are updated in place.
    cu_seqlens: int32 GPU tensor (doc-causal); key_bits: the key block's padding mask from
    ring_attn_pack_key_mask; stats: int64 GPU tensor of 3 counters (added to)."""
    _view3(q_blk, "q_blk")
    Bq, Hq, d = q_blk.shape
    _f32_buffer(O, (Hq, Bq, d), "O")
    _f32_buffer(m, (Hq, Bq), "m")
    _f32_buffer(l, (Hq, Bq), "l")
    qt, kt, vt = _tensor(q_blk, "q_blk"), _tensor(k_blk, "k_blk"), _tensor(v_blk, "v_blk")
    for x, name in ((O, "O"), (m, "m"), (l, "l")):
        _gpu(x, name)
    n_docs = 0
    if cu_seqlens is not None:
        _gpu(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous int32")
        n_docs = cu_seqlens.numel() - 1
    if stats is not None:
        _gpu(stats, "stats")
        if stats.dtype != torch.int64 or stats.numel() < 3:
            raise ValueError("stats must hold 3 int64 counters")
    if key_bits is not None:
        _gpu(key_bits, "key_bits")
        if key_bits.dtype != torch.int32 or key_bits.numel() < 2 * ((k_blk.shape[0] + 63) // 64):
            raise ValueError("key_bits must be the int32 words ring_attn_pack_key_mask writes for the block")
    st = load_library().ring_attn_step(ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), O.data_ptr(),
                                       m.data_ptr(), l.data_ptr(), int(bool(first_step)), float(scale),
                                       int(mask_mode), int(q_offset), int(kv_offset), int(pos_stride),
                                       _ptr(cu_seqlens), n_docs, _ptr(key_bits), _ptr(stats), _stream(stream))
    _check("ring_attn_step", st)


def ring_attn_pack_key_mask(key_valid: torch.Tensor, *, stream=None) -> torch.Tensor:
    """Key-padding mask of one key block ([n] bool / uint8 GPU tensor, may be strided, nonzero = the key
    takes part) as the int32 bit words ring_attn_step reads (2 * ceil(n / 64) words)."""
    _gpu(key_valid, "key_valid")
    if key_valid.dim() != 1 or key_valid.dtype not in (torch.bool, torch.uint8):
        raise ValueError("key_valid must be a 1-D bool or uint8 tensor")
    n = key_valid.shape[0]
    bits = torch.empty(max(2 * ((n + 63) // 64), 2), device=key_valid.device, dtype=torch.int32)
    _check("ring_attn_pack_key_mask",
           load_library().ring_attn_pack_key_mask(key_valid.data_ptr(), n, max(key_valid.stride(0), 1),
                                                  bits.data_ptr(), _stream(stream)))
    return bits


def _key_valid(key_valid, T: int):
    """A [T] key-padding mask as a contiguous uint8 GPU tensor (or None)."""
    if key_valid is None:
        return None
    _gpu(key_valid, "key_valid")
    if key_valid.dim() != 1 or key_valid.shape[0] != T or key_valid.dtype not in (torch.bool, torch.uint8):
        raise ValueError("key_valid must be a [T] bool or uint8 tensor")
    return key_valid.contiguous().view(torch.uint8)


def ring_attn_finalize(O, m, l, out, lse=None, *, stream=None):
    """out[u, h, :] = O[h, u, :] / l[h, u]; lse[h, u] = m + ln l.  out: [Bq, Hq, d] view."""
    if not isinstance(O, torch.Tensor) or O.dim() != 3:
        raise ValueError("O must be a [Hq, Bq, d] tensor")
    Hq, Bq, d = O.shape
    _f32_buffer(O, (Hq, Bq, d), "O")
    _f32_buffer(m, (Hq, Bq), "m")
    _f32_buffer(l, (Hq, Bq), "l")
    if not isinstance(out, torch.Tensor) or out.dim() != 3 or out.stride(2) != 1 or tuple(out.shape) != (Bq, Hq, d):
        raise ValueError("out must be a [Bq, Hq, d] view with unit last stride")
    if lse is not None:
        _f32_buffer(lse, (Hq, Bq), "lse")
    for x, name in ((O, "O"), (m, "m"), (l, "l"), (out, "out")):
        _gpu(x, name)
    if lse is not None:
        _gpu(lse, "lse")
    st = load_library().ring_attn_finalize(O.data_ptr(), m.data_ptr(), l.data_ptr(), Hq, Bq, d, out.data_ptr(),
                                           _dtype_code(out.dtype), out.stride(0), out.stride(1), _ptr(lse),
                                           _stream(stream))
    _check("ring_attn_finalize", st)


def ring_attn_merge(out_acc, lse_acc, out_blk, lse_blk, *, stream=None):
    """In-place log-sum-exp merge; out_* [rows, Hq, d] contiguous, lse_* [Hq, rows] fp32."""
    for x, name in ((out_acc, "out_acc"), (out_blk, "out_blk")):
        if not isinstance(x, torch.Tensor) or x.dim() != 3 or not x.is_contiguous():
            raise ValueError("%s must be a contiguous [rows, Hq, d] tensor" % name)
    if out_acc.dtype != out_blk.dtype or out_acc.shape != out_blk.shape:
        raise ValueError("out_acc and out_blk must match")
    rows, Hq, d = out_acc.shape
    _f32_buffer(lse_acc, (Hq, rows), "lse_acc")
    _f32_buffer(lse_blk, (Hq, rows), "lse_blk")
    for x, name in ((out_acc, "out_acc"), (lse_acc, "lse_acc"), (out_blk, "out_blk"), (lse_blk, "lse_blk")):
        _gpu(x, name)
    st = load_library().ring_attn_merge(out_acc.data_ptr(), lse_acc.data_ptr(), out_blk.data_ptr(),
                                        lse_blk.data_ptr(), _dtype_code(out_acc.dtype), Hq, rows, d,
                                        _stream(stream))
    _check("ring_attn_merge", st)


def ring_attn_forward_workspace_size(q, k, n_blocks: int, n_docs: int = 0, prefetch: bool = False) -> int:
    qt, kt = _tensor(q, "q"), _tensor(k, "k")
    return int(load_library().ring_attn_forward_workspace_size(ctypes.byref(qt), ctypes.byref(kt), int(n_blocks),
                                                               int(n_docs), int(bool(prefetch))))


def ring_attn_forward(q, k, v, out, lse, *, n_blocks: int, layout: int, mask_mode: int, max_ring_passes: int,
                      cu_seqlens_host=None, key_valid=None, scale: float, prefetch: bool, workspace: torch.Tensor,
                      want_stats: bool = False, stream=None):
    """The whole one-GPU ring; out [T, Hq, d] contiguous; lse [Hq, T] fp32 or None.
    Returns the tallies (dict) when want_stats (this synchronises the stream)."""
    _forward_operands(q, k, v, out, lse)
    qt, kt, vt = _tensor(q, "q"), _tensor(k, "k"), _tensor(v, "v")
    _gpu(out, "out")
    if lse is not None:
        _gpu(lse, "lse")
    _gpu(workspace, "workspace")
    cu_ptr, n_docs, cu_keep = None, 0, None
    if cu_seqlens_host is not None:
        cu_keep = torch.as_tensor(cu_seqlens_host).to(device="cpu", dtype=torch.int32).contiguous()
        cu_ptr, n_docs = cu_keep.data_ptr(), cu_keep.numel() - 1
    kv = _key_valid(key_valid, q.shape[0])
    stats = RaStats()
    st = load_library().ring_attn_forward(
        ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), out.data_ptr(), _dtype_code(out.dtype), _ptr(lse),
        int(n_blocks), int(layout), int(mask_mode), int(max_ring_passes), cu_ptr, n_docs, _ptr(kv), float(scale),
        int(bool(prefetch)), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        ctypes.byref(stats) if want_stats else None, _stream(stream))
    _check("ring_attn_forward", st)
    return stats.as_dict() if want_stats else None


def ring_attn_forward_noalloc(q, k, v, out, lse, *, n_blocks: int, layout: int, mask_mode: int,
                              max_ring_passes: int, cu_seqlens_host=None, key_valid=None, scale: float,
                              want_stats: bool = False, stream=None):
    """ring_attn_forward (no prefetch) in the library's fixed per-GPU scratch: no device memory is
    allocated, here or in the library.  key_valid, when given, must already be a contiguous [T]
    bool / uint8 GPU tensor.  Overlapping calls on one GPU race for the scratch."""
    _forward_operands(q, k, v, out, lse)
    qt, kt, vt = _tensor(q, "q"), _tensor(k, "k"), _tensor(v, "v")
    _gpu(out, "out")
    if lse is not None:
        _gpu(lse, "lse")
    cu_ptr, n_docs, cu_keep = None, 0, None
    if cu_seqlens_host is not None:
        cu_keep = torch.as_tensor(cu_seqlens_host).to(device="cpu", dtype=torch.int32).contiguous()
        cu_ptr, n_docs = cu_keep.data_ptr(), cu_keep.numel() - 1
    kv_ptr = None
    if key_valid is not None:
        _gpu(key_valid, "key_valid")
        if key_valid.dim() != 1 or key_valid.shape[0] != q.shape[0] or not key_valid.is_contiguous() \
                or key_valid.dtype not in (torch.bool, torch.uint8):
            raise ValueError("key_valid must be a contiguous [T] bool or uint8 tensor")
        kv_ptr = key_valid.data_ptr()
    stats = RaStats()
    st = load_library().ring_attn_forward_noalloc(
        ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), out.data_ptr(), _dtype_code(out.dtype), _ptr(lse),
        int(n_blocks), int(layout), int(mask_mode), int(max_ring_passes), cu_ptr, n_docs, kv_ptr, float(scale),
        ctypes.byref(stats) if want_stats else None, _stream(stream))
    _check("ring_attn_forward_noalloc", st)
    return stats.as_dict() if want_stats else None


def ring_attn_test_prefetch_delays(copy_delay_us: int, compute_delay_us: int):
    """Test hook: bounded waits before every prefetch step's copies (copy stream) and compute
    (caller's stream); 0 turns them off."""
    _check("ring_attn_test_prefetch_delays",
           load_library().ring_attn_test_prefetch_delays(int(copy_delay_us), int(compute_delay_us)))


def ring_attn_forward_noalloc_scratch_bytes() -> int:
    return int(load_library().ring_attn_forward_noalloc_scratch_bytes())


def ring_attn_backward_workspace_size(q, n_blocks: int, n_docs: int = 0) -> int:
    qt = _tensor(q, "q")
    return int(load_library().ring_attn_backward_workspace_size(ctypes.byref(qt), int(n_blocks), int(n_docs)))


def ring_attn_backward(q, k, v, out, dout, lse, dq, dk, dv, *, n_blocks: int, layout: int, mask_mode: int,
                       max_ring_passes: int, cu_seqlens_host=None, key_valid=None, scale: float,
                       workspace: torch.Tensor, stream=None):
    """Gradients of the ring forward: dq [T, Hq, d], dk / dv [T, Hkv, d] (contiguous, fp32 or the inputs' 16-bit type, written
    in full) from the forward's out [T, Hq, d] and lse [Hq, T] and the output gradient dout [T, Hq, d]."""
    qt, kt, vt = _tensor(q, "q"), _tensor(k, "k"), _tensor(v, "v")
    ot, gt = _tensor(out, "out"), _tensor(dout, "dout")
    _gpu(lse, "lse")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (q.shape[1], q.shape[0]):
        raise ValueError("lse must be contiguous float32 [Hq, T]")
    for x, name, shape in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape)):
        _gpu(x, name)
        if not x.is_contiguous() or tuple(x.shape) != tuple(shape):
            raise ValueError("%s must be contiguous with shape %s" % (name, tuple(shape)))
    if not (dq.dtype == dk.dtype == dv.dtype):
        raise ValueError("dq, dk, dv must share a dtype")
    _gpu(workspace, "workspace")
    cu_ptr, n_docs, cu_keep = None, 0, None
    if cu_seqlens_host is not None:
        cu_keep = torch.as_tensor(cu_seqlens_host).to(device="cpu", dtype=torch.int32).contiguous()
        cu_ptr, n_docs = cu_keep.data_ptr(), cu_keep.numel() - 1
    kv = _key_valid(key_valid, q.shape[0])
    st = load_library().ring_attn_backward(
        ctypes.byref(qt), ctypes.byref(kt), ctypes.byref(vt), ctypes.byref(ot), ctypes.byref(gt), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _dtype_code(dq.dtype), int(n_blocks), int(layout),
        int(mask_mode), int(max_ring_passes), cu_ptr, n_docs, _ptr(kv), float(scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("ring_attn_backward", st)


def ring_attn_plan(T: int, n_blocks: int, *, layout: int, mask_mode: int, max_ring_passes: int,
                   cu_seqlens_host=None, dtype: torch.dtype, head_dim: int) -> dict:
    """Host-only: tallies and allowed-pair count the forward would produce."""
    cu_ptr, n_docs, cu_keep = None, 0, None
    if cu_seqlens_host is not None:
        cu_keep = torch.as_tensor(cu_seqlens_host).to(device="cpu", dtype=torch.int32).contiguous()
        cu_ptr, n_docs = cu_keep.data_ptr(), cu_keep.numel() - 1
    stats = RaStats()
    st = load_library().ring_attn_plan(int(T), int(n_blocks), int(layout), int(mask_mode), int(max_ring_passes),
                                       cu_ptr, n_docs, _dtype_code(dtype), int(head_dim), ctypes.byref(stats))
    _check("ring_attn_plan", st)
    return stats.as_dict()


_LAYOUTS = {"contiguous": RA_LAYOUT_CONTIGUOUS, "striped": RA_LAYOUT_STRIPED}


def forward(q, k, v, *, n_blocks: int, layout: str = "contiguous", causal: bool = False, cu_seqlens=None,
            max_ring_passes: Optional[int] = None, scale: Optional[float] = None, prefetch: bool = False,
            out_dtype: Optional[torch.dtype] = None, return_lse: bool = False, return_stats: bool = False,
            key_valid: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Ring attention over q [T, Hq, d], k / v [T, Hkv, d] on one GPU as n_blocks virtual devices.
    cu_seqlens (documents, implies per-document causal) may be a CPU or GPU int tensor or a list;
    key_valid: optional [T] bool / uint8 GPU tensor, a key-padding mask (False = padded key)."""
    T, Hq, d = q.shape
    mask = RA_MASK_NONE
    if causal:
        mask = RA_MASK_CAUSAL
    if cu_seqlens is not None:
        mask = RA_MASK_DOC_CAUSAL
        cu_seqlens = torch.as_tensor(cu_seqlens).to(device="cpu", dtype=torch.int32)
    n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    P = n_blocks if max_ring_passes is None else max_ring_passes
    out = torch.empty(T, Hq, d, device=q.device, dtype=out_dtype or q.dtype)
    lse = torch.empty(Hq, T, device=q.device, dtype=torch.float32) if return_lse else None
    ws_bytes = ring_attn_forward_workspace_size(q, k, n_blocks, n_docs, prefetch)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    stats = ring_attn_forward(q, k, v, out, lse, n_blocks=n_blocks, layout=_LAYOUTS[layout], mask_mode=mask,
                              max_ring_passes=P, cu_seqlens_host=cu_seqlens, key_valid=key_valid, scale=scale,
                              prefetch=prefetch, workspace=workspace, want_stats=return_stats)
    res = [out]
    if return_lse:
        res.append(lse)
    if return_stats:
        res.append(stats)
    return res[0] if len(res) == 1 else tuple(res)


def forward_qkvpacked(qkv, **kw):
    """Ring attention over a packed [T, 3, H, d] tensor (read through strided views, no copy)."""
    if qkv.dim() != 4 or qkv.shape[1] != 3:
        raise ValueError("qkv must be [T, 3, H, d]")
    return forward(qkv[:, 0], qkv[:, 1], qkv[:, 2], **kw)


def backward(q, k, v, out, lse, dout, *, n_blocks: int, layout: str = "contiguous", causal: bool = False,
             cu_seqlens=None, max_ring_passes: Optional[int] = None, scale: Optional[float] = None,
             grad_dtype: torch.dtype = torch.float32, key_valid: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None):
    """(dq, dk, dv) of ``forward(q, k, v, ...)`` for the output gradient dout, given that call's out and lse
    (return_lse=True) and the same ring arguments."""
    T, Hq, d = q.shape
    mask = RA_MASK_NONE
    if causal:
        mask = RA_MASK_CAUSAL
    if cu_seqlens is not None:
        mask = RA_MASK_DOC_CAUSAL
        cu_seqlens = torch.as_tensor(cu_seqlens).to(device="cpu", dtype=torch.int32)
    n_docs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    P = n_blocks if max_ring_passes is None else max_ring_passes
    dq = torch.empty(T, Hq, d, device=q.device, dtype=grad_dtype)
    dk = torch.empty(k.shape, device=q.device, dtype=grad_dtype)
    dv = torch.empty(k.shape, device=q.device, dtype=grad_dtype)
    ws_bytes = ring_attn_backward_workspace_size(q, n_blocks, n_docs)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(ws_bytes, device=q.device, dtype=torch.uint8)
    ring_attn_backward(q, k, v, out, dout, lse, dq, dk, dv, n_blocks=n_blocks, layout=_LAYOUTS[layout],
                       mask_mode=mask, max_ring_passes=P, cu_seqlens_host=cu_seqlens, key_valid=key_valid,
                       scale=scale, workspace=workspace)
    return dq, dk, dv


__all__ = ["ring_attn_step", "ring_attn_finalize", "ring_attn_merge", "ring_attn_forward_workspace_size",
           "ring_attn_forward", "ring_attn_plan", "ring_attn_tile_shape", "ring_attn_backward_workspace_size",
           "ring_attn_backward", "ring_attn_pack_key_mask", "forward", "forward_qkvpacked", "backward",
           "ring_attn_forward_noalloc", "ring_attn_forward_noalloc_scratch_bytes", "load_library", "RingAttnError"]
