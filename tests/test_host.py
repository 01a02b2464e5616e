"""CPU tests of the C-ABI library's host side: it loads and exports every
symbol its header declares, its planner's tallies and pair counts equal the
oracle's brute force, and bad arguments are refused before any GPU work."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
import workloads as W
import ring_attention_step_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")


@pytest.fixture(scope="module")
def lib():
    return ra.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ring_attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for fn in ("ring_attn_step", "ring_attn_finalize", "ring_attn_merge", "ring_attn_forward",
               "ring_attn_forward_workspace_size", "ring_attn_plan", "ring_attn_tile_shape",
               "ring_attn_status_string", "ring_attn_backward", "ring_attn_backward_workspace_size"):
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    for fn in _declared_functions():
        assert hasattr(lib, fn), fn


def test_library_links_no_torch():
    import subprocess
    out = subprocess.run(["readelf", "-d", ra.library_path()], capture_output=True, text=True).stdout
    needed = re.findall(r"\[(.*?)\]", "\n".join(l for l in out.splitlines() if "NEEDED" in l))
    assert not any("torch" in n or "c10" in n for n in needed), needed


def test_status_strings(lib):
    for s in range(6):
        assert lib.ring_attn_status_string(s)


def test_tile_shapes():
    assert ra.ring_attn_tile_shape(torch.bfloat16, 128) == (256, 64)
    assert ra.ring_attn_tile_shape(torch.bfloat16, 64) == (256, 64)
    assert ra.ring_attn_tile_shape(torch.float32, 16) == (64, 64)
    with pytest.raises(ra.RingAttnError):
        ra.ring_attn_tile_shape(torch.bfloat16, 96)
    with pytest.raises(ra.RingAttnError):
        ra.ring_attn_tile_shape(torch.float32, 200)


PLAN_CASES = [
    # T, N, layout, mask, P, dtype, d, cu
    (32, 4, 0, 0, 4, torch.float32, 16, None),
    (1024, 16, 0, 0, 16, torch.float32, 2, None),
    (888, 3, 0, 1, 3, torch.bfloat16, 128, None),
    (888, 3, 1, 1, 3, torch.bfloat16, 128, None),
    (1200, 4, 0, 1, 2, torch.bfloat16, 64, None),
    (1200, 4, 1, 0, 3, torch.bfloat16, 64, None),
    (960, 4, 0, 2, 4, torch.bfloat16, 128, [0, 100, 101, 400, 700, 960]),
    (960, 4, 0, 2, 1, torch.float32, 8, [0, 100, 101, 400, 700, 960]),
    (4096, 8, 0, 2, 4, torch.bfloat16, 128, "random"),
    (640, 5, 1, 1, 9, torch.float32, 32, None),
]


@pytest.mark.parametrize("case", range(len(PLAN_CASES)))
def test_plan_matches_oracle_brute_force(case):
    T, N, layout, mask, P, dt, d, cu = PLAN_CASES[case]
    if cu == "random":
        cu = W.random_doc_cu_seqlens(T, 64, 700, seed=case).tolist()
    tq, tk = ra.ring_attn_tile_shape(dt, d)
    got = ra.ring_attn_plan(T, N, layout=layout, mask_mode=mask, max_ring_passes=P, cu_seqlens_host=cu,
                            dtype=dt, head_dim=d)
    want = oracle.tallies(T, N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=cu, tile_q=tq, tile_k=tk)
    for key, val in want.items():
        assert got[key] == val, key
    assert got["allowed_pairs"] == oracle.allowed_pairs(T, N, layout=layout, mask=mask, max_ring_passes=P,
                                                        cu_seqlens=cu)
    assert (got["tile_q"], got["tile_k"]) == (tq, tk)


@pytest.mark.parametrize("name", ["causal32k_h32_d128_8blk", "gqa_striped64k_h32kv8_d128_16blk",
                                  "varlen_packed128k_h32_d128_8blk_p4"])
def test_plan_matches_oracle_on_long_workloads(name):
    w = W.WORKLOADS[name]
    cu = W.doc_cu_seqlens(w.seed, w.T, *w.doc_len_range).tolist() if w.doc_len_range else None
    dt = torch.bfloat16
    got = ra.ring_attn_plan(w.T, w.n_blocks, layout=w.layout, mask_mode=w.mask, max_ring_passes=w.max_ring_passes,
                            cu_seqlens_host=cu, dtype=dt, head_dim=w.d)
    want = oracle.tallies(w.T, w.n_blocks, layout=w.layout, mask=w.mask, max_ring_passes=w.max_ring_passes,
                          cu_seqlens=cu, tile_q=got["tile_q"], tile_k=got["tile_k"])
    for key, val in want.items():
        assert got[key] == val, key
    if name != "varlen_packed128k_h32_d128_8blk_p4":
        assert got["allowed_pairs"] == w.T * (w.T + 1) // 2
    else:
        assert got["allowed_pairs"] == oracle.allowed_pairs(w.T, w.n_blocks, mask=w.mask,
                                                            max_ring_passes=w.max_ring_passes, cu_seqlens=cu)


def test_plan_rejects_bad_arguments():
    bad = [
        dict(T=30, n_blocks=4),                                  # T % N
        dict(T=32, n_blocks=4, max_ring_passes=0),
        dict(T=32, n_blocks=4, mask_mode=2),                     # doc mask without cu_seqlens
        dict(T=32, n_blocks=4, mask_mode=2, cu_seqlens_host=[0, 10, 31]),  # does not end at T
        dict(T=32, n_blocks=4, mask_mode=2, cu_seqlens_host=[0, 20, 10, 32]),  # decreasing
        dict(T=32, n_blocks=4, layout=7),
    ]
    for b in bad:
        kw = dict(layout=0, mask_mode=0, max_ring_passes=4, cu_seqlens_host=None, dtype=torch.float32, head_dim=16)
        kw.update({k: v for k, v in b.items() if k not in ("T", "n_blocks")})
        with pytest.raises(ra.RingAttnError) as e:
            ra.ring_attn_plan(b["T"], b["n_blocks"], **kw)
        assert e.value.status == ra.RA_E_ARG
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_plan(32, 4, layout=1, mask_mode=2, max_ring_passes=4, cu_seqlens_host=[0, 32],
                          dtype=torch.float32, head_dim=16)
    assert e.value.status == ra.RA_E_UNSUPPORTED


def _fake(T, H, d, dtype=ra.RA_BF16, ptr=1 << 20, st=None):
    st = st if st is not None else H * d
    return ra.RaTensor(ptr, dtype, T, H, d, st, d)


def test_forward_and_step_refuse_bad_arguments_before_any_gpu_work(lib):
    # Fake (never dereferenced) device addresses: every call below must fail
    # argument checks before touching the GPU.
    q, k, v = _fake(64, 4, 128), _fake(64, 2, 128), _fake(64, 2, 128)
    out, ws = ctypes.c_void_p(1 << 21), ctypes.c_void_p(1 << 22)
    F = lib.ring_attn_forward
    R = ctypes.byref

    def fwd(qq=q, kk=k, vv=v, n_blocks=4, layout=0, mask=1, P=4, cu=None, n_docs=0, scale=0.1, ws_bytes=1 << 40,
            out_dtype=ra.RA_BF16, o=out, kv=None):
        return F(R(qq), R(kk), R(vv), o, out_dtype, None, n_blocks, layout, mask, P, cu, n_docs, kv, scale, 0, ws,
                 ws_bytes, None, None)

    assert fwd(n_blocks=5) == ra.RA_E_ARG             # 64 % 5
    assert fwd(P=0) == ra.RA_E_ARG
    assert fwd(scale=0.0) == ra.RA_E_ARG
    assert fwd(scale=float("nan")) == ra.RA_E_ARG
    assert fwd(kk=_fake(64, 3, 128)) == ra.RA_E_ARG   # 4 % 3
    assert fwd(vv=_fake(60, 2, 128)) == ra.RA_E_ARG
    assert fwd(o=None) == ra.RA_E_ARG
    assert fwd(mask=2) == ra.RA_E_ARG                 # no cu_seqlens
    assert fwd(qq=_fake(64, 4, 96), kk=_fake(64, 2, 96), vv=_fake(64, 2, 96)) == ra.RA_E_UNSUPPORTED
    assert fwd(qq=_fake(64, 4, 128, ptr=(1 << 20) + 2)) == ra.RA_E_UNSUPPORTED  # misaligned bf16
    f32 = [_fake(64, 4, 16, ra.RA_F32), _fake(64, 2, 16, ra.RA_F32), _fake(64, 2, 16, ra.RA_F32)]
    assert fwd(*f32, out_dtype=ra.RA_BF16) == ra.RA_E_UNSUPPORTED
    h16 = [_fake(64, 4, 128, ra.RA_F16), _fake(64, 2, 128, ra.RA_F16), _fake(64, 2, 128, ra.RA_F16)]
    assert fwd(*h16, out_dtype=ra.RA_BF16) == ra.RA_E_UNSUPPORTED  # 16-bit out must be the inputs' type
    assert fwd(*h16, out_dtype=ra.RA_F16, ws_bytes=16) == ra.RA_E_WORKSPACE  # fp16 passes the checks
    assert fwd(h16[0], k, v) == ra.RA_E_ARG           # mixed input types
    assert fwd(out_dtype=3) == ra.RA_E_ARG
    assert fwd(ws_bytes=16) == ra.RA_E_WORKSPACE
    cu = (ctypes.c_int32 * 3)(0, 10, 64)
    assert fwd(mask=2, cu=cu, n_docs=2, layout=1) == ra.RA_E_UNSUPPORTED
    cu_bad = (ctypes.c_int32 * 3)(0, 70, 64)
    assert fwd(mask=2, cu=cu_bad, n_docs=2) == ra.RA_E_ARG

    S = lib.ring_attn_step
    state = ctypes.c_void_p(1 << 23)
    assert S(R(q), R(k), R(v), state, state, state, 1, -1.0, 0, 0, 0, 1, None, 0, None, None, None) == ra.RA_E_ARG
    assert S(R(q), R(k), R(v), None, state, state, 1, 0.1, 0, 0, 0, 1, None, 0, None, None, None) == ra.RA_E_ARG
    assert S(R(q), R(k), R(v), state, state, state, 1, 0.1, 0, 0, 0, 0, None, 0, None, None, None) == ra.RA_E_ARG
    assert S(R(q), R(k), R(v), state, state, state, 1, 0.1, 2, 0, 0, 1, None, 0, None, None, None) == ra.RA_E_ARG
    assert S(R(q), R(_fake(64, 2, 64)), R(v), state, state, state, 1, 0.1, 0, 0, 0, 1, None, 0, None, None,
             None) == ra.RA_E_ARG
    bits_misaligned = ctypes.c_void_p((1 << 24) + 4)
    assert S(R(q), R(k), R(v), state, state, state, 1, 0.1, 0, 0, 0, 1, None, 0, bits_misaligned, None,
             None) == ra.RA_E_ARG
    P_ = lib.ring_attn_pack_key_mask
    assert P_(None, 64, 1, ctypes.c_void_p(1 << 24), None) == ra.RA_E_ARG
    assert P_(ctypes.c_void_p(1 << 23), 64, 0, ctypes.c_void_p(1 << 24), None) == ra.RA_E_ARG
    assert P_(ctypes.c_void_p(1 << 23), 64, 1, bits_misaligned, None) == ra.RA_E_ARG


def test_empty_sequence_needs_no_buffers_and_launches_nothing(lib):
    """T = 0 (torch gives empty tensors a null data pointer): every entry point
    returns RA_OK before any GPU call, the forward's tallies all zero."""
    R = ctypes.byref
    q, k = _fake(0, 4, 128, ptr=0), _fake(0, 2, 128, ptr=0)
    ws = ctypes.c_void_p(1 << 22)
    st = ra.RaStats()
    assert lib.ring_attn_forward(R(q), R(k), R(k), None, ra.RA_BF16, None, 4, 0, 1, 4, None, 0, None, 0.1, 0, ws,
                                 1 << 40, R(st), None) == ra.RA_OK
    assert st.as_dict()["tiles_full"] == 0 and st.as_dict()["allowed_pairs"] == 0 and st.tile_q > 0
    assert lib.ring_attn_backward(R(q), R(k), R(k), R(q), R(q), None, None, None, None, ra.RA_F32, 4, 0, 1, 4,
                                  None, 0, None, 0.1, ws, 1 << 40, None) == ra.RA_OK
    assert lib.ring_attn_step(R(q), R(k), R(k), None, None, None, 1, 0.1, 1, 0, 0, 1, None, 0, None, None,
                              None) == ra.RA_OK
    # no workspace either
    assert lib.ring_attn_forward(R(q), R(k), R(k), None, ra.RA_BF16, None, 4, 0, 1, 4, None, 0, None, 0.1, 0, None,
                                 0, None, None) == ra.RA_OK
    assert lib.ring_attn_backward(R(q), R(k), R(k), R(q), R(q), None, None, None, None, ra.RA_F32, 4, 0, 1, 4,
                                  None, 0, None, 0.1, None, 0, None) == ra.RA_OK
    # an empty block's state, and an empty merge, with NULL pointers
    assert lib.ring_attn_finalize(None, None, None, 4, 0, 128, None, ra.RA_BF16, 512, 128, None, None) == ra.RA_OK
    assert lib.ring_attn_merge(None, None, None, None, ra.RA_BF16, 4, 0, 128, None) == ra.RA_OK
    # a non-empty one still needs them
    assert lib.ring_attn_finalize(None, None, None, 4, 1, 128, None, ra.RA_BF16, 512, 128, None, None) == ra.RA_E_ARG
    assert lib.ring_attn_merge(None, None, None, None, ra.RA_BF16, 4, 1, 128, None) == ra.RA_E_ARG


def test_workspace_size_grows_with_prefetch(lib):
    q, k = _fake(4096, 32, 128), _fake(4096, 8, 128)
    a = lib.ring_attn_forward_workspace_size(ctypes.byref(q), ctypes.byref(k), 8, 0, 0)
    b = lib.ring_attn_forward_workspace_size(ctypes.byref(q), ctypes.byref(k), 8, 0, 1)
    state = 4096 * 32 * 128 * 4 + 2 * 4096 * 32 * 4
    # prefetch adds the per-step state and the K / V^T double buffers
    assert b >= a + state + 2 * 2 * 4096 * 8 * 128 * 2


def _ws(lib, T, Hq, Hkv, d, N, dtype, prefetch=0):
    q, k = _fake(T, Hq, d, dtype), _fake(T, Hkv, d, dtype)
    return lib.ring_attn_forward_workspace_size(ctypes.byref(q), ctypes.byref(k), N, 0, prefetch)


def test_one_launch_workspace_has_no_per_step_state(lib):
    # Causal 32K tokens, 32 heads, d = 128, 8 blocks in bf16: the one-launch
    # ring keeps O / m / l in registers, so the workspace is the packed V^T
    # (32768 x 32 x 128 x 2 bytes, keys padded per block) and small tables;
    # the fp32 state planes (512 MiB + 8 MiB) appear only where the per-step
    # path can run.
    T, H, d, N = 32768, 32, 128, 8
    state = T * H * d * 4 + 2 * T * H * 4
    vt = T * H * d * 2
    ws16 = _ws(lib, T, H, H, d, N, ra.RA_BF16)
    assert vt <= ws16 < vt + (8 << 20)
    assert _ws(lib, T, H, H, d, N, ra.RA_F16) == ws16
    assert _ws(lib, T, H, H, d, N, ra.RA_F32) >= state               # fp32 inputs: per-step path
    assert _ws(lib, T, H, H, d, N, ra.RA_BF16, prefetch=1) >= ws16 + state
    assert _ws(lib, T, H, H, d, 128, ra.RA_BF16) >= vt + state       # chains longer than 64 blocks
    assert _ws(lib, T, H, H, d, 64, ra.RA_BF16) < vt + (8 << 20)


def test_backward_refuses_bad_arguments_before_any_gpu_work(lib):
    q, k, v = _fake(64, 4, 128), _fake(64, 2, 128), _fake(64, 2, 128)
    out, dout = _fake(64, 4, 128), _fake(64, 4, 128)
    lse, g, ws = ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 25), ctypes.c_void_p(1 << 26)
    R = ctypes.byref

    def bwd(qq=q, kk=k, vv=v, oo=out, gg=dout, ll=lse, dq=g, n_blocks=4, layout=0, mask=1, P=4, cu=None,
            n_docs=0, scale=0.1, ws_bytes=1 << 40, grad=ra.RA_F32):
        return lib.ring_attn_backward(R(qq), R(kk), R(vv), R(oo), R(gg), ll, dq, g, g, grad, n_blocks, layout,
                                      mask, P, cu, n_docs, None, scale, ws, ws_bytes, None)

    assert bwd(n_blocks=5) == ra.RA_E_ARG             # 64 % 5
    assert bwd(P=0) == ra.RA_E_ARG
    assert bwd(scale=-1.0) == ra.RA_E_ARG
    assert bwd(ll=None) == ra.RA_E_ARG
    assert bwd(dq=None) == ra.RA_E_ARG
    assert bwd(gg=_fake(64, 2, 128)) == ra.RA_E_ARG   # dout heads != q heads
    assert bwd(oo=_fake(32, 4, 128)) == ra.RA_E_ARG
    assert bwd(kk=_fake(64, 3, 128)) == ra.RA_E_ARG
    assert bwd(mask=2) == ra.RA_E_ARG                 # no cu_seqlens
    assert bwd(grad=7) == ra.RA_E_ARG
    f32 = dict(qq=_fake(64, 4, 16, ra.RA_F32), kk=_fake(64, 2, 16, ra.RA_F32), vv=_fake(64, 2, 16, ra.RA_F32),
               oo=_fake(64, 4, 16, ra.RA_F32), gg=_fake(64, 4, 16, ra.RA_F32))
    assert bwd(**f32) == ra.RA_E_UNSUPPORTED          # fp32 inputs: no backward kernel
    h16 = dict(qq=_fake(64, 4, 128, ra.RA_F16), kk=_fake(64, 2, 128, ra.RA_F16), vv=_fake(64, 2, 128, ra.RA_F16),
               gg=_fake(64, 4, 128, ra.RA_F16))
    assert bwd(grad=ra.RA_BF16, **h16) == ra.RA_E_UNSUPPORTED  # 16-bit gradients take the inputs' type
    assert bwd(oo=_fake(64, 4, 128, ra.RA_BF16), **h16) == ra.RA_E_UNSUPPORTED  # so does a 16-bit out
    assert bwd(oo=_fake(64, 4, 128, ra.RA_F16), grad=ra.RA_F16, ws_bytes=16, **h16) == ra.RA_E_WORKSPACE
    assert bwd(gg=_fake(64, 4, 128, ra.RA_F16)) == ra.RA_E_ARG  # dout type differs from q's
    assert bwd(qq=_fake(64, 4, 96), kk=_fake(64, 2, 96), vv=_fake(64, 2, 96), oo=_fake(64, 4, 96),
               gg=_fake(64, 4, 96)) == ra.RA_E_UNSUPPORTED
    assert bwd(qq=_fake(64, 4, 128, ptr=(1 << 20) + 2)) == ra.RA_E_UNSUPPORTED
    assert bwd(dq=ctypes.c_void_p((1 << 25) + 8)) == ra.RA_E_UNSUPPORTED
    big = dict(qq=_fake(128, 4, 128), kk=_fake(128, 2, 128), vv=_fake(128, 2, 128), oo=_fake(128, 4, 128),
               gg=_fake(128, 4, 128))
    assert bwd(n_blocks=128, P=1, **big) == ra.RA_E_UNSUPPORTED  # more ring blocks than lanes
    huge = dict(qq=_fake(1 << 31, 4, 128), kk=_fake(1 << 31, 2, 128), vv=_fake(1 << 31, 2, 128),
                oo=_fake(1 << 31, 4, 128), gg=_fake(1 << 31, 4, 128))
    assert bwd(n_blocks=64, P=1, **huge) == ra.RA_E_UNSUPPORTED  # positions beyond 32 bits
    long_blk = dict(qq=_fake(1 << 21, 4, 128), kk=_fake(1 << 21, 2, 128), vv=_fake(1 << 21, 2, 128),
                    oo=_fake(1 << 21, 4, 128), gg=_fake(1 << 21, 4, 128))
    assert bwd(n_blocks=1, P=1, **long_blk) == ra.RA_E_UNSUPPORTED  # 2^21 rows in one block
    assert bwd(ws_bytes=16) == ra.RA_E_WORKSPACE
    cu = (ctypes.c_int32 * 3)(0, 10, 64)
    assert bwd(mask=2, cu=cu, n_docs=2, layout=1) == ra.RA_E_UNSUPPORTED


def test_backward_workspace_size(lib):
    q = _fake(4096, 32, 128)
    n = lib.ring_attn_backward_workspace_size(ctypes.byref(q), 8, 0)
    assert n >= 4096 * 32 * 4 + 2 * 8 * 8 * 8
    assert lib.ring_attn_backward_workspace_size(ctypes.byref(q), 3, 0) == 0   # 4096 % 3
    assert lib.ring_attn_backward_workspace_size(ctypes.byref(q), 8, 1000) > n


def test_noalloc_forward_refuses_shapes_beyond_its_scratch_before_any_gpu_work(lib):
    # 65536 tokens x 8 kv heads x d 128 in bf16: the packed V^T alone is
    # 128 MiB, over the fixed 64 MiB scratch; fake (never dereferenced)
    # addresses, refused before any HIP call.
    assert lib.ring_attn_forward_noalloc_scratch_bytes() == 64 << 20
    q, k = _fake(65536, 8, 128), _fake(65536, 8, 128)
    R = ctypes.byref
    assert lib.ring_attn_forward_noalloc(R(q), R(k), R(k), ctypes.c_void_p(1 << 21), ra.RA_BF16, None, 8, 0, 1, 8,
                                         None, 0, None, 0.1, None, None) == ra.RA_E_TOO_LARGE


def test_prefetch_delay_hook_bounds(lib):
    assert lib.ring_attn_test_prefetch_delays(100001, 0) == ra.RA_E_ARG
    assert lib.ring_attn_test_prefetch_delays(0, 100001) == ra.RA_E_ARG
    assert lib.ring_attn_test_prefetch_delays(0, 0) == ra.RA_OK
