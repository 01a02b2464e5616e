"""GPU test of ring_attn_forward_noalloc, through the C ABI: on consecutive
calls (each smaller than the one before) its out, lse and tallies equal those
of ring_attn_forward with a caller-allocated workspace, bit for bit, since
both run the same kernels on the same inputs.  The fixed scratch keeps the
previous call's contents, so the later, smaller calls also show that nothing
stale leaks into a result."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_step_amd as mod
    mod.load_library()
    return mod


def _say(*a):
    print("[case]", *a, flush=True)


# (name, T, Hq, Hkv, d, N, dtype, layout, mask, passes, docs, key padding), largest first
CASES = [
    ("bf16 causal 8192x8/2 d128 N4", 8192, 8, 2, 128, 4, "bf16", 0, 1, 4, False, False),
    ("bf16 doc-causal 2048x4 d64 N2 padded", 2048, 4, 4, 64, 2, "bf16", 0, 2, 2, True, True),
    ("f16 striped causal 1024x4/1 d128 N8 P3", 1024, 4, 1, 128, 8, "f16", 1, 1, 3, False, False),
    ("fp32 causal 256x2 d32 N4", 256, 2, 2, 32, 4, "f32", 0, 1, 4, False, False),
]


def _run_pair(ra, case, seed):
    name, T, Hq, Hkv, d, N, dt, layout, mask, P, docs, pad = case
    q, k, v = (x.cuda() for x in W.random_qkv(T, Hq, Hkv, d, dt, seed))
    cu = W.random_doc_cu_seqlens(T, 100, 700, seed) if docs else None
    kv = W.random_key_valid(T, seed).cuda() if pad else None
    scale = d ** -0.5
    kw = dict(n_blocks=N, layout=layout, mask_mode=mask, max_ring_passes=P, cu_seqlens_host=cu, key_valid=kv,
              scale=scale, want_stats=True)
    n_docs = 0 if cu is None else cu.numel() - 1
    ws = torch.empty(ra.ring_attn_forward_workspace_size(q, k, N, n_docs, False), device="cuda", dtype=torch.uint8)
    out_ref = torch.full((T, Hq, d), float("nan"), device="cuda", dtype=q.dtype)
    lse_ref = torch.full((Hq, T), float("nan"), device="cuda")
    st_ref = ra.ring_attn_forward(q, k, v, out_ref, lse_ref, prefetch=False, workspace=ws, **kw)
    out = torch.full_like(out_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    st = ra.ring_attn_forward_noalloc(q, k, v, out, lse, **kw)
    torch.cuda.synchronize()
    _say(name, "seed", seed, "max |diff|", float((out.float() - out_ref.float()).abs().max()))
    assert torch.equal(out, out_ref), name
    assert torch.equal(lse, lse_ref), name
    assert st == st_ref, name


def test_noalloc_forward_equals_forward_on_shrinking_calls(ra):
    assert ra.ring_attn_forward_noalloc_scratch_bytes() == 64 << 20
    for i, case in enumerate(CASES):
        _say("noalloc vs forward", case[0])
        _run_pair(ra, case, 1000 + i)
    # and the largest again after the small ones
    _say("noalloc vs forward", CASES[0][0], "again")
    _run_pair(ra, CASES[0], 2000)


def test_noalloc_forward_refuses_shapes_beyond_its_scratch(ra):
    T, Hq, d = 65536, 8, 128
    q = torch.empty(T, Hq, d, device="cuda", dtype=torch.bfloat16)
    out = torch.empty_like(q)
    with pytest.raises(ra.RingAttnError) as e:
        ra.ring_attn_forward_noalloc(q, q, q, out, None, n_blocks=8, layout=0, mask_mode=1, max_ring_passes=8,
                                     scale=0.1)
    assert e.value.status == ra.RA_E_TOO_LARGE
