"""GPU parity of the ring backward (ring_attn_backward through the C ABI)
against the fp64 oracle's gradients on the same seeded inputs.

The GPU path takes the forward's own out and lse (bf16 inputs, fp32
accumulation, P and dS rounded to bf16 as matrix-core operands); the oracle
recomputes everything in fp64.  Tolerance (fp32 gradients compared with the
oracle): max |diff| <= 2e-2 and mean |diff| <= 1e-2, the forward's bf16 bar;
for fp16 inputs those bounds times 2^-11 / 2^-8 = 1/8 (the ratio of the unit
roundoffs).  16-bit gradients are the round-to-nearest-even of the fp32
ones, bit for bit.

Full sizes: dout is zero outside a seeded sample of (head, token) rows, so
every gradient is exactly those rows' terms, which the oracle computes at
any length; dq must vanish exactly on every other row.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from bounds import backward_bounds as _rounding_bounds
from bounds import backward_bounds_rows as _rounding_bounds_rows

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 1e-2
TOL16 = {"bf16": (BF16_MAX, BF16_MEAN), "f16": (BF16_MAX / 8, BF16_MEAN / 8)}
TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def ra():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_step_amd as mod
    mod.load_library()
    return mod


def _say(*a):
    print("[case]", *a, flush=True)


def _check(got, ref, what, dt="bf16"):
    diff = np.abs(got - ref)
    _say(what, dt, "max", float(diff.max()), "mean", float(diff.mean()), "max|ref|", float(np.abs(ref).max()))
    tmax, tmean = TOL16[dt]
    assert diff.max() <= tmax and diff.mean() <= tmean, (what, dt, diff.max(), diff.mean())


def _check_bound(got, ref, bound, what):
    """err <= bound, widened by 2^-10 of itself and 1e-6 for the fp32 terms
    (P itself carries ~1e-7 relative error before its 16-bit rounding).  A
    key that one query reaches has dv = P dout: its error is one rounding of
    P, so the bound is approached there by construction."""
    err = np.abs(got - ref)
    lim = bound * (1 + 2.0 ** -10) + 1e-6
    ratio = float((err / lim).max())
    _say(what, "max err", float(err.max()), "max err / bound", ratio)
    assert (err <= lim).all(), (what, float(err.max()), ratio)


BWD_SMALL = [
    # T, N, Hq, Hkv, d, layout, mask, P, docs, forward out dtype
    (888, 3, 4, 2, 128, 0, 1, 3, None, "bf16"),     # B = 296: ragged tiles on both sides
    (888, 3, 4, 4, 128, 0, 0, 3, None, "bf16"),
    (888, 3, 4, 1, 128, 1, 1, 3, None, "f32"),      # striped, MQA
    (1200, 4, 2, 2, 64, 0, 1, 4, None, "bf16"),
    (1200, 4, 4, 2, 64, 1, 1, 2, None, "bf16"),     # striped with a pass limit
    (1024, 4, 2, 2, 128, 0, 0, 1, None, "bf16"),    # own block only
    (960, 4, 2, 2, 128, 0, 2, 4, [0, 100, 101, 400, 700, 960], "bf16"),
    (2048, 4, 2, 1, 128, 0, 2, 2, "random", "f32"),
    (256, 1, 2, 2, 128, 0, 1, 1, None, "bf16"),     # one virtual device
    (520, 8, 2, 2, 128, 1, 1, 8, None, "bf16"),     # B = 65: 1-row ragged tails
    (1024, 8, 16, 8, 128, 1, 1, 8, None, "bf16"),   # striped, heads a multiple of 8: tile-major items, kv groups per XCD
]


def _fwd_bwd(ra, q, k, v, dout, *, N, lay, mask, P, docs, out_dtype, grad_dtype=torch.float32, key_valid=None):
    out, lse = ra.forward(q, k, v, n_blocks=N, layout=lay, causal=mask == 1, cu_seqlens=docs, max_ring_passes=P,
                          out_dtype=out_dtype, return_lse=True, key_valid=key_valid)
    return ra.backward(q, k, v, out, lse, dout, n_blocks=N, layout=lay, causal=mask == 1, cu_seqlens=docs,
                       max_ring_passes=P, grad_dtype=grad_dtype, key_valid=key_valid)




@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(BWD_SMALL)))
def test_16bit_backward_small(ra, case, dt):
    T, N, Hq, Hkv, d, layout, mask, P, docs, odt = BWD_SMALL[case]
    if docs == "random":
        docs = W.random_doc_cu_seqlens(T, 16, 900, seed=case).tolist()
    _say(dt, "backward small", BWD_SMALL[case])
    t16 = TORCH16[dt]
    qh, kh, vh = W.random_qkv(T, Hq, Hkv, d, dt, 2000 + case)
    gh = W.random_dout(T, Hq, d, dt, 2000 + case)
    q, k, v, g = (x.cuda() for x in (qh, kh, vh, gh))
    lay = "striped" if layout == 1 else "contiguous"
    kw = dict(N=N, lay=lay, mask=mask, P=P, docs=docs, out_dtype=t16 if odt == "bf16" else torch.float32)
    dq, dk, dv = _fwd_bwd(ra, q, k, v, g, **kw)
    ref = oracle.backward(qh, kh, vh, gh, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs)
    bounds = _rounding_bounds(qh, kh, vh, gh, N, layout, mask, P, docs, dt)
    for name, got, r, bd in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, bounds):
        _check(got.cpu().double().numpy(), r, name, dt)
        _check_bound(got.cpu().double().numpy(), r, bd, name)
    # 16-bit gradients: the same values rounded to nearest even
    bq, bk, bv = _fwd_bwd(ra, q, k, v, g, grad_dtype=t16, **kw)
    for got, f in zip((bq, bk, bv), (dq, dk, dv)):
        assert got.dtype == t16 and torch.equal(got, f.to(t16))


KP_BWD = [
    # T, N, Hq, Hkv, d, layout, mask, P, docs
    (888, 3, 4, 2, 128, 0, 1, 3, None),
    (888, 3, 4, 1, 128, 1, 1, 3, None),
    (1200, 4, 2, 2, 64, 0, 0, 4, None),
    (960, 4, 2, 2, 128, 0, 2, 4, [0, 100, 101, 400, 700, 960]),
]


def _key_valid(T, seed, frac=0.3):
    return W.random_key_valid(T, seed, frac)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(KP_BWD)))
def test_16bit_backward_key_padding(ra, case, dt):
    T, N, Hq, Hkv, d, layout, mask, P, docs = KP_BWD[case]
    _say(dt, "backward key padding", KP_BWD[case])
    t16 = TORCH16[dt]
    qh, kh, vh = W.random_qkv(T, Hq, Hkv, d, dt, 4000 + case)
    gh = W.random_dout(T, Hq, d, dt, 4000 + case)
    kv = _key_valid(T, 4000 + case)
    q, k, v, g = (x.cuda() for x in (qh, kh, vh, gh))
    lay = "striped" if layout == 1 else "contiguous"
    kvd = kv.cuda()
    out, lse = ra.forward(q, k, v, n_blocks=N, layout=lay, causal=mask == 1, cu_seqlens=docs, max_ring_passes=P,
                          out_dtype=t16, return_lse=True, key_valid=kvd)
    dq, dk, dv = ra.backward(q, k, v, out, lse, g, n_blocks=N, layout=lay, causal=mask == 1, cu_seqlens=docs,
                             max_ring_passes=P, key_valid=kvd)
    ref = oracle.backward(qh, kh, vh, gh, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs,
                          key_valid=kv)
    # Rows left with two or three keys carry large dS: the per-element bound
    # from the arithmetic is the bar there, with the mean bar of the others.
    bounds = _rounding_bounds(qh, kh, vh, gh, N, layout, mask, P, docs, dt, key_valid=kv)
    for name, got, r, bd in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, bounds):
        gn = got.cpu().double().numpy()
        _check_bound(gn, r, bd, name)
        assert np.abs(gn - r).mean() <= TOL16[dt][1], (name, float(np.abs(gn - r).mean()))
    assert not dk[~kvd].any() and not dv[~kvd].any()


@pytest.mark.parametrize("layout", [0, 1])
def test_backward_at_the_longest_ring_chain(ra, layout):
    """n_blocks = 64, the most ring blocks a chain table holds (one per
    lane): 24-row blocks, every tile ragged, forward and backward."""
    T, N, H, d = 64 * 24, 64, 2, 128
    _say("bf16 backward 64 blocks", layout)
    qh, kh, vh = W.random_qkv(T, H, H, d, "bf16", 5000 + layout)
    gh = W.random_dout(T, H, d, "bf16", 5000 + layout)
    q, k, v, g = (x.cuda() for x in (qh, kh, vh, gh))
    lay = "striped" if layout == 1 else "contiguous"
    dq, dk, dv = _fwd_bwd(ra, q, k, v, g, N=N, lay=lay, mask=1, P=N, docs=None, out_dtype=torch.bfloat16)
    ref = oracle.backward(qh, kh, vh, gh, n_blocks=N, layout=layout, mask=1)
    bounds = _rounding_bounds(qh, kh, vh, gh, N, layout, 1, N, None, "bf16")
    for name, got, r, bd in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, bounds):
        gn = got.cpu().double().numpy()
        _check(gn, r, name)
        _check_bound(gn, r, bd, name)
    with pytest.raises(ra.RingAttnError):  # one block more than a chain table holds
        T2 = 65 * 16
        q2, k2, v2 = (x.cuda() for x in W.random_qkv(T2, H, H, d, "bf16", 1))
        o2, l2 = ra.forward(q2, k2, v2, n_blocks=65, causal=True, return_lse=True)
        ra.backward(q2, k2, v2, o2, l2, torch.zeros_like(q2), n_blocks=65, causal=True)


def test_bf16_backward_packed_qkv_views(ra):
    """Strided q / k / v views of one [T, 3, H, d] tensor give the gradients of
    contiguous copies, bit for bit."""
    T, H, d, N = 1024, 2, 128, 4
    qh, kh, vh = W.random_qkv(T, H, H, d, "bf16", 77)
    gh = W.random_dout(T, H, d, "bf16", 77)
    _say("bf16 backward packed views", T, H, d, N)
    qkv = torch.stack([qh, kh, vh], dim=1).cuda()  # [T, 3, H, d]
    g = gh.cuda()
    kw = dict(N=N, lay="contiguous", mask=1, P=N, docs=None, out_dtype=torch.bfloat16)
    a = _fwd_bwd(ra, qkv[:, 0], qkv[:, 1], qkv[:, 2], g, **kw)
    b = _fwd_bwd(ra, qkv[:, 0].contiguous(), qkv[:, 1].contiguous(), qkv[:, 2].contiguous(), g, **kw)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bf16_backward_is_deterministic(ra):
    T, Hq, Hkv, d, N = 1536, 4, 2, 128, 3
    qh, kh, vh = W.random_qkv(T, Hq, Hkv, d, "bf16", 91)
    gh = W.random_dout(T, Hq, d, "bf16", 91)
    q, k, v, g = (x.cuda() for x in (qh, kh, vh, gh))
    _say("bf16 backward determinism", T, Hq, Hkv, d, N)
    kw = dict(N=N, lay="striped", mask=1, P=N, docs=None, out_dtype=torch.bfloat16)
    a = _fwd_bwd(ra, q, k, v, g, **kw)
    b = _fwd_bwd(ra, q, k, v, g, **kw)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _sample_pairs(w, rng, heads, n_per_head):
    B = w.block
    pairs = set()
    for h in heads:
        toks = [0, 1, B - 1, B, w.T - 1, w.T // 2] + list(rng.integers(0, w.T, size=n_per_head))
        pairs.update((int(h), int(t)) for t in toks)
    pairs = sorted(pairs)
    return np.array([p[0] for p in pairs]), np.array([p[1] for p in pairs])


@pytest.mark.parametrize("name,dt,padded", [("causal32k_h32_d128_8blk", "bf16", False),
                                            ("gqa_striped64k_h32kv8_d128_16blk", "bf16", False),
                                            ("varlen_packed128k_h32_d128_8blk_p4", "bf16", False),
                                            ("causal32k_h32_d128_8blk", "f16", False),
                                            ("gqa_striped64k_h32kv8_d128_16blk", "bf16", True)])
def test_long_workload_sparse_dout(ra, name, dt, padded):
    w = dataclasses.replace(W.WORKLOADS[name], dtype=dt)
    kv = W.random_key_valid(w.T, w.seed, 0.1) if padded else None
    _say(name, "generating inputs")
    x = W.make_inputs(w)
    if w.packed:
        qkv = x["qkv"].cuda()
        q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    else:
        q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    cu = x.get("cu_seqlens")
    group = w.Hq // w.Hkv
    rng = np.random.default_rng(w.seed + 100)
    # one query head in each of two kv heads
    kv_sel = sorted(rng.choice(w.Hkv, size=2, replace=False).tolist())
    q_sel = [g * group + int(rng.integers(0, group)) for g in kv_sel]
    heads, toks = _sample_pairs(w, rng, q_sel, 26)
    full = W.random_dout(w.T, w.Hq, w.d, dt, w.seed)
    dout = torch.zeros_like(full)
    dout[toks, heads] = full[toks, heads]
    lay = "striped" if w.layout else "contiguous"
    _say(name, "forward + backward on", len(toks), "rows of heads", q_sel)
    dq, dk, dv = _fwd_bwd(ra, q, k, v, dout.cuda(), N=w.n_blocks, lay=lay, mask=w.mask, P=w.max_ring_passes,
                          docs=cu, out_dtype=TORCH16[dt], key_valid=None if kv is None else kv.cuda())
    torch.cuda.synchronize()
    # oracle on the selected heads only, each query head with its own kv head
    sub_q = x["q"][:, q_sel]
    sub_k = x["k"][:, kv_sel]
    sub_v = x["v"][:, kv_sel]
    sub_g = dout[:, q_sel].contiguous()
    idx = {h: n for n, h in enumerate(q_sel)}
    _say(name, "oracle")
    ref_dq, ref_dk, ref_dv = oracle.backward(sub_q, sub_k, sub_v, sub_g, n_blocks=w.n_blocks, layout=w.layout,
                                             mask=w.mask, max_ring_passes=w.max_ring_passes, cu_seqlens=cu,
                                             scale=w.scale, rows=(np.array([idx[int(h)] for h in heads]), toks),
                                             rows_dkdv=True, key_valid=kv)
    got = (dq.cpu()[toks, heads].double().numpy(), dk.cpu()[:, kv_sel].double().numpy(),
           dv.cpu()[:, kv_sel].double().numpy())
    if kv is None:
        for gn, r, what in zip(got, (ref_dq, ref_dk, ref_dv), ("dq rows", "dk", "dv")):
            _check(gn, r, name + " " + what, dt)
    else:
        # rows left with few keys by the padding: the per-element bound, and the mean bar
        bounds = _rounding_bounds_rows(sub_q, sub_k, sub_v, sub_g, w.n_blocks, w.layout, w.mask,
                                       w.max_ring_passes, cu, dt, np.array([idx[int(h)] for h in heads]), toks,
                                       key_valid=kv)
        for gn, r, bd, what in zip(got, (ref_dq, ref_dk, ref_dv), bounds, ("dq rows", "dk", "dv")):
            _check_bound(gn, r, bd, name + " " + what)
            assert np.abs(gn - r).mean() <= TOL16[dt][1], (what, float(np.abs(gn - r).mean()))
        assert not dk[~kv.cuda()].any() and not dv[~kv.cuda()].any()
    # every other row and kv head: exactly zero
    dq_rest = dq.clone()
    dq_rest[toks, heads] = 0
    assert not dq_rest.any()
    others = [g for g in range(w.Hkv) if g not in kv_sel]
    assert not dk[:, others].any() and not dv[:, others].any()
