"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same
seeded inputs.  Tolerances (fp32 outputs compared with the oracle):
  fp32 inputs: max |diff| <= 1e-5;
  bf16 inputs (fp32 accumulation): max |diff| <= 2e-2 and mean |diff| <= 1e-2;
  fp16 inputs: the bf16 bounds scaled by the ratio of the two unit roundoffs
    (2^-11 / 2^-8 = 1/8): max |diff| <= 2.5e-3 and mean |diff| <= 1.25e-3;
  tallies: exact.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from bounds import forward_bound, forward_bound_rows

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_MAX, BF16_MEAN = 2e-2, 1e-2
TOL16 = {"bf16": (BF16_MAX, BF16_MEAN), "f16": (BF16_MAX / 8, BF16_MEAN / 8), "f32": (F32_TOL, F32_TOL)}
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


def _dev(*xs):
    return [x.cuda() for x in xs]


def _check_fwd_bound(out, ref, bound, what):
    """Every element within the first-order rounding bound of the 16-bit
    forward (widened by 2^-10 of itself and 1e-6 for the fp32 terms)."""
    err = np.abs(out - ref)
    lim = bound * (1 + 2.0 ** -10) + 1e-6
    _say(what, "max err / bound", float((err / lim).max()))
    assert (err <= lim).all(), (what, float(err.max()), float((err / lim).max()))


def _check_bf16(out, ref, what, dt="bf16"):
    diff = np.abs(out - ref)
    _say(what, dt, "max", float(diff.max()), "mean", float(diff.mean()))
    tmax, tmean = TOL16[dt]
    assert diff.max() <= tmax and diff.mean() <= tmean, (what, dt, diff.max(), diff.mean())


# ---------------------------------------------------------------------------
# fp32 path: the pages' two worked examples
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["p4_ring4_b8_d16", "p2_1024tok_d2_16blk"])
def test_f32_worked_examples_forward(ra, name):
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    _say(name)
    q, k, v = _dev(x["q"], x["k"], x["v"])
    out, lse, st = ra.forward(q, k, v, n_blocks=w.n_blocks, scale=w.scale, return_lse=True, return_stats=True)
    ref = oracle.forward(x["q"], x["k"], x["v"], n_blocks=w.n_blocks, scale=w.scale)
    assert np.abs(out.cpu().double().numpy() - ref["out"]).max() <= F32_TOL
    assert np.abs(lse.cpu().double().numpy() - ref["lse"]).max() <= F32_TOL
    tal = oracle.tallies(w.T, w.n_blocks, tile_q=st["tile_q"], tile_k=st["tile_k"])
    assert all(st[k_] == v_ for k_, v_ in tal.items())


@pytest.mark.parametrize("name", ["p4_ring4_b8_d16", "p2_1024tok_d2_16blk"])
def test_f32_step_by_step_state(ra, name):
    """Drive ring_attn_step in ring order; after step s the state of device i
    must be the oracle's state over blocks i, i-1, ..., i-s."""
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    N, B = w.n_blocks, w.block
    q, k, v = _dev(x["q"], x["k"], x["v"])
    O = torch.empty(N, 1, B, w.d, device="cuda")
    m = torch.empty(N, 1, B, device="cuda")
    l = torch.empty(N, 1, B, device="cuda")
    for s in range(N):
        _say(name, "step", s)
        for i in range(N):
            j = (i - s) % N
            ra.ring_attn_step(q[i * B:(i + 1) * B], k[j * B:(j + 1) * B], v[j * B:(j + 1) * B], O[i], m[i], l[i],
                              first_step=(s == 0), scale=w.scale, q_offset=i * B, kv_offset=j * B)
        ref = oracle.forward(x["q"], x["k"], x["v"], n_blocks=N, scale=w.scale, max_ring_passes=s + 1)
        got_m = m.cpu().double().numpy().reshape(1, -1)
        got_l = l.cpu().double().numpy().reshape(1, -1)
        got_O = O.cpu().double().numpy().reshape(-1, w.d)
        assert np.abs(got_m - ref["m"]).max() <= F32_TOL
        assert np.abs(got_l / ref["l"] - 1).max() <= F32_TOL
        assert np.abs(got_O / got_l.reshape(-1, 1) - ref["out"][:, 0]).max() <= F32_TOL
    out = torch.empty(w.T, 1, w.d, device="cuda")
    lse = torch.empty(N, 1, B, device="cuda")
    for i in range(N):
        ra.ring_attn_finalize(O[i], m[i], l[i], out[i * B:(i + 1) * B], lse[i])
    ref = oracle.forward(x["q"], x["k"], x["v"], n_blocks=N, scale=w.scale)
    assert np.abs(out.cpu().double().numpy() - ref["out"]).max() <= F32_TOL
    assert np.abs(lse.cpu().double().numpy().reshape(1, -1) - ref["lse"]).max() <= F32_TOL


def test_f32_merge_path_equals_forward(ra):
    """Each step on a fresh state, finalised, then merged through lse."""
    w = W.WORKLOADS["p4_ring4_b8_d16"]
    x = W.make_inputs(w)
    N, B, d = w.n_blocks, w.block, w.d
    q, k, v = _dev(x["q"], x["k"], x["v"])
    acc = torch.empty(w.T, 1, d, device="cuda")
    lse_acc = torch.empty(1, w.T, device="cuda")
    O = torch.empty(1, B, d, device="cuda")
    m = torch.empty(1, B, device="cuda")
    l = torch.empty(1, B, device="cuda")
    part = torch.empty(B, 1, d, device="cuda")
    lse_p = torch.empty(1, B, device="cuda")
    for i in range(N):
        for s in range(N):
            j = (i - s) % N
            ra.ring_attn_step(q[i * B:(i + 1) * B], k[j * B:(j + 1) * B], v[j * B:(j + 1) * B], O, m, l,
                              first_step=True, scale=w.scale, q_offset=i * B, kv_offset=j * B)
            if s == 0:
                ra.ring_attn_finalize(O, m, l, acc[i * B:(i + 1) * B], lse_acc[:, i * B:(i + 1) * B])
            else:
                ra.ring_attn_finalize(O, m, l, part, lse_p)
                a_blk = acc[i * B:(i + 1) * B].clone()
                l_blk = lse_acc[:, i * B:(i + 1) * B].clone()
                ra.ring_attn_merge(a_blk, l_blk, part, lse_p)
                acc[i * B:(i + 1) * B] = a_blk
                lse_acc[:, i * B:(i + 1) * B] = l_blk
    ref = oracle.forward(x["q"], x["k"], x["v"], n_blocks=N, scale=w.scale)
    assert np.abs(acc.cpu().double().numpy() - ref["out"]).max() <= F32_TOL
    assert np.abs(lse_acc.cpu().double().numpy() - ref["lse"]).max() <= F32_TOL


def test_f32_fully_masked_step_leaves_empty_state(ra):
    q, k, v = _dev(*W.random_qkv(16, 2, 2, 8, "f32", 3))
    O = torch.full((2, 8, 8), 7.0, device="cuda")
    m = torch.full((2, 8), 7.0, device="cuda")
    l = torch.full((2, 8), 7.0, device="cuda")
    stats = torch.zeros(3, dtype=torch.int64, device="cuda")
    # queries at positions 0..7, keys at 8..15: causal allows nothing
    ra.ring_attn_step(q[:8], k[8:], v[8:], O, m, l, first_step=True, scale=0.3, mask_mode=ra.RA_MASK_CAUSAL,
                      q_offset=0, kv_offset=8, stats=stats)
    assert torch.isneginf(m).all() and (l == 0).all() and (O == 0).all()
    assert stats.tolist() == [1, 0, 0]
    out = torch.empty(8, 2, 8, device="cuda")
    lse = torch.empty(2, 8, device="cuda")
    ra.ring_attn_finalize(O, m, l, out, lse)
    assert (out == 0).all() and torch.isneginf(lse).all()


def _key_valid(T, seed, frac=0.3):
    return W.random_key_valid(T, seed, frac)


# ---------------------------------------------------------------------------
# bf16 matrix-core path on small shapes (several tiles, ragged tails)
# ---------------------------------------------------------------------------

SMALL = [
    # T, N, Hq, Hkv, d, layout, mask, P, docs
    (888, 3, 4, 2, 128, 0, 1, 3, None),       # B = 296: ragged q and k tiles
    (888, 3, 4, 4, 128, 0, 0, 3, None),
    (888, 3, 4, 1, 128, 1, 1, 3, None),       # striped, MQA
    (1200, 4, 2, 2, 64, 0, 1, 4, None),
    (1200, 4, 4, 2, 64, 1, 1, 2, None),       # striped with a pass limit
    (1024, 4, 2, 2, 128, 0, 0, 1, None),      # own block only
    (960, 4, 2, 2, 128, 0, 2, 4, [0, 100, 101, 400, 700, 960]),
    (2048, 4, 2, 1, 128, 0, 2, 2, "random"),
    (256, 1, 2, 2, 128, 0, 1, 1, None),       # one virtual device
    (520, 8, 2, 2, 128, 1, 1, 8, None),       # B = 65: a single 1-key ragged tail
    (1024, 4, 8, 1, 128, 0, 1, 4, None),      # 8 query heads per kv head: 32-row work items
    (900, 3, 6, 2, 64, 1, 1, 3, None),        # groups of 3: one head per item, striped
    (1200, 4, 8, 2, 128, 0, 2, 2, [0, 130, 700, 1200]),  # 4 heads per item, doc-causal, P < N
    (1024, 8, 16, 8, 128, 1, 1, 8, None),     # striped, groups a multiple of 8: q-tile-major items per XCD
]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_16bit_forward_small(ra, case, dt):
    T, N, Hq, Hkv, d, layout, mask, P, docs = SMALL[case]
    if docs == "random":
        docs = W.random_doc_cu_seqlens(T, 16, 900, seed=case).tolist()
    _say(dt, "small", SMALL[case])
    qh, kh, vh = W.random_qkv(T, Hq, Hkv, d, dt, 1000 + case)
    q, k, v = _dev(qh, kh, vh)
    lay = "striped" if layout == 1 else "contiguous"
    out, lse, st = ra.forward(q, k, v, n_blocks=N, layout=lay, causal=mask == 1, cu_seqlens=docs,
                              max_ring_passes=P, out_dtype=torch.float32, return_lse=True, return_stats=True)
    ref = oracle.forward(qh, kh, vh, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs)
    _check_bf16(out.cpu().double().numpy(), ref["out"], "out", dt)
    _check_fwd_bound(out.cpu().double().numpy(), ref["out"], forward_bound(qh, kh, vh, N, layout, mask, P, docs, dt),
                     "out")
    assert np.abs(lse.cpu().double().numpy() - ref["lse"]).max() <= 1e-3
    tal = oracle.tallies(T, N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs,
                         tile_q=st["tile_q"], tile_k=st["tile_k"])
    for key, val in tal.items():
        assert st[key] == val, key
    # 16-bit output is the round-to-nearest-even of the fp32 one, bit for bit
    out16 = ra.forward(q, k, v, n_blocks=N, layout=lay, causal=mask == 1, cu_seqlens=docs, max_ring_passes=P)
    assert out16.dtype == TORCH16[dt]
    assert torch.equal(out16, out.to(TORCH16[dt]))


def test_16bit_forward_host_tables_stay_valid_when_the_host_runs_ahead(ra):
    """Twelve doc-causal forwards with different document tables are enqueued
    behind a long GPU wait, so the host runs more calls ahead than the
    library's ring of pinned staging buffers holds and each buffer is refilled
    only after its earlier copies were consumed; every result must equal the
    same call made on an idle GPU, bit for bit."""
    T, N, Hq, Hkv, d = 1200, 4, 4, 2, 64
    qh, kh, vh = W.random_qkv(T, Hq, Hkv, d, "bf16", 77)
    q, k, v = _dev(qh, kh, vh)
    tables = [W.random_doc_cu_seqlens(T, 40, 700, seed=300 + i) for i in range(12)]
    n_docs = max(t.numel() - 1 for t in tables)
    ws = torch.empty(ra.ring_attn_forward_workspace_size(q, k, N, n_docs), dtype=torch.uint8, device="cuda")
    kw = dict(n_blocks=N, layout=0, mask_mode=2, max_ring_passes=N, scale=d ** -0.5, prefetch=False, workspace=ws)
    expect = []
    for t in tables:
        o = torch.empty(T, Hq, d, dtype=torch.float32, device="cuda")
        ra.ring_attn_forward(q, k, v, o, None, cu_seqlens_host=t.clone(), **kw)
        torch.cuda.synchronize()
        expect.append(o)
    outs = [torch.full((T, Hq, d), float("nan"), device="cuda") for _ in tables]
    torch.cuda.synchronize()
    torch.cuda._sleep(200_000_000)  # the stream stays busy while the calls below are enqueued
    for t, o in zip(tables, outs):
        host = t.clone()
        ra.ring_attn_forward(q, k, v, o, None, cu_seqlens_host=host, **kw)
        host.fill_(T)  # the caller's array may change once the call has returned
    torch.cuda.synchronize()
    _say("host-ahead forwards", len(tables), "documents up to", n_docs)
    for i, (o, e) in enumerate(zip(outs, expect)):
        assert torch.equal(o, e), i


KP_SMALL = [
    # T, N, Hq, Hkv, d, layout, mask, P, docs
    (888, 3, 4, 2, 128, 0, 1, 3, None),       # ragged tiles
    (888, 3, 4, 1, 128, 1, 1, 3, None),       # striped
    (1200, 4, 4, 2, 64, 0, 0, 4, None),       # no mask beyond the padding
    (960, 4, 2, 2, 128, 0, 2, 4, [0, 100, 101, 400, 700, 960]),
    (1200, 4, 4, 2, 64, 1, 1, 2, None),       # striped with a pass limit
]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(KP_SMALL)))
def test_16bit_forward_key_padding(ra, case, dt):
    T, N, Hq, Hkv, d, layout, mask, P, docs = KP_SMALL[case]
    _say(dt, "key padding", KP_SMALL[case])
    qh, kh, vh = W.random_qkv(T, Hq, Hkv, d, dt, 3000 + case)
    kv = _key_valid(T, 3000 + case)
    q, k, v = _dev(qh, kh, vh)
    lay = "striped" if layout == 1 else "contiguous"
    kw = dict(n_blocks=N, layout=lay, causal=mask == 1, cu_seqlens=docs, max_ring_passes=P, out_dtype=torch.float32,
              return_lse=True)
    ref = oracle.forward(qh, kh, vh, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs,
                         key_valid=kv)
    bound = forward_bound(qh, kh, vh, N, layout, mask, P, docs, dt, key_valid=kv)
    for prefetch in (False, True):
        out, lse = ra.forward(q, k, v, key_valid=kv.cuda(), prefetch=prefetch, **kw)
        _check_bf16(out.cpu().double().numpy(), ref["out"], "out prefetch=%d" % prefetch, dt)
        _check_fwd_bound(out.cpu().double().numpy(), ref["out"], bound, "out prefetch=%d" % prefetch)
        got_lse = lse.cpu().double().numpy()
        empty = np.isneginf(ref["lse"])
        assert np.array_equal(np.isneginf(got_lse), empty)
        assert np.abs(got_lse[~empty] - ref["lse"][~empty]).max() <= 1e-3
    # an all-true mask changes nothing, bit for bit
    a_ = ra.forward(q, k, v, **kw)
    b_ = ra.forward(q, k, v, key_valid=torch.ones(T, dtype=torch.bool, device="cuda"), **kw)
    assert torch.equal(a_[0], b_[0]) and torch.equal(a_[1], b_[1])


def test_f32_forward_key_padding(ra):
    T, N, H, d = 512, 4, 2, 40
    qh, kh, vh = W.random_qkv(T, H, H, d, "f32", 3100)
    kv = _key_valid(T, 3100)
    _say("f32 key padding", T, N, H, d)
    for mask, lay in ((1, "contiguous"), (1, "striped"), (0, "contiguous")):
        out, lse = ra.forward(*_dev(qh, kh, vh), n_blocks=N, layout=lay, causal=mask == 1, key_valid=kv.cuda(),
                              return_lse=True)
        ref = oracle.forward(qh, kh, vh, n_blocks=N, layout=1 if lay == "striped" else 0, mask=mask, key_valid=kv)
        assert np.abs(out.cpu().double().numpy() - ref["out"]).max() <= F32_TOL


def test_pack_key_mask_bits(ra):
    """Bit words of ring_attn_pack_key_mask, from a strided view, against the
    definition (bit w % 32 of word w / 32 is key w's flag, zero past n)."""
    g = torch.Generator().manual_seed(3200)
    for n in (1, 63, 64, 65, 300):
        full = torch.rand(3 * n, generator=g) > 0.5
        view = full.cuda()[1::3]
        bits = ra.ring_attn_pack_key_mask(view).cpu().numpy().view(np.uint32)
        flags = full[1::3].numpy()
        want = np.zeros(2 * ((n + 63) // 64), dtype=np.uint32)
        for w in range(n):
            want[w // 32] |= np.uint32(int(flags[w]) << (w % 32))
        assert np.array_equal(bits, want), n


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_16bit_step_api_key_bits(ra, dt):
    """ring_attn_step with a key block's packed padding bits (striped block
    as strided views): the state must equal the oracle's block state."""
    T, N, Hq, d = 1024, 4, 2, 128
    qh, kh, vh = W.random_qkv(T, Hq, Hq, d, dt, 3300)
    kv = _key_valid(T, 3300)
    q, k, v = _dev(qh, kh, vh)
    i, j = 2, 1
    B = T // N
    O = torch.empty(Hq, B, d, device="cuda")
    m = torch.empty(Hq, B, device="cuda")
    l = torch.empty(Hq, B, device="cuda")
    bits = ra.ring_attn_pack_key_mask(kv.cuda()[j::N])
    ra.ring_attn_step(q[i::N], k[j::N], v[j::N], O, m, l, first_step=True, scale=1 / math.sqrt(d),
                      mask_mode=ra.RA_MASK_CAUSAL, q_offset=i, kv_offset=j, pos_stride=N, key_bits=bits)
    ref = oracle.block(qh[i::N], kh[j::N], vh[j::N], np.arange(B) * N + i, np.arange(B) * N + j,
                       mask=oracle.MASK_CAUSAL, key_valid=kv[j::N])
    got_l = l.cpu().double().numpy()
    ok = ref["l"] > 0
    assert np.array_equal(got_l > 0, ok)
    out = (O.cpu().double().numpy() / np.where(ok, got_l, 1)[..., None])
    _check_bf16(out[ok], ref["out"][ok], "key-bits step", dt)


@pytest.mark.parametrize("N", [64, 65])
def test_forward_at_and_past_the_longest_ring_chain(ra, N):
    """64 ring blocks run as one launch (one chain block per lane); 65 take
    one launch per ring step.  Both against the oracle, with the tallies."""
    T, H, d = N * 24, 2, 128
    _say("bf16 forward blocks", N)
    qh, kh, vh = W.random_qkv(T, H, H, d, "bf16", 5100 + N)
    for layout in (0, 1):
        out, lse, st = ra.forward(*_dev(qh, kh, vh), n_blocks=N, layout="striped" if layout else "contiguous",
                                  causal=True, out_dtype=torch.float32, return_lse=True, return_stats=True)
        ref = oracle.forward(qh, kh, vh, n_blocks=N, layout=layout, mask=oracle.MASK_CAUSAL)
        _check_bf16(out.cpu().double().numpy(), ref["out"], "out %d blocks layout %d" % (N, layout))
        assert np.abs(lse.cpu().double().numpy() - ref["lse"]).max() <= 1e-3
        tal = oracle.tallies(T, N, layout=layout, mask=oracle.MASK_CAUSAL, tile_q=st["tile_q"], tile_k=st["tile_k"])
        for key, val in tal.items():
            assert st[key] == val, key


def test_empty_sequence(ra):
    """T = 0 through the binding: empty out and lse, zero tallies, empty gradients."""
    _say("empty sequence")
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        q = torch.empty(0, 4, 128, device="cuda", dtype=dt)
        k = torch.empty(0, 2, 128, device="cuda", dtype=dt)
        out, lse, st = ra.forward(q, k, k, n_blocks=4, causal=True, return_lse=True, return_stats=True)
        assert out.shape == (0, 4, 128) and lse.shape == (4, 0) and st["tiles_partial"] == 0
        if dt != torch.float32:
            dq, dk, dv = ra.backward(q, k, k, out, lse, q, n_blocks=4, causal=True)
            assert dq.shape == (0, 4, 128) and dk.shape == (0, 2, 128) and dv.shape == (0, 2, 128)
    torch.cuda.synchronize()


def test_bf16_ring_late_score_jumps(ra):
    """Scores that jump far above a row's running reference late in its chain:
    under a causal ring, device i visits blocks i, i-1, ..., 0, so keys of
    block 0 scaled by 8 raise the row maximum by tens of log2 units at the end
    of every chain, and one key on a query's own direction raises it by
    hundreds (2^(jump) would overflow fp32).  The one-launch ring takes P
    against the current reference and must fall back to the maximum (with S
    recomputed from the K tile) on exactly such tiles."""
    T, N, H, d = 1024, 4, 2, 128
    qh, kh, vh = W.random_qkv(T, H, H, d, "bf16", 4242)
    kf = kh.float()
    B = T // N
    kf[:B] *= 8.0
    kf[B // 2, 0] = (qh[T - 1, 0].float() * 24.0)  # a very large score for the last query row of head 0
    kh = kf.to(torch.bfloat16)
    _say("bf16 late score jumps", T, N, H, d)
    q, k, v = _dev(qh, kh, vh)
    out, lse = ra.forward(q, k, v, n_blocks=N, causal=True, out_dtype=torch.float32, return_lse=True)
    ref = oracle.forward(qh, kh, vh, n_blocks=N, mask=oracle.MASK_CAUSAL)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    _check_bf16(out.cpu().double().numpy(), ref["out"], "out")
    lse_err = np.abs(lse.cpu().double().numpy() - ref["lse"])
    _say("lse max err", float(lse_err.max()), "max |lse|", float(np.abs(ref["lse"]).max()))
    assert lse_err.max() <= 1e-3


def test_bf16_packed_qkv_views(ra):
    T, H, d = 1024, 2, 128
    qh, kh, vh = W.random_qkv(T, H, H, d, "bf16", 77, packed=True)
    qkv = torch.stack([qh, kh, vh], dim=1).cuda()
    out = ra.forward_qkvpacked(qkv, n_blocks=4, causal=True, out_dtype=torch.float32)
    ref = oracle.forward(qh, kh, vh, n_blocks=4, mask=oracle.MASK_CAUSAL)
    _check_bf16(out.cpu().double().numpy(), ref["out"], "packed")


@pytest.mark.parametrize("copy_us,compute_us", [(400, 0), (0, 400), (250, 250)])
def test_prefetch_event_ordering_under_forced_delays(ra, copy_us, compute_us):
    """The prefetch path's double buffer under adversarial timing: a bounded
    wait before every step's copies (copies land late: a step that did not
    wait for them would read the buffer's previous contents) or before every
    step's compute (compute runs late: a copy that did not wait for the step
    reading its buffer would overwrite it mid-read).  Results stay bit-exact:
    fp32 equals prefetch = 0, and the 16-bit path equals its undelayed self."""
    w = W.WORKLOADS["p2_1024tok_d2_16blk"]
    x = W.make_inputs(w)
    q32, k32, v32 = _dev(x["q"], x["k"], x["v"])
    kw32 = dict(n_blocks=w.n_blocks, scale=w.scale, causal=True, return_lse=True)
    qh, kh, vh = W.random_qkv(2048, 4, 2, 128, "bf16", 77)
    q16, k16, v16 = _dev(qh, kh, vh)
    kw16 = dict(n_blocks=8, causal=True, out_dtype=torch.float32, return_lse=True)
    base32 = ra.forward(q32, k32, v32, prefetch=False, **kw32)
    base16 = ra.forward(q16, k16, v16, prefetch=True, **kw16)
    torch.cuda.synchronize()
    _say("prefetch delays copy", copy_us, "us, compute", compute_us, "us")
    try:
        ra.ring_attn_test_prefetch_delays(copy_us, compute_us)
        for rep in range(2):
            got32 = ra.forward(q32, k32, v32, prefetch=True, **kw32)
            got16 = ra.forward(q16, k16, v16, prefetch=True, **kw16)
            torch.cuda.synchronize()
            assert torch.equal(got32[0], base32[0]) and torch.equal(got32[1], base32[1]), rep
            assert torch.equal(got16[0], base16[0]) and torch.equal(got16[1], base16[1]), rep
    finally:
        ra.ring_attn_test_prefetch_delays(0, 0)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_16bit_prefetch_matches_one_launch_ring(ra, dt):
    """The side-stream prefetch path (one launch per ring step, state through
    HBM between steps) and the default one-launch ring (state in registers)
    round differently, so both are held to the oracle and to each other."""
    for layout, docs in (("contiguous", None), ("striped", None), ("contiguous", [0, 300, 301, 1024])):
        qkv = W.random_qkv(1024, 4, 2, 128, dt, 5, packed=False)
        q, k, v = _dev(*qkv)
        kw = dict(n_blocks=4, layout=layout, causal=docs is None, cu_seqlens=docs, return_lse=True,
                  out_dtype=torch.float32)
        a, la = ra.forward(q, k, v, prefetch=False, **kw)
        b, lb = ra.forward(q, k, v, prefetch=True, **kw)
        torch.cuda.synchronize()
        _say("prefetch", dt, layout, docs is not None)
        lay = oracle.LAYOUT_STRIPED if layout == "striped" else oracle.LAYOUT_CONTIGUOUS
        mask = oracle.MASK_CAUSAL if docs is None else oracle.MASK_DOC_CAUSAL
        ref = oracle.forward(*qkv, n_blocks=4, layout=lay, mask=mask, cu_seqlens=docs)
        for x, lx in ((a, la), (b, lb)):
            _check_bf16(x.cpu().double().numpy(), ref["out"], "prefetch", dt)
            assert np.abs(lx.cpu().double().numpy() - ref["lse"]).max() <= 1e-3
        # The two paths differ in where P is rounded to 16 bits (relative to
        # the running reference maximum, which a state hand-off resets): they
        # agree to that rounding level, not bitwise.
        dif = (a - b).abs()
        assert dif.max().item() <= 1e-2 and dif.mean().item() <= 5e-4
        assert (la - lb).abs().max().item() <= 1e-3


def _ring_steps(ra, q, k, v, N, B, d, Hq, scale, order, state=None, mask=1):
    O, m, l = state if state is not None else (torch.empty(N, Hq, B, d, device="cuda"),
                                              torch.empty(N, Hq, B, device="cuda"),
                                              torch.empty(N, Hq, B, device="cuda"))
    for (i, j, first) in order:
        ra.ring_attn_step(q[i * B:(i + 1) * B], k[j * B:(j + 1) * B], v[j * B:(j + 1) * B], O[i], m[i], l[i],
                          first_step=first, scale=scale, mask_mode=mask, q_offset=i * B, kv_offset=j * B)
    return O, m, l


def test_bf16_resume_from_saved_state_is_bit_identical(ra):
    """The (O, m, l) triple is the whole resume state: copy it to the host
    after step 2, wipe the device copy, restore and finish the ring."""
    N, B, Hq, d = 4, 256, 2, 128
    q, k, v = _dev(*W.random_qkv(N * B, Hq, Hq, d, "bf16", 9))
    sched = [(i, (i - s) % N, s == 0) for s in range(N) for i in range(N)]
    full = _ring_steps(ra, q, k, v, N, B, d, Hq, 0.088, sched, mask=0)
    cut = 3 * N
    part = _ring_steps(ra, q, k, v, N, B, d, Hq, 0.088, sched[:cut], mask=0)
    saved = [x.cpu() for x in part]
    for x in part:
        x.fill_(float("nan"))
    restored = [x.cuda() for x in saved]
    resumed = _ring_steps(ra, q, k, v, N, B, d, Hq, 0.088, sched[cut:], state=restored, mask=0)
    for a, b in zip(full, resumed):
        assert torch.equal(a, b)


def test_bf16_shuffled_step_order_within_tolerance(ra):
    N, B, Hq, d = 4, 200, 2, 128
    qh, kh, vh = W.random_qkv(N * B, Hq, Hq, d, "bf16", 10)
    q, k, v = _dev(qh, kh, vh)
    rng = np.random.default_rng(0)
    sched = []
    for i in range(N):
        js = rng.permutation(N)
        sched += [(i, int(j), n == 0) for n, j in enumerate(js)]
    O, m, l = _ring_steps(ra, q, k, v, N, B, d, Hq, 1 / math.sqrt(d), sched, mask=1)
    out = torch.empty(N * B, Hq, d, device="cuda")
    for i in range(N):
        ra.ring_attn_finalize(O[i], m[i], l[i], out[i * B:(i + 1) * B])
    ref = oracle.forward(qh, kh, vh, n_blocks=N, mask=oracle.MASK_CAUSAL)
    _check_bf16(out.cpu().double().numpy(), ref["out"], "shuffled")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_16bit_step_api_striped_positions(ra, dt):
    """ring_attn_step on striped blocks given as strided views, positions
    q_offset + u * N; the state must equal the oracle's block state."""
    T, N, Hq, d = 1024, 4, 2, 128
    qh, kh, vh = W.random_qkv(T, Hq, Hq, d, dt, 11)
    q, k, v = _dev(qh, kh, vh)
    i, j = 1, 3
    B = T // N
    O = torch.empty(Hq, B, d, device="cuda")
    m = torch.empty(Hq, B, device="cuda")
    l = torch.empty(Hq, B, device="cuda")
    ra.ring_attn_step(q[i::N], k[j::N], v[j::N], O, m, l, first_step=True, scale=1 / math.sqrt(d),
                      mask_mode=ra.RA_MASK_CAUSAL, q_offset=i, kv_offset=j, pos_stride=N)
    ref = oracle.block(qh[i::N], kh[j::N], vh[j::N], np.arange(B) * N + i, np.arange(B) * N + j,
                       mask=oracle.MASK_CAUSAL)
    got_l = l.cpu().double().numpy()
    ok = ref["l"] > 0
    assert np.array_equal(got_l > 0, ok)
    out = (O.cpu().double().numpy() / np.where(ok, got_l, 1)[..., None])
    _check_bf16(out[ok], ref["out"][ok], "striped step", dt)
    assert np.abs(m.cpu().double().numpy()[ok] - ref["m"][ok]).max() <= 1e-3


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_16bit_finalize_and_merge_round_the_fp32_results(ra, dt):
    """ring_attn_finalize / ring_attn_merge with a 16-bit out: the finalized
    output is the fp32 one rounded to nearest even, and so is the merge of two
    16-bit partial outputs (the merge computes in fp32 either way)."""
    g = torch.Generator().manual_seed(12)
    Hq, B, d = 2, 300, 128
    O = torch.randn(Hq, B, d, generator=g).cuda()
    m = torch.randn(Hq, B, generator=g).cuda()
    l = (torch.rand(Hq, B, generator=g) + 0.5).cuda()
    l[0, :7] = 0  # rows that saw no key: out 0, lse -inf
    o32 = torch.empty(B, Hq, d, device="cuda")
    o16 = torch.empty(B, Hq, d, device="cuda", dtype=TORCH16[dt])
    lse = torch.empty(Hq, B, device="cuda")
    ra.ring_attn_finalize(O, m, l, o32, lse)
    ra.ring_attn_finalize(O, m, l, o16)
    assert torch.equal(o16, o32.to(TORCH16[dt]))
    assert torch.isinf(lse[0, :7]).all() and not o32[:7, 0].any()
    # merge (o16, lse) with a second partial result
    ob = torch.randn(B, Hq, d, generator=g).to(TORCH16[dt]).cuda()
    lb = torch.randn(Hq, B, generator=g).cuda()
    acc16, lacc16 = o16.clone(), lse.clone()
    acc32, lacc32 = o16.float(), lse.clone()
    ra.ring_attn_merge(acc16, lacc16, ob, lb)
    ra.ring_attn_merge(acc32, lacc32, ob.float(), lb)
    torch.cuda.synchronize()
    assert torch.equal(lacc16, lacc32)
    assert torch.equal(acc16, acc32.to(TORCH16[dt]))
    # both against the oracle's merge of the same two partial results: the
    # fp32 one within a few fp32 roundings of the operands, the 16-bit one
    # within the 16-bit rounding of the result on top (unit roundoff u)
    oa, ob64 = o16.double().cpu().numpy(), ob.double().cpu().numpy()
    ro, rl = oracle.merge(oa, lse.t().double().cpu().numpy(), ob64, lb.t().double().cpu().numpy())
    f32_err = 2.0 ** -21 * (np.abs(oa) + np.abs(ob64) + 1.0)
    e32 = np.abs(acc32.double().cpu().numpy() - ro)
    e16 = np.abs(acc16.double().cpu().numpy() - ro)
    u = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}[dt]
    _say(dt, "merge vs oracle: fp32 err / tol", float((e32 / f32_err).max()), "16-bit err / tol",
         float((e16 / (u * np.abs(ro) + f32_err)).max()))
    assert (e32 <= f32_err).all()
    assert (e16 <= u * np.abs(ro) + f32_err).all()
    got_l = lacc32.t().double().cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert (np.abs(got_l[fin] - rl[fin]) <= 2.0 ** -21 * (1 + np.abs(rl[fin]))).all()


@pytest.mark.parametrize("name", ["p4_ring4_b8_d16", "p2_1024tok_d2_16blk"])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("mask", [0, 1])
def test_f32_prefetch_is_bit_identical(ra, name, layout, mask):
    """fp32 inputs: the prefetching per-step path (its 2-D copies of K and V
    into the double buffer) gives exactly the results of prefetch = 0, and
    both meet the fp32 bar against the oracle."""
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    _say("f32 prefetch", name, "layout", layout, "mask", mask)
    q, k, v = _dev(x["q"], x["k"], x["v"])
    lay = "striped" if layout == 1 else "contiguous"
    kw = dict(n_blocks=w.n_blocks, layout=lay, causal=mask == 1, scale=w.scale, return_lse=True)
    a_out, a_lse = ra.forward(q, k, v, prefetch=False, **kw)
    b_out, b_lse = ra.forward(q, k, v, prefetch=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)
    ref = oracle.forward(x["q"], x["k"], x["v"], n_blocks=w.n_blocks, layout=layout, mask=mask, scale=w.scale)
    assert np.abs(a_out.cpu().double().numpy() - ref["out"]).max() <= F32_TOL
    assert np.abs(a_lse.cpu().double().numpy() - ref["lse"]).max() <= F32_TOL


F32_MASKED = [
    # T, N, Hq, Hkv, d, layout, mask, P, docs
    (960, 4, 2, 1, 40, 0, 2, 4, [0, 100, 101, 400, 700, 960]),   # doc-causal, GQA
    (960, 4, 2, 2, 40, 0, 2, 2, [0, 100, 101, 400, 700, 960]),   # doc-causal, P < N
    (2048, 4, 2, 2, 64, 0, 2, 3, "random"),
    (1024, 8, 2, 2, 64, 0, 1, 3, None),                          # causal, P < N
    (1024, 8, 4, 2, 64, 1, 1, 3, None),                          # striped causal, P < N
    (1000, 4, 2, 2, 16, 0, 0, 2, None),                          # no mask, P < N, ragged tiles
]


@pytest.mark.parametrize("case", range(len(F32_MASKED)))
def test_f32_doc_causal_and_pass_limits(ra, case):
    """The fp32 kernel under document-causal masks and ring pass limits
    against the oracle at the fp32 bar, with and without prefetch (bit-equal)."""
    T, N, Hq, Hkv, d, layout, mask, P, docs = F32_MASKED[case]
    if docs == "random":
        docs = W.random_doc_cu_seqlens(T, 16, 900, seed=case).tolist()
    _say("f32 masked", F32_MASKED[case][:8])
    qh, kh, vh = W.random_qkv(T, Hq, Hkv, d, "f32", 4000 + case)
    q, k, v = _dev(qh, kh, vh)
    lay = "striped" if layout == 1 else "contiguous"
    kw = dict(n_blocks=N, layout=lay, causal=mask == 1, cu_seqlens=docs, max_ring_passes=P, return_lse=True)
    out, lse = ra.forward(q, k, v, prefetch=False, **kw)
    out_p, lse_p = ra.forward(q, k, v, prefetch=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, out_p) and torch.equal(lse, lse_p)
    ref = oracle.forward(qh, kh, vh, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs)
    assert np.abs(out.cpu().double().numpy() - ref["out"]).max() <= F32_TOL
    got_lse = lse.cpu().double().numpy()
    empty = np.isneginf(ref["lse"])
    assert np.array_equal(np.isneginf(got_lse), empty)
    assert np.abs(got_lse[~empty] - ref["lse"][~empty]).max() <= F32_TOL


# ---------------------------------------------------------------------------
# Full-size long-context workloads, in the benchmark's launch configuration:
# sampled rows against the oracle, tallies exactly.
# ---------------------------------------------------------------------------

def _sample_rows(w, rng, n=48):
    B = w.block
    toks = [0, 1, B - 1, B, w.T - 1, w.T // 2]
    toks += list(rng.integers(0, w.T, size=n - len(toks)))
    heads = list(rng.integers(0, w.Hq, size=len(toks)))
    return np.asarray(heads), np.asarray(toks)


# Two query heads per long workload whose every row is checked; for the GQA
# one they read different kv heads (group of 4: kv heads 1 and 5).
FULL_HEADS = {"causal32k_h32_d128_8blk": (3, 29), "gqa_striped64k_h32kv8_d128_16blk": (5, 22),
              "varlen_packed128k_h32_d128_8blk_p4": (3, 29)}


@pytest.mark.parametrize("name", list(FULL_HEADS))
def test_long_workload_every_row_of_two_heads(ra, name):
    """The benchmark launch at full size (every virtual device and query tile
    of the two heads): each output element within the first-order rounding
    bound of the 16-bit forward against the fp64 oracle, each lse within its
    fp32 summation bound, -inf exactly where a row takes no key.  On the
    causal 32K workload the prefetching per-step path is checked the same
    way against the same oracle rows."""
    w = W.WORKLOADS[name]
    _say(name, "generating inputs")
    x = W.make_inputs(w)
    if w.packed:
        qkv = x["qkv"].cuda()
        q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    else:
        q, k, v = _dev(x["q"], x["k"], x["v"])
    cu = x.get("cu_seqlens")
    layout = "striped" if w.layout else "contiguous"
    runs = {}
    for prefetch in ((False, True) if name == "causal32k_h32_d128_8blk" else (False,)):
        _say(name, "forward, prefetch", prefetch)
        out, lse = ra.forward(q, k, v, n_blocks=w.n_blocks, layout=layout, causal=w.mask == 1, cu_seqlens=cu,
                              max_ring_passes=w.max_ring_passes, out_dtype=torch.float32, return_lse=True,
                              prefetch=prefetch)
        torch.cuda.synchronize()
        runs[prefetch] = (out.cpu(), lse.cpu())
        del out, lse
    del q, k, v
    torch.cuda.empty_cache()
    hs = FULL_HEADS[name]
    heads = np.repeat(np.asarray(hs), w.T)
    toks = np.tile(np.arange(w.T), len(hs))
    group = w.Hq // w.Hkv
    qs = x["q"][:, list(hs)]
    ks = x["k"][:, [h // group for h in hs]]
    vs = x["v"][:, [h // group for h in hs]]
    local = np.repeat(np.arange(len(hs)), w.T)
    _say(name, "oracle on", len(toks), "rows")
    ref = oracle.forward(qs, ks, vs, n_blocks=w.n_blocks, layout=w.layout, mask=w.mask,
                         max_ring_passes=w.max_ring_passes, cu_seqlens=cu, scale=w.scale, rows=(local, toks))
    _say(name, "bounds")
    bound, n_keys, lse_tol = forward_bound_rows(qs, ks, vs, w.n_blocks, w.layout, w.mask, w.max_ring_passes, cu,
                                                w.dtype, local, toks, ref["lse"])
    empty = n_keys == 0
    assert np.array_equal(np.isneginf(ref["lse"]), empty)
    for prefetch, (out, lse) in runs.items():
        what = "%s prefetch=%s" % (name, prefetch)
        got = out[toks, heads].double().numpy()
        _check_fwd_bound(got, ref["out"], bound, what)
        got_lse = lse[heads, toks].double().numpy()
        assert np.array_equal(np.isneginf(got_lse), empty), what
        err = np.abs(got_lse[~empty] - ref["lse"][~empty])
        _say(what, "lse max err / tol", float((err / lse_tol[~empty]).max()))
        assert (err <= lse_tol[~empty]).all(), what


@pytest.mark.parametrize("name,dt,padded", [("causal32k_h32_d128_8blk", "f16", False),
                                            ("gqa_striped64k_h32kv8_d128_16blk", "bf16", True)])
def test_long_workload_sampled_rows(ra, name, dt, padded):
    w = dataclasses.replace(W.WORKLOADS[name], dtype=dt)
    kv = _key_valid(w.T, w.seed, frac=0.1) if padded else None
    _say(name, "generating inputs")
    x = W.make_inputs(w)
    if w.packed:
        qkv = x["qkv"].cuda()
        q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    else:
        q, k, v = _dev(x["q"], x["k"], x["v"])
    cu = x.get("cu_seqlens")
    _say(name, "forward")
    out, lse, st = ra.forward(q, k, v, n_blocks=w.n_blocks, layout="striped" if w.layout else "contiguous",
                              causal=w.mask == 1, cu_seqlens=cu, max_ring_passes=w.max_ring_passes,
                              out_dtype=torch.float32, return_lse=True, return_stats=True,
                              key_valid=None if kv is None else kv.cuda())
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (kv is not None or torch.isfinite(lse).all())
    rng = np.random.default_rng(w.seed)
    heads, toks = _sample_rows(w, rng)
    group = w.Hq // w.Hkv
    # oracle on the sampled heads only: q head h reads kv head h // group
    uh = sorted(set(int(h) for h in heads))
    qs = x["q"][:, uh]
    ks = x["k"][:, [h // group for h in uh]]
    vs = x["v"][:, [h // group for h in uh]]
    idx = {h: n for n, h in enumerate(uh)}
    _say(name, "oracle on", len(toks), "rows")
    ref = oracle.forward(qs, ks, vs, n_blocks=w.n_blocks, layout=w.layout, mask=w.mask,
                         max_ring_passes=w.max_ring_passes, cu_seqlens=cu, scale=w.scale,
                         rows=(np.array([idx[int(h)] for h in heads]), toks), key_valid=kv)
    got = out.cpu()[toks, heads].double().numpy()
    _check_bf16(got, ref["out"], name, dt)
    got_lse = lse.cpu()[heads, toks].double().numpy()
    empty = np.isneginf(ref["lse"])
    assert np.array_equal(np.isneginf(got_lse), empty)
    assert np.abs(got_lse[~empty] - ref["lse"][~empty]).max() <= 1e-3
    tal = oracle.tallies(w.T, w.n_blocks, layout=w.layout, mask=w.mask, max_ring_passes=w.max_ring_passes,
                         cu_seqlens=cu, tile_q=st["tile_q"], tile_k=st["tile_k"])
    for key, val in tal.items():
        assert st[key] == val, key
