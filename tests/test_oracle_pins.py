"""Pins for the fp64 oracle: every check here compares it with something other
than itself -- the pages' two worked examples re-run as the pages describe
them, a library softmax-attention routine on cases that reduce to it, closed
forms, invariants of softmax, and hand-derived tallies.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa64(q, k, v, mask=None, scale=None, is_causal=False):
    """torch's scaled-dot-product attention in fp64 on the CPU; q [Tq, H, d], k/v [Tk, H, d]."""
    qh, kh, vh = (x.double().permute(1, 0, 2) for x in (q, k, v))
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale, is_causal=is_causal)
    return o.permute(1, 0, 2).numpy()


# ---------------------------------------------------------------------------
# Worked example of the Ultralytics "Ring Attention" page (section "Come
# funziona"): 4 devices x block 8 x dim 16, seed 0, randn(3, 32, 16), scores
# scaled by 1/sqrt(dim), weights exp(score) with no maximum subtracted, each
# device's numerator and denominator accumulated over its ring order.
# ---------------------------------------------------------------------------

def _ring_order_sums(q, k, v, n_dev, scale, dtype):
    """Every device's rows as (sum of weighted values) / (sum of weights), the
    block terms added in ring order: at step s device i holds key block
    (i - s) mod n_dev.  q, k, v: [T, dim] tensors."""
    q, k, v = (t.to(dtype) for t in (q, k, v))
    B = q.shape[0] // n_dev
    rows = []
    for dev in range(n_dev):
        visits = [(dev - s) % n_dev for s in range(n_dev)]
        weight = [torch.exp(scale * q[dev * B:(dev + 1) * B] @ k[j * B:(j + 1) * B].T) for j in visits]
        numer = torch.zeros(B, v.shape[1], dtype=dtype)
        denom = torch.zeros(B, 1, dtype=dtype)
        for wgt, j in zip(weight, visits):
            numer = numer + wgt @ v[j * B:(j + 1) * B]
            denom = denom + wgt.sum(dim=1, keepdim=True)
        rows.append(numer / denom)
    return torch.cat(rows)


def test_p4_worked_example_equals_oracle_fp64():
    w = W.WORKLOADS["p4_ring4_b8_d16"]
    x = W.make_inputs(w)
    q, k, v = (t[:, 0] for t in (x["q"], x["k"], x["v"]))
    ring = _ring_order_sums(q, k, v, 4, 1 / 16 ** 0.5, torch.float64).numpy()
    r = oracle.forward(x["q"], x["k"], x["v"], n_blocks=4, scale=w.scale)
    assert np.abs(r["out"][:, 0] - ring).max() < 1e-12


def test_p4_worked_example_fp32_agrees_with_full_attention():
    # The page reports that its fp32 ring result equals full attention to an
    # absolute 1e-5; the same holds here against a library attention routine
    # and against the fp64 oracle.
    w = W.WORKLOADS["p4_ring4_b8_d16"]
    x = W.make_inputs(w)
    q, k, v = (t[:, 0] for t in (x["q"], x["k"], x["v"]))
    ring32 = _ring_order_sums(q, k, v, 4, 1 / 16 ** 0.5, torch.float32)
    lib32 = F.scaled_dot_product_attention(q[None], k[None], v[None], scale=1 / 16 ** 0.5)[0]
    assert (ring32 - lib32).abs().max() < 1e-5
    r = oracle.forward(x["q"], x["k"], x["v"], n_blocks=4, scale=w.scale)
    assert np.abs(r["out"][:, 0] - ring32.double().numpy()).max() < 1e-5
    # the page's sizes: an 8x8 score block per device, 32 tokens in all
    assert (w.block, w.T) == (8, 32)


# ---------------------------------------------------------------------------
# "Ring Attention simulation" gist: 1024 tokens, d_head 2, 16 workers, no
# scaling; keys are folded in one at a time into a normalised running output
# with a running maximum and weight sum; device i takes its own block first,
# then the blocks of devices i-1, i-2, ...
# ---------------------------------------------------------------------------

def _fold_keys(scores, vals, state):
    """Fold keys one by one into (out, ref, wsum): out is the softmax-weighted
    mean of the values folded so far, ref the largest score seen, wsum the sum
    of exp(score - ref).  scores [rows, keys], vals [keys, dim]."""
    out, ref, wsum = state
    for t in range(scores.shape[1]):
        s_t = scores[:, t:t + 1]
        new_ref = np.maximum(ref, s_t)
        kept = wsum * np.exp(ref - new_ref)  # earlier weights against the new reference
        w_t = np.exp(s_t - new_ref)
        wsum = kept + w_t
        out = (out * kept + w_t * vals[t]) / wsum
        ref = new_ref
    return out, ref, wsum


def _keywise_ring(x, n_dev, n_steps):
    q, k, v = (t[:, 0].double().numpy() for t in (x["q"], x["k"], x["v"]))
    B = q.shape[0] // n_dev
    outs, refs, sums = [], [], []
    for dev in range(n_dev):
        state = (np.zeros((B, q.shape[1])), np.full((B, 1), -np.inf), np.zeros((B, 1)))
        for s in range(n_steps):
            j = (dev - s) % n_dev
            state = _fold_keys(q[dev * B:(dev + 1) * B] @ k[j * B:(j + 1) * B].T, v[j * B:(j + 1) * B], state)
        outs.append(state[0])
        refs.append(state[1][:, 0])
        sums.append(state[2][:, 0])
    return np.concatenate(outs), np.concatenate(refs), np.concatenate(sums)


def test_p2_recurrence_equals_oracle_all_steps():
    w = W.WORKLOADS["p2_1024tok_d2_16blk"]
    x = W.make_inputs(w)
    o, m, d = _keywise_ring(x, 16, 16)
    r = oracle.forward(x["q"], x["k"], x["v"], n_blocks=16, scale=1.0)
    assert np.abs(r["out"][:, 0] - o).max() < 1e-12
    assert np.abs(r["m"][0] - m).max() < 1e-12
    assert np.abs(r["l"][0] / d - 1).max() < 1e-12


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_p2_partial_ring_state_equals_oracle_with_pass_limit(steps):
    # After `steps` ring steps a device has seen blocks i, i-1, ..., i-steps+1:
    # the oracle's max_ring_passes = steps must give the same state.
    w = W.WORKLOADS["p2_1024tok_d2_16blk"]
    x = W.make_inputs(w)
    o, m, d = _keywise_ring(x, 16, steps)
    r = oracle.forward(x["q"], x["k"], x["v"], n_blocks=16, scale=1.0, max_ring_passes=steps)
    assert np.abs(r["out"][:, 0] - o).max() < 1e-12
    assert np.abs(r["m"][0] - m).max() < 1e-12
    assert np.abs(r["l"][0] / d - 1).max() < 1e-12


def test_p2_fp32_claim_holds():
    # The gist asserts allclose(correct, output, rtol=1e-4, atol=1e-6) in fp32.
    w = W.WORKLOADS["p2_1024tok_d2_16blk"]
    x = W.make_inputs(w)
    q, k, v = (t[:, 0] for t in (x["q"], x["k"], x["v"]))
    correct = F.softmax(q @ k.T, dim=-1) @ v
    r = oracle.forward(x["q"], x["k"], x["v"], n_blocks=16, scale=1.0)
    assert torch.allclose(correct.double(), torch.from_numpy(r["out"][:, 0]), rtol=1e-4, atol=1e-6)


# ---------------------------------------------------------------------------
# Cases that reduce to a library attention routine.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,N,Hq,Hkv,d,seed", [(24, 3, 2, 2, 8, 0), (40, 4, 4, 2, 5, 1), (33, 1, 3, 1, 16, 2)])
def test_no_mask_and_causal_equal_sdpa(T, N, Hq, Hkv, d, seed):
    q, k, v = W.random_qkv(T, Hq, Hkv, d, "f32", seed)
    rep = Hq // Hkv
    kk, vv = k.repeat_interleave(rep, dim=1), v.repeat_interleave(rep, dim=1)
    for mask, causal in ((oracle.MASK_NONE, False), (oracle.MASK_CAUSAL, True)):
        r = oracle.forward(q, k, v, n_blocks=N, mask=mask)
        ref = _sdpa64(q, kk, vv, is_causal=causal)
        assert np.abs(r["out"] - ref).max() < 1e-12


def test_bf16_inputs_decode_exactly():
    q, k, v = W.random_qkv(32, 2, 2, 8, "bf16", 7)
    r = oracle.forward(q, k, v, n_blocks=4, mask=oracle.MASK_CAUSAL)
    ref = _sdpa64(q.float(), k.float(), v.float(), is_causal=True)
    assert np.abs(r["out"] - ref).max() < 1e-12


@pytest.mark.parametrize("mask", [0, 1])
def test_key_padding_equals_sdpa_with_boolean_mask(mask):
    """Key-padding mask: torch's fp64 attention with the boolean mask
    (causal and key_valid); rows left with no key give out 0, lse -inf."""
    T, N, H, d = 48, 4, 2, 8
    q, k, v = W.random_qkv(T, H, H, d, "f32", 31 + mask)
    kv = torch.rand(T, generator=torch.Generator().manual_seed(5)) > 0.4
    kv[0] = False  # under the causal mask, row 0 keeps no key
    r = oracle.forward(q, k, v, n_blocks=N, mask=mask, key_valid=kv)
    allowed = kv[None, :].expand(T, T).clone()
    if mask:
        allowed &= torch.ones(T, T, dtype=torch.bool).tril()
    has = allowed.any(dim=1)
    ref = _sdpa64(q, k, v, mask=allowed)
    assert np.abs(r["out"][has.numpy()] - ref[has.numpy()]).max() < 1e-12
    assert not r["out"][~has.numpy()].any() and np.isneginf(r["lse"][:, ~has.numpy()]).all()
    assert bool((~has).any()) == bool(mask)


def test_key_padding_all_valid_is_no_mask_and_drops_keys_exactly():
    T, N, H, d = 40, 4, 2, 8
    q, k, v = W.random_qkv(T, H, H, d, "f32", 33)
    a = oracle.forward(q, k, v, n_blocks=N, mask=1)
    b = oracle.forward(q, k, v, n_blocks=N, mask=1, key_valid=torch.ones(T, dtype=torch.bool))
    assert all(np.array_equal(a[x], b[x]) for x in ("out", "lse", "m", "l", "O"))
    # one block against one block: padding equals removing the padded rows
    kv = torch.tensor([i % 3 != 1 for i in range(T)])
    pos = np.arange(T)
    c = oracle.block(q, k, v, pos, pos, key_valid=kv)
    e = oracle.block(q, k[kv], v[kv], pos, pos[kv.numpy()])
    assert np.abs(c["out"] - e["out"]).max() < 1e-13 and np.abs(c["lse"] - e["lse"]).max() < 1e-13


def test_f16_inputs_decode_exactly():
    """fp16 values off the bf16 grid (10-bit fractions), subnormal and near
    the top of the binary16 range reach the oracle unchanged: its result
    equals fp64 attention on torch's own fp16 -> fp64 conversion."""
    q, k, v = (x * 0.37 for x in W.random_qkv(32, 2, 2, 8, "f32", 8))
    q, k, v = q.half(), k.half(), v.half()
    v[3, 0, 0], v[5, 1, 2], v[9, 0, 7] = 6.0e-8, -3.1e-5, 6.0e4   # subnormal, subnormal, large
    assert (q.float() != q.float().to(torch.bfloat16).float()).any()
    r = oracle.forward(q, k, v, n_blocks=4, mask=oracle.MASK_CAUSAL)
    ref = _sdpa64(q.double(), k.double(), v.double(), is_causal=True)
    assert np.abs(r["out"] - ref).max() <= 1e-12 * max(1.0, float(np.abs(ref).max()))
    g = W.random_dout(32, 2, 8, "f16", 8)
    dq, dk, dv = oracle.backward(q, k, v, g, n_blocks=4, mask=oracle.MASK_CAUSAL)
    dq32, dk32, dv32 = oracle.backward(q.float(), k.float(), v.float(), g.float(), n_blocks=4,
                                       mask=oracle.MASK_CAUSAL)
    assert np.array_equal(dq, dq32) and np.array_equal(dk, dk32) and np.array_equal(dv, dv32)


@pytest.mark.parametrize("N", [2, 4, 8])
def test_striped_causal_full_ring_is_plain_causal(N):
    # The mask is defined on original token order; the striped assignment only
    # changes which device holds a token, so after all N passes the result is
    # plain causal attention.
    T = 8 * N
    q, k, v = W.random_qkv(T, 2, 1, 8, "f32", 10 + N)
    r = oracle.forward(q, k, v, n_blocks=N, layout=oracle.LAYOUT_STRIPED, mask=oracle.MASK_CAUSAL)
    ref = _sdpa64(q, k.repeat_interleave(2, 1), v.repeat_interleave(2, 1), is_causal=True)
    assert np.abs(r["out"] - ref).max() < 1e-12


def test_doc_causal_equals_per_document_causal():
    cu = [0, 7, 8, 20, 31, 48]
    T = 48
    q, k, v = W.random_qkv(T, 3, 3, 6, "f32", 21)
    r = oracle.forward(q, k, v, n_blocks=4, mask=oracle.MASK_DOC_CAUSAL, cu_seqlens=cu)
    for a, b in zip(cu[:-1], cu[1:]):
        ref = _sdpa64(q[a:b], k[a:b], v[a:b], is_causal=True)
        assert np.abs(r["out"][a:b] - ref).max() < 1e-12


def _ring_schedule_keys(i, N, P):
    """Key blocks device i holds during the first P steps: (i - s) mod N."""
    return [(i - s) % N for s in range(min(P, N))]


@pytest.mark.parametrize("layout", [oracle.LAYOUT_CONTIGUOUS, oracle.LAYOUT_STRIPED])
@pytest.mark.parametrize("mask", [oracle.MASK_NONE, oracle.MASK_CAUSAL])
@pytest.mark.parametrize("P", [1, 2, 3])
def test_pass_limit_equals_attention_over_visited_blocks(layout, mask, P):
    N, B = 4, 6
    T = N * B
    q, k, v = W.random_qkv(T, 2, 2, 4, "f32", 100 + P)
    r = oracle.forward(q, k, v, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P)
    tok = (lambda blk: np.arange(B) * N + blk) if layout == oracle.LAYOUT_STRIPED else \
        (lambda blk: np.arange(B) + blk * B)
    for i in range(N):
        rows = tok(i)
        keys = np.concatenate([tok(j) for j in _ring_schedule_keys(i, N, P)])
        bool_mask = None
        if mask == oracle.MASK_CAUSAL:
            bool_mask = torch.from_numpy(keys[None, :] <= rows[:, None])
        ref = _sdpa64(q[rows], k[keys], v[keys], mask=bool_mask)
        assert np.abs(r["out"][rows] - ref).max() < 1e-12


def test_gqa_head_map_is_consecutive_groups():
    # q heads 0..3 share kv head 0, 4..7 share kv head 1 (repeat_interleave).
    q, k, v = W.random_qkv(16, 8, 2, 4, "f32", 5)
    r = oracle.forward(q, k, v, n_blocks=2, mask=oracle.MASK_CAUSAL)
    for h in range(8):
        ref = _sdpa64(q[:, h:h + 1], k[:, h // 4:h // 4 + 1], v[:, h // 4:h // 4 + 1], is_causal=True)
        assert np.abs(r["out"][:, h:h + 1] - ref).max() < 1e-12


def test_strided_views_read_like_contiguous():
    qkv = torch.randn(20, 3, 2, 8, generator=torch.Generator().manual_seed(3))
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    r1 = oracle.forward(q, k, v, n_blocks=4, mask=oracle.MASK_CAUSAL)
    r2 = oracle.forward(q.contiguous(), k.contiguous(), v.contiguous(), n_blocks=4, mask=oracle.MASK_CAUSAL)
    assert np.array_equal(r1["out"], r2["out"]) and np.array_equal(r1["lse"], r2["lse"])


# ---------------------------------------------------------------------------
# Invariants and closed forms (shift invariance of softmax: Zhihu article,
# local vs. global softmax section).
# ---------------------------------------------------------------------------

def test_key_shift_invariance_and_lse_shift():
    # Keys on a 1/8 grid and a shift on a 16 grid: k + u is exact in fp32, so
    # every score of row t moves by exactly scale * q_t . u.
    T, H, d = 32, 2, 8
    g = torch.Generator().manual_seed(11)
    q = torch.randn(T, H, d, generator=g)
    k = torch.round(torch.randn(T, H, d, generator=g) * 8) / 8
    v = torch.randn(T, H, d, generator=g)
    u = torch.round(torch.randn(d, generator=g) * 10) * 16
    scale = 1 / math.sqrt(d)
    base = oracle.forward(q, k, v, n_blocks=4, mask=oracle.MASK_CAUSAL)
    shifted = oracle.forward(q, k + u, v, n_blocks=4, mask=oracle.MASK_CAUSAL)
    shift = scale * (q.double() @ u.double()).numpy().T  # [H, T]
    # scores are ~1e2..1e3 here: an exp without the max subtracted would overflow
    assert np.abs(shift).max() > 100
    assert np.abs(shifted["out"] - base["out"]).max() < 1e-9
    assert np.isfinite(shifted["lse"]).all()
    assert np.abs(shifted["lse"] - base["lse"] - shift).max() < 1e-9


def test_value_shift_and_convexity():
    T, H, d = 24, 2, 5
    q, k, v = W.random_qkv(T, H, H, d, "f32", 13)
    v = torch.round(v * 64) / 64  # on a grid so that v + c is exact in fp32
    c = torch.tensor([1.5, -2.0, 0.25, 8.0, -0.5])
    a = oracle.forward(q, k, v, n_blocks=3, mask=oracle.MASK_CAUSAL)
    b = oracle.forward(q, k, v + c, n_blocks=3, mask=oracle.MASK_CAUSAL)
    assert np.abs(b["out"] - a["out"] - c.numpy()).max() < 1e-12
    assert np.array_equal(a["lse"], b["lse"])
    vv = v.double().numpy()
    for t in range(T):
        for h in range(H):
            assert (a["out"][t, h] <= vv[:t + 1, h].max(0) + 1e-12).all()
            assert (a["out"][t, h] >= vv[:t + 1, h].min(0) - 1e-12).all()


def test_zero_queries_give_running_mean_and_log_count():
    T, H, d = 20, 2, 3
    _, k, v = W.random_qkv(T, H, H, d, "f32", 14)
    q = torch.zeros(T, H, d)
    r = oracle.forward(q, k, v, n_blocks=4, mask=oracle.MASK_CAUSAL)
    vv = v.double().numpy()
    cum_mean = np.cumsum(vv, axis=0) / np.arange(1, T + 1)[:, None, None]
    assert np.abs(r["out"] - cum_mean).max() < 1e-13
    assert np.abs(r["lse"] - np.log(np.arange(1, T + 1))[None, :]).max() < 1e-13
    assert np.array_equal(r["m"], np.zeros((H, T)))
    assert np.abs(r["l"] - np.arange(1, T + 1)[None, :]).max() == 0


def test_first_token_sees_only_itself_and_identical_keys_average():
    T, H, d = 16, 1, 4
    q, k, v = W.random_qkv(T, H, H, d, "f32", 15)
    r = oracle.forward(q, k, v, n_blocks=2, mask=oracle.MASK_CAUSAL)
    assert np.array_equal(r["out"][0], v[0].double().numpy())
    k_same = k[:1].expand(T, H, d).contiguous()
    r2 = oracle.forward(q, k_same, v, n_blocks=2, mask=oracle.MASK_NONE)
    assert np.abs(r2["out"] - v.double().numpy().mean(0, keepdims=True)).max() < 1e-13


# ---------------------------------------------------------------------------
# Block state, finalize and merge.
# ---------------------------------------------------------------------------

def test_block_state_merged_over_ring_equals_forward():
    N, B, H, d = 4, 8, 2, 6
    T = N * B
    q, k, v = W.random_qkv(T, H, H, d, "f32", 16)
    full = oracle.forward(q, k, v, n_blocks=N, mask=oracle.MASK_CAUSAL)
    for i in range(N):
        out, lse = None, None
        for s in range(N):
            j = (i - s) % N
            r = oracle.block(q[i * B:(i + 1) * B], k[j * B:(j + 1) * B], v[j * B:(j + 1) * B],
                             np.arange(B) + i * B, np.arange(B) + j * B, mask=oracle.MASK_CAUSAL)
            o_b, l_b = r["out"].transpose(1, 0, 2), r["lse"]
            if out is None:
                out, lse = o_b, l_b
            else:
                out, lse = oracle.merge(out, lse.T, o_b, l_b.T)
                lse = lse.T
        assert np.abs(out - full["out"][i * B:(i + 1) * B]).max() < 1e-13
        assert np.abs(lse - full["lse"][:, i * B:(i + 1) * B]).max() < 1e-13


def test_block_fully_masked_rows_are_empty():
    q, k, v = W.random_qkv(8, 1, 1, 4, "f32", 17)
    r = oracle.block(q, k, v, np.arange(8), np.arange(8) + 8, mask=oracle.MASK_CAUSAL)
    assert np.array_equal(r["out"], np.zeros_like(r["out"]))
    assert np.isneginf(r["lse"]).all() and np.isneginf(r["m"]).all()
    assert np.array_equal(r["l"], np.zeros_like(r["l"]))
    out, lse = oracle.finalize(r["O"], r["m"], r["l"])
    assert np.array_equal(out, np.zeros_like(out)) and np.isneginf(lse).all()


def test_finalize_matches_definition_closed_form():
    # Q = 0: m = 0, l = number of keys, O = sum of values -> out = mean, lse = ln n.
    _, k, v = W.random_qkv(12, 1, 1, 3, "f32", 18)
    q = torch.zeros(12, 1, 3)
    r = oracle.block(q, k, v, np.arange(12), np.arange(12), mask=oracle.MASK_NONE)
    out, lse = oracle.finalize(r["O"], r["m"], r["l"])
    assert np.abs(out[0] - v.double().numpy()[:, 0].mean(0)).max() < 1e-14
    assert np.abs(lse - math.log(12)).max() < 1e-14


def test_merge_of_any_partition_equals_direct():
    rng = np.random.default_rng(19)
    T, H, d = 30, 2, 4
    q, k, v = W.random_qkv(T, H, H, d, "f32", 19)
    keys = rng.permutation(T)
    a_idx, b_idx = np.sort(keys[:11]), np.sort(keys[11:])
    pos = np.arange(T)
    direct = oracle.block(q, k, v, pos, pos, mask=oracle.MASK_CAUSAL)
    ra = oracle.block(q, k[a_idx], v[a_idx], pos, a_idx, mask=oracle.MASK_CAUSAL)
    rb = oracle.block(q, k[b_idx], v[b_idx], pos, b_idx, mask=oracle.MASK_CAUSAL)
    out, lse = oracle.merge(ra["out"], ra["lse"], rb["out"], rb["lse"])
    assert np.abs(out - direct["out"]).max() < 1e-13
    assert np.abs(lse - direct["lse"]).max() < 1e-13
    out2, lse2 = oracle.merge(rb["out"], rb["lse"], ra["out"], ra["lse"])
    assert np.abs(out2 - out).max() < 1e-15 and np.abs(lse2 - lse).max() < 1e-15


def test_merge_associative_and_empty_is_identity():
    rng = np.random.default_rng(20)
    o = [rng.normal(size=(5, 3)) for _ in range(3)]
    l = [rng.normal(size=5) * 3 for _ in range(3)]
    x1 = oracle.merge(*oracle.merge(o[0], l[0], o[1], l[1]), o[2], l[2])
    x2 = oracle.merge(o[0], l[0], *oracle.merge(o[1], l[1], o[2], l[2]))
    assert np.abs(x1[0] - x2[0]).max() < 1e-14 and np.abs(x1[1] - x2[1]).max() < 1e-14
    e_out, e_lse = np.zeros((5, 3)), np.full(5, -np.inf)
    y = oracle.merge(o[0], l[0], e_out, e_lse)
    assert np.array_equal(y[0], o[0]) and np.array_equal(y[1], l[0])
    z = oracle.merge(e_out, e_lse, e_out, e_lse)
    assert np.array_equal(z[0], e_out) and np.isneginf(z[1]).all()


# ---------------------------------------------------------------------------
# Tallies and pair counts.
# ---------------------------------------------------------------------------

def _causal_diag_tiles(B, tq, tk):
    """Closed form for a square causal block split into tq x tk tiles, tq a
    multiple of tk: q-tile a has a*r full tiles and r partial ones (r = tq/tk)."""
    r, nq = tq // tk, B // tq
    full = r * nq * (nq - 1) // 2
    part = r * nq
    return (nq * (B // tk)) - full - part, full, part


@pytest.mark.parametrize("N,B,tq,tk", [(8, 4096, 128, 64), (4, 512, 64, 64), (3, 256, 128, 32)])
def test_tallies_contiguous_causal_closed_form(N, B, tq, tk):
    t = oracle.tallies(N * B, N, mask=oracle.MASK_CAUSAL, tile_q=tq, tile_k=tk)
    per_block = (B // tq) * (B // tk)
    s, f, p = _causal_diag_tiles(B, tq, tk)
    lower = N * (N - 1) // 2
    assert t["block_pairs_visited"] == N * N
    assert (t["block_pairs_skipped"], t["block_pairs_full"], t["block_pairs_partial"]) == (lower, lower, N)
    assert t["tiles_skipped"] == lower * per_block + N * s
    assert t["tiles_full"] == lower * per_block + N * f
    assert t["tiles_partial"] == N * p


@pytest.mark.parametrize("N,B,tq,tk", [(16, 256, 64, 32), (4, 128, 32, 32)])
def test_tallies_striped_causal_closed_form(N, B, tq, tk):
    # Every striped block pair is about half allowed: nothing skipped or full
    # at block level; inside, each pair looks like a causal diagonal block.
    t = oracle.tallies(N * B, N, layout=oracle.LAYOUT_STRIPED, mask=oracle.MASK_CAUSAL, tile_q=tq, tile_k=tk)
    s, f, p = _causal_diag_tiles(B, tq, tk)
    assert (t["block_pairs_visited"], t["block_pairs_skipped"], t["block_pairs_full"],
            t["block_pairs_partial"]) == (N * N, 0, 0, N * N)
    assert (t["tiles_skipped"], t["tiles_full"], t["tiles_partial"]) == (N * N * s, N * N * f, N * N * p)


@pytest.mark.parametrize("N,B", [(4, 6), (3, 5)])
def test_tallies_striped_unit_tiles_count_pairs(N, B):
    # With 1x1 tiles every tile is one (query, key) pair: block pair (r, s)
    # allows B(B+1)/2 pairs when s <= r (diagonal included) and B(B-1)/2 when
    # s > r, which sums to T(T+1)/2.
    T = N * B
    t = oracle.tallies(T, N, layout=oracle.LAYOUT_STRIPED, mask=oracle.MASK_CAUSAL, tile_q=1, tile_k=1)
    incl = N * (N + 1) // 2 * (B * (B + 1) // 2)
    strict = N * (N - 1) // 2 * (B * (B - 1) // 2)
    assert incl + strict == T * (T + 1) // 2
    assert t["tiles_full"] == incl + strict
    assert t["tiles_skipped"] == T * T - (incl + strict) and t["tiles_partial"] == 0


@pytest.mark.parametrize("P", [1, 3, 8, 20])
def test_tallies_no_mask_and_visit_count(P):
    N, B = 8, 96
    t = oracle.tallies(N * B, N, mask=oracle.MASK_NONE, max_ring_passes=P, tile_q=64, tile_k=64)
    v = N * min(P, N)
    assert t["block_pairs_visited"] == v and t["block_pairs_full"] == v
    assert t["tiles_full"] == v * 4 and t["tiles_skipped"] == 0 and t["tiles_partial"] == 0


def test_tallies_and_pairs_doc_causal_golden():
    g = json.load(open(os.path.join(GOLDEN, "doc_causal_tallies_T16_N2.json")))
    for case in g["cases"]:
        t = oracle.tallies(g["T"], g["n_blocks"], mask=oracle.MASK_DOC_CAUSAL,
                           max_ring_passes=case["max_ring_passes"], cu_seqlens=g["cu_seqlens"],
                           tile_q=g["tile_q"], tile_k=g["tile_k"])
        assert t == case["tallies"]
        n = oracle.allowed_pairs(g["T"], g["n_blocks"], mask=oracle.MASK_DOC_CAUSAL,
                                 max_ring_passes=case["max_ring_passes"], cu_seqlens=g["cu_seqlens"])
        assert n == case["allowed_pairs"]


def test_varlen_workload_block_tallies_structure():
    # Documents are at most one block long, so with 8 blocks and 4 passes:
    # 8 own-block pairs partial, wrapped and distance-2/3 pairs skipped, and a
    # distance-1 pair is partial exactly when a document crosses the boundary.
    w = W.WORKLOADS["varlen_packed128k_h32_d128_8blk_p4"]
    cu = W.doc_cu_seqlens(w.seed, w.T, *w.doc_len_range)
    assert cu[0] == 0 and cu[-1] == w.T and np.all(np.diff(cu) >= 1) and np.all(np.diff(cu) <= 16384)
    B = w.block
    crossed = sum(1 for kb in range(1, w.n_blocks) if (kb * B) not in set(cu.tolist()))
    n = 2048  # scale the brute force down: same documents relative to blocks, smaller rows
    assert B % n == 0
    t = oracle.tallies(w.T, w.n_blocks, mask=w.mask, max_ring_passes=w.max_ring_passes,
                       cu_seqlens=cu, tile_q=B, tile_k=B)
    assert t["block_pairs_visited"] == 32
    assert t["block_pairs_partial"] == 8 + crossed
    assert t["block_pairs_skipped"] == 24 - crossed
    assert t["block_pairs_full"] == 0


@pytest.mark.parametrize("layout", [oracle.LAYOUT_CONTIGUOUS, oracle.LAYOUT_STRIPED])
def test_allowed_pairs_closed_forms(layout):
    T, N = 256, 8
    assert oracle.allowed_pairs(T, N, layout=layout, mask=oracle.MASK_CAUSAL) == T * (T + 1) // 2
    for P in (1, 3, 8):
        assert oracle.allowed_pairs(T, N, layout=layout, mask=oracle.MASK_NONE, max_ring_passes=P) == \
            N * min(P, N) * (T // N) ** 2
    cu = [0, 10, 100, 101, 256]
    lens = np.diff(cu)
    assert oracle.allowed_pairs(T, N, mask=oracle.MASK_DOC_CAUSAL, cu_seqlens=cu) == \
        int((lens * (lens + 1) // 2).sum())
