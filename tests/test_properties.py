"""Property sweeps (Hypothesis) over small rings, T <= 512 tokens, every
mask, layout and pass limit, with document splits and key padding drawn as
well.  CPU: the planner's tallies and allowed-pair count equal the oracle's
brute force; the oracle equals a library attention routine under the same
visibility rule.  GPU: the forward meets its bar against the oracle.
Examples are derandomized (the same sequence every run) and the GPU sweep
does not shrink: it stops at the first failing example and prints it."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import oracle
import workloads as W
from bounds import allowed, forward_bound

SWEEP = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                 suppress_health_check=[HealthCheck.too_slow])


@st.composite
def rings(draw, max_T=512):
    """(T, N, layout, mask, P, docs): N ring blocks of B tokens, T = N B <= max_T."""
    N = draw(st.integers(1, 9))
    B = draw(st.integers(1, max_T // N))
    T = N * B
    mask = draw(st.sampled_from([0, 1, 2]))
    layout = 0 if mask == 2 else draw(st.sampled_from([0, 1]))  # documents: contiguous blocks only
    P = draw(st.integers(1, N))
    docs = None
    if mask == 2:
        n_cut = draw(st.integers(0, min(5, T - 1)))
        cuts = sorted(draw(st.sets(st.integers(1, T - 1), min_size=n_cut, max_size=n_cut))) if T > 1 else []
        docs = [0] + cuts + [T]
    return T, N, layout, mask, P, docs


@SWEEP
@given(ring=rings(), dt=st.sampled_from([torch.bfloat16, torch.float32]), d=st.sampled_from([64, 128]))
def test_planner_equals_oracle_brute_force(ring, dt, d):
    import ring_attention_step_amd as ra
    T, N, layout, mask, P, docs = ring
    tq, tk = ra.ring_attn_tile_shape(dt, d)
    got = ra.ring_attn_plan(T, N, layout=layout, mask_mode=mask, max_ring_passes=P, cu_seqlens_host=docs,
                            dtype=dt, head_dim=d)
    want = oracle.tallies(T, N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs, tile_q=tq, tile_k=tk)
    for key, val in want.items():
        assert got[key] == val, (key, ring)
    assert got["allowed_pairs"] == oracle.allowed_pairs(T, N, layout=layout, mask=mask, max_ring_passes=P,
                                                        cu_seqlens=docs) == int(allowed(T, N, layout, mask, P,
                                                                                        docs).sum())


@SWEEP
@given(ring=rings(max_T=256), heads=st.sampled_from([(1, 1), (2, 1), (4, 2)]), d=st.integers(1, 24),
       pad=st.booleans(), seed=st.integers(0, 2 ** 16))
def test_oracle_equals_library_attention_under_the_same_mask(ring, heads, d, pad, seed):
    """Rows with at least one visible key: the oracle's out equals torch's
    fp64 scaled-dot-product attention with the visibility rule as a boolean
    mask, and its lse equals logsumexp of the visible scores; rows with none
    get out 0 and lse -inf."""
    T, N, layout, mask, P, docs = ring
    Hq, Hkv = heads
    q, k, v = W.random_qkv(T, Hq, Hkv, d, "f32", seed)
    kv = W.random_key_valid(T, seed, 0.3).numpy() if pad and T > 1 else None
    ok = allowed(T, N, layout, mask, P, docs, kv)
    r = oracle.forward(q, k, v, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs,
                       key_valid=kv)
    scale = 1.0 / math.sqrt(d)
    live = ok.any(axis=1)
    g = Hq // Hkv
    for h in range(Hq):
        qh, kh, vh = (x[:, i].double() for x, i in ((q, h), (k, h // g), (v, h // g)))
        if live.any():
            m = torch.from_numpy(ok[live])
            o = F.scaled_dot_product_attention(qh[live][None], kh[None], vh[None], attn_mask=m[None], scale=scale)[0]
            assert np.abs(r["out"][live, h] - o.numpy()).max() < 1e-12
            s = (scale * qh[live] @ kh.T).masked_fill(~m, -math.inf)
            assert np.abs(r["lse"][h, live] - torch.logsumexp(s, dim=1).numpy()).max() < 1e-12
        assert not r["out"][~live, h].any() and np.isneginf(r["lse"][h, ~live]).all()


@pytest.mark.gpu
@settings(max_examples=40, deadline=None, derandomize=True, database=None, phases=[Phase.explicit, Phase.generate],
          suppress_health_check=[HealthCheck.too_slow])
@given(ring=rings(), heads=st.sampled_from([(1, 1), (2, 1), (4, 2), (2, 2), (4, 1), (8, 1), (16, 2), (6, 2)]),
       kind=st.sampled_from(["bf16-64", "bf16-128", "f16-128", "f32-16", "f32-40"]), pad=st.booleans(),
       prefetch=st.booleans(), seed=st.integers(0, 2 ** 16))
def test_gpu_forward_meets_its_bar_on_any_small_ring(ring, heads, kind, pad, prefetch, seed):
    """Heads cover every work-item shape of the one-launch ring: 1, 2, 4 and 8
    query heads per item (groups of 1, 2, 4 and 8), and a group of 3.
    16-bit inputs: every output element within the first-order rounding
    bound of the 16-bit forward; fp32 inputs: within 1e-5; lse within 1e-3
    (16-bit) or 1e-5 (fp32); -inf exactly where a row sees no key."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_step_amd as ra
    T, N, layout, mask, P, docs = ring
    Hq, Hkv = heads
    dt, d = kind.split("-")
    d = int(d)
    print("[case]", ring, heads, kind, "pad", pad, "prefetch", prefetch, "seed", seed, flush=True)
    qh, kh, vh = W.random_qkv(T, Hq, Hkv, d, dt, seed)
    kv = W.random_key_valid(T, seed, 0.3) if pad and T > 1 else None
    out, lse = ra.forward(qh.cuda(), kh.cuda(), vh.cuda(), n_blocks=N, layout="striped" if layout else "contiguous",
                          causal=mask == 1, cu_seqlens=docs, max_ring_passes=P, out_dtype=torch.float32,
                          return_lse=True, prefetch=prefetch, key_valid=None if kv is None else kv.cuda())
    torch.cuda.synchronize()
    ref = oracle.forward(qh, kh, vh, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs,
                         key_valid=None if kv is None else kv.numpy())
    got = out.cpu().double().numpy()
    if dt == "f32":
        assert np.abs(got - ref["out"]).max() <= 1e-5
        lse_tol = 1e-5
    else:
        b = forward_bound(qh, kh, vh, N, layout, mask, P, docs, dt, key_valid=None if kv is None else kv.numpy())
        assert (np.abs(got - ref["out"]) <= b * (1 + 2.0 ** -10) + 1e-6).all()
        lse_tol = 1e-3
    gl = lse.cpu().double().numpy()
    empty = np.isneginf(ref["lse"])
    assert np.array_equal(np.isneginf(gl), empty)
    assert (np.abs(gl[~empty] - ref["lse"][~empty]) <= lse_tol).all()
