"""Pins of the oracle's backward (ring_oracle.c, ro_backward) against what
does not depend on it:

* central finite differences of the forward oracle's sum(out * dout) in every
  element of q, k and v (the perturbations are the exact differences of the
  float32 inputs, so only the O(h^2) truncation remains);
* fp64 reverse-mode autodiff of plain masked softmax attention written here
  with torch (a library routine), the allowed-pair matrix built here from the
  ring schedule (blocks b = t // B or t % N, key block visible from query
  block when (b_q - b_k) mod N < min(P, N)) and the mask (causal: key <= query;
  doc-causal: also the same document).
"""
import math

import numpy as np
import pytest
import torch

import oracle

CASES = [
    # T, N, Hq, Hkv, d, layout, mask, P, docs
    (12, 3, 2, 1, 3, 0, 1, 3, None),
    (12, 4, 2, 2, 3, 1, 1, 2, None),
    (12, 3, 1, 1, 4, 0, 2, 3, [0, 5, 12]),
    (8, 2, 2, 1, 2, 0, 0, 1, None),
]


def _inputs(T, Hq, Hkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(T, Hq, d, generator=g)
    k = torch.randn(T, Hkv, d, generator=g)
    v = torch.randn(T, Hkv, d, generator=g)
    do = torch.randn(T, Hq, d, generator=g)
    return q, k, v, do


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_matches_finite_differences(case):
    T, N, Hq, Hkv, d, layout, mask, P, docs = CASES[case]
    q, k, v, do = _inputs(T, Hq, Hkv, d, 10 + case)
    kw = dict(n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs)
    dq, dk, dv = oracle.backward(q, k, v, do, **kw)
    dod = do.double().numpy()

    def f(qq, kk, vv):
        return float((oracle.forward(qq, kk, vv, **kw)["out"] * dod).sum())

    h = 1e-3
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        tensors = [q.clone(), k.clone(), v.clone()]
        X = tensors[which]
        num = np.zeros(X.shape)
        for idx in np.ndindex(*X.shape):
            x0 = X[idx].item()
            X[idx] = x0 + h
            xp = X[idx].item()
            fp = f(*tensors)
            X[idx] = x0 - h
            xm = X[idx].item()
            fm = f(*tensors)
            X[idx] = x0
            num[idx] = (fp - fm) / (xp - xm)
        err = np.abs(num - grad).max()
        assert err <= 2e-6 * (1.0 + np.abs(num).max()), (which, err)


def _allowed(T, N, layout, mask, P, docs):
    t = torch.arange(T)
    B = T // N
    blk = t % N if layout == 1 else t // B
    step = (blk[:, None] - blk[None, :]) % N
    ok = step < min(P, N)
    if mask >= 1:
        ok &= t[None, :] <= t[:, None]
    if mask == 2:
        doc = torch.bucketize(t, torch.tensor(docs[1:]), right=True)
        ok &= doc[:, None] == doc[None, :]
    return ok


AUTOGRAD_CASES = [
    (64, 4, 4, 2, 8, 0, 1, 4, None),
    (64, 8, 2, 1, 8, 1, 1, 3, None),
    (60, 3, 2, 2, 8, 0, 2, 2, [0, 7, 8, 33, 60]),
    (48, 4, 2, 1, 5, 0, 0, 4, None),
]


def _key_valid(T, seed):
    """About a third of the keys padded, key 0 among them (so under a causal
    mask row 0 has no key left)."""
    kv = torch.rand(T, generator=torch.Generator().manual_seed(seed)) > 0.35
    kv[0] = False
    return kv


@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("case", range(len(AUTOGRAD_CASES)))
def test_backward_matches_fp64_autograd(case, padded):
    T, N, Hq, Hkv, d, layout, mask, P, docs = AUTOGRAD_CASES[case]
    q, k, v, do = _inputs(T, Hq, Hkv, d, 50 + case)
    kv = _key_valid(T, 90 + case) if padded else None
    dq, dk, dv = oracle.backward(q, k, v, do, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P,
                                 cu_seqlens=docs, key_valid=kv)
    ok = _allowed(T, N, layout, mask, P, docs)
    if padded:
        ok &= kv[None, :]
    qd, kd, vd = (x.double().requires_grad_(True) for x in (q, k, v))
    grp = Hq // Hkv
    outs = []
    for hh in range(Hq):
        g = hh // grp
        s = (qd[:, hh] @ kd[:, g].T) / math.sqrt(d)
        s = s.masked_fill(~ok, float("-inf"))
        has = ok.any(dim=1, keepdim=True)
        p = torch.where(has, torch.softmax(torch.where(has, s, torch.zeros_like(s)), dim=1), torch.zeros_like(s))
        p = p.masked_fill(~ok, 0.0)
        outs.append(p @ vd[:, g])
    out = torch.stack(outs, dim=1)
    (out * do.double()).sum().backward()
    for got, want in ((dq, qd.grad), (dk, kd.grad), (dv, vd.grad)):
        want = want.numpy()
        assert np.abs(got - want).max() <= 1e-10 * (1.0 + np.abs(want).max())


def test_padded_keys_get_no_gradient_and_no_weight():
    """A padded key changes nothing: its dk and dv are exactly zero, and dq of
    every row equals the gradients of the same ring without that key's
    influence (its k and v replaced by garbage change no other gradient)."""
    T, N, Hq, Hkv, d = 32, 4, 2, 1, 6
    q, k, v, do = _inputs(T, Hq, Hkv, d, 77)
    kv = _key_valid(T, 78)
    dq, dk, dv = oracle.backward(q, k, v, do, n_blocks=N, mask=1, key_valid=kv)
    assert not dk[~kv.numpy()].any() and not dv[~kv.numpy()].any()
    k2, v2 = k.clone(), v.clone()
    k2[~kv] = 1e3
    v2[~kv] = -7.0
    dq2, dk2, dv2 = oracle.backward(q, k2, v2, do, n_blocks=N, mask=1, key_valid=kv)
    assert np.array_equal(dq, dq2) and np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_zero_output_gradient_gives_zero_gradients():
    q, k, v, do = _inputs(16, 2, 1, 4, 99)
    dq, dk, dv = oracle.backward(q, k, v, torch.zeros_like(do), n_blocks=4, mask=oracle.MASK_CAUSAL)
    assert not dq.any() and not dk.any() and not dv.any()


def test_bf16_inputs_decode_exactly():
    """bf16 q, k, v, dout give the gradients of their exact fp64 values."""
    q, k, v, do = (x.to(torch.bfloat16) for x in _inputs(32, 2, 2, 8, 7))
    a = oracle.backward(q, k, v, do, n_blocks=4, mask=oracle.MASK_CAUSAL)
    b = oracle.backward(q.float(), k.float(), v.float(), do.float(), n_blocks=4, mask=oracle.MASK_CAUSAL)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_dq_rows_equal_full_rows(case):
    """The sampled-row entry returns exactly the full backward's dq rows (a
    row's dq depends on that row alone)."""
    T, N, Hq, Hkv, d, layout, mask, P, docs = CASES[case]
    q, k, v, dout = _inputs(T, Hq, Hkv, d, 70 + case)
    kw = dict(n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs)
    dq, _, _ = oracle.backward(q, k, v, dout, **kw)
    rng = np.random.default_rng(case)
    heads, toks = rng.integers(0, Hq, 9), rng.integers(0, T, 9)
    pairs = sorted(set(zip(heads.tolist(), toks.tolist())))
    heads, toks = np.array([p[0] for p in pairs]), np.array([p[1] for p in pairs])
    got = oracle.backward(q, k, v, dout, rows=(heads, toks), **kw)
    assert got.shape == (len(pairs), d)
    assert np.array_equal(got, dq[toks, heads])


@pytest.mark.parametrize("case", range(len(CASES)))
def test_row_terms_equal_full_gradients_of_a_sparse_dout(case):
    """dout zero outside a few rows: the rows entry's dk / dv (those rows'
    terms only) equal the full backward's, and its dq rows equal the full dq
    rows; the full dq is zero on every other row."""
    T, N, Hq, Hkv, d, layout, mask, P, docs = CASES[case]
    q, k, v, dout = _inputs(T, Hq, Hkv, d, 90 + case)
    rng = np.random.default_rng(10 + case)
    pairs = sorted(set(zip(rng.integers(0, Hq, 6).tolist(), rng.integers(0, T, 6).tolist())))
    heads, toks = np.array([p[0] for p in pairs]), np.array([p[1] for p in pairs])
    sparse = torch.zeros_like(dout)
    sparse[toks, heads] = dout[toks, heads]
    kw = dict(n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs)
    dq, dk, dv = oracle.backward(q, k, v, sparse, **kw)
    dq_r, dk_r, dv_r = oracle.backward(q, k, v, sparse, rows=(heads, toks), rows_dkdv=True, **kw)
    assert np.allclose(dk_r, dk, rtol=0, atol=1e-12) and np.allclose(dv_r, dv, rtol=0, atol=1e-12)
    assert np.array_equal(dq_r, dq[toks, heads])
    rest = np.ones((T, Hq), bool)
    rest[toks, heads] = False
    assert not dq[rest].any()
