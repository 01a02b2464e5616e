"""First-order rounding bounds of the 16-bit GPU path, per output element,
computed in fp64 from the oracle's results (test infrastructure: the GPU
parity tests compare against these; nothing here is on the product path)."""
import numpy as np
import torch

import oracle

U16 = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}  # unit roundoff of the 16-bit type (8 / 11 significant bits)


def allowed(T, N, layout, mask, P, docs, key_valid=None):
    """[T, T] allowed (query, key) pairs: ring visibility, mask, key padding."""
    t = np.arange(T)
    B = T // N
    blk = t % N if layout == 1 else t // B
    ok = (blk[:, None] - blk[None, :]) % N < min(P, N)
    if mask >= 1:
        ok &= t[None, :] <= t[:, None]
    if mask == 2:
        doc = np.searchsorted(np.asarray(docs[1:]), t, side="right")
        ok &= doc[:, None] == doc[None, :]
    if key_valid is not None:
        ok &= np.asarray(key_valid, dtype=bool)[None, :]
    return ok


def backward_bounds(qh, kh, vh, gh, N, layout, mask, P, docs, dt, key_valid=None):
    """First-order bounds on the 16-bit backward's error, per gradient element.
    With u the unit roundoff of the 16-bit type and, per (query t, key j),
    P, dP = dout.v, D = dout.out, dS = P (dP - D) from the fp64 oracle:
      the kernels round dS to 16 bits (and the dK side may use a 16-bit P),
      <= 2 u |dS|;  D comes from the forward's 16-bit out, whose error is
      <= u |out| (its rounding) + u sum_j P |v_j| (the forward's 16-bit P),
      so |dD| <= u sum_c |dout_c| (|out_c| + (P |v|)_c) and dS moves by P |dD|;
      dv uses a 16-bit P: <= u P |dout|.
    Hence |d dq_t| <= scale sum_j w_tj |k_j|, |d dk_j| <= scale sum_t w_tj |q_t|
    with w = 2 u |dS| + P |dD|, and |d dv_j| <= u sum_t P_tj |dout_t|.  fp32
    accumulation adds terms of order 2^-24 times the sums, far below these."""
    T, Hq, d = qh.shape
    Hkv = kh.shape[1]
    scale = 1.0 / np.sqrt(d)
    q, k, v, g = (x.double().numpy() for x in (qh, kh, vh, gh))
    ref = oracle.forward(qh, kh, vh, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs,
                         key_valid=key_valid)
    out, lse = ref["out"], ref["lse"]
    ok = allowed(T, N, layout, mask, P, docs, key_valid)
    u = U16[dt]
    bq, bk, bv = np.zeros((T, Hq, d)), np.zeros((T, Hkv, d)), np.zeros((T, Hkv, d))
    grp = Hq // Hkv
    for h in range(Hq):
        gk = h // grp
        use = ok & np.isfinite(lse[h])[:, None]
        s = scale * (q[:, h] @ k[:, gk].T)
        Pm = np.where(use, np.exp(np.where(use, s - lse[h][:, None], -np.inf)), 0.0)
        dS = Pm * (g[:, h] @ v[:, gk].T - (g[:, h] * out[:, h]).sum(1)[:, None])
        dD = u * (np.abs(g[:, h]) * (np.abs(out[:, h]) + Pm @ np.abs(v[:, gk]))).sum(1)[:, None]
        w = 2 * u * np.abs(dS) + Pm * dD
        bq[:, h] += scale * (w @ np.abs(k[:, gk]))
        bk[:, gk] += scale * (w.T @ np.abs(q[:, h]))
        bv[:, gk] += u * (Pm.T @ np.abs(g[:, h]))
    return bq, bk, bv


def forward_bound(qh, kh, vh, N, layout, mask, P, docs, dt, key_valid=None):
    """Bound on |out - out_exact| for the fp32 output of the 16-bit forward:
    the kernel rounds each weight P_j (relative to its running reference) to
    16 bits before the P.V product and divides by the unrounded fp32 sum, so
    out moves by at most u sum_j p_j |v_j| with p the normalised weights."""
    T, Hq, d = qh.shape
    Hkv = kh.shape[1]
    scale = 1.0 / np.sqrt(d)
    q, k, v = (x.double().numpy() for x in (qh, kh, vh))
    ref = oracle.forward(qh, kh, vh, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs,
                         key_valid=key_valid)
    ok = allowed(T, N, layout, mask, P, docs, key_valid)
    u = U16[dt]
    b = np.zeros((T, Hq, d))
    grp = Hq // Hkv
    for h in range(Hq):
        gk = h // grp
        lse = ref["lse"][h]
        use = ok & np.isfinite(lse)[:, None]
        p = np.where(use, np.exp(np.where(use, scale * (q[:, h] @ k[:, gk].T) - lse[:, None], -np.inf)), 0.0)
        b[:, h] = u * (p @ np.abs(v[:, gk]))
    return b


def backward_bounds_rows(q, k, v, g, N, layout, mask, P, docs, dt, heads, toks, key_valid=None):
    """backward_bounds for a dout that is zero outside the listed (head, token)
    rows, each head h of q reading kv head h of k / v: dq bounds of those rows
    [n, d], and dk / dv bounds [T, H, d] summed over those rows only."""
    T, H, d = q.shape
    scale = 1.0 / np.sqrt(d)
    u = U16[dt]
    qn, kn, vn, gn = (x.double().numpy() for x in (q, k, v, g))
    ref = oracle.forward(q, k, v, n_blocks=N, layout=layout, mask=mask, max_ring_passes=P, cu_seqlens=docs,
                         rows=(heads, toks), key_valid=key_valid)
    t_all = np.arange(T)
    B = T // N
    blk = t_all % N if layout == 1 else t_all // B
    doc = np.searchsorted(np.asarray(docs[1:]), t_all, side="right") if mask == 2 else None
    kvm = None if key_valid is None else np.asarray(key_valid, dtype=bool)
    bq = np.zeros((len(toks), d))
    bk, bv = np.zeros((T, H, d)), np.zeros((T, H, d))
    for r, (h, t) in enumerate(zip(heads, toks)):
        ok = (blk[t] - blk) % N < min(P, N)
        if mask >= 1:
            ok &= t_all <= t
        if mask == 2:
            ok &= doc == doc[t]
        if kvm is not None:
            ok &= kvm
        if not np.isfinite(ref["lse"][r]):
            continue
        Pr = np.where(ok, np.exp(np.where(ok, scale * (kn[:, h] @ qn[t, h]) - ref["lse"][r], -np.inf)), 0.0)
        dS = Pr * (vn[:, h] @ gn[t, h] - gn[t, h] @ ref["out"][r])
        dD = u * (np.abs(gn[t, h]) * (np.abs(ref["out"][r]) + Pr @ np.abs(vn[:, h]))).sum()
        w = 2 * u * np.abs(dS) + Pr * dD
        bq[r] = scale * (w @ np.abs(kn[:, h]))
        bk[:, h] += scale * np.outer(w, np.abs(qn[t, h]))
        bv[:, h] += u * np.outer(Pr, np.abs(gn[t, h]))
    return bq, bk, bv


def forward_bound_rows(qh, kh, vh, N, layout, mask, P, docs, dt, heads, toks, lse, key_valid=None, chunk=512):
    """forward_bound for the listed (head, token) rows only, without a [T, T]
    matrix: each chunk of one head's rows is scored against the key range its
    mask can allow.  lse: the oracle's lse of those rows.  Returns the bound
    [n, d] and, per row, the number of keys it takes (n_keys) and the fp32
    error bound of its lse:
      the kernel's l is a recursive fp32 sum of n_keys positive terms,
      |d ln l| <= (n_keys + 8) 2^-24 (a few rescales and the final ln add
      8 more roundings); the scores are fp32 sums of d exact 16-bit products,
      |d s| <= scale d 2^-24 sum_i |q_i| max_j |k_j,i|, which moves lse by as
      much; and the result is an fp32 number, 2^-24 |lse|.
    The weights are evaluated in fp32 on torch's threaded CPU ops (their
    relative error, below 1e-5, is covered by widening the bound by 1e-3)."""
    T, Hq, d = qh.shape
    Hkv = kh.shape[1]
    grp = Hq // Hkv
    scale = 1.0 / np.sqrt(d)
    u = U16[dt]
    heads, toks = np.asarray(heads), np.asarray(toks)
    t_all = torch.arange(T)
    B = T // N
    blk = t_all % N if layout == 1 else t_all // B
    doc = torch.searchsorted(torch.as_tensor(np.asarray(docs[1:]), dtype=torch.int64), t_all, right=True) \
        if mask == 2 else None
    starts = np.asarray(docs[:-1]) if mask == 2 else None
    kvm = None if key_valid is None else torch.as_tensor(np.asarray(key_valid, dtype=bool))
    passes = min(P, N)
    lse_all = np.asarray(lse)
    bound = np.zeros((len(toks), d))
    n_keys = np.zeros(len(toks), dtype=np.int64)
    lse_tol = np.zeros(len(toks))
    for h in np.unique(heads):
        g = int(h) // grp
        q = qh[:, int(h)].float()
        k = kh[:, g].float()
        va = vh[:, g].float().abs()
        kmax = k.abs().max(dim=0).values.double().numpy()
        sel = np.nonzero(heads == h)[0]
        sel = sel[np.argsort(toks[sel], kind="stable")]
        for c0 in range(0, len(sel), chunk):
            idx = sel[c0:c0 + chunk]
            rt_np = toks[idx]
            rt = torch.as_tensor(rt_np)
            lo, hi = 0, T
            if mask >= 1:
                hi = int(rt_np.max()) + 1
            if mask == 2:
                lo = int(starts[int(doc[int(rt_np.min())])])
            keys = torch.arange(lo, hi)
            ok = torch.ones(len(idx), hi - lo, dtype=torch.bool)
            if passes < N:
                ok &= (blk[rt][:, None] - blk[keys][None, :]) % N < passes
            if mask >= 1:
                ok &= keys[None, :] <= rt[:, None]
            if mask == 2:
                ok &= doc[keys][None, :] == doc[rt][:, None]
            if kvm is not None:
                ok &= kvm[keys][None, :]
            lr = torch.as_tensor(lse_all[idx])
            fin = torch.isfinite(lr)
            ok &= fin[:, None]
            s = (q[rt] @ k[keys].T) * scale - torch.where(fin, lr, torch.zeros_like(lr)).float()[:, None]
            p = torch.where(ok, torch.exp(s), torch.zeros_like(s))
            bound[idx] = (u * (1 + 1e-3)) * (p @ va[keys]).double().numpy()
            n_keys[idx] = ok.sum(dim=1).numpy()
            qa = q[rt].double().abs().numpy()
            lr_np = lse_all[idx]
            lse_tol[idx] = (2.0 ** -24) * (n_keys[idx] + 8) + scale * d * 2.0 ** -24 * (qa @ kmax) \
                + 2.0 ** -24 * np.where(np.isfinite(lr_np), np.abs(lr_np), 0.0)
    return bound, n_keys, lse_tol
