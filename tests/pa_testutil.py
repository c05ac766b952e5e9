"""Helpers shared by the tests: independent references used to pin the oracle,
and comparison helpers for the parity tests.

The brute-force reference here never pages anything: it runs torch's
scaled_dot_product_attention (with its own GQA handling) in float64 on dense,
per-request K / V, with an explicit causal mask aligned to the sequence end.
The paged inputs for the oracle are produced from the same dense tensors by
`scatter_pages`, which writes the documented cache layouts directly.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F


def round_to(x: torch.Tensor, dtype) -> torch.Tensor:
    return x.to(dtype)


def dense_request(gen, nq, ctx, Hq, Hkv, Dqk, Dv, dtype):
    """Dense q [nq, Hq, Dqk], K [L, Hkv, Dqk], V [L, Hkv, Dv] for one request."""
    L = nq + ctx
    q = torch.randn(nq, Hq, Dqk, generator=gen).to(dtype)
    K = torch.randn(L, Hkv, Dqk, generator=gen).to(dtype)
    V = torch.randn(L, Hkv, Dv, generator=gen).to(dtype)
    return q, K, V


def scatter_pages(Ks, Vs, P, gen, spare=1, layout="mha", max_pages=None):
    """Write per-request dense K / V into a page pool in a random physical order.

    MHA: k_cache[page, h, slot, d], v_cache[page, h, d, slot].
    MLA: latent[page, slot, d] (Ks only; V is its column prefix).
    Unused pool pages and unused tail slots hold NaN.  Returns
    (k_cache, v_cache, block_table int32 [B, max_pages]).
    """
    npg = [(K.shape[0] + P - 1) // P for K in Ks]
    used = sum(npg)
    pool = used + spare
    perm = torch.randperm(pool, generator=gen)
    maxp = max(npg + [1]) if max_pages is None else max_pages
    filler = int(perm[used]) if spare else 0
    bt = torch.full((len(Ks), maxp), filler, dtype=torch.int32)
    dt = Ks[0].dtype
    if layout == "mla":
        D = Ks[0].shape[-1]
        kc = torch.full((pool, P, D), float("nan"), dtype=dt)
        vc = kc
    else:
        Hkv, Dqk = Ks[0].shape[1], Ks[0].shape[2]
        Dv = Vs[0].shape[2]
        kc = torch.full((pool, Hkv, P, Dqk), float("nan"), dtype=dt)
        vc = torch.full((pool, Hkv, Dv, P), float("nan"), dtype=dt)
    off = 0
    for b, K in enumerate(Ks):
        for t in range(K.shape[0]):
            lp, slot = divmod(t, P)
            if slot == 0:
                bt[b, lp] = perm[off]
                off += 1
            page = int(bt[b, lp])
            if layout == "mla":
                kc[page, slot, :] = K[t, 0, :]
            else:
                kc[page, :, slot, :] = K[t]
                vc[page, :, :, slot] = Vs[b][t]
    return kc, vc, bt


def causal_mask(nq, L):
    """Bool [nq, L]: query j (at position L - nq + j) sees keys 0 .. L - nq + j."""
    c = L - nq
    j = torch.arange(nq).unsqueeze(1)
    t = torch.arange(L).unsqueeze(0)
    return t <= c + j


def prefix_mask(nq, L, prefix):
    """Bool [nq, L]: causal, plus keys 0 .. prefix - 1 visible to every query."""
    return causal_mask(nq, L) | (torch.arange(L).unsqueeze(0) < prefix)


def sdpa_reference(q, K, V, scale, mask=None):
    """float64 torch SDPA (GQA via enable_gqa) with the end-aligned causal mask, or
    with `mask` (bool [nq, L], True = visible) when given.

    q [nq, Hq, Dqk], K [L, Hkv, Dqk], V [L, Hkv, Dv] -> out [nq, Hq, Dv], lse [nq, Hq].
    """
    nq, L = q.shape[0], K.shape[0]
    qd = q.double().permute(1, 0, 2).unsqueeze(0)
    kd = K.double().permute(1, 0, 2).unsqueeze(0)
    vd = V.double().permute(1, 0, 2).unsqueeze(0)
    mask = causal_mask(nq, L) if mask is None else mask
    out = F.scaled_dot_product_attention(qd, kd, vd, attn_mask=mask, scale=scale, enable_gqa=True)
    g = q.shape[1] // K.shape[1]
    kx = kd.repeat_interleave(g, dim=1)
    s = torch.matmul(qd, kx.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return out[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


def errors(got, ref):
    """(max abs error, relative RMS error) over all elements."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    d = g - r
    mx = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.sqrt(np.sum(r * r)))
    rel = float(np.sqrt(np.sum(d * d)) / den) if den > 0 else float(np.sqrt(np.sum(d * d)))
    return mx, rel


def finite_lse_err(got, ref):
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(r)), "-inf pattern differs"
    m = np.isfinite(r)
    return float(np.max(np.abs(g[m] - r[m]))) if m.any() else 0.0
