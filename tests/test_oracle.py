"""Pins for the fp64 CPU oracle (no GPU).

Each test ties the oracle to something other than itself: torch's float64
scaled_dot_product_attention on dense, never-paged inputs; closed forms;
invariances the mathematics fixes; hand-derived worked examples.  The set is
chosen so that a dropped term, a wrong sign, a wrong index (causal offset,
GQA head mapping, page / slot / layout index, split range) or a transposed
operand fails at least one test; `test_oracle_mutants.py` checks that claim by
planting such mistakes in a copy of the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from pa_testutil import dense_request, prefix_mask, scatter_pages, sdpa_reference

TOL = 1e-12
HERE = os.path.dirname(os.path.abspath(__file__))


def _build_case(seed, specs, Hq, Hkv, Dqk, Dv, P, dtype=torch.float32, layout="mha", spare=1):
    """specs: list of (nq, ctx).  Returns dense tensors plus the paged inputs."""
    gen = torch.Generator().manual_seed(seed)
    qs, Ks, Vs = [], [], []
    for nq, ctx in specs:
        if layout == "mla":
            q, K, _ = dense_request(gen, nq, ctx, Hq, 1, Dqk, Dv, dtype)
            V = K[:, :, :Dv]
        else:
            q, K, V = dense_request(gen, nq, ctx, Hq, Hkv, Dqk, Dv, dtype)
        qs.append(q)
        Ks.append(K)
        Vs.append(V)
    kc, vc, bt = scatter_pages(Ks, Vs, P, gen, spare=spare, layout=layout)
    qsl = np.zeros(len(specs) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum([s[0] for s in specs])
    seq = np.array([s[0] + s[1] for s in specs], dtype=np.int32)
    qcat = torch.cat(qs, 0) if sum(s[0] for s in specs) else torch.zeros(0, Hq, Dqk, dtype=dtype)
    return dict(q=qcat, qs=qs, Ks=Ks, Vs=Vs, kc=kc, vc=vc, bt=bt, qsl=qsl, seq=seq)


def _run(c, scale, Hkv, Dv, layout="mha", rows=None):
    lay = oracle.LAYOUT_MLA if layout == "mla" else oracle.LAYOUT_MHA
    return oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], scale,
                            Hkv, head_dim_v=Dv, layout=lay, rows=rows)


CASES = [
    # seed, specs (nq, ctx), Hq, Hkv, Dqk, Dv, P
    (1, [(1, 0), (1, 9), (5, 0), (3, 7)], 4, 2, 8, 8, 4),
    (2, [(2, 30), (1, 39), (7, 3)], 6, 2, 8, 5, 16),
    (3, [(4, 0), (1, 1)], 3, 1, 4, 4, 1),
    (4, [(0, 5), (6, 10), (1, 0)], 2, 2, 16, 16, 4),
    (5, [(16, 17), (1, 31)], 8, 4, 8, 8, 16),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", CASES)
def test_bruteforce_against_torch_sdpa(case, dtype):
    """Paged fp64 oracle == float64 torch SDPA on the dense, unpaged inputs."""
    seed, specs, Hq, Hkv, Dqk, Dv, P = case
    c = _build_case(seed, specs, Hq, Hkv, Dqk, Dv, P, dtype)
    scale = 1.0 / math.sqrt(Dqk) * 1.3
    out, lse = _run(c, scale, Hkv, Dv)
    i0 = 0
    for (nq, ctx), q, K, V in zip(specs, c["qs"], c["Ks"], c["Vs"]):
        if nq == 0:
            continue
        ro, rl = sdpa_reference(q, K, V, float(np.float32(scale)))
        np.testing.assert_allclose(out[i0:i0 + nq], ro, atol=TOL, rtol=0)
        np.testing.assert_allclose(lse[i0:i0 + nq], rl, atol=TOL, rtol=0)
        i0 += nq
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_page_permutation_is_bitwise_invariant():
    specs = [(3, 20), (1, 44), (6, 0)]
    a = _build_case(11, specs, 4, 2, 8, 8, 4)
    out_a, lse_a = _run(a, 0.4, 2, 8)
    # same dense tensors, different physical page order and pool size
    gen = torch.Generator().manual_seed(999)
    kc, vc, bt = scatter_pages(a["Ks"], a["Vs"], 4, gen, spare=5)
    b = dict(a, kc=kc, vc=vc, bt=bt)
    out_b, lse_b = _run(b, 0.4, 2, 8)
    assert not np.array_equal(a["bt"].numpy(), bt.numpy()[:, :a["bt"].shape[1]])
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


@pytest.mark.parametrize("S", [1, 2, 3, 7, 64])
def test_split_then_merge_equals_unsplit(S):
    specs = [(1, 0), (1, 12), (1, 37), (1, 63)]
    c = _build_case(21, specs, 4, 2, 8, 8, 4)
    out, lse = _run(c, 0.35, 2, 8)
    q = c["q"].reshape(len(specs), 4, 8)
    po, pl = oracle.decode_split(q, c["kc"], c["vc"], c["bt"], c["seq"], 0.35, S, 2, head_dim_v=8)
    mo, ml = oracle.merge_lse(po, pl)
    np.testing.assert_allclose(mo, out, atol=TOL, rtol=0)
    np.testing.assert_allclose(ml, lse, atol=TOL, rtol=0)
    for b, L in enumerate(c["seq"]):
        pages = (int(L) + 3) // 4
        for s in range(S):
            if s >= pages:  # more partitions than pages: the extra ones are empty
                assert np.all(np.isneginf(pl[b, :, s])) and np.all(po[b, :, s] == 0)


def test_split_partials_match_sdpa_on_their_ranges():
    """Each partial is plain attention over its own key range (checked with SDPA on
    the dense keys), and the ranges tile [0, L) contiguously on page boundaries."""
    specs = [(1, 40), (1, 9)]
    c = _build_case(23, specs, 4, 1, 8, 8, 4)
    S = 3
    q = c["q"].reshape(2, 4, 8)
    po, pl = oracle.decode_split(q, c["kc"], c["vc"], c["bt"], c["seq"], 0.5, S, 1, head_dim_v=8)
    for b, L in enumerate(c["seq"]):
        L = int(L)
        prev = 0
        for s in range(S):
            t0, t1 = oracle.split_range(L, 4, S, s)
            assert t0 == prev and t0 % 4 == 0 and t0 <= t1 <= L
            prev = t1
            if t1 > t0:
                K = c["Ks"][b][t0:t1]
                V = c["Vs"][b][t0:t1]
                ro, rl = sdpa_reference(c["qs"][b], K, V, 0.5)
                np.testing.assert_allclose(po[b, :, s], ro[0], atol=TOL, rtol=0)
                np.testing.assert_allclose(pl[b, :, s], rl[0], atol=TOL, rtol=0)
        assert prev == L
        sizes = [oracle.split_range(L, 4, S, s) for s in range(S)]
        nonempty = [t1 - t0 for t0, t1 in sizes if t1 > t0]
        assert all(n == nonempty[0] for n in nonempty[:-1])


# decode, decode, extend, prefill, extend: rows with few and many visible keys
CHUNK_SPECS = [(1, 0), (1, 12), (4, 9), (6, 0), (3, 30)]


@pytest.mark.parametrize("C", [1, 3, 4, 16, 64])
def test_chunked_then_merge_equals_unchunked(C):
    """Chunked-context partials merged by LSE give plain attention; a chunk past
    every request's keys is empty (zeros, -inf) for every row."""
    c = _build_case(31, CHUNK_SPECS, 4, 2, 8, 8, 4)
    out, lse = _run(c, 0.35, 2, 8)
    S = max((int(L) + C - 1) // C for L in c["seq"]) + 1
    po, pl = oracle.chunked_partials(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.35,
                                     C, S, 2, head_dim_v=8)
    mo, ml = oracle.merge_lse(po, pl)
    np.testing.assert_allclose(mo, out, atol=TOL, rtol=0)
    np.testing.assert_allclose(ml, lse, atol=TOL, rtol=0)
    assert np.all(np.isneginf(pl[:, :, S - 1])) and np.all(po[:, :, S - 1] == 0)


@pytest.mark.parametrize("mask,prefix", [(oracle.MASK_FULL, None), (oracle.MASK_PREFIX, [0, 4, 11, 30, 15, 2])])
def test_masked_chunks_merge_to_masked_attention(mask, prefix):
    """Chunk partials under the full and prefix masks merge to the masked attention."""
    specs = [(1, 0), (1, 12), (4, 9), (6, 0), (3, 30), (7, 5)]
    c = _build_case(35, specs, 4, 2, 8, 8, 4)
    pfx = None if prefix is None else np.asarray(prefix, np.int32)
    out, lse = oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.35, 2,
                                head_dim_v=8, mask=mask, prefix_lens=pfx)
    po, pl = oracle.chunked_partials(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.35,
                                     5, 8, 2, head_dim_v=8, mask=mask, prefix_lens=pfx)
    mo, ml = oracle.merge_lse(po, pl)
    np.testing.assert_allclose(mo, out, atol=TOL, rtol=0)
    np.testing.assert_allclose(ml, lse, atol=TOL, rtol=0)


def test_chunked_partials_match_sdpa_on_visible_keys():
    """Each chunk partial of a row is attention over the chunk's keys that the row's
    token sees (SDPA on the dense keys); chunks it cannot see are empty."""
    specs = [(5, 7), (1, 20), (9, 0)]
    c = _build_case(33, specs, 4, 2, 8, 8, 4)
    C, S = 6, 6
    po, pl = oracle.chunked_partials(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.5,
                                     C, S, 2, head_dim_v=8)
    i = 0
    empty = 0
    for b, (nq, ctx) in enumerate(specs):
        for j in range(nq):
            pos = ctx + j
            for s in range(S):
                t0, t1 = s * C, min(s * C + C, pos + 1)
                if t1 <= t0:
                    assert np.all(np.isneginf(pl[i, :, s])) and np.all(po[i, :, s] == 0)
                    empty += 1
                    continue
                ro, rl = sdpa_reference(c["qs"][b][j:j + 1], c["Ks"][b][t0:t1], c["Vs"][b][t0:t1], 0.5)
                np.testing.assert_allclose(po[i, :, s], ro[0], atol=TOL, rtol=0)
                np.testing.assert_allclose(pl[i, :, s], rl[0], atol=TOL, rtol=0)
            i += 1
    assert empty > 0 and i == c["q"].shape[0]


MASK_SPECS = [(1, 0), (1, 12), (4, 9), (6, 0), (3, 30), (7, 5)]


def _masked(c, mask, prefix=None, scale=0.45):
    lay = oracle.LAYOUT_MHA
    return oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], scale, 2,
                            head_dim_v=8, layout=lay, mask=mask,
                            prefix_lens=None if prefix is None else np.asarray(prefix, np.int32))


def test_full_mask_equals_unmasked_sdpa():
    """MASK_FULL: every new token sees all keys of its request (SDPA with no mask)."""
    c = _build_case(41, MASK_SPECS, 4, 2, 8, 8, 4)
    out, lse = _masked(c, oracle.MASK_FULL)
    i0 = 0
    for (nq, ctx), q, K, V in zip(MASK_SPECS, c["qs"], c["Ks"], c["Vs"]):
        full = torch.ones(nq, nq + ctx, dtype=torch.bool)
        ro, rl = sdpa_reference(q, K, V, float(np.float32(0.45)), mask=full)
        np.testing.assert_allclose(out[i0:i0 + nq], ro, atol=TOL, rtol=0)
        np.testing.assert_allclose(lse[i0:i0 + nq], rl, atol=TOL, rtol=0)
        i0 += nq


@pytest.mark.parametrize("prefixes", [[0, 5, 9, 3, 20, 2], [1, 13, 13, 6, 33, 12], [2, 40, 1, 4, 7, 11]])
def test_prefix_mask_matches_sdpa(prefixes):
    """MASK_PREFIX: causal plus a bidirectional prefix of prefix_lens[b] keys (lengths
    below, inside and past the new tokens, and past the end of the request)."""
    c = _build_case(43, MASK_SPECS, 4, 2, 8, 8, 4)
    out, lse = _masked(c, oracle.MASK_PREFIX, prefixes)
    i0 = 0
    for (nq, ctx), q, K, V, pf in zip(MASK_SPECS, c["qs"], c["Ks"], c["Vs"], prefixes):
        m = prefix_mask(nq, nq + ctx, pf)
        ro, rl = sdpa_reference(q, K, V, float(np.float32(0.45)), mask=m)
        np.testing.assert_allclose(out[i0:i0 + nq], ro, atol=TOL, rtol=0)
        np.testing.assert_allclose(lse[i0:i0 + nq], rl, atol=TOL, rtol=0)
        i0 += nq


def test_mask_special_cases_reduce_to_causal_or_full():
    """An empty prefix is causal and a prefix covering every key is full, bit for
    bit; decode rows (one new token) see every key under all three masks."""
    c = _build_case(45, MASK_SPECS, 4, 2, 8, 8, 4)
    causal = _masked(c, oracle.MASK_CAUSAL)
    full = _masked(c, oracle.MASK_FULL)
    zero = _masked(c, oracle.MASK_PREFIX, [0] * len(MASK_SPECS))
    big = _masked(c, oracle.MASK_PREFIX, [10 ** 6] * len(MASK_SPECS))
    for a, b in ((causal, zero), (full, big)):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    qsl = c["qsl"]
    for i, (nq, ctx) in enumerate(MASK_SPECS):
        if nq == 1:
            r = qsl[i]
            assert np.array_equal(causal[0][r], full[0][r])
    assert not np.allclose(causal[0], full[0])


def _sdpa_with_sink(q, K, V, scale, sinks):
    """float64 attention with the causal mask and, per query head h, one extra key of
    zero key and value whose logit is sinks[h] (an additive bias on SDPA)."""
    nq, L, Hkv = q.shape[0], K.shape[0], K.shape[1]
    Kx = torch.cat([K.double(), torch.zeros(1, Hkv, K.shape[2], dtype=torch.float64)], 0)
    Vx = torch.cat([V.double(), torch.zeros(1, Hkv, V.shape[2], dtype=torch.float64)], 0)
    Hq = q.shape[1]
    bias = torch.full((Hq, nq, L + 1), float("-inf"), dtype=torch.float64)
    vis = torch.cat([torch.ones(nq, L, dtype=torch.bool), torch.zeros(nq, 1, dtype=torch.bool)], 1)
    vis[:, :L] = torch.arange(L).unsqueeze(0) <= (L - nq + torch.arange(nq)).unsqueeze(1)
    bias[:, vis] = 0.0
    bias[:, :, L] = torch.as_tensor(np.asarray(sinks, np.float64)).unsqueeze(1)
    qd = q.double().permute(1, 0, 2).unsqueeze(0)
    kd = Kx.permute(1, 0, 2).unsqueeze(0)
    vd = Vx.permute(1, 0, 2).unsqueeze(0)
    out = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=bias.unsqueeze(0),
                                                           scale=scale, enable_gqa=True)
    g = Hq // Hkv
    s = torch.matmul(qd, kd.repeat_interleave(g, dim=1).transpose(-1, -2)) * scale + bias.unsqueeze(0)
    lse = torch.logsumexp(s, dim=-1)
    return out[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


def test_sinks_match_sdpa_with_an_extra_zero_key():
    """A sink logit per query head acts as one more key with zero value (checked with
    SDPA and an additive bias), for sinks far below, near and far above the scores."""
    c = _build_case(47, MASK_SPECS, 4, 2, 8, 8, 4)
    sinks = np.array([-30.0, -0.7, 1.3, 25.0], dtype=np.float32)
    out, lse = oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.45, 2,
                                head_dim_v=8, sinks=sinks)
    i0 = 0
    for (nq, ctx), q, K, V in zip(MASK_SPECS, c["qs"], c["Ks"], c["Vs"]):
        ro, rl = _sdpa_with_sink(q, K, V, float(np.float32(0.45)), sinks)
        np.testing.assert_allclose(out[i0:i0 + nq], ro, atol=TOL, rtol=0)
        np.testing.assert_allclose(lse[i0:i0 + nq], rl, atol=TOL, rtol=0)
        i0 += nq


def test_minus_infinite_sinks_change_nothing():
    c = _build_case(49, MASK_SPECS, 4, 2, 8, 8, 4)
    a = oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.45, 2, head_dim_v=8)
    b = oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.45, 2, head_dim_v=8,
                         sinks=np.full(4, -np.inf, np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_constant_value_rows_sum_to_one():
    """V = const => out = const for every row (softmax rows sum to 1)."""
    specs = [(1, 30), (4, 5), (9, 0)]
    c = _build_case(31, specs, 4, 2, 8, 8, 4)
    vc = torch.where(torch.isnan(c["vc"]), c["vc"], torch.full_like(c["vc"], 2.5))
    out, _ = _run(dict(c, vc=vc), 0.7, 2, 8)
    np.testing.assert_allclose(out, 2.5, atol=1e-14, rtol=0)


def test_length_one_context_returns_v0():
    specs = [(1, 0)]
    c = _build_case(41, specs, 4, 2, 8, 8, 16)
    out, lse = _run(c, 0.25, 2, 8)
    q, K, V = c["qs"][0].double(), c["Ks"][0].double(), c["Vs"][0].double()
    for h in range(4):
        kvh = h // 2
        assert np.array_equal(out[0, h], V[0, kvh].numpy())
        s0 = 0.25 * float(np.dot(q[0, h].numpy(), K[0, kvh].numpy()))
        assert abs(lse[0, h] - s0) <= 1e-15 * max(1.0, abs(s0))
    # the first token of a prefill also sees only key 0
    c = _build_case(42, [(5, 0)], 4, 2, 8, 8, 4)
    out, _ = _run(c, 0.25, 2, 8)
    for h in range(4):
        assert np.array_equal(out[0, h], c["Vs"][0][0, h // 2].double().numpy())


def test_equal_keys_give_mean_of_visible_values():
    specs = [(3, 6)]
    c = _build_case(51, specs, 2, 1, 8, 8, 4)
    K = c["Ks"][0]
    Keq = K[:1].expand_as(K).clone()
    gen = torch.Generator().manual_seed(52)
    kc, vc, bt = scatter_pages([Keq], c["Vs"], 4, gen)
    out, lse = _run(dict(c, kc=kc, vc=vc, bt=bt), 0.3, 1, 8)
    V = c["Vs"][0].double().numpy()
    q = c["qs"][0].double().numpy()
    for j in range(3):
        pos = 6 + j
        for h in range(2):
            np.testing.assert_allclose(out[j, h], V[:pos + 1, 0].mean(0), atol=1e-14, rtol=0)
            s = float(np.float32(0.3)) * float(np.dot(q[j, h], Keq[0, 0].double().numpy()))
            assert abs(lse[j, h] - (s + math.log(pos + 1))) <= 1e-13


def test_zero_query_gives_mean_and_log_count():
    specs = [(4, 3), (1, 10)]
    c = _build_case(61, specs, 4, 2, 8, 8, 4)
    q0 = torch.zeros_like(c["q"])
    out, lse = _run(dict(c, q=q0), 0.9, 2, 8)
    i0 = 0
    for (nq, ctx), V in zip(specs, c["Vs"]):
        Vd = V.double().numpy()
        for j in range(nq):
            n = ctx + j + 1
            for h in range(4):
                np.testing.assert_allclose(out[i0 + j, h], Vd[:n, h // 2].mean(0), atol=1e-14)
                assert abs(lse[i0 + j, h] - math.log(n)) <= 1e-14
        i0 += nq


def test_decode_equals_last_prefill_row_and_extend_matches_prefill():
    gen = torch.Generator().manual_seed(71)
    Hq, Hkv, D, P = 4, 2, 8, 4
    q, K, V = dense_request(gen, 10, 0, Hq, Hkv, D, D, torch.float32)
    kc, vc, bt = scatter_pages([K], [V], P, gen)

    def run(qpart, nq, L):
        return oracle.attention(qpart, kc, vc, bt, np.array([L], np.int32),
                                np.array([0, nq], np.int32), 0.4, Hkv)

    full_o, full_l = run(q, 10, 10)
    dec_o, dec_l = run(q[9:], 1, 10)               # decode: last token over 10 keys
    assert np.array_equal(dec_o[0], full_o[9]) and np.array_equal(dec_l[0], full_l[9])
    ext_o, ext_l = run(q[6:], 4, 10)               # extend: 4 new tokens on 6 cached
    assert np.array_equal(ext_o, full_o[6:]) and np.array_equal(ext_l, full_l[6:])
    pre_o, _ = run(q[:7], 7, 7)                    # a shorter prefill = leading rows
    assert np.array_equal(pre_o, full_o[:7])


def test_gqa_equals_replicated_mha():
    specs = [(3, 9), (1, 20)]
    c = _build_case(81, specs, 8, 2, 8, 8, 4)
    out_g, lse_g = _run(c, 0.3, 2, 8)
    Ks = [K.repeat_interleave(4, dim=1) for K in c["Ks"]]
    Vs = [V.repeat_interleave(4, dim=1) for V in c["Vs"]]
    gen = torch.Generator().manual_seed(82)
    kc, vc, bt = scatter_pages(Ks, Vs, 4, gen)
    out_m, lse_m = _run(dict(c, kc=kc, vc=vc, bt=bt), 0.3, 8, 8)
    assert np.array_equal(out_g, out_m) and np.array_equal(lse_g, lse_m)


def test_request_order_permutation():
    specs = [(1, 14), (5, 3), (2, 0), (1, 30)]
    c = _build_case(91, specs, 4, 2, 8, 8, 4)
    out, lse = _run(c, 0.3, 2, 8)
    order = [2, 0, 3, 1]
    specs2 = [specs[i] for i in order]
    gen = torch.Generator().manual_seed(92)
    kc, vc, bt = scatter_pages([c["Ks"][i] for i in order], [c["Vs"][i] for i in order], 4, gen)
    q2 = torch.cat([c["qs"][i] for i in order], 0)
    qsl = np.zeros(5, np.int32)
    qsl[1:] = np.cumsum([s[0] for s in specs2])
    seq = np.array([a + b for a, b in specs2], np.int32)
    out2, lse2 = oracle.attention(q2, kc, vc, bt, seq, qsl, 0.3, 2)
    starts = np.concatenate([[0], np.cumsum([s[0] for s in specs])])
    i0 = 0
    for i in order:
        n = specs[i][0]
        assert np.array_equal(out2[i0:i0 + n], out[starts[i]:starts[i] + n])
        assert np.array_equal(lse2[i0:i0 + n], lse[starts[i]:starts[i] + n])
        i0 += n


def test_mla_latent_layout_matches_sdpa_and_mha_layout():
    """MLA: keys are the full latent rows, values their first Dv columns."""
    specs = [(1, 20), (1, 0), (1, 64)]
    Hq, Dqk, Dv, P = 8, 12, 8, 8
    c = _build_case(101, specs, Hq, 1, Dqk, Dv, P, torch.bfloat16, layout="mla")
    out, lse = _run(c, 0.2, 1, Dv, layout="mla")
    for b, (q, K) in enumerate(zip(c["qs"], c["Ks"])):
        ro, rl = sdpa_reference(q, K, K[:, :, :Dv], float(np.float32(0.2)))
        np.testing.assert_allclose(out[b:b + 1], ro, atol=TOL, rtol=0)
        np.testing.assert_allclose(lse[b:b + 1], rl, atol=TOL, rtol=0)
    gen = torch.Generator().manual_seed(102)
    kc, vc, bt = scatter_pages(c["Ks"], [K[:, :, :Dv] for K in c["Ks"]], P, gen)
    out_m, lse_m = _run(dict(c, kc=kc, vc=vc, bt=bt), 0.2, 1, Dv)
    np.testing.assert_allclose(out_m, out, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse_m, lse, atol=1e-14, rtol=0)


def test_merge_closed_forms():
    o = np.array([[[1.0, 2.0], [5.0, -3.0]]])          # [rows=1, S=2, Dv=2]
    l = np.array([[0.0, math.log(3.0)]])                # weights 1 : 3
    out, lse = oracle.merge_lse(o, l)
    np.testing.assert_allclose(out[0], [(1 + 15) / 4, (2 - 9) / 4], atol=1e-15)
    assert abs(lse[0] - math.log(4.0)) < 1e-15
    # one empty partition: the other passes through
    out, lse = oracle.merge_lse(o, np.array([[-np.inf, 0.5]]))
    np.testing.assert_array_equal(out[0], [5.0, -3.0])
    assert lse[0] == 0.5
    # all empty: zeros and -inf, never NaN
    out, lse = oracle.merge_lse(o, np.array([[-np.inf, -np.inf]]))
    assert np.all(out == 0) and np.isneginf(lse[0])
    # large equal lse values do not overflow
    out, lse = oracle.merge_lse(o, np.array([[800.0, 800.0]]))
    np.testing.assert_allclose(out[0], [3.0, -0.5], atol=1e-15)
    assert abs(lse[0] - (800.0 + math.log(2.0))) < 1e-12


def test_invalid_inputs_are_rejected():
    c = _build_case(111, [(2, 3)], 4, 2, 8, 8, 4)
    bad = c["seq"].copy()
    bad[0] = 1  # seq_len < q_len
    with pytest.raises(ValueError):
        oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], bad, c["qsl"], 0.3, 2)
    bt = c["bt"].clone()
    bt[0, 0] = 10 ** 6
    with pytest.raises(ValueError):
        oracle.attention(c["q"], c["kc"], c["vc"], bt, c["seq"], c["qsl"], 0.3, 2)
    with pytest.raises(ValueError):
        oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.3, 3)


def _alibi_bias(nq, L, slopes, mode, vis):
    """[Hq, nq, L] additive bias for torch SDPA: the ALiBi term on visible keys
    (positions: new token j at L - nq + j), -inf elsewhere."""
    pos = (L - nq + torch.arange(nq, dtype=torch.float64)).unsqueeze(1)
    dist = (pos - torch.arange(L, dtype=torch.float64).unsqueeze(0)).abs()
    f = dist.sqrt() if mode == oracle.ALIBI_SQRT else dist
    m = torch.as_tensor(np.asarray(slopes, np.float64)).view(-1, 1, 1)
    bias = -m * f.unsqueeze(0)
    return bias.masked_fill(~vis.unsqueeze(0), float("-inf"))


def _sdpa_bias(q, K, V, scale, bias):
    Hq, Hkv = q.shape[1], K.shape[1]
    qd = q.double().permute(1, 0, 2).unsqueeze(0)
    kd = K.double().permute(1, 0, 2).unsqueeze(0)
    vd = V.double().permute(1, 0, 2).unsqueeze(0)
    out = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=bias.unsqueeze(0),
                                                           scale=scale, enable_gqa=True)
    s = torch.matmul(qd, kd.repeat_interleave(Hq // Hkv, dim=1).transpose(-1, -2)) * scale
    lse = torch.logsumexp(s + bias.unsqueeze(0), dim=-1)
    return out[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


ALIBI_SLOPES = np.array([0.5, 0.0625, 1.5, 0.25], dtype=np.float32)


@pytest.mark.parametrize("mode", [oracle.ALIBI_LINEAR, oracle.ALIBI_SQRT])
@pytest.mark.parametrize("mask,prefix", [(oracle.MASK_CAUSAL, None), (oracle.MASK_FULL, None),
                                         (oracle.MASK_PREFIX, [2, 13, 13, 6, 33, 12])])
def test_alibi_matches_sdpa_with_an_additive_bias(mode, mask, prefix):
    """ALiBi (linear and sqrt) under every mask: torch SDPA with the bias as an
    additive attention mask on dense, unpaged inputs."""
    c = _build_case(53, MASK_SPECS, 4, 2, 8, 8, 4)
    out, lse = oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.45, 2,
                                head_dim_v=8, mask=mask,
                                prefix_lens=None if prefix is None else np.asarray(prefix, np.int32),
                                alibi_slopes=ALIBI_SLOPES, alibi_mode=mode)
    i0 = 0
    for i, ((nq, ctx), q, K, V) in enumerate(zip(MASK_SPECS, c["qs"], c["Ks"], c["Vs"])):
        L = nq + ctx
        if mask == oracle.MASK_FULL:
            vis = torch.ones(nq, L, dtype=torch.bool)
        elif mask == oracle.MASK_PREFIX:
            vis = prefix_mask(nq, L, prefix[i])
        else:
            vis = torch.arange(L).unsqueeze(0) <= (L - nq + torch.arange(nq)).unsqueeze(1)
        ro, rl = _sdpa_bias(q, K, V, float(np.float32(0.45)), _alibi_bias(nq, L, ALIBI_SLOPES, mode, vis))
        np.testing.assert_allclose(out[i0:i0 + nq], ro, atol=TOL, rtol=0)
        np.testing.assert_allclose(lse[i0:i0 + nq], rl, atol=TOL, rtol=0)
        i0 += nq


def test_alibi_zero_slopes_change_nothing():
    c = _build_case(55, MASK_SPECS, 4, 2, 8, 8, 4)
    a = oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.45, 2, head_dim_v=8)
    for mode in (oracle.ALIBI_LINEAR, oracle.ALIBI_SQRT):
        b = oracle.attention(c["q"], c["kc"], c["vc"], c["bt"], c["seq"], c["qsl"], 0.45, 2,
                             head_dim_v=8, alibi_slopes=np.zeros(4, np.float32), alibi_mode=mode)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_alibi_decode_equals_last_prefill_row():
    """Positions under ALiBi: a decode over L keys is the last row of a prefill of L
    tokens, and an extend's rows are the matching prefill rows."""
    gen = torch.Generator().manual_seed(57)
    Hq, Hkv, D, P = 4, 2, 8, 4
    q, K, V = dense_request(gen, 10, 0, Hq, Hkv, D, D, torch.float32)
    kc, vc, bt = scatter_pages([K], [V], P, gen)
    for mode in (oracle.ALIBI_LINEAR, oracle.ALIBI_SQRT):
        def run(qpart, nq, L):
            return oracle.attention(qpart, kc, vc, bt, np.array([L], np.int32),
                                    np.array([0, nq], np.int32), 0.4, Hkv,
                                    alibi_slopes=ALIBI_SLOPES, alibi_mode=mode)
        full_o, full_l = run(q, 10, 10)
        dec_o, dec_l = run(q[9:], 1, 10)
        assert np.array_equal(dec_o[0], full_o[9]) and np.array_equal(dec_l[0], full_l[9])
        ext_o, ext_l = run(q[6:], 4, 10)
        assert np.array_equal(ext_o, full_o[6:]) and np.array_equal(ext_l, full_l[6:])


def _load_golden():
    with open(os.path.join(HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _load_golden(), ids=lambda e: e["name"])
def test_hand_worked_examples(ex):
    """Tiny cases whose results were derived by hand (see the fixture's notes)."""
    P, Hq, Hkv = ex["page_size"], ex["num_q_heads"], ex["num_kv_heads"]
    q = np.array(ex["q"], dtype=np.float32)
    kc = np.array(ex["k_cache"], dtype=np.float32)
    vc = np.array(ex["v_cache"], dtype=np.float32)
    bt = np.array(ex["block_table"], dtype=np.int32)
    seq = np.array(ex["seq_lens"], dtype=np.int32)
    qsl = np.array(ex["query_start_loc"], dtype=np.int32)
    mode = {"linear": oracle.ALIBI_LINEAR, "sqrt": oracle.ALIBI_SQRT}.get(ex.get("alibi_mode"),
                                                                        oracle.ALIBI_NONE)
    slopes = np.array(ex["alibi_slopes"], np.float32) if mode != oracle.ALIBI_NONE else None
    out, lse = oracle.attention(q, kc, vc, bt, seq, qsl, ex["scale"], Hkv,
                                head_dim_v=vc.shape[2], alibi_slopes=slopes, alibi_mode=mode)
    np.testing.assert_allclose(out, np.array(ex["expected_out"]), atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, np.array(ex["expected_lse"]), atol=1e-12, rtol=0)
