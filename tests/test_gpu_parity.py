"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs.

Tolerances of the parity contract: bf16 max |err| <= 2e-2 and relative RMS
<= 5e-3 over the output tensor; fp32 max |err| <= 1e-5; LSE within 1e-3
(natural log).  Index handling must be exact: unused pages and the slots past
each sequence end hold NaN, so any stray read shows up as a non-finite output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_attention_kv_pa_amd as pa
from paged_attention_kv_pa_amd import workload
from pa_testutil import errors, finite_lse_err

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_REL, F32_MAX, LSE_TOL = 2e-2, 5e-3, 1e-5, 1e-3
DEV = torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def check_out(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), "%s: non-finite output" % what
    mx, rel = errors(got, ref)
    say("%s: max_abs=%.3e rel_rms=%.3e" % (what, mx, rel))
    if dtype == torch.float32:
        assert mx <= F32_MAX, "%s: max_abs %.3e" % (what, mx)
    else:
        assert mx <= BF16_MAX and rel <= BF16_REL, "%s: max_abs %.3e rel %.3e" % (what, mx, rel)


def check_lse(got, ref, what):
    e = finite_lse_err(got, ref)
    say("%s: lse max_abs=%.3e" % (what, e))
    assert e <= LSE_TOL


def run_forward(b, g=None, **kw):
    g = g if g is not None else b.to(DEV)
    lse = torch.full((b.num_tokens, b.num_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    out = pa.pa_forward(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.query_start_loc,
                        b.scale, lse=lse, max_seq_len=max(b.seq_lens_list + [1]),
                        max_q_len=max(b.q_lens + [1]), **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def oracle_forward(b, rows=None):
    lay = oracle.LAYOUT_MLA if b.layout == "mla" else oracle.LAYOUT_MHA
    return oracle.attention(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                            b.query_start_loc, b.scale, b.num_kv_heads,
                            head_dim_v=b.head_dim_v, layout=lay, rows=rows)


def forward_parity(b, what, rows=None, ref=None):
    """pa_forward against the oracle (ref: a precomputed oracle (out, lse) of b)."""
    say("case %s: B=%d T=%d keys=%d" % (what, b.num_seqs, b.num_tokens, sum(b.seq_lens_list)))
    got, glse = run_forward(b)
    ref, rlse = oracle_forward(b, rows) if ref is None else ref
    if rows is not None:
        sel = np.asarray(rows, dtype=bool)
        got, ref, glse, rlse = got[sel], ref[sel], glse[sel], rlse[sel]
    check_out(got, ref, b.dtype, what)
    check_lse(glse, rlse, what)
    return got


# ---------------------------------------------------------------- fp32 (tiny)

@pytest.mark.parametrize("case", [0, 1, 2])
def test_tiny_f32_decode_forward(case):
    b = workload.tiny_f32_decode(case)
    forward_parity(b, "tiny_f32_decode/%d" % case)


@pytest.mark.parametrize("S", [1, 3, 8, 40])
def test_tiny_f32_decode_split_and_merge(S):
    b = workload.tiny_f32_decode(0)
    g = b.to(DEV)
    say("case tiny_f32 split S=%d" % S)
    po, pl = pa.pa_decode_split(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.scale, S)
    out = pa.pa_merge_lse(po, pl, out_dtype=torch.float32)
    lse = torch.empty(pl.shape[:2], dtype=torch.float32, device=DEV)
    pa.pa_merge_lse(po, pl, lse=lse, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rpo, rpl = oracle.decode_split(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.scale,
                                   S, b.num_kv_heads)
    check_out(po.cpu().numpy(), rpo, torch.float32, "f32 partials S=%d" % S)
    check_lse(pl.cpu().numpy(), rpl, "f32 partial lse S=%d" % S)
    ref, rlse = oracle_forward(b)
    check_out(out.cpu().numpy(), ref, torch.float32, "f32 merged S=%d" % S)
    check_lse(lse.cpu().numpy(), rlse, "f32 merged lse S=%d" % S)


# ------------------------------------------------------- Llama-3.1-8B decode

@pytest.mark.parametrize("case", [0, 1, 2, 3])
def test_llama_decode_forward_full_size(case):
    b = workload.llama_decode(case)
    forward_parity(b, "llama_decode/%d" % case)


@pytest.mark.parametrize("batch", [1030, 2000])
def test_decode_more_requests_than_the_kernel_plans(batch):
    # decode-only batches above 1024 requests go through the planner kernel;
    # smaller ones are planned inside the persistent kernel (the cases above)
    b = workload.llama_decode(3, batch=batch, lo=1, hi=300)
    forward_parity(b, "llama decode, %d short requests" % batch)


@pytest.mark.parametrize("P", [8, 24, 48])
def test_decode_page_sizes(P):
    # decode items and split partitions over pages that hold a multiple of 8
    # keys, not always a power of two: one 32-key step can touch up to four
    # pages, and ranges end anywhere inside a page
    b = workload.make_batch([1] * 9, [0, 6, 7, 8, 30, 32, 199, 999, 2499], num_q_heads=32,
                            num_kv_heads=8, head_dim_qk=128, page_size=P, seed=70 + P)
    forward_parity(b, "decode pages P=%d" % P)
    g = b.to(DEV)
    say("case decode split pages P=%d" % P)
    po, pl = pa.pa_decode_split(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.scale, 5)
    torch.cuda.synchronize()
    rpo, rpl = oracle.decode_split(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.scale,
                                   5, b.num_kv_heads)
    check_out(po.cpu().numpy(), rpo, torch.bfloat16, "bf16 partials P=%d" % P)
    check_lse(pl.cpu().numpy(), rpl, "bf16 partial lse P=%d" % P)


@pytest.mark.parametrize("S", [1, 2, 7, 64, 200])
def test_llama_decode_split_matches_oracle_partials(S):
    b = workload.llama_decode(3, batch=8)
    g = b.to(DEV)
    say("case llama split S=%d" % S)
    po, pl = pa.pa_decode_split(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.scale, S)
    out = pa.pa_merge_lse(po, pl)
    torch.cuda.synchronize()
    rpo, rpl = oracle.decode_split(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.scale,
                                   S, b.num_kv_heads)
    check_out(po.cpu().numpy(), rpo, torch.bfloat16, "bf16 partials S=%d" % S)
    check_lse(pl.cpu().numpy(), rpl, "bf16 partial lse S=%d" % S)
    ref, _ = oracle_forward(b)
    check_out(out.float().cpu().numpy(), ref, torch.bfloat16, "bf16 merged S=%d" % S)


@pytest.mark.parametrize("Hq,Hkv,D,S", [(64, 2, 128, 1), (64, 2, 128, 5), (64, 1, 64, 3)])
def test_decode_split_wide_groups(Hq, Hkv, D, S):
    # more query heads per KV head than one decode tile holds: the split
    # kernel runs these rows through the prefill-mode item
    b = workload.make_batch([1, 1, 1], [2900, 77, 1500], num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim_qk=D, page_size=16, seed=Hq + D + S)
    g = b.to(DEV)
    say("case wide split Hq=%d Hkv=%d D=%d S=%d" % (Hq, Hkv, D, S))
    po, pl = pa.pa_decode_split(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.scale, S)
    out = pa.pa_merge_lse(po, pl)
    torch.cuda.synchronize()
    rpo, rpl = oracle.decode_split(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.scale,
                                   S, b.num_kv_heads)
    check_out(po.cpu().numpy(), rpo, torch.bfloat16, "wide partials S=%d" % S)
    check_lse(pl.cpu().numpy(), rpl, "wide partial lse S=%d" % S)
    ref, _ = oracle_forward(b)
    check_out(out.float().cpu().numpy(), ref, torch.bfloat16, "wide merged S=%d" % S)


@pytest.mark.parametrize("D,P", [(64, 16), (128, 8), (128, 32)])
def test_prefill_multi_item_shapes(D, P):
    # several 256-row items per (request, KV head), key ranges over many
    # copy tiles with a ragged last tile, for the other head dim and pages
    b = workload.make_batch([300, 37, 1], [700, 0, 900], num_q_heads=32, num_kv_heads=4,
                            head_dim_qk=D, page_size=P, seed=D + P)
    forward_parity(b, "prefill items D=%d P=%d" % (D, P))


# ------------------------------------------------- long-context split decode

@pytest.mark.parametrize("batch,S,lengths", [(1, 64, None), (4, 32, None), (16, 16, None),
                                             (1, 64, [32768]), (1, 64, [131072])])
def test_long_context_split_full_size(batch, S, lengths):
    b = workload.llama_long(batch=batch, lengths=lengths, device=DEV)
    say("case llama_long B=%d S=%d keys=%d" % (b.num_seqs, S, sum(b.seq_lens_list)))
    po, pl = pa.pa_decode_split(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.scale, S)
    out = pa.pa_merge_lse(po, pl)
    lse = torch.empty(pl.shape[:2], dtype=torch.float32, device=DEV)
    pa.pa_merge_lse(po, pl, out=torch.empty_like(out), lse=lse)
    torch.cuda.synchronize()
    h = b.to("cpu")
    ref, rlse = oracle_forward(h)
    check_out(out.float().cpu().numpy(), ref, torch.bfloat16, "long B=%d S=%d" % (batch, S))
    check_lse(lse.cpu().numpy(), rlse, "long B=%d S=%d" % (batch, S))
    # the same batch through pa_forward (its planner splits internally)
    got, glse = run_forward(h, g=b)
    check_out(got, ref, torch.bfloat16, "long pa_forward B=%d" % batch)
    check_lse(glse, rlse, "long pa_forward B=%d" % batch)


# ------------------------------------------------------ full and prefix masks

def masked_parity(b, mask, prefixes, what, sinks=None, alibi=None, alibi_mode=pa.PA_ALIBI_NONE):
    """pa_forward_masked against the oracle (alibi: the slopes, with alibi_mode)."""
    say("case %s: B=%d T=%d keys=%d mask=%d prefixes=%s sinks=%s alibi=%d" % (
        what, b.num_seqs, b.num_tokens, sum(b.seq_lens_list), mask, prefixes, sinks is not None,
        alibi_mode))
    g = b.to(DEV)
    pl = None if prefixes is None else torch.tensor(prefixes, dtype=torch.int32, device=DEV)
    sk = None if sinks is None else torch.tensor(sinks, dtype=torch.float32, device=DEV)
    al = None if alibi is None else torch.tensor(alibi, dtype=torch.float32, device=DEV)
    lse = torch.full((b.num_tokens, b.num_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    out = pa.pa_forward_masked(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                               g.query_start_loc, b.scale, mask, prefix_lens=pl, sinks=sk, lse=lse,
                               max_seq_len=max(b.seq_lens_list + [1]),
                               max_q_len=max(b.q_lens + [1]), alibi_slopes=al,
                               alibi_mode=alibi_mode)
    torch.cuda.synchronize()
    ref, rlse = oracle.attention(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                                 b.query_start_loc, b.scale, b.num_kv_heads, mask=mask,
                                 prefix_lens=None if prefixes is None else np.asarray(prefixes, np.int32),
                                 sinks=sinks, head_dim_v=b.head_dim_v,
                                 alibi_slopes=None if alibi is None else np.asarray(alibi, np.float32),
                                 alibi_mode=alibi_mode)
    got = out.float().cpu().numpy()
    check_out(got, ref, b.dtype, what)
    check_lse(lse.cpu().numpy(), rlse, what)
    return got


# decode, a two-token request (8 decode-mode rows), extend, prefill, prefill over 3 row blocks
MASK_Q, MASK_C = [1, 2, 300, 37, 190], [900, 40, 700, 0, 0]


@pytest.mark.parametrize("mask,prefixes", [
    (pa.PA_MASK_FULL, None),
    (pa.PA_MASK_PREFIX, [0, 41, 750, 20, 100]),     # inside the new tokens / the cache / none
    (pa.PA_MASK_PREFIX, [5000, 10, 1000, 37, 190]),  # past the end, covering every key
    (pa.PA_MASK_PREFIX, [-3, 42, 1, 64, 129]),
])
def test_masked_forward_matches_oracle(mask, prefixes):
    b = workload.make_batch(MASK_Q, MASK_C, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=601)
    masked_parity(b, mask, prefixes, "masked bf16")


@pytest.mark.parametrize("Hq,Hkv,D,P", [(32, 4, 64, 16), (64, 4, 128, 8), (16, 16, 128, 32)])
def test_masked_forward_shapes(Hq, Hkv, D, P):
    b = workload.make_batch([3, 1, 270], [50, 500, 260], num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim_qk=D, page_size=P, seed=Hq + Hkv + D + P)
    masked_parity(b, pa.PA_MASK_FULL, None, "full Hq=%d Hkv=%d D=%d P=%d" % (Hq, Hkv, D, P))
    masked_parity(b, pa.PA_MASK_PREFIX, [40, 0, 400], "prefix Hq=%d Hkv=%d D=%d P=%d" % (Hq, Hkv, D, P))


@pytest.mark.parametrize("mask,prefixes", [(pa.PA_MASK_FULL, None), (pa.PA_MASK_PREFIX, [3, 9, 0])])
def test_masked_forward_f32(mask, prefixes):
    b = workload.make_batch([4, 1, 7], [20, 33, 0], num_q_heads=8, num_kv_heads=2, head_dim_qk=64,
                            page_size=16, dtype=torch.float32, seed=607)
    masked_parity(b, mask, prefixes, "masked fp32")


def test_masked_causal_is_pa_forward_bitwise():
    b = workload.make_batch(MASK_Q, MASK_C, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=611)
    g = b.to(DEV)
    kw = dict(max_seq_len=max(b.seq_lens_list), max_q_len=max(b.q_lens))
    a = pa.pa_forward(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.query_start_loc,
                      b.scale, **kw)
    c = pa.pa_forward_masked(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                             g.query_start_loc, b.scale, pa.PA_MASK_CAUSAL, **kw)
    z = pa.pa_forward_masked(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                             g.query_start_loc, b.scale, pa.PA_MASK_PREFIX,
                             prefix_lens=torch.zeros(b.num_seqs, dtype=torch.int32, device=DEV), **kw)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(a.view(torch.int16), z.view(torch.int16))


def sink_logits(Hq, seed):
    """Sink logits far below, near and far above the scaled scores, and one -inf."""
    g = np.random.default_rng(seed)
    s = g.normal(0.0, 2.0, Hq).astype(np.float32)
    s[0], s[1], s[2] = -40.0, 30.0, -np.inf
    return s


@pytest.mark.parametrize("mask,prefixes", [(pa.PA_MASK_CAUSAL, None), (pa.PA_MASK_FULL, None),
                                           (pa.PA_MASK_PREFIX, [0, 41, 750, 20, 100])])
def test_sinks_forward_matches_oracle(mask, prefixes):
    b = workload.make_batch(MASK_Q, MASK_C, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=613)
    masked_parity(b, mask, prefixes, "sinks bf16", sinks=sink_logits(32, 1))


def test_sinks_in_split_decode_merge():
    # pa_decode_split partials merged by pa_merge_lse with sink logits
    b = workload.llama_decode(3, batch=8)
    g = b.to(DEV)
    sk = sink_logits(32, 11)
    po, pl = pa.pa_decode_split(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.scale, 7)
    lse = torch.empty(pl.shape[:2], dtype=torch.float32, device=DEV)
    out = pa.pa_merge_lse(po, pl, lse=lse, sinks=torch.from_numpy(sk).to(DEV))
    torch.cuda.synchronize()
    ref, rlse = oracle.attention(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                                 b.query_start_loc, b.scale, b.num_kv_heads, sinks=sk)
    check_out(out.float().cpu().numpy(), ref, torch.bfloat16, "split merge with sinks")
    check_lse(lse.cpu().numpy(), rlse, "split merge with sinks")


def test_sinks_on_split_decode_rows():
    # few long decode requests: pa_forward splits their keys, and the sink enters
    # in the merge of the partial rows
    b = workload.llama_decode(3, batch=4)
    masked_parity(b, pa.PA_MASK_CAUSAL, None, "sinks split decode", sinks=sink_logits(32, 2))


def test_sinks_f32():
    b = workload.make_batch([4, 1, 7], [20, 33, 0], num_q_heads=8, num_kv_heads=2, head_dim_qk=64,
                            page_size=16, dtype=torch.float32, seed=617)
    masked_parity(b, pa.PA_MASK_CAUSAL, None, "sinks fp32", sinks=sink_logits(8, 3))


# ------------------------------------------------------------- ALiBi (sqrt)

@pytest.mark.parametrize("mode", [pa.PA_ALIBI_SQRT, pa.PA_ALIBI_LINEAR])
@pytest.mark.parametrize("mask,prefixes", [(pa.PA_MASK_CAUSAL, None), (pa.PA_MASK_FULL, None),
                                           (pa.PA_MASK_PREFIX, [0, 41, 750, 20, 100])])
def test_alibi_forward_matches_oracle(mode, mask, prefixes):
    b = workload.make_batch(MASK_Q, MASK_C, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=1301)
    masked_parity(b, mask, prefixes, "alibi", alibi=workload.alibi_slopes(32), alibi_mode=mode)


@pytest.mark.parametrize("Hq,Hkv,D,P,dtype", [(12, 4, 64, 16, torch.bfloat16),
                                              (16, 16, 128, 32, torch.bfloat16),
                                              (8, 2, 64, 16, torch.float32)])
def test_alibi_shapes_and_fp32(Hq, Hkv, D, P, dtype):
    b = workload.make_batch([3, 1, 270, 4], [50, 500, 260, 0], num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim_qk=D, page_size=P, dtype=dtype, seed=1311 + Hq + D)
    masked_parity(b, pa.PA_MASK_CAUSAL, None, "alibi sqrt Hq=%d D=%d %s" % (Hq, D, dtype),
                  alibi=workload.alibi_slopes(Hq), alibi_mode=pa.PA_ALIBI_SQRT,
                  sinks=sink_logits(Hq, 7))


def test_alibi_decode_only_with_split_rows():
    # long decode rows split over several partitions: the bias follows the key, not
    # the partition
    b = workload.llama_decode(3, batch=6)
    masked_parity(b, pa.PA_MASK_CAUSAL, None, "alibi sqrt decode", alibi=workload.alibi_slopes(32),
                  alibi_mode=pa.PA_ALIBI_SQRT)


# Decode-only calls of at most 512 keys whose (request, KV head) pairs fit the
# grid run one workgroup per pair over all its keys (no plan, no split, no merge
# launch): that path with every option of pa_forward_masked and every head shape.
SINGLE_Q, SINGLE_C = [1, 1, 1, 1, 1], [0, 37, 255, 400, 511]


@pytest.mark.parametrize("feature", ["causal", "full", "prefix", "sinks", "alibi_sqrt",
                                     "alibi_linear"])
def test_single_pass_decode_options(feature):
    b = workload.make_batch(SINGLE_Q, SINGLE_C, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=1401)
    mask = {"full": pa.PA_MASK_FULL, "prefix": pa.PA_MASK_PREFIX}.get(feature, pa.PA_MASK_CAUSAL)
    prefixes = [0, 10, 300, 1000, 5] if feature == "prefix" else None
    sinks = sink_logits(32, 21) if feature == "sinks" else None
    mode = {"alibi_sqrt": pa.PA_ALIBI_SQRT, "alibi_linear": pa.PA_ALIBI_LINEAR}.get(
        feature, pa.PA_ALIBI_NONE)
    alibi = workload.alibi_slopes(32) if mode != pa.PA_ALIBI_NONE else None
    masked_parity(b, mask, prefixes, "single-pass decode %s" % feature, sinks=sinks, alibi=alibi,
                  alibi_mode=mode)


@pytest.mark.parametrize("Hq,Hkv,Dqk,Dv,P", [(64, 4, 128, 128, 16), (32, 8, 64, 64, 8),
                                             (16, 16, 192, 128, 64), (128, 8, 128, 128, 32)])
def test_single_pass_decode_shapes(Hq, Hkv, Dqk, Dv, P):
    b = workload.make_batch(SINGLE_Q, SINGLE_C, num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim_qk=Dqk, head_dim_v=Dv, page_size=P, seed=1403 + Hq + Dqk)
    forward_parity(b, "single-pass decode Hq=%d Hkv=%d D=%d/%d P=%d" % (Hq, Hkv, Dqk, Dv, P))
    masked_parity(b, pa.PA_MASK_CAUSAL, None, "single-pass decode sinks Hq=%d D=%d/%d" % (
        Hq, Dqk, Dv), sinks=sink_logits(Hq, 23))


def test_alibi_stays_off_the_chunked_route():
    # few long extends (pa_forward would take the chunked route): with ALiBi the call
    # runs on the persistent kernel
    b = workload.make_batch([100, 1, 30], [12000, 20000, 9000], num_q_heads=8, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=1321)
    masked_parity(b, pa.PA_MASK_CAUSAL, None, "alibi sqrt long extends",
                  alibi=workload.alibi_slopes(8), alibi_mode=pa.PA_ALIBI_SQRT)


def test_full_mask_qwen3_scaled():
    b = workload.qwen3_mixed(1, n_decode=6, n_extend=2, n_prefill=2, dec=(1024, 4096),
                             ext_q=(256, 600), ext_c=(4096, 8192), pre_q=(512, 1500))
    masked_parity(b, pa.PA_MASK_FULL, None, "full mask qwen3 scaled")


# ------------------------------------------- chunked-context processing

def chunked_parity(b, C, what, S=None, rows=None, mask=pa.PA_MASK_CAUSAL, prefixes=None,
                   ref=None, partials=True):
    """pa_forward_chunked partials against the oracle's chunk partials, and their
    pa_merge_lse against plain attention (rows: optional sample of output rows;
    ref: a precomputed oracle (out, lse); partials=False skips the partials)."""
    g = b.to(DEV)
    pfx = None if prefixes is None else np.asarray(prefixes, np.int32)
    dpfx = None if prefixes is None else torch.tensor(prefixes, dtype=torch.int32, device=DEV)
    Lmax = max(b.seq_lens_list + [1])
    S = (Lmax + C - 1) // C if S is None else S
    say("case %s: B=%d T=%d keys=%d C=%d S=%d" % (what, b.num_seqs, b.num_tokens,
                                                  sum(b.seq_lens_list), C, S))
    po, pl = pa.pa_forward_chunked(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                                   g.query_start_loc, b.scale, C, num_chunks=S, max_seq_len=Lmax,
                                   max_q_len=max(b.q_lens + [1]), mask=mask, prefix_lens=dpfx)
    lse = torch.empty(pl.shape[:2], dtype=torch.float32, device=DEV)
    out = pa.pa_merge_lse(po, pl, lse=lse)
    torch.cuda.synchronize()
    po, pl = po.cpu().numpy(), pl.cpu().numpy()
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    if rows is None and partials:
        rpo, rpl = oracle.chunked_partials(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                                           b.query_start_loc, b.scale, C, S, b.num_kv_heads,
                                           mask=mask, prefix_lens=pfx, head_dim_v=b.head_dim_v)
        check_out(po, rpo, torch.bfloat16, "%s partials" % what)
        check_lse(pl, rpl, "%s partial lse" % what)
    if ref is None:
        ref, rlse = oracle.attention(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                                     b.query_start_loc, b.scale, b.num_kv_heads, rows=rows,
                                     mask=mask, prefix_lens=pfx, head_dim_v=b.head_dim_v)
    else:
        ref, rlse = ref
    if rows is not None:
        sel = np.asarray(rows, dtype=bool)
        got, ref, glse, rlse = got[sel], ref[sel], glse[sel], rlse[sel]
    check_out(got, ref, torch.bfloat16, "%s merged" % what)
    check_lse(glse, rlse, "%s merged" % what)


@pytest.mark.parametrize("C", [64, 256, 1024])
def test_chunked_mixed_batch_matches_oracle(C):
    # decode, short decode, extend, prefill, prefill over several row blocks
    b = workload.make_batch([1, 1, 300, 37, 520], [900, 50, 700, 0, 0], num_q_heads=32,
                            num_kv_heads=8, head_dim_qk=128, page_size=16, seed=500 + C)
    chunked_parity(b, C, "chunked mixed")


@pytest.mark.parametrize("Hq,Hkv,D,P,C", [(32, 4, 64, 16, 128), (32, 8, 128, 8, 64),
                                          (64, 4, 128, 32, 192), (16, 16, 128, 16, 320)])
def test_chunked_head_and_page_shapes(Hq, Hkv, D, P, C):
    b = workload.make_batch([70, 1, 129], [400, 333, 64], num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim_qk=D, page_size=P, seed=Hq + Hkv + D + P + C)
    chunked_parity(b, C, "chunked Hq=%d Hkv=%d D=%d P=%d" % (Hq, Hkv, D, P))


@pytest.mark.parametrize("mask,prefixes", [(pa.PA_MASK_FULL, None),
                                           (pa.PA_MASK_PREFIX, [0, 60, 800, 20, 300])])
def test_chunked_masks_match_oracle(mask, prefixes):
    b = workload.make_batch([1, 1, 300, 37, 520], [900, 50, 700, 0, 0], num_q_heads=32,
                            num_kv_heads=8, head_dim_qk=128, page_size=16, seed=531)
    chunked_parity(b, 256, "chunked mask %d" % mask, mask=mask, prefixes=prefixes)


def test_chunked_extra_chunks_are_empty():
    b = workload.make_batch([5, 1], [60, 190], num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=77)
    chunked_parity(b, 64, "chunked extra chunks", S=9)  # 4 chunks would cover 196 keys


def test_chunked_long_context_extend():
    # the case chunking is for: a long cached context under few new tokens
    b = workload.make_batch([200, 1, 64], [20000, 30000, 9000], num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=91)
    chunked_parity(b, 4096, "chunked long extend")


def test_forward_runs_few_long_extends_as_chunks():
    # few long requests with new tokens: pa_forward itself runs them as chunk
    # partials + merge (its prefill items alone could not fill the GPU)
    b = workload.make_batch([200, 1, 64], [20000, 30000, 9000], num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=93)
    forward_parity(b, "pa_forward on few long extends")


@pytest.mark.parametrize("mask,prefixes,with_sinks", [(pa.PA_MASK_FULL, None, True),
                                                      (pa.PA_MASK_PREFIX, [20100, 5, 9030], False),
                                                      (pa.PA_MASK_CAUSAL, None, True)])
def test_forward_chunked_route_masks_and_sinks(mask, prefixes, with_sinks):
    # the same few long extends under the other masks and with sinks: the chunk
    # kernel takes the mask, the merge folds the sinks in
    b = workload.make_batch([200, 1, 64], [20000, 30000, 9000], num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=95)
    masked_parity(b, mask, prefixes, "routed mask %d" % mask,
                  sinks=sink_logits(32, 9) if with_sinks else None)


_LONG_EXTEND = {}


def long_extend_case():
    """The bench's chunked-extend workload (256 new tokens on 131072 cached tokens,
    Llama-3.1-8B heads) and its oracle result over every row, computed once."""
    if not _LONG_EXTEND:
        b = workload.llama_long_extend(0)
        say("oracle: long extend, all %d rows x %d heads" % (b.num_tokens, b.num_q_heads))
        _LONG_EXTEND["b"] = b
        _LONG_EXTEND["ref"] = oracle_forward(b)
    return _LONG_EXTEND["b"], _LONG_EXTEND["ref"]


def test_forward_long_extend_full_size_all_rows():
    b, ref = long_extend_case()
    forward_parity(b, "pa_forward long extend full size (all rows)", ref=ref)


@pytest.mark.parametrize("chunks", [8, 17])
def test_chunked_long_extend_full_size_all_rows(chunks):
    # partials are compared at smaller sizes (test_chunked_long_context_extend);
    # 8 chunks (one work item per compute unit) is the configuration the bench times
    b, ref = long_extend_case()
    L = max(b.seq_lens_list)
    C = ((L + chunks - 1) // chunks + 63) // 64 * 64
    chunked_parity(b, C, "chunked long extend full size, %d chunks (all rows)" % chunks, ref=ref,
                   partials=False)


LONG_MIX = dict(n_decode=6, n_extend=2, n_prefill=2, dec=(1024, 4096), ext_q=(256, 500),
                ext_c=(4096, 8192), pre_q=(512, 1200))


@pytest.mark.parametrize("mask,prefixes,with_sinks,alibi", [
    (pa.PA_MASK_CAUSAL, None, False, False),
    (pa.PA_MASK_FULL, None, True, False),
    (pa.PA_MASK_PREFIX, [0] * 10 + [131000], False, False),
    (pa.PA_MASK_CAUSAL, None, True, True)])
def test_long_extend_cut_into_chunks_inside_a_mixed_batch(mask, prefixes, with_sinks, alibi):
    # a scaled Qwen3 mixed batch plus one extend of 8 new tokens on 131072 cached
    # ones: the planner cuts that request (>= 100K keys) into 32K-key chunks whose
    # partial rows the chunk merge combines, inside the same persistent call
    b = workload.qwen3_mixed_with_long_extend(1, new_tokens=8, cached=131072, **LONG_MIX)
    masked_parity(b, mask, prefixes, "long extend in mixed batch mask %d" % mask,
                  sinks=sink_logits(64, 13) if with_sinks else None,
                  alibi=workload.alibi_slopes(64) if alibi else None,
                  alibi_mode=pa.PA_ALIBI_SQRT if alibi else pa.PA_ALIBI_NONE)


def padded_call(b, route_expected):
    """pa_forward with 7 padding rows past query_start_loc[B] in q, out and lse: the
    padding rows of out / lse must keep their sentinel bytes."""
    g = b.to(DEV)
    T, Hq, D = b.num_tokens, b.num_q_heads, b.head_dim_v
    qp = torch.cat([g.q, torch.full((7, Hq, b.head_dim_qk), float("nan"), dtype=b.dtype,
                                    device=DEV)]).contiguous()
    out = torch.full((T + 7, Hq, D), 3.0, dtype=b.dtype, device=DEV)
    lse = torch.full((T + 7, Hq), -7.0, dtype=torch.float32, device=DEV)
    maxL, maxq = max(b.seq_lens_list), max(b.q_lens)
    dims = pa.make_dims(qp, g.k_cache, g.v_cache, g.block_table, g.seq_lens, T + 7,
                        max_seq_len=maxL, max_q_len=maxq)
    # the chunked route adds its partials to the workspace of the same dims
    decode_dims = pa.make_dims(qp, g.k_cache, g.v_cache, g.block_table, g.seq_lens, T + 7,
                               max_seq_len=maxL, max_q_len=1)
    assert (pa.pa_workspace_size(dims) > pa.pa_workspace_size(decode_dims)) == route_expected
    pa.pa_forward(qp, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.query_start_loc,
                  b.scale, out=out, lse=lse, max_seq_len=maxL, max_q_len=maxq)
    torch.cuda.synchronize()
    assert torch.all(out[T:].float() == 3.0), "padding rows of out were written"
    assert torch.all(lse[T:] == -7.0), "padding rows of lse were written"
    ref, rlse = oracle_forward(b)
    check_out(out[:T].float().cpu().numpy(), ref, b.dtype, "padded call (route %s)" % route_expected)
    check_lse(lse[:T].cpu().numpy(), rlse, "padded call (route %s)" % route_expected)


def test_padding_rows_untouched_on_the_chunked_route():
    b = workload.make_batch([200, 1, 64], [20000, 30000, 9000], num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=97)
    padded_call(b, True)


def test_padding_rows_untouched_on_the_persistent_path():
    b = workload.make_batch([1, 37, 130, 1], [300, 0, 90, 2000], num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=98)
    padded_call(b, False)


# --------------------------------------------------- Qwen3 mixed batch (MHA)

def test_qwen3_mixed_scaled_all_rows():
    b = workload.qwen3_mixed(1, n_decode=12, n_extend=2, n_prefill=2, dec=(1024, 4096),
                             ext_q=(256, 600), ext_c=(4096, 8192), pre_q=(512, 1500))
    forward_parity(b, "qwen3_mixed scaled")


def test_qwen3_mixed_full_size_sampled_rows():
    b = workload.qwen3_mixed(0)
    T, Hq = b.num_tokens, b.num_q_heads
    rows = np.zeros((T, Hq), dtype=bool)
    qsl = b.query_start_loc.numpy()
    for i in range(b.num_seqs):  # every decode row, first/last row of each request, a stride
        s, e = qsl[i], qsl[i + 1]
        rows[s, :] = True
        rows[e - 1, :] = True
        rows[s:e:97, ::5] = True
    forward_parity(b, "qwen3_mixed full (sampled rows)", rows=rows)


# ------------------------------------------------------- DeepSeek-R1 MLA

def mla_parity(b, what, S=0, heads=None):
    say("case %s: B=%d keys=%d S=%d" % (what, b.num_seqs, sum(b.seq_lens_list), S))
    g = b.to(DEV)
    lse = torch.empty(b.num_seqs, b.num_q_heads, dtype=torch.float32, device=DEV)
    out = pa.mla_decode(g.q, g.k_cache, g.block_table, g.seq_lens, b.scale, lse=lse, num_splits=S,
                        max_seq_len=max(b.seq_lens_list))
    torch.cuda.synchronize()
    rows = None
    if heads is not None:
        rows = np.zeros((b.num_seqs, b.num_q_heads), dtype=bool)
        rows[:, heads] = True
    ref, rlse = oracle_forward(b, rows)
    got, glse = out.float().cpu().numpy(), lse.cpu().numpy()
    if rows is not None:
        got, ref, glse, rlse = got[rows], ref[rows], glse[rows], rlse[rows]
    check_out(got, ref, torch.bfloat16, what)
    check_lse(glse, rlse, what)


@pytest.mark.parametrize("S", [0, 1, 3, 16])
def test_mla_scaled(S):
    b = workload.deepseek_mla(1, batch=6, lo=1, hi=1500)
    mla_parity(b, "mla scaled", S=S)


def test_mla_balanced_many_short_requests():
    # more tiles than workgroups: ranges hold several requests, some cut in two
    b = workload.deepseek_mla(2, batch=600, lo=1, hi=40)
    mla_parity(b, "mla balanced, 600 short requests", S=0)


@pytest.mark.parametrize("page,heads", [(16, 64), (8, 16), (256, 128), (32, 48), (64, 112)])
def test_mla_balanced_pages_and_heads(page, heads):
    # (head counts that leave some of the 16-head waves without rows)
    # fewer tiles than workgroups: most requests spread over several workgroups
    lens = [1, 33, 700, 5, 2000, 64, 63, 32, 31]
    b = workload.make_batch([1] * len(lens), [x - 1 for x in lens], num_q_heads=heads,
                            num_kv_heads=1, head_dim_qk=576, head_dim_v=512, page_size=page,
                            dtype=torch.bfloat16, layout="mla", scale=1.0 / math.sqrt(192.0),
                            seed=41 + page, name="mla_pages")
    mla_parity(b, "mla balanced page %d heads %d" % (page, heads), S=0)


def test_mla_full_size_all_heads():
    b = workload.deepseek_mla(0)
    mla_parity(b, "mla full size, all 128 heads")


# --------------------------------------------------------------- edge cases

@pytest.mark.parametrize("Hq,Hkv", [(16, 16), (32, 8)])
def test_f32_unequal_head_dims(Hq, Hkv):
    # non-absorbed MLA-shaped heads (query/key 192 = 128 + 64 rotary, value 128) on the
    # fp32 path: prefill, extend and decode rows
    b = workload.make_batch([1, 37, 130], [300, 0, 90], num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim_qk=192, head_dim_v=128, page_size=16,
                            dtype=torch.float32, seed=701 + Hq)
    forward_parity(b, "fp32 Dqk 192 Dv 128 Hq=%d Hkv=%d" % (Hq, Hkv))


# ------------------- MLA prefill / extend, non-absorbed (query/key 192, value 128)

F2 = dict(head_dim_qk=192, head_dim_v=128, scale=1.0 / math.sqrt(192.0))


@pytest.mark.parametrize("Hq,Hkv,P", [(16, 16, 64), (16, 4, 16), (8, 1, 8)])
def test_f2_mixed_forward(Hq, Hkv, P):
    # decode, a 3-token request, extend, prefill and a prefill over 3 row blocks (G = 1)
    b = workload.make_batch([1, 3, 300, 40, 520], [900, 50, 700, 0, 0], num_q_heads=Hq,
                            num_kv_heads=Hkv, page_size=P, seed=900 + Hq + Hkv + P, **F2)
    forward_parity(b, "bf16 Dqk 192 Dv 128 Hq=%d Hkv=%d P=%d" % (Hq, Hkv, P))


def test_f2_all_128_heads():
    b = workload.make_batch([1, 130, 64], [200, 100, 0], num_q_heads=128, num_kv_heads=128,
                            page_size=64, seed=931, **F2)
    forward_parity(b, "bf16 Dqk 192 Dv 128, 128 heads")


def test_f2_deepseek_prefill_scaled():
    b = workload.deepseek_mha_prefill(1, n_extend=2, n_prefill=2, ext_q=(200, 400),
                                      ext_c=(1000, 3000), pre_q=(300, 700), heads=16)
    forward_parity(b, "deepseek non-absorbed prefill + extend, scaled, 16 heads")


def test_f2_decode_only_batch():
    b = workload.make_batch([1] * 7, [5, 900, 3000, 64, 127, 2000, 40], num_q_heads=32,
                            num_kv_heads=8, page_size=16, seed=941, **F2)
    forward_parity(b, "bf16 Dqk 192 Dv 128 decode-only")


@pytest.mark.parametrize("mask,prefixes,with_sinks", [(pa.PA_MASK_FULL, None, False),
                                                      (pa.PA_MASK_PREFIX, [0, 41, 750, 20, 100], True),
                                                      (pa.PA_MASK_CAUSAL, None, True)])
def test_f2_masks_and_sinks(mask, prefixes, with_sinks):
    b = workload.make_batch(MASK_Q, MASK_C, num_q_heads=16, num_kv_heads=8, page_size=16,
                            seed=951, **F2)
    masked_parity(b, mask, prefixes, "f2 mask %d sinks %s" % (mask, with_sinks),
                  sinks=sink_logits(16, 5) if with_sinks else None)


def test_f2_chunked_and_routed():
    b = workload.make_batch([200, 1, 64], [20000, 30000, 9000], num_q_heads=4, num_kv_heads=4,
                            page_size=16, seed=961, **F2)
    chunked_parity(b, 4096, "f2 chunked long extend")
    forward_parity(b, "f2 pa_forward routed through chunks")


@pytest.mark.parametrize("Hq,Hkv,S", [(16, 4, 5), (16, 16, 1), (64, 2, 3)])
def test_f2_decode_split(Hq, Hkv, S):
    b = workload.make_batch([1] * 5, [300, 1, 2000, 77, 900], num_q_heads=Hq, num_kv_heads=Hkv,
                            page_size=16, seed=971 + S, **F2)
    g = b.to(DEV)
    say("case f2 decode split Hq=%d Hkv=%d S=%d" % (Hq, Hkv, S))
    po, pl = pa.pa_decode_split(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.scale, S)
    lse = torch.empty(pl.shape[:2], dtype=torch.float32, device=DEV)
    out = pa.pa_merge_lse(po, pl, lse=lse)
    torch.cuda.synchronize()
    rpo, rpl = oracle.decode_split(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.scale,
                                   S, b.num_kv_heads, head_dim_v=128)
    check_out(po.cpu().numpy(), rpo, torch.bfloat16, "f2 partials")
    check_lse(pl.cpu().numpy(), rpl, "f2 partial lse")
    ref, rlse = oracle_forward(b)
    check_out(out.float().cpu().numpy(), ref, torch.bfloat16, "f2 split merged")
    check_lse(lse.cpu().numpy(), rlse, "f2 split merged")


def test_edge_empty_requests_single_keys_and_exact_pages():
    b = workload.make_batch([1, 0, 1, 3, 0, 16, 1, 1], [0, 5, 15, 13, 0, 0, 31, 47],
                            num_q_heads=32, num_kv_heads=8, head_dim_qk=128, page_size=16, seed=11)
    forward_parity(b, "edge mix")


def test_edge_empty_requests_in_chunked_masked_and_routed_calls():
    # requests with no new token (one of them with no key at all) between real ones
    b = workload.make_batch([1, 0, 40, 0, 3], [0, 5, 100, 0, 13], num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=13)
    chunked_parity(b, 64, "edge chunked")
    masked_parity(b, pa.PA_MASK_FULL, None, "edge full mask", sinks=sink_logits(32, 7))
    masked_parity(b, pa.PA_MASK_PREFIX, [0, 3, 120, 0, 16], "edge prefix mask")
    # the same shape of batch with long contexts, so that pa_forward takes its chunked route
    r = workload.make_batch([1, 0, 40, 0, 3], [9000, 5, 10000, 0, 13], num_q_heads=32,
                            num_kv_heads=8, head_dim_qk=128, page_size=16, seed=14)
    forward_parity(r, "edge routed")
    masked_parity(r, pa.PA_MASK_PREFIX, [0, 3, 9500, 0, 16], "edge routed prefix", sinks=sink_logits(32, 8))


@pytest.mark.parametrize("Hq,Hkv,D,P", [(32, 8, 64, 16), (64, 2, 128, 16), (16, 16, 128, 32),
                                        (8, 1, 128, 64), (12, 4, 64, 8), (32, 8, 128, 24),
                                        (16, 2, 64, 40)])
def test_head_and_page_shapes(Hq, Hkv, D, P):
    b = workload.make_batch([1, 5, 40, 1, 130], [700, 100, 0, 3, 60], num_q_heads=Hq,
                            num_kv_heads=Hkv, head_dim_qk=D, page_size=P, seed=Hq * 7 + P)
    forward_parity(b, "shapes Hq=%d Hkv=%d D=%d P=%d" % (Hq, Hkv, D, P))


def test_request_order_permutation_bitwise():
    # [decode : extend : prefill] reordered: every request's rows move with it and
    # come out bit for bit the same (the decode items' key partitions of this batch
    # do not depend on a request's place in it)
    b = workload.make_batch([1, 1, 1, 300, 37, 1, 520, 2], [900, 50, 2500, 700, 0, 4000, 0, 30],
                            num_q_heads=32, num_kv_heads=8, head_dim_qk=128, page_size=16,
                            seed=1201)
    order = [6, 3, 0, 7, 5, 1, 4, 2]
    pb, src = workload.permute_requests(b, order)
    say("case request order %s" % order)
    got, glse = run_forward(b)
    pgot, plse = run_forward(pb)
    # (bf16 outputs widened exactly to fp32: equal floats are equal bit patterns)
    assert np.array_equal(pgot, got[src.numpy()]), "permuted outputs differ"
    assert np.array_equal(plse, glse[src.numpy()])
    ref, rlse = oracle_forward(pb)
    check_out(pgot, ref, b.dtype, "permuted batch")
    check_lse(plse, rlse, "permuted batch")


def test_request_order_permutation_large_batch():
    # a decode batch large enough that the last requests get finer key partitions:
    # reversing it changes the partitions, so outputs permute within tolerance
    b = workload.llama_decode(3, batch=48)
    order = list(range(47, -1, -1))
    pb, src = workload.permute_requests(b, order)
    got, glse = run_forward(b)
    pgot, plse = run_forward(pb)
    ref, rlse = oracle_forward(pb)
    check_out(pgot, ref, b.dtype, "reversed decode batch")
    check_lse(plse, rlse, "reversed decode batch")
    mx = float(np.max(np.abs(pgot - got[src.numpy()])))
    say("reversed decode batch: max |permuted - original| = %.3e" % mx)
    assert mx <= 2 * BF16_MAX


@pytest.mark.parametrize("fill", [0x00, 0xAB])
def test_decode_workspace_state_between_calls(fill):
    # A decode-only call plans itself and takes its items from a queue counter
    # that the previous call's merge left at zero, next to a marker.  A fresh
    # workspace (any bytes) has no marker: that call takes a fixed item sequence.
    # Both kinds of call, and a call after a prefill call on the same workspace,
    # give the same bits.
    b = workload.llama_decode(3, batch=40)
    g = b.to(DEV)
    kw = dict(max_seq_len=max(b.seq_lens_list), max_q_len=1)
    dims = pa.make_dims(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.num_tokens, **kw)
    ws = torch.full((pa.pa_workspace_size(dims),), fill, dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(3):
        outs.append(pa.pa_forward(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                                  g.query_start_loc, b.scale, workspace=ws, **kw))
    m = workload.make_batch([1, 37, 130], [300, 0, 90], num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=5).to(DEV)
    mws = ws[:pa.pa_workspace_size(pa.make_dims(m.q, m.k_cache, m.v_cache, m.block_table,
                                                m.seq_lens, m.num_tokens, max_seq_len=220,
                                                max_q_len=130))]
    pa.pa_forward(m.q, m.k_cache, m.v_cache, m.block_table, m.seq_lens, m.query_start_loc,
                  m.scale, workspace=mws, max_seq_len=220, max_q_len=130)
    outs.append(pa.pa_forward(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                              g.query_start_loc, b.scale, workspace=ws, **kw))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    ref, _ = oracle_forward(b)
    check_out(outs[0].float().cpu().numpy(), ref, b.dtype, "decode, workspace filled 0x%02x" % fill)


def test_forward_without_workspace_shares_one_per_stream():
    # calls that pass no workspace reuse one kept by the binding, so the second
    # call finds the queue marker the first one left; the bits do not change
    b = workload.llama_decode(3, batch=24)
    g = b.to(DEV)
    kw = dict(max_seq_len=max(b.seq_lens_list), max_q_len=1)
    from paged_attention_kv_pa_amd import binding
    binding._ws_cache.clear()
    o1 = pa.pa_forward(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.query_start_loc,
                       b.scale, **kw)
    assert len(binding._ws_cache) == 1
    ws = next(iter(binding._ws_cache.values()))
    o2 = pa.pa_forward(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.query_start_loc,
                       b.scale, **kw)
    torch.cuda.synchronize()
    assert next(iter(binding._ws_cache.values())) is ws
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ref, _ = oracle_forward(b)
    check_out(o2.float().cpu().numpy(), ref, b.dtype, "decode, shared workspace")


def test_page_permutation_invariance_bitwise():
    a = workload.make_batch([1, 9, 70], [400, 33, 0], num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=5)
    out_a, lse_a = run_forward(a)
    # move every page to a new physical slot and remap the table
    perm = torch.randperm(a.num_pages, generator=torch.Generator().manual_seed(9))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(a.num_pages)
    b = workload.Batch(**{**a.__dict__})
    b.k_cache = a.k_cache[inv]
    b.v_cache = a.v_cache[inv]
    b.block_table = perm[a.block_table.long()].to(torch.int32)
    out_b, lse_b = run_forward(b)
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


def test_determinism_bitwise():
    b = workload.qwen3_mixed(2, n_decode=6, n_extend=1, n_prefill=1, dec=(500, 3000),
                             ext_q=(100, 300), ext_c=(500, 900), pre_q=(200, 400))
    g = b.to(DEV)
    o1, l1 = run_forward(b, g)
    o2, l2 = run_forward(b, g)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_split_count_larger_than_pages_gives_empty_partitions():
    b = workload.make_batch([1, 1], [4, 40], num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=13)
    g = b.to(DEV)
    po, pl = pa.pa_decode_split(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.scale, 9)
    torch.cuda.synchronize()
    pl = pl.cpu().numpy()
    po = po.cpu().numpy()
    assert np.isneginf(pl[0, :, 1:]).all() and (po[0, :, 1:] == 0).all()
    assert np.isneginf(pl[1, :, 3:]).all() and np.isfinite(pl[1, :, :3]).all()


# ------------------------------------------------------------ graph replay

def test_graph_capture_replay_with_new_lengths():
    """One captured pa_forward (planner + persistent kernel + merge) replayed
    after rewriting seq_lens, query_start_loc and block_table in place."""
    Hq, Hkv, D, P = 32, 8, 128, 16
    specs = [([1, 1, 20, 1], [900, 40, 30, 2000]), ([1, 7, 1, 1], [60, 100, 2500, 5]),
             ([3, 1, 1, 15], [10, 1200, 0, 700])]
    batches = [workload.make_batch(q, c, num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D,
                                   page_size=P, seed=100 + i, max_pages_per_seq=200,
                                   pool_pages=700) for i, (q, c) in enumerate(specs)]
    T = max(b.num_tokens for b in batches)
    # fixed-capacity device buffers
    q = torch.zeros(T, Hq, D, dtype=torch.bfloat16, device=DEV)
    kc = batches[0].k_cache.to(DEV).clone()
    vc = batches[0].v_cache.to(DEV).clone()
    bt = torch.zeros(4, 200, dtype=torch.int32, device=DEV)
    sl = torch.zeros(4, dtype=torch.int32, device=DEV)
    qsl = torch.zeros(5, dtype=torch.int32, device=DEV)
    out = torch.zeros(T, Hq, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(T, Hq, dtype=torch.float32, device=DEV)
    dims_kw = dict(max_seq_len=200 * P, max_q_len=T)
    ws = torch.empty(pa.pa_workspace_size(pa.make_dims(q, kc, vc, bt, sl, T, **dims_kw)),
                     dtype=torch.uint8, device=DEV)

    def load(b):
        q.zero_()
        q[:b.num_tokens].copy_(b.q)
        kc.copy_(b.k_cache)
        vc.copy_(b.v_cache)
        bt.copy_(b.block_table)
        sl.copy_(b.seq_lens)
        qsl.copy_(torch.cat([b.query_start_loc,
                             b.query_start_loc[-1:].expand(5 - b.query_start_loc.numel())]))

    def call():
        pa.pa_forward(q, kc, vc, bt, sl, qsl, batches[0].scale, out=out, lse=lse, workspace=ws,
                      **dims_kw)

    load(batches[0])
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, b in enumerate(batches):
            say("graph replay %d batch %d" % (rep, i))
            load(b)
            out.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            g_out = out[:b.num_tokens].float().cpu().numpy()
            g_lse = lse[:b.num_tokens].cpu().numpy()
            e_out, e_lse = run_forward(b)  # eager on a fresh copy
            assert np.array_equal(g_out, e_out) and np.array_equal(g_lse, e_lse)
            ref, rlse = oracle_forward(b)
            check_out(g_out, ref, torch.bfloat16, "graph batch %d" % i)
            check_lse(g_lse, rlse, "graph batch %d" % i)


def test_graph_replay_masked_sinks_and_chunked():
    """A captured pa_forward_masked (prefix mask, sinks) and a captured pa_forward_chunked +
    pa_merge_lse, replayed after rewriting the batch, the prefix lengths and the sinks."""
    Hq, Hkv, D, P = 32, 8, 128, 16
    specs = [([1, 9, 130], [700, 40, 200]), ([3, 1, 60], [10, 1500, 90])]
    batches = [workload.make_batch(q, c, num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D,
                                   page_size=P, seed=200 + i, max_pages_per_seq=120,
                                   pool_pages=300) for i, (q, c) in enumerate(specs)]
    prefixes = [[5, 30, 100], [0, 2000, 77]]
    sinks = [sink_logits(Hq, 5), sink_logits(Hq, 6)]
    T, C, S = max(b.num_tokens for b in batches), 256, 8
    q = torch.zeros(T, Hq, D, dtype=torch.bfloat16, device=DEV)
    kc = batches[0].k_cache.to(DEV).clone()
    vc = batches[0].v_cache.to(DEV).clone()
    bt = torch.zeros(3, 120, dtype=torch.int32, device=DEV)
    sl = torch.zeros(3, dtype=torch.int32, device=DEV)
    qsl = torch.zeros(4, dtype=torch.int32, device=DEV)
    pl = torch.zeros(3, dtype=torch.int32, device=DEV)
    sk = torch.zeros(Hq, dtype=torch.float32, device=DEV)
    out = torch.zeros(T, Hq, D, dtype=torch.bfloat16, device=DEV)
    cout = torch.zeros(T, Hq, D, dtype=torch.bfloat16, device=DEV)
    po = torch.zeros(T, Hq, S, D, dtype=torch.float32, device=DEV)
    plse = torch.zeros(T, Hq, S, dtype=torch.float32, device=DEV)
    kw = dict(max_seq_len=120 * P, max_q_len=T)
    ws = torch.empty(pa.pa_workspace_size(pa.make_dims(q, kc, vc, bt, sl, T, **kw)),
                     dtype=torch.uint8, device=DEV)

    def load(i):
        b = batches[i]
        q.zero_()
        q[:b.num_tokens].copy_(b.q)
        kc.copy_(b.k_cache)
        vc.copy_(b.v_cache)
        bt.copy_(b.block_table)
        sl.copy_(b.seq_lens)
        qsl.copy_(b.query_start_loc)
        pl.copy_(torch.tensor(prefixes[i], dtype=torch.int32))
        sk.copy_(torch.from_numpy(sinks[i]))

    def call():
        pa.pa_forward_masked(q, kc, vc, bt, sl, qsl, batches[0].scale, pa.PA_MASK_PREFIX,
                             prefix_lens=pl, sinks=sk, out=out, workspace=ws, **kw)
        pa.pa_forward_chunked(q, kc, vc, bt, sl, qsl, batches[0].scale, C, num_chunks=S,
                              part_out=po, part_lse=plse, **kw)
        pa.pa_merge_lse(po, plse, out=cout)

    load(0)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, b in enumerate(batches):
            say("masked / chunked graph replay %d batch %d" % (rep, i))
            load(i)
            out.fill_(float("nan"))
            cout.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            g = out[:b.num_tokens].float().cpu().numpy()
            gc = cout[:b.num_tokens].float().cpu().numpy()
            ref, _ = oracle.attention(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                                      b.query_start_loc, b.scale, b.num_kv_heads,
                                      mask=oracle.MASK_PREFIX,
                                      prefix_lens=np.asarray(prefixes[i], np.int32), sinks=sinks[i])
            check_out(g, ref, torch.bfloat16, "graph masked batch %d" % i)
            cref, _ = oracle_forward(b)
            check_out(gc, cref, torch.bfloat16, "graph chunked batch %d" % i)


def test_sinks_llama_decode_full_size():
    # the headline decode batch (B 64, L~U[500,8192]) with sink logits
    b = workload.llama_decode(3)
    masked_parity(b, pa.PA_MASK_CAUSAL, None, "sinks llama decode full size", sinks=sink_logits(32, 4))


def test_validate_reports_bad_rows():
    b = workload.make_batch([1, 2], [10, 30], num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=17)
    g = b.to(DEV)
    dims = pa.make_dims(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.num_tokens,
                        max_seq_len=32, max_q_len=2)
    assert pa.pa_validate(g.block_table, g.seq_lens, g.query_start_loc, dims) == -1
    bad = g.block_table.clone()
    bad[1, 0] = b.num_pages + 5
    assert pa.pa_validate(bad, g.seq_lens, g.query_start_loc, dims) == 1
    sl = g.seq_lens.clone()
    sl[0] = 0  # shorter than its one new token
    assert pa.pa_validate(g.block_table, sl, g.query_start_loc, dims) == 0
