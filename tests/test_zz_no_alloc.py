"""pa_forward_noalloc (the entry point for callers that cannot allocate) against
pa_forward on the same inputs, through the C ABI: two calls in a row, the
second on a smaller batch, each bit for bit equal to pa_forward's output and
log-sum-exp, and within the parity tolerances of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_attention_kv_pa_amd as pa
from paged_attention_kv_pa_amd import workload
from pa_testutil import errors, finite_lse_err

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def both(b):
    g = b.to(DEV)
    T, Hq = b.num_tokens, b.num_q_heads
    kw = dict(max_seq_len=max(b.seq_lens_list), max_q_len=max(b.q_lens))
    out_a = torch.full((T, Hq, b.head_dim_v), float("nan"), dtype=b.dtype, device=DEV)
    lse_a = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=DEV)
    out_b, lse_b = torch.empty_like(out_a).fill_(float("nan")), torch.empty_like(lse_a).fill_(float("nan"))
    print("case %s: B=%d T=%d" % (b.name, b.num_seqs, T), flush=True)
    pa.pa_forward_noalloc(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                          g.query_start_loc, b.scale, out_a, lse=lse_a, **kw)
    pa.pa_forward(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, g.query_start_loc,
                  b.scale, out=out_b, lse=lse_b, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "outputs differ"
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32)), "lse differ"
    ref, rlse = oracle.attention(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens,
                                 b.query_start_loc, b.scale, b.num_kv_heads)
    mx, rel = errors(out_a.float().cpu().numpy(), ref)
    assert mx <= 2e-2 and rel <= 5e-3, (mx, rel)
    assert finite_lse_err(lse_a.cpu().numpy(), rlse) <= 1e-3


def test_noalloc_matches_pa_forward_on_two_calls():
    # a full-size Llama-3.1-8B decode batch, then a smaller mixed batch
    both(workload.llama_decode(3))
    both(workload.make_batch([1, 37, 130, 1, 2], [300, 0, 90, 2000, 40], num_q_heads=32,
                             num_kv_heads=8, head_dim_qk=128, page_size=16, seed=808,
                             name="small mixed"))


def test_noalloc_refuses_calls_beyond_its_workspace():
    # 1024 decode requests on 8 KV heads: room for pa_forward's split partials
    # of that many (request, KV head) pairs is about 100 MB, more than the
    # library's 64 MiB array
    n = 1024
    b = workload.make_batch([1] * n, [47] * n, num_q_heads=32, num_kv_heads=8,
                            head_dim_qk=128, page_size=16, seed=7, name="noalloc_big")
    g = b.to(DEV)
    dims = pa.make_dims(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens, b.num_tokens,
                        max_seq_len=48, max_q_len=1)
    assert pa.pa_workspace_size(dims) > pa.pa_noalloc_max_workspace()
    out = torch.empty(b.num_tokens, b.num_q_heads, b.head_dim_v, dtype=b.dtype, device=DEV)
    with pytest.raises(pa.PaError) as e:
        pa.pa_forward_noalloc(g.q, g.k_cache, g.v_cache, g.block_table, g.seq_lens,
                              g.query_start_loc, b.scale, out, max_seq_len=48, max_q_len=1)
    assert e.value.status == pa.binding.PA_ERR_WORKSPACE
