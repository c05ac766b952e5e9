"""Seeded synthetic inputs for paged attention.

This module only draws random numbers and lays them out in the documented
cache layouts; it holds none of the attention arithmetic.  Both the HIP path
and the CPU oracle are fed from it (the oracle is never imported here).

Workload shapes follow the pages' workloads:
  * Llama-3.1-8B decode (32 query / 8 KV heads, head dim 128) at 500 input
    tokens — "vLLM Triton Attention Backend Deep Dive", section
    "Benchmarks and results";
  * Qwen3-235B MHA (64 / 4 heads, dim 128) and DeepSeek-R1 MLA (128 heads on
    one 576-wide latent, 512 of it the value) at 64 concurrent requests —
    "vLLM AMD ROCm Attention Backend Optimization", sections
    "Performance benchmarks" and "AITER MLA backend";
  * a mixed continuous batch ordered decode, extend, prefill — same page,
    sections "The challenge of mixed inference workloads" and "Batch
    reordering".

Recipe (all integers inclusive):
  * lengths are drawn with torch.randint on a CPU generator seeded with the
    case seed; physical pages are a random permutation of the pool drawn from
    the same generator; requests take pages from the permutation in order;
  * q and the caches are N(0, 1) drawn in fp32 and rounded to the storage
    dtype (round-to-nearest-even for bf16) on a generator of the target
    device seeded with seed + 1;
  * every pool page no request uses, every unused block-table entry (which
    points at such a page) and every slot of a last page past the sequence end
    is filled with NaN ("poison"), so an index mistake shows up as NaN.

Cache layouts (element at page p, slot s, KV head h, column d):
  key   k_cache[p, h, s, d]          shape [pages, Hkv, P, D]
  value v_cache[p, h, d, s]          shape [pages, Hkv, D, P]
  MLA   latent[p, s, d]              shape [pages, P, 576]; value = d < 512
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

BF16 = torch.bfloat16
F32 = torch.float32


@dataclasses.dataclass
class Batch:
    """One batch of paged-attention inputs (all tensors on `device`)."""
    q: torch.Tensor                 # [T, Hq, Dqk]
    k_cache: torch.Tensor           # MHA [pages, Hkv, P, Dqk]; MLA latent [pages, P, Dqk]
    v_cache: torch.Tensor           # MHA [pages, Hkv, Dv, P];  MLA: same tensor as k_cache
    block_table: torch.Tensor       # int32 [B, max_pages]
    seq_lens: torch.Tensor          # int32 [B]  total KV length incl. new tokens
    query_start_loc: torch.Tensor   # int32 [B + 1]
    scale: float
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    layout: str                     # "mha" or "mla"
    q_lens: List[int]
    ctx_lens: List[int]             # cached tokens before the new ones
    name: str = ""

    @property
    def num_seqs(self) -> int:
        return len(self.q_lens)

    @property
    def num_tokens(self) -> int:
        return int(sum(self.q_lens))

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def seq_lens_list(self) -> List[int]:
        return [c + q for c, q in zip(self.ctx_lens, self.q_lens)]

    @property
    def dtype(self) -> torch.dtype:
        return self.q.dtype

    def to(self, device) -> "Batch":
        f = lambda t: t.to(device)
        kc = f(self.k_cache)
        vc = kc if self.v_cache is self.k_cache else f(self.v_cache)
        return dataclasses.replace(self, q=f(self.q), k_cache=kc, v_cache=vc,
                                   block_table=f(self.block_table), seq_lens=f(self.seq_lens),
                                   query_start_loc=f(self.query_start_loc))


def _randn(shape, dtype, gen, device, chunk=1 << 26):
    """N(0, 1) drawn in fp32 in chunks, rounded to `dtype`."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, dtype=F32, device=device).to(dtype)
    return out


def make_batch(q_lens: Sequence[int], ctx_lens: Sequence[int], *, num_q_heads: int,
               num_kv_heads: int, head_dim_qk: int, head_dim_v: Optional[int] = None,
               page_size: int, dtype=BF16, layout: str = "mha", scale: Optional[float] = None,
               seed: int = 0, pool_pages: Optional[int] = None, spare_pages: int = 2,
               max_pages_per_seq: Optional[int] = None, poison: bool = True,
               device="cpu", name: str = "") -> Batch:
    """Build a batch for the given per-request new-token and cached-token counts."""
    q_lens = [int(x) for x in q_lens]
    ctx_lens = [int(x) for x in ctx_lens]
    assert len(q_lens) == len(ctx_lens)
    B = len(q_lens)
    Dqk = int(head_dim_qk)
    Dv = Dqk if head_dim_v is None else int(head_dim_v)
    P = int(page_size)
    Hq, Hkv = int(num_q_heads), int(num_kv_heads)
    if layout == "mla":
        assert Hkv == 1 and Dv <= Dqk
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    seq = [c + q for c, q in zip(ctx_lens, q_lens)]
    npg = [(L + P - 1) // P for L in seq]
    used = sum(npg)
    pool = used + spare_pages if pool_pages is None else int(pool_pages)
    assert pool >= used + (1 if poison else 0), "pool too small"
    maxp = max(npg + [1]) if max_pages_per_seq is None else int(max_pages_per_seq)
    assert maxp >= max(npg + [0])

    gcpu = torch.Generator(device="cpu").manual_seed(int(seed))
    perm = torch.randperm(pool, generator=gcpu).to(torch.int32)
    spare = perm[used:]
    filler = int(spare[0]) if spare.numel() else 0
    bt = torch.full((B, maxp), filler, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    qsl = torch.zeros(B + 1, dtype=torch.int32)
    qsl[1:] = torch.cumsum(torch.tensor(q_lens, dtype=torch.int64), 0).to(torch.int32)
    T = int(qsl[-1])

    gdev = torch.Generator(device=device).manual_seed(int(seed) + 1)
    q = _randn((T, Hq, Dqk), dtype, gdev, device)
    if layout == "mla":
        kc = _randn((pool, P, Dqk), dtype, gdev, device)
        vc = kc
    else:
        kc = _randn((pool, Hkv, P, Dqk), dtype, gdev, device)
        vc = _randn((pool, Hkv, Dv, P), dtype, gdev, device)

    if poison:
        nan = float("nan")
        if spare.numel():
            sp = spare.to(device=device, dtype=torch.int64)
            kc[sp] = nan
            if vc is not kc:
                vc[sp] = nan
        for b in range(B):
            tail = seq[b] % P
            if npg[b] and tail:
                last = int(bt[b, npg[b] - 1])
                if layout == "mla":
                    kc[last, tail:, :] = nan
                else:
                    kc[last, :, tail:, :] = nan
                    vc[last, :, :, tail:] = nan

    return Batch(q=q, k_cache=kc, v_cache=vc, block_table=bt.to(device),
                 seq_lens=torch.tensor(seq, dtype=torch.int32, device=device),
                 query_start_loc=qsl.to(device), scale=float(scale), num_q_heads=Hq,
                 num_kv_heads=Hkv, head_dim_qk=Dqk, head_dim_v=Dv, page_size=P,
                 layout=layout, q_lens=q_lens, ctx_lens=ctx_lens, name=name)


def sub_batch(b: Batch, requests: Sequence[int]) -> Batch:
    """The given consecutive requests of `b` as a batch of their own (same cache pool)."""
    r = list(requests)
    assert r == list(range(r[0], r[-1] + 1)), "requests must be consecutive"
    qsl = b.query_start_loc
    t0, t1 = int(qsl[r[0]]), int(qsl[r[-1] + 1])
    return dataclasses.replace(
        b, q=b.q[t0:t1], block_table=b.block_table[r[0]:r[-1] + 1].contiguous(),
        seq_lens=b.seq_lens[r[0]:r[-1] + 1].contiguous(),
        query_start_loc=(qsl[r[0]:r[-1] + 2] - t0).contiguous(),
        q_lens=b.q_lens[r[0]:r[-1] + 1], ctx_lens=b.ctx_lens[r[0]:r[-1] + 1],
        name=b.name + "[%d:%d]" % (r[0], r[-1] + 1))


def permute_requests(b: Batch, order: Sequence[int]) -> Batch:
    """The requests of `b` in the given order (same cache pool): request i of the
    result is request order[i] of `b`, with its query rows, block-table row and
    lengths.  Returns the batch and, as a LongTensor, the row of `b` each result
    token comes from."""
    order = [int(i) for i in order]
    assert sorted(order) == list(range(b.num_seqs)), "order must be a permutation"
    qsl = [int(x) for x in b.query_start_loc.cpu()]
    src = torch.tensor([t for i in order for t in range(qsl[i], qsl[i + 1])], dtype=torch.int64)
    q_lens = [b.q_lens[i] for i in order]
    new_qsl = torch.zeros(b.num_seqs + 1, dtype=torch.int32)
    new_qsl[1:] = torch.cumsum(torch.tensor(q_lens, dtype=torch.int64), 0).to(torch.int32)
    idx = torch.tensor(order, dtype=torch.int64, device=b.block_table.device)
    pb = dataclasses.replace(
        b, q=b.q[src.to(b.q.device)].contiguous(), block_table=b.block_table[idx].contiguous(),
        seq_lens=b.seq_lens[idx.to(b.seq_lens.device)].contiguous(),
        query_start_loc=new_qsl.to(b.query_start_loc.device), q_lens=q_lens,
        ctx_lens=[b.ctx_lens[i] for i in order], name=b.name + "[permuted]")
    return pb, src


def _randint(gen, lo, hi, n):
    """n integers uniform in [lo, hi] (inclusive)."""
    return [int(x) for x in torch.randint(int(lo), int(hi) + 1, (n,), generator=gen)]


def case_seed(config: int, case: int) -> int:
    return 1000 * int(config) + int(case)


# --------------------------------------------------------------------------
# The five workloads.  Each returns a Batch; `scale_down` shrinks lengths and
# batch for parity runs the oracle finishes in seconds (shapes of heads,
# head dims and page sizes are never changed).
# --------------------------------------------------------------------------

def tiny_f32_decode(case: int = 0, device="cpu") -> Batch:
    """4 sequences, L ~ U[1, 300], one new token each, 8/2 heads, dim 64, page 16,
    a 128-page pool in random order, fp32, scale 1/8."""
    seed = case_seed(1, case)
    g = torch.Generator().manual_seed(seed + 7)
    L = _randint(g, 1, 300, 4)
    return make_batch([1] * 4, [x - 1 for x in L], num_q_heads=8, num_kv_heads=2,
                      head_dim_qk=64, page_size=16, dtype=F32, scale=1.0 / 8.0, seed=seed,
                      pool_pages=128, device=device, name="tiny_f32_decode/%d" % case)


LLAMA_CASES = {0: (1, "fixed"), 1: (64, "fixed"), 2: (1, "uniform"), 3: (64, "uniform")}


def llama_decode(case: int = 3, device="cpu", batch: Optional[int] = None,
                 lo: int = 500, hi: int = 8192) -> Batch:
    """Llama-3.1-8B decode: 32/8 heads, dim 128, page 16, bf16, scale 1/sqrt(128).
    Cases: 0 = B1 L500, 1 = B64 L500, 2 = B1 L~U[500, 8192], 3 = B64 L~U[500, 8192]."""
    B, kind = LLAMA_CASES[case]
    if batch is not None:
        B = batch
    seed = case_seed(2, case)
    g = torch.Generator().manual_seed(seed + 7)
    L = [lo] * B if kind == "fixed" else _randint(g, lo, hi, B)
    return make_batch([1] * B, [x - 1 for x in L], num_q_heads=32, num_kv_heads=8,
                      head_dim_qk=128, page_size=16, dtype=BF16, seed=seed, device=device,
                      name="llama_decode/%d" % case)


def llama_long(batch: int = 1, case: int = 0, device="cpu", lengths: Optional[Sequence[int]] = None,
               lo: int = 32768, hi: int = 131072) -> Batch:
    """Long-context split-KV decode, Llama-3.1-8B heads, L ~ U[32K, 128K] (or given)."""
    seed = case_seed(3, case)
    g = torch.Generator().manual_seed(seed + 7)
    L = list(lengths) if lengths is not None else _randint(g, lo, hi, batch)
    return make_batch([1] * len(L), [x - 1 for x in L], num_q_heads=32, num_kv_heads=8,
                      head_dim_qk=128, page_size=16, dtype=BF16, seed=seed, device=device,
                      name="llama_long/%d" % case)


def llama_long_extend(case: int = 0, device="cpu", new_tokens: int = 256,
                      cached: int = 131072) -> Batch:
    """Long-context extend with Llama-3.1-8B heads: new_tokens new tokens on a cached
    context of `cached` tokens (one request), page 16, bf16."""
    return make_batch([new_tokens], [cached], num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                      page_size=16, dtype=BF16, seed=case_seed(3, 100 + case), device=device,
                      name="llama_long_extend/%d" % case)


def qwen3_mixed(case: int = 0, device="cpu", n_decode: int = 48, n_extend: int = 8,
                n_prefill: int = 8, dec=(1024, 16384), ext_q=(256, 2048),
                ext_c=(4096, 32768), pre_q=(512, 8192)) -> Batch:
    """Qwen3-235B mixed batch ordered [decode : extend : prefill]; 64/4 heads, dim 128,
    page 16, bf16, causal, scale 1/sqrt(128)."""
    seed = case_seed(4, case)
    g = torch.Generator().manual_seed(seed + 7)
    dL = _randint(g, dec[0], dec[1], n_decode)
    eq = _randint(g, ext_q[0], ext_q[1], n_extend)
    ec = _randint(g, ext_c[0], ext_c[1], n_extend)
    pq = _randint(g, pre_q[0], pre_q[1], n_prefill)
    q_lens = [1] * n_decode + eq + pq
    ctx = [x - 1 for x in dL] + ec + [0] * n_prefill
    return make_batch(q_lens, ctx, num_q_heads=64, num_kv_heads=4, head_dim_qk=128,
                      page_size=16, dtype=BF16, seed=seed, device=device,
                      name="qwen3_mixed/%d" % case)


def deepseek_mla(case: int = 0, device="cpu", batch: int = 64, lo: int = 1024,
                 hi: int = 32768) -> Batch:
    """DeepSeek-R1 absorbed MLA decode: 128 heads on one 576-wide latent (value = first
    512 columns), page 64, bf16, scale 1/sqrt(192), L ~ U[1K, 32K]."""
    seed = case_seed(5, case)
    g = torch.Generator().manual_seed(seed + 7)
    L = _randint(g, lo, hi, batch)
    return make_batch([1] * batch, [x - 1 for x in L], num_q_heads=128, num_kv_heads=1,
                      head_dim_qk=576, head_dim_v=512, page_size=64, dtype=BF16,
                      layout="mla", scale=1.0 / math.sqrt(192.0), seed=seed, device=device,
                      name="deepseek_mla/%d" % case)


def qwen3_mixed_with_long_extend(case: int = 0, device="cpu", new_tokens: int = 256,
                                 cached: int = 131072, **mix) -> Batch:
    """The Qwen3-235B mixed batch (keyword arguments as for qwen3_mixed) with one
    more extend request after it: `new_tokens` new tokens on `cached` cached
    ones (a context of at least 100K keys, which pa_forward cuts into key
    chunks inside the batch)."""
    base = qwen3_mixed(case, n_decode=mix.get("n_decode", 48), n_extend=mix.get("n_extend", 8),
                       n_prefill=mix.get("n_prefill", 8), dec=mix.get("dec", (1024, 16384)),
                       ext_q=mix.get("ext_q", (256, 2048)), ext_c=mix.get("ext_c", (4096, 32768)),
                       pre_q=mix.get("pre_q", (512, 8192)))
    return make_batch(base.q_lens + [new_tokens], base.ctx_lens + [cached], num_q_heads=64,
                      num_kv_heads=4, head_dim_qk=128, page_size=16, dtype=BF16,
                      seed=case_seed(4, 200 + case), device=device,
                      name="qwen3_mixed_with_long_extend/%d" % case)


def deepseek_mha_prefill(case: int = 0, device="cpu", n_extend: int = 8, n_prefill: int = 8,
                         ext_q=(256, 2048), ext_c=(4096, 32768), pre_q=(512, 8192),
                         heads: int = 128, page_size: int = 64) -> Batch:
    """DeepSeek-R1 MLA prefill / extend on the uncompressed representation
    ("Hybrid processing strategy": prefill and extend run non-absorbed, as MHA):
    `heads` query heads each with its own key / value head, query / key 192 wide
    (128 + 64 rotary), value 128 wide, page 64, bf16, scale 1/sqrt(192); requests
    ordered [extend : prefill] with the extend / prefill lengths of the Qwen3 mix."""
    seed = case_seed(6, case)
    g = torch.Generator().manual_seed(seed + 7)
    eq = _randint(g, ext_q[0], ext_q[1], n_extend)
    ec = _randint(g, ext_c[0], ext_c[1], n_extend)
    pq = _randint(g, pre_q[0], pre_q[1], n_prefill)
    return make_batch(eq + pq, ec + [0] * n_prefill, num_q_heads=heads, num_kv_heads=heads,
                      head_dim_qk=192, head_dim_v=128, page_size=page_size, dtype=BF16,
                      scale=1.0 / math.sqrt(192.0), seed=seed, device=device,
                      name="deepseek_mha_prefill/%d" % case)


def alibi_slopes(num_heads: int) -> List[float]:
    """The per-head ALiBi slopes published with ALiBi (Press et al., "Train Short,
    Test Long", 2022): for n a power of two, the geometric sequence
    2^(-8 (h + 1) / n), h = 0 .. n - 1; for other n, the n' = 2^floor(log2 n)
    slopes of n' heads followed by every other slope (the 1st, 3rd, ...) of the
    2 n' sequence, n - n' of them.  Inputs of the ALiBi calls (the kernels take
    any slopes)."""
    def pow2(n):
        return [2.0 ** (-8.0 * (h + 1) / n) for h in range(n)]
    n = int(num_heads)
    if n <= 0:
        return []
    base = 1 << (n.bit_length() - 1)
    if base == n:
        return pow2(n)
    return pow2(base) + pow2(2 * base)[0::2][:n - base]


def algorithmic_bytes(b: Batch) -> int:
    """Bytes a perfect kernel moves: each visible K/V element once (the MLA latent
    once), q, out, lse (fp32) and 4 bytes per used block-table entry."""
    es = b.q.element_size()
    keys = sum(b.seq_lens_list)
    if b.layout == "mla":
        kv = keys * b.head_dim_qk * es
    else:
        kv = keys * b.num_kv_heads * (b.head_dim_qk + b.head_dim_v) * es
    T = b.num_tokens
    qo = T * b.num_q_heads * (b.head_dim_qk + b.head_dim_v) * es + T * b.num_q_heads * 4
    tbl = sum((L + b.page_size - 1) // b.page_size for L in b.seq_lens_list) * 4
    return int(kv + qo + tbl)


def algorithmic_flops(b: Batch) -> int:
    """2 * Hq * (Dqk + Dv) flops per unmasked (query, key) pair."""
    pairs = sum(q * c + q * (q + 1) // 2 for q, c in zip(b.q_lens, b.ctx_lens))
    return int(2 * b.num_q_heads * (b.head_dim_qk + b.head_dim_v) * pairs)
