"""Writes worked_examples.json: tiny paged-attention cases whose results are
derived by hand, in closed form, from the definition of attention (scores
s_t = scale * q . k_t, weights exp(s_t) / sum exp, lse = ln sum exp(s_t)).

The pages the method is taken from print no worked example, so these cases
are hand-made.  Nothing here calls the HIP library or the oracle: the
expected values are the closed forms below, evaluated with `math`.

Layouts: k_cache[page][kv_head][slot][dim], v_cache[page][kv_head][dim][slot].
Pool pages no request uses and slots past a sequence end hold 1000.0, which
would visibly change a result if an index mistake read them.
"""
import json
import math
import os

E = math.e
X = 1000.0


def three_token_prefill():
    # one request, 3 new tokens, nothing cached; keys k0=[0,0], k1=[1,0], k2=[2,0];
    # every query is [1,0] so the scores are 0, 1, 2 (scale 1); values
    # v0=[1,0], v1=[0,1], v2=[1,1].  Token j sees keys 0..j:
    #   j=0: out = v0,                               lse = 0
    #   j=1: out = (v0 + e v1) / (1 + e),            lse = ln(1 + e)
    #   j=2: out = (v0 + e v1 + e^2 v2)/(1+e+e^2),   lse = ln(1 + e + e^2)
    # page size 2: logical page 0 (tokens 0,1) -> physical 2, logical page 1
    # (token 2) -> physical 0; physical page 1 unused.
    k_cache = [[[[2, 0], [X, X]]], [[[X, X], [X, X]]], [[[0, 0], [1, 0]]]]
    v_cache = [[[[1, X], [1, X]]], [[[X, X], [X, X]]], [[[1, 0], [0, 1]]]]
    z1, z2 = 1 + E, 1 + E + E * E
    out = [[[1.0, 0.0]], [[1 / z1, E / z1]], [[(1 + E * E) / z2, (E + E * E) / z2]]]
    lse = [[0.0], [math.log(z1)], [math.log(z2)]]
    return dict(name="three_token_prefill", page_size=2, num_q_heads=1, num_kv_heads=1,
                scale=1.0, q=[[[1, 0]], [[1, 0]], [[1, 0]]], k_cache=k_cache,
                v_cache=v_cache, block_table=[[2, 0]], seq_lens=[3], query_start_loc=[0, 3],
                expected_out=out, expected_lse=lse)


def gqa_two_decodes():
    # two decode requests, 2 query heads on 1 KV head, head dim 2, value dim 1.
    # Request A: 2 keys kA=[0,0],[0,1], values 4, -2.
    #   head 0, q=[0,0]: scores 0,0 -> out = (4-2)/2 = 1,        lse = ln 2
    #   head 1, q=[0,2]: scores 0,2 -> out = (4-2e^2)/(1+e^2),   lse = ln(1+e^2)
    # Request B: 1 key [3,3], value 7 -> out = 7;
    #   head 0, q=[1,0]: lse = 3;  head 1, q=[0,-1]: lse = -3
    # A -> physical page 1, B -> physical page 2, page 0 unused.
    k_cache = [[[[X, X], [X, X]]], [[[0, 0], [0, 1]]], [[[3, 3], [X, X]]]]
    v_cache = [[[[X, X]]], [[[4, -2]]], [[[7, X]]]]
    out = [[[1.0], [(4 - 2 * E * E) / (1 + E * E)]], [[7.0], [7.0]]]
    lse = [[math.log(2.0), math.log(1 + E * E)], [3.0, -3.0]]
    return dict(name="gqa_two_decodes", page_size=2, num_q_heads=2, num_kv_heads=1,
                scale=1.0, q=[[[0, 0], [0, 2]], [[1, 0], [0, -1]]], k_cache=k_cache,
                v_cache=v_cache, block_table=[[1], [2]], seq_lens=[2, 1],
                query_start_loc=[0, 1, 2], expected_out=out, expected_lse=lse)


def alibi_extend(mode):
    # ALiBi reading: the logit of the key at position t for the query at position
    # p gets -m_h |p - t| (linear) or -m_h sqrt|p - t| (sqrt).  One request, 2 new
    # tokens on 1 cached key (positions 1 and 2), 2 query heads on 1 KV head with
    # slopes m = 0.5 and 1.0, every query 0 (so q . k = 0 and the weights are the
    # bias terms alone), values 8, 4, 2 (value dim 1).  Weights per visible key:
    #   token 0 (p = 1), keys 0, 1:    e^{-m d(1)}, 1         (d(1) = 1 both modes)
    #   token 1 (p = 2), keys 0, 1, 2: e^{-m d(2)}, e^{-m}, 1 (d(2) = 2 or sqrt 2)
    # out = sum w v / sum w, lse = ln sum w.  Page size 2: logical page 0 (tokens
    # 0, 1) -> physical 1, logical page 1 (token 2) -> physical 0.
    d2 = 2.0 if mode == "linear" else math.sqrt(2.0)
    vals = [8.0, 4.0, 2.0]
    out, lse = [], []
    for p, n in ((1, 2), (2, 3)):
        orow, lrow = [], []
        for m in (0.5, 1.0):
            w = [math.exp(-m * 1.0), 1.0] if p == 1 else [math.exp(-m * d2), math.exp(-m), 1.0]
            z = sum(w)
            orow.append([sum(wi * vi for wi, vi in zip(w, vals[:n])) / z])
            lrow.append(math.log(z))
        out.append(orow)
        lse.append(lrow)
    k_cache = [[[[5, 6], [X, X]]], [[[1, 2], [3, 4]]]]
    v_cache = [[[[2, X]]], [[[8, 4]]]]
    return dict(name="alibi_%s_extend_two_heads" % mode, page_size=2, num_q_heads=2,
                num_kv_heads=1, scale=1.0, q=[[[0, 0], [0, 0]], [[0, 0], [0, 0]]],
                k_cache=k_cache, v_cache=v_cache, block_table=[[1, 0]], seq_lens=[3],
                query_start_loc=[0, 2], alibi_mode=mode, alibi_slopes=[0.5, 1.0],
                expected_out=out, expected_lse=lse)


if __name__ == "__main__":
    doc = {"source": "hand-derived closed forms; the pages print no worked example",
           "examples": [three_token_prefill(), gqa_two_decodes(), alibi_extend("linear"),
                        alibi_extend("sqrt")]}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "worked_examples.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)
