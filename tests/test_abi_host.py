"""Host-side tests of the C ABI (no GPU): the library loads, exports every
entry point include/pa.h declares, and rejects bad arguments on the host
before any HIP call; plus checks of the seeded input generator."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import paged_attention_kv_pa_amd as pa
from paged_attention_kv_pa_amd import binding, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"PA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    names = set(_declared())
    assert {"pa_forward", "pa_forward_masked", "pa_forward_chunked", "pa_decode_split",
            "pa_merge_lse", "mla_decode",
            "pa_workspace_size",
            "mla_workspace_size", "pa_validate", "pa_status_string", "pa_last_hip_error"} <= names


def test_library_loads_and_exports_every_declared_symbol():
    lib = ctypes.CDLL(pa.library_path())
    for name in _declared():
        assert hasattr(lib, name), name


def test_debug_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(binding._DEBUG_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_set_debug_switches_the_library():
    try:
        pa.set_debug(True)
        assert pa.library_path().endswith("libpa_debug.so")
        assert pa.library().pa_workspace_size(None) == 0
    finally:
        pa.set_debug(False)
    assert pa.library_path() == binding._RELEASE_PATH


def test_status_strings():
    for code in range(6):
        s = pa.pa_status_string(code)
        assert isinstance(s, str) and s and s != "unknown status"
    assert pa.pa_status_string(99) == "unknown status"


def _dims(**kw):
    d = binding.PaDims()
    base = dict(num_seqs=4, num_tokens=4, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                head_dim_v=128, page_size=16, num_pages=100, max_pages_per_seq=20,
                max_seq_len=320, max_q_len=1, dtype=binding.PA_BF16)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def _fwd(d, ws_bytes=1 << 40, q=FAKE, lse=None):
    lib = pa.library()
    return lib.pa_forward(q, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, lse, ctypes.byref(d), FAKE,
                          ws_bytes, None)


def test_workspace_size_host_function():
    assert pa.library().pa_workspace_size(None) == 0
    d = _dims()
    s1 = pa.pa_workspace_size(d)
    assert s1 > 0
    s2 = pa.pa_workspace_size(_dims(num_seqs=64, num_tokens=64))
    assert s2 > s1
    assert pa.pa_workspace_size(_dims(dtype=binding.PA_F32)) > 0
    assert pa.pa_workspace_size(_dims(num_q_heads=30)) == 0  # Hq % Hkv != 0


@pytest.mark.parametrize("field,value", [
    ("num_seqs", -1), ("num_q_heads", 0), ("num_kv_heads", 0), ("num_q_heads", 30),
    ("head_dim_qk", 0), ("page_size", 0), ("num_pages", 0), ("max_pages_per_seq", 0),
    ("dtype", 7), ("max_seq_len", 10 ** 6), ("max_q_len", 10 ** 6)])
def test_forward_rejects_bad_dims(field, value):
    assert _fwd(_dims(**{field: value})) == binding.PA_ERR_INVALID_ARG


def test_forward_rejects_null_pointers_and_dims():
    assert _fwd(_dims(), q=None) == binding.PA_ERR_INVALID_ARG
    lib = pa.library()
    assert lib.pa_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, None, FAKE, 1, None) \
        == binding.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(head_dim_qk=96, head_dim_v=96), dict(head_dim_v=64),
                                dict(head_dim_qk=192, head_dim_v=192),
                                dict(head_dim_qk=128, head_dim_v=192),
                                dict(page_size=12, max_pages_per_seq=30), dict(page_size=512, max_pages_per_seq=20),
                                dict(dtype=binding.PA_F32, head_dim_qk=512, head_dim_v=512)])
def test_forward_reports_unsupported(kw):
    assert _fwd(_dims(**kw)) == binding.PA_ERR_UNSUPPORTED


def test_forward_accepts_the_non_absorbed_mla_head_dims():
    # query / key 192 (128 + 64 rotary), value 128: supported in bf16; the call gets
    # past every host check (the workspace check is the last one)
    d = _dims(head_dim_qk=192, head_dim_v=128, num_q_heads=16, num_kv_heads=16)
    assert pa.pa_workspace_size(d) > 0
    assert _fwd(d, ws_bytes=0) == binding.PA_ERR_WORKSPACE


def test_forward_checks_workspace_before_launch():
    d = _dims()
    need = pa.pa_workspace_size(d)
    assert _fwd(d, ws_bytes=need - 1) == binding.PA_ERR_WORKSPACE
    lib = pa.library()
    assert lib.pa_forward(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, ctypes.byref(d),
                          None, need, None) == binding.PA_ERR_WORKSPACE


def test_empty_batch_is_a_no_op():
    assert _fwd(_dims(num_seqs=0, num_tokens=0)) == binding.PA_OK


def test_decode_split_argument_checks():
    lib = pa.library()
    d = _dims()
    call = lambda S, dd=d: lib.pa_decode_split(FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, S, FAKE, FAKE,
                                               ctypes.byref(dd), None)
    assert call(0) == binding.PA_ERR_INVALID_ARG
    assert call(257) == binding.PA_ERR_INVALID_ARG
    assert call(4, _dims(num_tokens=5)) == binding.PA_ERR_INVALID_ARG  # T != B
    assert call(4, _dims(head_dim_qk=80, head_dim_v=80)) == binding.PA_ERR_UNSUPPORTED
    assert call(4, _dims(num_seqs=0, num_tokens=0)) == binding.PA_OK
    # a bf16 partition is one work item of at most 256 rows: wider groups are refused
    assert call(4, _dims(num_q_heads=512, num_kv_heads=1)) == binding.PA_ERR_UNSUPPORTED
    assert call(4, _dims(num_q_heads=512, num_kv_heads=1, num_seqs=0, num_tokens=0)) == \
        binding.PA_ERR_UNSUPPORTED


def test_make_dims_takes_max_q_len_from_query_start_loc():
    # without max_q_len the binding reads the longest request off query_start_loc, so
    # a decode batch keeps the decode-only kernel (max_q_len * Hq / Hkv <= 16)
    b = workload.make_batch([1] * 6, [3000] * 6, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                            page_size=16, seed=5, poison=False)
    d = binding.make_dims(b.q, b.k_cache, b.v_cache, b.block_table, b.seq_lens, b.num_tokens,
                          query_start_loc=b.query_start_loc)
    assert d.max_q_len == 1
    m = workload.make_batch([1, 7, 0, 3], [20, 5, 9, 0], num_q_heads=8, num_kv_heads=2,
                            head_dim_qk=64, page_size=16, seed=6, poison=False)
    d = binding.make_dims(m.q, m.k_cache, m.v_cache, m.block_table, m.seq_lens, m.num_tokens,
                          query_start_loc=m.query_start_loc)
    assert d.max_q_len == 7
    d = binding.make_dims(m.q, m.k_cache, m.v_cache, m.block_table, m.seq_lens, m.num_tokens,
                          max_q_len=9, query_start_loc=m.query_start_loc)
    assert d.max_q_len == 9


def test_masked_forward_argument_checks():
    lib = pa.library()
    d = _dims()

    def call(mask, prefix, dd=d, slopes=None, alibi=0):
        return lib.pa_forward_masked(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, mask, prefix, None,
                                     slopes, alibi, 0.1, FAKE, None, ctypes.byref(dd), FAKE,
                                     1 << 40, None)
    bad = binding.PA_ERR_INVALID_ARG
    assert call(3, None) == bad and call(-1, None) == bad
    assert call(binding.PA_MASK_PREFIX, None) == bad   # prefix mask without prefix lengths
    assert call(binding.PA_MASK_FULL, FAKE) == bad     # prefix lengths with another mask
    assert call(binding.PA_MASK_CAUSAL, FAKE) == bad
    # ALiBi: a known mode with slopes, or neither; bf16 keys up to 128 wide
    assert call(binding.PA_MASK_CAUSAL, None, slopes=None, alibi=binding.PA_ALIBI_SQRT) == bad
    assert call(binding.PA_MASK_CAUSAL, None, slopes=FAKE, alibi=binding.PA_ALIBI_NONE) == bad
    assert call(binding.PA_MASK_CAUSAL, None, slopes=FAKE, alibi=3) == bad
    f2 = _dims(head_dim_qk=192, head_dim_v=128)
    assert call(binding.PA_MASK_CAUSAL, None, f2, slopes=FAKE, alibi=binding.PA_ALIBI_LINEAR) == \
        binding.PA_ERR_UNSUPPORTED
    empty = _dims(num_seqs=0, num_tokens=0)
    assert call(binding.PA_MASK_FULL, None, empty) == binding.PA_OK
    assert call(binding.PA_MASK_FULL, None, empty, slopes=FAKE, alibi=binding.PA_ALIBI_SQRT) == \
        binding.PA_OK
    assert call(binding.PA_MASK_PREFIX, FAKE, empty) == binding.PA_OK


def test_chunked_argument_checks():
    lib = pa.library()
    d = _dims(num_tokens=40, max_q_len=37)

    def call(C, S, dd=d, qsl=FAKE):
        return lib.pa_forward_chunked(FAKE, FAKE, FAKE, FAKE, FAKE, qsl, 0.1, C, S, FAKE, FAKE,
                                      binding.PA_MASK_CAUSAL, None, ctypes.byref(dd), None)
    bad = binding.PA_ERR_INVALID_ARG
    assert call(0, 8) == bad and call(32, 10) == bad and call(100, 4) == bad  # not a multiple of 64
    assert call(64, 0) == bad and call(64, 257) == bad
    assert call(64, 4) == bad  # 4 chunks of 64 keys do not cover max_seq_len = 320
    assert call(64, 5, qsl=None) == bad
    assert call(64, 5, _dims(num_tokens=40, max_q_len=37, dtype=binding.PA_F32)) == binding.PA_ERR_UNSUPPORTED
    assert call(64, 5, _dims(num_tokens=40, max_q_len=37, head_dim_qk=80, head_dim_v=80)) == \
        binding.PA_ERR_UNSUPPORTED
    dd = _dims(num_tokens=40, max_q_len=37)
    masked = lambda m, pfx: lib.pa_forward_chunked(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 64, 5,
                                                   FAKE, FAKE, m, pfx, ctypes.byref(dd), None)
    assert masked(3, None) == bad and masked(binding.PA_MASK_PREFIX, None) == bad
    assert masked(binding.PA_MASK_FULL, FAKE) == bad
    assert call(64, 5, _dims(num_seqs=0, num_tokens=0, max_q_len=0)) == binding.PA_OK
    assert call(64, 5, _dims(num_tokens=0, max_q_len=0)) == binding.PA_OK


def test_merge_argument_checks():
    lib = pa.library()
    m = lambda rows, S, Dv, dt: lib.pa_merge_lse(FAKE, FAKE, rows, S, Dv, FAKE, None, dt, None, 0,
                                                 None)
    assert m(-1, 4, 128, 1) == binding.PA_ERR_INVALID_ARG
    assert m(4, 0, 128, 1) == binding.PA_ERR_INVALID_ARG
    assert m(4, 300, 128, 1) == binding.PA_ERR_INVALID_ARG
    assert m(4, 4, 0, 1) == binding.PA_ERR_INVALID_ARG
    assert m(4, 4, 128, 5) == binding.PA_ERR_INVALID_ARG
    assert m(0, 4, 128, 1) == binding.PA_OK
    assert lib.pa_merge_lse(None, FAKE, 4, 4, 128, FAKE, None, 1, None, 0, None) == binding.PA_ERR_INVALID_ARG
    assert lib.pa_merge_lse(FAKE, FAKE, 4, 4, 128, FAKE, None, 1, FAKE, 0, None) == binding.PA_ERR_INVALID_ARG


def test_mla_argument_checks():
    lib = pa.library()
    base = dict(num_seqs=4, num_tokens=4, num_q_heads=128, num_kv_heads=1, head_dim_qk=576,
                head_dim_v=512, page_size=64, num_pages=100, max_pages_per_seq=20,
                max_seq_len=1280, max_q_len=1)

    def call(S=4, **kw):
        b = dict(base)
        b.update(kw)
        d = _dims(**b)
        return lib.mla_decode(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, S, ctypes.byref(d), FAKE,
                              1 << 40, None)

    assert call(head_dim_qk=512) == binding.PA_ERR_UNSUPPORTED
    assert call(num_kv_heads=2, num_q_heads=128) == binding.PA_ERR_UNSUPPORTED
    assert call(num_q_heads=120) == binding.PA_ERR_UNSUPPORTED
    assert call(num_q_heads=256) == binding.PA_ERR_UNSUPPORTED
    assert call(dtype=binding.PA_F32) == binding.PA_ERR_UNSUPPORTED
    assert call(num_tokens=5) == binding.PA_ERR_INVALID_ARG
    assert call(S=65) == binding.PA_ERR_INVALID_ARG
    assert call(num_seqs=0, num_tokens=0) == binding.PA_OK
    d = _dims(**base)
    assert pa.mla_workspace_size(d, 1) > 0
    assert pa.mla_workspace_size(d, 8) > pa.mla_workspace_size(d, 2)
    assert lib.mla_decode(FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, 8, ctypes.byref(d), FAKE,
                          16, None) == binding.PA_ERR_WORKSPACE


# ---- seeded input generator -------------------------------------------------

def test_generator_is_deterministic_and_pages_are_exclusive():
    a = workload.llama_decode(3, batch=6, hi=900)
    b = workload.llama_decode(3, batch=6, hi=900)
    assert torch.equal(a.block_table, b.block_table) and torch.equal(a.seq_lens, b.seq_lens)
    assert torch.equal(a.q.view(torch.int16), b.q.view(torch.int16))
    used = []
    for i, L in enumerate(a.seq_lens_list):
        n = (L + a.page_size - 1) // a.page_size
        used += a.block_table[i, :n].tolist()
    assert len(used) == len(set(used))  # no physical page serves two requests
    spare = sorted(set(range(a.num_pages)) - set(used))
    assert spare, "at least one poison page"
    assert torch.isnan(a.k_cache[spare].float()).all() and torch.isnan(a.v_cache[spare].float()).all()
    for i, L in enumerate(a.seq_lens_list):  # unused table entries point at poison
        n = (L + a.page_size - 1) // a.page_size
        assert set(a.block_table[i, n:].tolist()) <= set(spare)


def test_generator_poisons_tail_slots_only():
    b = workload.make_batch([1, 3], [20, 0], num_q_heads=4, num_kv_heads=2, head_dim_qk=64,
                            page_size=16, seed=3)
    for i, L in enumerate(b.seq_lens_list):
        n = (L + 15) // 16
        last = int(b.block_table[i, n - 1])
        tail = L % 16
        kc = b.k_cache[last].float()
        vc = b.v_cache[last].float()
        assert not torch.isnan(kc[:, :tail or 16]).any()
        assert not torch.isnan(vc[:, :, :tail or 16]).any()
        if tail:
            assert torch.isnan(kc[:, tail:]).all() and torch.isnan(vc[:, :, tail:]).all()
    assert not torch.isnan(b.q.float()).any()


def test_workload_shapes():
    c = workload.tiny_f32_decode(0)
    assert c.q.dtype == torch.float32 and c.num_pages == 128 and c.num_seqs == 4
    assert all(1 <= L <= 300 for L in c.seq_lens_list)
    m = workload.qwen3_mixed(0, n_decode=3, n_extend=2, n_prefill=2, dec=(20, 40), ext_q=(3, 5),
                             ext_c=(10, 20), pre_q=(5, 9))
    assert m.q_lens[:3] == [1, 1, 1] and all(c == 0 for c in m.ctx_lens[-2:])
    assert int(m.query_start_loc[-1]) == m.num_tokens == m.q.shape[0]
    d = workload.deepseek_mla(0, batch=2, lo=70, hi=90)
    assert d.k_cache is d.v_cache and d.k_cache.shape[1:] == (64, 576)


def test_standard_alibi_slopes():
    # the geometric slopes published with ALiBi: 8 heads 1/2 .. 1/256, 16 heads
    # 2^-0.5 .. 2^-8, and for 12 heads the 8-head slopes then 2^-0.5, 2^-1.5, 2^-2.5, 2^-3.5
    assert workload.alibi_slopes(8) == [2.0 ** -k for k in range(1, 9)]
    assert workload.alibi_slopes(16) == [2.0 ** (-0.5 * k) for k in range(1, 17)]
    assert workload.alibi_slopes(12) == [2.0 ** -k for k in range(1, 9)] + \
        [2.0 ** -0.5, 2.0 ** -1.5, 2.0 ** -2.5, 2.0 ** -3.5]
    assert workload.alibi_slopes(1) == [2.0 ** -8]
