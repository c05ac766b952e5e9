"""fp64 CPU oracle for paged causal attention — TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark may import this package.  The product path (the HIP library and its
Python binding) never imports, links or runs anything here, and this package
imports nothing from the product.

The arithmetic lives in ``pa_oracle.c`` (plain C, fp64, OpenMP over
(request, KV head) pairs); this module builds it with gcc and marshals numpy
arrays through ctypes.  See ``pa_oracle.c`` for what is computed and which
passage of the pages each step follows.

Inputs are the exact bf16 / fp32 values of the device tensors: bf16 arrays are
passed as their raw 16-bit patterns (numpy ``uint16``) and widened exactly in
C.  Outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "libpa_oracle.so")

F32, BF16 = 0, 1
LAYOUT_MHA, LAYOUT_MLA = 0, 1
MASK_CAUSAL, MASK_FULL, MASK_PREFIX = 0, 1, 2
ALIBI_NONE, ALIBI_LINEAR, ALIBI_SQRT = 0, 1, 2
_ERRORS = {1: "invalid sizes", 2: "invalid request data (lengths or block table)",
           3: "out of memory"}

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile pa_oracle.c into libpa_oracle.so with gcc (-O2 -fopenmp)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            # PA_ORACLE_LIB: another build of pa_oracle.c (a sanitizer build, say)
            path = os.environ.get("PA_ORACLE_LIB")
            if not path:
                path = build(force=False)
            lib = ctypes.CDLL(path)
            p, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
            lib.orc_attention.argtypes = [p, p, p, i32, p, p, p] + [i32] * 9 + [f32, p, p, p, i32]
            lib.orc_attention.restype = i32
            lib.orc_attention_masked.argtypes = [p, p, p, i32, p, p, p] + [i32] * 9 + [f32, i32, p,
                                                                                     p, p, i32, p, p,
                                                                                     p, i32]
            lib.orc_attention_masked.restype = i32
            lib.orc_decode_split.argtypes = [p, p, p, i32, p, p] + [i32] * 9 + [f32, i32, p, p, i32]
            lib.orc_decode_split.restype = i32
            lib.orc_chunked_partials.argtypes = [p, p, p, i32, p, p, p] + [i32] * 9 + [f32, i32, i32,
                                                                                    p, p, i32]
            lib.orc_chunked_partials.restype = i32
            lib.orc_chunked_partials_masked.argtypes = ([p, p, p, i32, p, p, p] + [i32] * 9 +
                                                        [f32, i32, i32, i32, p, p, p, i32])
            lib.orc_chunked_partials_masked.restype = i32
            lib.orc_merge_lse.argtypes = [p, p, i32, i32, i32, p, p]
            lib.orc_merge_lse.restype = i32
            lib.orc_split_range.argtypes = [i32, i32, i32, i32, ctypes.POINTER(i32),
                                            ctypes.POINTER(i32)]
            lib.orc_split_range.restype = None
            lib.orc_max_threads.argtypes = []
            lib.orc_max_threads.restype = i32
            _lib = lib
    return _lib


def max_threads() -> int:
    """Number of OpenMP threads the oracle uses by default."""
    return int(_load().orc_max_threads())


def _raw(x):
    """Return (contiguous numpy array, dtype code) holding the exact input values."""
    try:
        import torch  # only for conversion of torch CPU tensors
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.view(torch.int16).numpy().view(np.uint16)), BF16
            if x.dtype == torch.float32:
                return np.ascontiguousarray(x.numpy()), F32
            if x.dtype == torch.int32:
                return np.ascontiguousarray(x.numpy()), None
            raise TypeError("unsupported tensor dtype %s" % x.dtype)
    except ImportError:
        pass
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), F32
    if x.dtype == np.int32:
        return np.ascontiguousarray(x), None
    raise TypeError("unsupported array dtype %s" % x.dtype)


def _i32(x):
    a, _ = _raw(x)
    if a.dtype != np.int32:
        raise TypeError("index arrays must be int32")
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _check(rc):
    if rc != 0:
        raise ValueError("oracle: " + _ERRORS.get(rc, "error %d" % rc))


def attention(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale,
              num_kv_heads, head_dim_v=None, layout=LAYOUT_MHA, rows=None,
              nthreads=None, mask=MASK_CAUSAL, prefix_lens=None, sinks=None,
              alibi_slopes=None, alibi_mode=ALIBI_NONE):
    """Paged attention over a varlen batch, in fp64: causal, or MASK_FULL / MASK_PREFIX
    (prefix_lens int32 [B]) as defined in pa_oracle.c; sinks: optional float32 [Hq]
    sink logits; alibi_mode ALIBI_LINEAR / ALIBI_SQRT with alibi_slopes float32 [Hq]:
    the ALiBi bias of pa_oracle.c.

    q: [T, Hq, Dqk]; k_cache / v_cache in the layouts of pa_oracle.c
    (for LAYOUT_MLA pass the latent cache as both); block_table [B, max_pages];
    seq_lens [B]; query_start_loc [B + 1]; rows: optional bool [T, Hq] mask of
    the rows to compute (others come back as NaN).
    Returns (out [T, Hq, Dv] float64, lse [T, Hq] float64).
    """
    lib = _load()
    qa, dt = _raw(q)
    ka, dk = _raw(k_cache)
    va, dv = _raw(v_cache)
    if not (dt == dk == dv) or dt is None:
        raise TypeError("q, k_cache and v_cache must share one float dtype")
    bt, sl, qs = _i32(block_table), _i32(seq_lens), _i32(query_start_loc)
    T, Hq, Dqk = qa.shape
    B = sl.shape[0]
    if qs.shape[0] != B + 1 or bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("inconsistent batch arrays")
    Dv = Dqk if head_dim_v is None else int(head_dim_v)
    if layout == LAYOUT_MHA:
        num_pages, P = ka.shape[0], ka.shape[2]
    else:
        num_pages, P = ka.shape[0], ka.shape[1]
    out = np.full((T, Hq, Dv), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64)
    sel = None
    if rows is not None:
        sel = np.ascontiguousarray(np.asarray(rows, dtype=np.uint8).reshape(T, Hq))
    nt = max_threads() if nthreads is None else int(nthreads)
    if mask == MASK_CAUSAL and prefix_lens is None and sinks is None and alibi_mode == ALIBI_NONE:
        rc = lib.orc_attention(_ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(bt), _ptr(sl), _ptr(qs),
                               B, Hq, int(num_kv_heads), Dqk, Dv, P, num_pages, bt.shape[1],
                               layout, float(scale), _ptr(sel), _ptr(out), _ptr(lse), nt)
    else:
        pfx = None
        if prefix_lens is not None:
            pfx = _i32(prefix_lens)
            if pfx.shape != (B,):
                raise ValueError("prefix_lens must have B entries")
        snk = None
        if sinks is not None:
            snk = np.ascontiguousarray(np.asarray(sinks, dtype=np.float32))
            if snk.shape != (Hq,):
                raise ValueError("sinks must have Hq entries")
        slp = None
        if alibi_mode != ALIBI_NONE:
            slp = np.ascontiguousarray(np.asarray(alibi_slopes, dtype=np.float32))
            if slp.shape != (Hq,):
                raise ValueError("alibi_slopes must have Hq entries")
        rc = lib.orc_attention_masked(_ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(bt), _ptr(sl),
                                      _ptr(qs), B, Hq, int(num_kv_heads), Dqk, Dv, P, num_pages,
                                      bt.shape[1], layout, float(scale), int(mask), _ptr(pfx),
                                      _ptr(snk), _ptr(slp), int(alibi_mode), _ptr(sel),
                                      _ptr(out), _ptr(lse), nt)
    _check(rc)
    return out, lse


def decode_split(q, k_cache, v_cache, block_table, seq_lens, scale, num_splits,
                 num_kv_heads, head_dim_v=None, layout=LAYOUT_MHA, nthreads=None):
    """Split-KV decode partials (one query token per request), in fp64.

    Returns (part_out [B, Hq, S, Dv], part_lse [B, Hq, S]).
    """
    lib = _load()
    qa, dt = _raw(q)
    ka, dk = _raw(k_cache)
    va, dv = _raw(v_cache)
    if not (dt == dk == dv) or dt is None:
        raise TypeError("q, k_cache and v_cache must share one float dtype")
    bt, sl = _i32(block_table), _i32(seq_lens)
    B, Hq, Dqk = qa.shape
    Dv = Dqk if head_dim_v is None else int(head_dim_v)
    num_pages, P = (ka.shape[0], ka.shape[2]) if layout == LAYOUT_MHA else (ka.shape[0], ka.shape[1])
    S = int(num_splits)
    po = np.zeros((B, Hq, S, Dv), dtype=np.float64)
    pl = np.zeros((B, Hq, S), dtype=np.float64)
    nt = max_threads() if nthreads is None else int(nthreads)
    rc = lib.orc_decode_split(_ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(bt), _ptr(sl), B, Hq,
                              int(num_kv_heads), Dqk, Dv, P, num_pages, bt.shape[1], layout,
                              float(scale), S, _ptr(po), _ptr(pl), nt)
    _check(rc)
    return po, pl


def chunked_partials(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale,
                     chunk_keys, num_chunks, num_kv_heads, head_dim_v=None, layout=LAYOUT_MHA,
                     nthreads=None, mask=MASK_CAUSAL, prefix_lens=None):
    """Chunked-context partials of a varlen batch, in fp64 (see orc_chunked_partials).

    Chunk s covers keys [s C, (s + 1) C) of every request; each row gets the partial
    over the keys of the chunk it sees (zeros and -inf when there are none).
    Returns (part_out [T, Hq, S, Dv], part_lse [T, Hq, S]).
    """
    lib = _load()
    qa, dt = _raw(q)
    ka, dk = _raw(k_cache)
    va, dv = _raw(v_cache)
    if not (dt == dk == dv) or dt is None:
        raise TypeError("q, k_cache and v_cache must share one float dtype")
    bt, sl, qs = _i32(block_table), _i32(seq_lens), _i32(query_start_loc)
    T, Hq, Dqk = qa.shape
    B = sl.shape[0]
    if qs.shape[0] != B + 1 or bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("inconsistent batch arrays")
    Dv = Dqk if head_dim_v is None else int(head_dim_v)
    num_pages, P = (ka.shape[0], ka.shape[2]) if layout == LAYOUT_MHA else (ka.shape[0], ka.shape[1])
    S = int(num_chunks)
    po = np.full((T, Hq, S, Dv), np.nan, dtype=np.float64)
    pl = np.full((T, Hq, S), np.nan, dtype=np.float64)
    nt = max_threads() if nthreads is None else int(nthreads)
    if mask == MASK_CAUSAL and prefix_lens is None:
        rc = lib.orc_chunked_partials(_ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(bt), _ptr(sl),
                                      _ptr(qs), B, Hq, int(num_kv_heads), Dqk, Dv, P, num_pages,
                                      bt.shape[1], layout, float(scale), int(chunk_keys), S,
                                      _ptr(po), _ptr(pl), nt)
    else:
        pfx = None if prefix_lens is None else _i32(prefix_lens)
        rc = lib.orc_chunked_partials_masked(_ptr(qa), _ptr(ka), _ptr(va), dt, _ptr(bt), _ptr(sl),
                                             _ptr(qs), B, Hq, int(num_kv_heads), Dqk, Dv, P,
                                             num_pages, bt.shape[1], layout, float(scale),
                                             int(chunk_keys), S, int(mask), _ptr(pfx), _ptr(po),
                                             _ptr(pl), nt)
    _check(rc)
    return po, pl


def merge_lse(part_out, part_lse):
    """Log-sum-exp merge over the split axis.

    part_out [..., S, Dv], part_lse [..., S] (float64) -> (out [..., Dv], lse [...]).
    """
    lib = _load()
    po = np.ascontiguousarray(np.asarray(part_out, dtype=np.float64))
    pl = np.ascontiguousarray(np.asarray(part_lse, dtype=np.float64))
    lead = pl.shape[:-1]
    S, Dv = po.shape[-2], po.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    out = np.zeros(lead + (Dv,), dtype=np.float64)
    lse = np.zeros(lead, dtype=np.float64)
    _check(lib.orc_merge_lse(_ptr(po), _ptr(pl), rows, S, Dv, _ptr(out), _ptr(lse)))
    return out, lse


def split_range(L, P, S, s):
    """Key range [t0, t1) of partition s of S for a sequence of L keys."""
    a, b = ctypes.c_int(), ctypes.c_int()
    _load().orc_split_range(int(L), int(P), int(S), int(s), ctypes.byref(a), ctypes.byref(b))
    return a.value, b.value
