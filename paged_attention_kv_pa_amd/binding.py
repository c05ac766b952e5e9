"""ctypes binding of libpa.so (declared in include/pa.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; shapes and dtypes are read off the tensors to fill the
`pa_dims` descriptor; every computation happens in the library's kernels.
The library is loaded on first call; if it is missing or cannot be loaded
the call raises (no CPU or PyTorch fallback exists).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the same library (a sanitizer build of
# the host code, for instance) to load in place of the in-tree libpa.so.
_RELEASE_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_PKG, "libpa.so")
_DEBUG_PATH = os.path.join(_PKG, "libpa_debug.so")
_LIB_PATH = _RELEASE_PATH

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_DEVICE_DATA = range(6)
PA_F32, PA_BF16 = 0, 1


class PaDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "num_tokens", "num_q_heads", "num_kv_heads", "head_dim_qk", "head_dim_v",
        "page_size", "num_pages", "max_pages_per_seq", "max_seq_len", "max_q_len", "dtype")]


class PaError(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = "%s: %s" % (where, pa_status_string(status))
        if status == PA_ERR_HIP:
            msg += " (hipError_t %d)" % hip_error
        super().__init__(msg)


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB_PATH


def set_debug(enabled: bool) -> None:
    """Send later calls to libpa_debug.so (the PA_DEBUG build: block-table
    entries outside the page pool are reported as PA_ERR_DEVICE_DATA) or back
    to libpa.so."""
    global _lib, _LIB_PATH
    with _lock:
        path = _DEBUG_PATH if enabled else _RELEASE_PATH
        if path != _LIB_PATH:
            _LIB_PATH, _lib = path, None


def library():
    """Load the selected library (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError("%s is not built (run paged_attention_kv_pa_amd.build.build())"
                                   % os.path.basename(_LIB_PATH))
            lib = ctypes.CDLL(_LIB_PATH)
            p, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
            dp = ctypes.POINTER(PaDims)
            lib.pa_workspace_size.argtypes = [dp]
            lib.pa_workspace_size.restype = sz
            lib.pa_forward.argtypes = [p, p, p, p, p, p, f32, p, p, dp, p, sz, p]
            lib.pa_forward.restype = i32
            lib.pa_forward_masked.argtypes = [p, p, p, p, p, p, i32, p, p, p, i32, f32, p, p, dp, p,
                                              sz, p]
            lib.pa_forward_masked.restype = i32
            lib.pa_forward_noalloc.argtypes = [p, p, p, p, p, p, f32, p, p, dp, p]
            lib.pa_forward_noalloc.restype = i32
            lib.pa_noalloc_max_workspace.argtypes = []
            lib.pa_noalloc_max_workspace.restype = sz
            lib.pa_decode_split.argtypes = [p, p, p, p, p, f32, i32, p, p, dp, p]
            lib.pa_decode_split.restype = i32
            lib.pa_forward_chunked.argtypes = [p, p, p, p, p, p, f32, i32, i32, p, p, i32, p, dp, p]
            lib.pa_forward_chunked.restype = i32
            lib.pa_merge_lse.argtypes = [p, p, i32, i32, i32, p, p, i32, p, i32, p]
            lib.pa_merge_lse.restype = i32
            lib.mla_workspace_size.argtypes = [dp, i32]
            lib.mla_workspace_size.restype = sz
            lib.mla_decode.argtypes = [p, p, p, p, f32, p, p, i32, dp, p, sz, p]
            lib.mla_decode.restype = i32
            lib.pa_validate.argtypes = [p, p, p, dp, ctypes.POINTER(i32), p]
            lib.pa_validate.restype = i32
            lib.pa_status_string.argtypes = [i32]
            lib.pa_status_string.restype = ctypes.c_char_p
            lib.pa_set_kernel_events.argtypes = [p, p]
            lib.pa_set_kernel_events.restype = i32
            lib.pa_last_hip_error.argtypes = []
            lib.pa_last_hip_error.restype = i32
            _lib = lib
    return _lib


def pa_status_string(status: int) -> str:
    return library().pa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != PA_OK:
        raise PaError(status, where, library().pa_last_hip_error() if status == PA_ERR_HIP else 0)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


# pa_forward leaves its work-queue state in the first bytes of its workspace
# for the next call on it; a workspace that is new (or was written by others
# since) makes the call take a fixed item order instead, which balances worse.
# Calls that pass no workspace therefore share one per (device, stream),
# grown when a call needs more.  Work on one stream is ordered, so calls on it
# never use the shared workspace at the same time.  Calls made while a graph is
# being captured get a workspace of their own, which the graph keeps.
_ws_cache = {}


def _shared_workspace(device, need, stream):
    if torch.cuda.is_current_stream_capturing():
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    key = (device.index, _stream(device, stream).value)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_F32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t.dtype)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def make_dims(q, k_cache, v_cache, block_table, seq_lens, num_tokens, *, layout="mha",
              head_dim_v=None, max_seq_len=None, max_q_len=None, query_start_loc=None) -> PaDims:
    """Fill a pa_dims from tensor shapes and host-side capacities.

    max_seq_len defaults to the block-table capacity (max_pages * P).  max_q_len
    defaults to the longest request of query_start_loc when that is given (one
    small device-to-host copy of the B + 1 offsets, which waits for the stream),
    else to num_tokens.  The default matters for speed: a batch whose requests
    all decode (max_q_len * Hq / Hkv <= 16) runs the decode-only kernel, which
    an over-estimated max_q_len would turn off.
    """
    B = int(seq_lens.shape[0])
    Hq, Dqk = int(q.shape[1]), int(q.shape[2])
    if layout == "mla":
        num_pages, P = int(k_cache.shape[0]), int(k_cache.shape[1])
        Hkv = 1
        Dv = 512 if head_dim_v is None else int(head_dim_v)
    else:
        num_pages, Hkv, P = int(k_cache.shape[0]), int(k_cache.shape[1]), int(k_cache.shape[2])
        Dv = int(v_cache.shape[2])
    maxp = int(block_table.shape[1])
    d = PaDims()
    d.num_seqs = B
    d.num_tokens = int(num_tokens)
    d.num_q_heads = Hq
    d.num_kv_heads = Hkv
    d.head_dim_qk = Dqk
    d.head_dim_v = Dv
    d.page_size = P
    d.num_pages = num_pages
    d.max_pages_per_seq = maxp
    d.max_seq_len = int(max_seq_len) if max_seq_len is not None else maxp * P
    if max_q_len is not None:
        d.max_q_len = int(max_q_len)
    elif query_start_loc is not None and int(query_start_loc.shape[0]) > 1:
        qs = query_start_loc.detach().to("cpu", torch.int64)
        d.max_q_len = max(0, int((qs[1:] - qs[:-1]).max()))
    else:
        d.max_q_len = min(int(num_tokens), d.max_seq_len)
    d.dtype = _dtype_code(q)
    return d


def _check_common(q, k_cache, v_cache, block_table, seq_lens):
    dev = q.device
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        _need(t.device == dev, "%s is on %s, q on %s" % (name, t.device, dev))
        _need(t.is_contiguous(), "%s must be contiguous" % name)
    _need(dev.type == "cuda", "tensors must be on a GPU")
    _need(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32,
          "block_table and seq_lens must be int32")
    _need(k_cache.dtype == q.dtype and v_cache.dtype == q.dtype, "q and caches must share a dtype")


def pa_workspace_size(dims: PaDims) -> int:
    return int(library().pa_workspace_size(ctypes.byref(dims)))


def mla_workspace_size(dims: PaDims, num_splits: int = 0) -> int:
    return int(library().mla_workspace_size(ctypes.byref(dims), int(num_splits)))


PA_MASK_CAUSAL, PA_MASK_FULL, PA_MASK_PREFIX = 0, 1, 2
PA_ALIBI_NONE, PA_ALIBI_LINEAR, PA_ALIBI_SQRT = 0, 1, 2


def pa_forward(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, out=None,
               lse=None, workspace=None, max_seq_len=None, max_q_len=None, stream=None):
    """Paged causal attention over a varlen batch (see pa_forward in include/pa.h).

    q [T, Hq, D]; k_cache [pages, Hkv, P, D]; v_cache [pages, Hkv, D, P];
    block_table int32 [B, max_pages]; seq_lens int32 [B]; query_start_loc int32 [B+1].
    Returns out ([T, Hq, D], allocated if not given).  Without `workspace`, calls on one
    (device, stream) share a workspace the binding keeps (see _shared_workspace).
    """
    return _forward(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, out, lse,
                    workspace, max_seq_len, max_q_len, stream, None, None, None, None, 0)


def pa_forward_masked(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, mask,
                      prefix_lens=None, sinks=None, out=None, lse=None, workspace=None,
                      max_seq_len=None, max_q_len=None, stream=None, alibi_slopes=None,
                      alibi_mode=None):
    """pa_forward with mask PA_MASK_CAUSAL, PA_MASK_FULL or PA_MASK_PREFIX (prefix_lens
    int32 [B] on the device for the last), optional sink logits (float32 [Hq] on the
    device) and an optional ALiBi bias (alibi_slopes float32 [Hq] on the device;
    alibi_mode PA_ALIBI_LINEAR or PA_ALIBI_SQRT, default PA_ALIBI_SQRT when slopes are
    given); see pa_forward_masked in include/pa.h."""
    for name, t in (("sinks", sinks), ("alibi_slopes", alibi_slopes)):
        if t is not None:
            _need(t.dtype == torch.float32 and t.is_contiguous() and t.device == q.device
                  and tuple(t.shape) == (int(q.shape[1]),), "%s must be contiguous float32 [Hq]" % name)
    if alibi_mode is None:
        alibi_mode = PA_ALIBI_NONE if alibi_slopes is None else PA_ALIBI_SQRT
    if prefix_lens is not None:
        _need(prefix_lens.dtype == torch.int32 and prefix_lens.is_contiguous()
              and prefix_lens.device == q.device and tuple(prefix_lens.shape) == (int(seq_lens.shape[0]),),
              "prefix_lens must be contiguous int32 [B] on q's device")
    return _forward(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, out, lse,
                    workspace, max_seq_len, max_q_len, stream, int(mask), prefix_lens, sinks,
                    alibi_slopes, int(alibi_mode))


def _forward(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, out, lse,
             workspace, max_seq_len, max_q_len, stream, mask, prefix_lens, sinks, alibi_slopes,
             alibi_mode):
    _check_common(q, k_cache, v_cache, block_table, seq_lens)
    _need(query_start_loc.dtype == torch.int32 and query_start_loc.is_contiguous()
          and query_start_loc.device == q.device, "query_start_loc must be contiguous int32 on q's device")
    _need(q.dim() == 3 and k_cache.dim() == 4 and v_cache.dim() == 4, "bad tensor ranks")
    _need(query_start_loc.shape[0] == seq_lens.shape[0] + 1, "query_start_loc must have B + 1 entries")
    T = int(q.shape[0])
    dims = make_dims(q, k_cache, v_cache, block_table, seq_lens, T, max_seq_len=max_seq_len,
                     max_q_len=max_q_len, query_start_loc=query_start_loc)
    if out is None:
        out = torch.empty(T, dims.num_q_heads, dims.head_dim_v, dtype=q.dtype, device=q.device)
    _need(out.is_contiguous() and out.dtype == q.dtype and out.shape == (T, dims.num_q_heads, dims.head_dim_v),
          "bad out tensor")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (T, dims.num_q_heads),
              "bad lse tensor")
    need = pa_workspace_size(dims)
    if workspace is None:
        workspace = _shared_workspace(q.device, need, stream)
    nbytes = workspace.numel() * workspace.element_size()
    if mask is None:
        st = library().pa_forward(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                  _ptr(seq_lens), _ptr(query_start_loc), float(scale), _ptr(out),
                                  _ptr(lse), ctypes.byref(dims), _ptr(workspace), nbytes,
                                  _stream(q.device, stream))
        _check(st, "pa_forward")
    else:
        st = library().pa_forward_masked(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                         _ptr(seq_lens), _ptr(query_start_loc), mask,
                                         _ptr(prefix_lens), _ptr(sinks), _ptr(alibi_slopes),
                                         alibi_mode, float(scale), _ptr(out), _ptr(lse),
                                         ctypes.byref(dims), _ptr(workspace), nbytes,
                                         _stream(q.device, stream))
        _check(st, "pa_forward_masked")
    return out


def pa_forward_noalloc(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale, out,
                       lse=None, max_seq_len=None, max_q_len=None, stream=None):
    """pa_forward on the library's own per-GPU workspace (see pa_forward_noalloc in
    include/pa.h): nothing is allocated, so `out` must be given."""
    _check_common(q, k_cache, v_cache, block_table, seq_lens)
    _need(query_start_loc.dtype == torch.int32 and query_start_loc.is_contiguous()
          and query_start_loc.device == q.device, "query_start_loc must be contiguous int32 on q's device")
    _need(q.dim() == 3 and k_cache.dim() == 4 and v_cache.dim() == 4, "bad tensor ranks")
    _need(query_start_loc.shape[0] == seq_lens.shape[0] + 1, "query_start_loc must have B + 1 entries")
    T = int(q.shape[0])
    dims = make_dims(q, k_cache, v_cache, block_table, seq_lens, T, max_seq_len=max_seq_len,
                     max_q_len=max_q_len, query_start_loc=query_start_loc)
    _need(out is not None and out.is_contiguous() and out.dtype == q.dtype
          and tuple(out.shape) == (T, dims.num_q_heads, dims.head_dim_v), "bad out tensor")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.is_contiguous() and lse.shape == (T, dims.num_q_heads),
              "bad lse tensor")
    st = library().pa_forward_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(query_start_loc), float(scale),
                                      _ptr(out), _ptr(lse), ctypes.byref(dims),
                                      _stream(q.device, stream))
    _check(st, "pa_forward_noalloc")
    return out


def pa_noalloc_max_workspace() -> int:
    return int(library().pa_noalloc_max_workspace())


def pa_decode_split(q, k_cache, v_cache, block_table, seq_lens, scale, num_splits, part_out=None,
                    part_lse=None, max_seq_len=None, stream=None):
    """Split-KV decode partials (see pa_decode_split in include/pa.h).

    q [B, Hq, D].  Returns (part_out [B, Hq, S, D] fp32, part_lse [B, Hq, S] fp32).
    """
    _check_common(q, k_cache, v_cache, block_table, seq_lens)
    B = int(seq_lens.shape[0])
    _need(q.dim() == 3 and q.shape[0] == B, "q must be [B, Hq, D]")
    dims = make_dims(q, k_cache, v_cache, block_table, seq_lens, B, max_seq_len=max_seq_len,
                     max_q_len=1)
    S = int(num_splits)
    shape = (B, dims.num_q_heads, S, dims.head_dim_v)
    if part_out is None:
        part_out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty(shape[:3], dtype=torch.float32, device=q.device)
    _need(part_out.shape == shape and part_out.dtype == torch.float32 and part_out.is_contiguous(),
          "bad part_out")
    _need(part_lse.shape == shape[:3] and part_lse.dtype == torch.float32 and part_lse.is_contiguous(),
          "bad part_lse")
    st = library().pa_decode_split(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                   _ptr(seq_lens), float(scale), S, _ptr(part_out),
                                   _ptr(part_lse), ctypes.byref(dims), _stream(q.device, stream))
    _check(st, "pa_decode_split")
    return part_out, part_lse


def pa_forward_chunked(q, k_cache, v_cache, block_table, seq_lens, query_start_loc, scale,
                       chunk_keys, num_chunks=None, part_out=None, part_lse=None, max_seq_len=None,
                       max_q_len=None, stream=None, mask=PA_MASK_CAUSAL, prefix_lens=None):
    """Chunked-context partials (see pa_forward_chunked in include/pa.h).

    num_chunks defaults to ceil(max_seq_len / chunk_keys).  Returns
    (part_out [T, Hq, S, D] fp32, part_lse [T, Hq, S] fp32); pa_merge_lse of the pair
    gives pa_forward's output.
    """
    _check_common(q, k_cache, v_cache, block_table, seq_lens)
    _need(query_start_loc.dtype == torch.int32 and query_start_loc.is_contiguous()
          and query_start_loc.device == q.device, "query_start_loc must be contiguous int32 on q's device")
    _need(q.dim() == 3 and k_cache.dim() == 4 and v_cache.dim() == 4, "bad tensor ranks")
    _need(query_start_loc.shape[0] == seq_lens.shape[0] + 1, "query_start_loc must have B + 1 entries")
    T = int(q.shape[0])
    dims = make_dims(q, k_cache, v_cache, block_table, seq_lens, T, max_seq_len=max_seq_len,
                     max_q_len=max_q_len, query_start_loc=query_start_loc)
    C = int(chunk_keys)
    S = (dims.max_seq_len + C - 1) // C if num_chunks is None else int(num_chunks)
    S = max(S, 1)
    shape = (T, dims.num_q_heads, S, dims.head_dim_v)
    if part_out is None:
        part_out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty(shape[:3], dtype=torch.float32, device=q.device)
    _need(tuple(part_out.shape) == shape and part_out.dtype == torch.float32 and part_out.is_contiguous(),
          "bad part_out")
    _need(tuple(part_lse.shape) == shape[:3] and part_lse.dtype == torch.float32 and part_lse.is_contiguous(),
          "bad part_lse")
    st = library().pa_forward_chunked(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                      _ptr(seq_lens), _ptr(query_start_loc), float(scale), C, S,
                                      _ptr(part_out), _ptr(part_lse), int(mask), _ptr(prefix_lens),
                                      ctypes.byref(dims), _stream(q.device, stream))
    _check(st, "pa_forward_chunked")
    return part_out, part_lse


def pa_merge_lse(part_out, part_lse, out=None, lse=None, out_dtype=torch.bfloat16, stream=None,
                 sinks=None):
    """Log-sum-exp merge of partials over the split axis (see pa_merge_lse in include/pa.h).

    part_out [..., S, Dv] fp32, part_lse [..., S] fp32 -> out [..., Dv] in out_dtype.
    """
    _need(part_out.dtype == torch.float32 and part_lse.dtype == torch.float32, "partials must be fp32")
    _need(part_out.is_contiguous() and part_lse.is_contiguous(), "partials must be contiguous")
    _need(part_out.shape[:-1] == part_lse.shape, "part_out / part_lse shapes disagree")
    lead = tuple(part_lse.shape[:-1])
    S, Dv = int(part_out.shape[-2]), int(part_out.shape[-1])
    rows = 1
    for x in lead:
        rows *= int(x)
    if out is None:
        out = torch.empty(lead + (Dv,), dtype=out_dtype, device=part_out.device)
    _need(out.is_contiguous() and tuple(out.shape) == lead + (Dv,), "bad out")
    code = _dtype_code(out)
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == lead, "bad lse")
    Hq = 0
    if sinks is not None:
        _need(part_lse.dim() >= 2, "sinks need partials shaped [..., Hq, S]")
        Hq = int(part_lse.shape[-2])
        _need(sinks.dtype == torch.float32 and sinks.is_contiguous() and tuple(sinks.shape) == (Hq,)
              and sinks.device == part_out.device, "sinks must be contiguous float32 [Hq]")
    st = library().pa_merge_lse(_ptr(part_out), _ptr(part_lse), rows, S, Dv, _ptr(out), _ptr(lse),
                                code, _ptr(sinks), Hq, _stream(part_out.device, stream))
    _check(st, "pa_merge_lse")
    return out


def mla_decode(q, kv_cache, block_table, seq_lens, scale, out=None, lse=None, num_splits=0,
               workspace=None, max_seq_len=None, stream=None):
    """Absorbed MLA decode (see mla_decode in include/pa.h).

    q [B, Hq, 576] bf16; kv_cache [pages, P, 576] bf16 -> out [B, Hq, 512] bf16.
    """
    _check_common(q, kv_cache, kv_cache, block_table, seq_lens)
    B = int(seq_lens.shape[0])
    _need(q.dim() == 3 and q.shape[0] == B and kv_cache.dim() == 3, "bad tensor ranks")
    dims = make_dims(q, kv_cache, kv_cache, block_table, seq_lens, B, layout="mla",
                     max_seq_len=max_seq_len, max_q_len=1)
    if out is None:
        out = torch.empty(B, dims.num_q_heads, 512, dtype=q.dtype, device=q.device)
    _need(out.is_contiguous() and tuple(out.shape) == (B, dims.num_q_heads, 512), "bad out")
    if lse is not None:
        _need(lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (B, dims.num_q_heads),
              "bad lse")
    need = mla_workspace_size(dims, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = library().mla_decode(_ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(seq_lens),
                              float(scale), _ptr(out), _ptr(lse), int(num_splits),
                              ctypes.byref(dims), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _stream(q.device, stream))
    _check(st, "mla_decode")
    return out


def pa_validate(block_table, seq_lens, query_start_loc, dims: PaDims, stream=None):
    """Synchronous check of the index arrays; returns -1 if valid, else the first bad request."""
    bad = ctypes.c_int32(-1)
    st = library().pa_validate(_ptr(block_table), _ptr(seq_lens), _ptr(query_start_loc),
                               ctypes.byref(dims), ctypes.byref(bad),
                               _stream(block_table.device, stream))
    if st == PA_ERR_DEVICE_DATA:
        return int(bad.value)
    _check(st, "pa_validate")
    return -1
