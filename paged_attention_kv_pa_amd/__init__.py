"""MI355X (gfx950) paged-attention engine.

Every step of the computation runs in the HIP kernels of ``libpa.so``; the
Python layer (``binding``) only marshals torch device tensors into the C ABI
declared in ``include/pa.h``.  Functions carry the names of the C entry
points.  The library is loaded on first use and a missing or unloadable
library raises — there is no fallback.
"""
from .binding import (PA_ALIBI_LINEAR, PA_ALIBI_NONE, PA_ALIBI_SQRT, PA_MASK_CAUSAL, PA_MASK_FULL,
                      PA_MASK_PREFIX, PaError, pa_decode_split,
                      pa_forward, pa_forward_chunked, pa_forward_masked, pa_forward_noalloc,
                      pa_merge_lse, pa_noalloc_max_workspace,
                      pa_status_string,
                      pa_validate, pa_workspace_size, mla_decode, mla_workspace_size,
                      library, library_path, make_dims, set_debug)

__all__ = ["PaError", "pa_forward", "pa_forward_masked", "pa_forward_chunked", "pa_decode_split",
           "pa_forward_noalloc", "pa_noalloc_max_workspace",
           "pa_merge_lse", "PA_MASK_CAUSAL", "PA_MASK_FULL", "PA_MASK_PREFIX",
           "PA_ALIBI_NONE", "PA_ALIBI_LINEAR", "PA_ALIBI_SQRT",
           "mla_decode",
           "pa_workspace_size", "mla_workspace_size", "pa_validate", "pa_status_string",
           "library", "library_path", "make_dims", "set_debug"]
