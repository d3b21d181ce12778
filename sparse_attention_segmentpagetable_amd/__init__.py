"""SegPagedAttention on AMD MI355X (gfx950).

A KV cache paged per (layer, KV head, segment) -- global heads keep the whole
context, local heads only their sink and recent window, retrieval heads a given
token set -- and mask-free prefill/decode kernels that read each head's own
pages. The compute path is libsegpaged.so (HIP, gfx950); this package is its
ctypes binding.
"""
from .segpaged import (DENSE, GLOBAL, LIB_PATH, LOCAL, NOALLOC_SCRATCH_BYTES, RETRIEVAL, Plan,
                       SegPagedError, Sizes, Stats, append, build, decode, decode_noalloc,
                       export_pages, import_pages, library, prefill, select_topp, stream_elems)

__all__ = ["Plan", "build", "append", "prefill", "decode", "decode_noalloc", "select_topp",
           "export_pages", "NOALLOC_SCRATCH_BYTES",
           "import_pages", "stream_elems", "library", "SegPagedError", "Sizes", "Stats",
           "GLOBAL", "LOCAL", "RETRIEVAL", "DENSE", "LIB_PATH"]
