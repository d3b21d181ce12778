"""Thin binding of libsegpaged_probe.so (include/segpaged_probe.h): the rate
probes used to report achieved rates against what gfx950 sustains. Argument
marshalling only; measurement support, not part of the attention path."""
from __future__ import annotations

import ctypes
import os

from .segpaged import SegPagedError, _ptr, _stream

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_PKG, "lib", "libsegpaged_probe.so")
SEED_ELEMS = 32768  # bf16 operands the MFMA probe reads
_LIB = None


def library():
    global _LIB
    if _LIB is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        lib.segpaged_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.c_void_p, ctypes.c_void_p]
        lib.segpaged_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        _LIB = lib
    return _LIB


def mfma_bf16(seed, iters: int, workgroups: int, out, stream=None):
    """segpaged_probe_mfma_bf16: workgroups * 8 * iters * 8 * 32768 flops."""
    import torch
    if seed.numel() < SEED_ELEMS or out.numel() < workgroups * 512:
        raise ValueError("seed needs 32768 bf16, out workgroups * 512 fp32")
    rc = library().segpaged_probe_mfma_bf16(_ptr(seed, "seed", torch.bfloat16), iters, workgroups,
                                            _ptr(out, "out", torch.float32), _stream(stream))
    if rc != 0:
        raise SegPagedError(rc, "segpaged_probe_mfma_bf16")


def hbm_read(src, workgroups: int, out, depth: int = 8, stream=None):
    """segpaged_probe_hbm_read over all of src (read as fp32), `depth` loads in
    flight per thread."""
    import torch
    if out.numel() < workgroups:
        raise ValueError("out needs workgroups fp32")
    nbytes = src.numel() * src.element_size()
    rc = library().segpaged_probe_hbm_read(_ptr(src, "src"), nbytes, workgroups, depth,
                                           _ptr(out, "out", torch.float32), _stream(stream))
    if rc != 0:
        raise SegPagedError(rc, "segpaged_probe_hbm_read")
