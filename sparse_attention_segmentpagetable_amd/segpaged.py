"""Thin Python binding of libsegpaged.so (include/segpaged.h): argument
marshalling only. Every step of the hot path runs in the library's HIP kernels;
there is no Python or CPU fallback. torch supplies device memory and streams.

The entry points keep the C names: Plan (segpaged_plan_create / _sizes /
_table_host / _stats / _destroy), build, prefill, decode.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# SEGPAGED_LIB names another build of the same C ABI (e.g. the host planner built
# with address and undefined-behaviour sanitizers); entry points it lacks raise
# when called
LIB_PATH = os.environ.get("SEGPAGED_LIB") or os.path.join(_PKG, "lib", "libsegpaged.so")

GLOBAL, LOCAL, RETRIEVAL, DENSE = 0, 1, 2, 3
STATUS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "ENOSPACE", -4: "EHIP", -5: "ESTATE"}

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


class SegPagedError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_lib().segpaged_status_str(status).decode()})")


class _Spec(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("seq_len", _i32p), ("first_query_pos", _i32p), ("kind", _i32p),
                ("sink", _i32p), ("window", _i32p), ("retr_offsets", _i64p),
                ("retr_pos", _i32p), ("free_list", _i32p), ("free_list_len", ctypes.c_int64),
                ("capacity_pages", ctypes.c_int64), ("decode_split_tokens", ctypes.c_int32),
                ("append_capacity", ctypes.c_int32),
                ("append_chunk", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("doc_group", _i32p), ("doc_len", _i32p)]


class Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_pages", "pool_pages", "pool_bytes", "table_int32s", "table_len", "num_units",
        "q_rows", "kv_rows", "decode_items", "prefill_items", "decode_workspace_bytes",
        "prefill_workspace_bytes", "select_workspace_bytes")]

    def as_dict(self) -> Dict[str, int]:
        return {n: getattr(self, n) for n, _ in self._fields_}


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "units", "pages", "retained_tokens", "decode_tokens", "prefill_pairs", "q_rows",
        "decode_items", "prefill_items")]

    def as_dict(self) -> Dict[str, int]:
        return {n: getattr(self, n) for n, _ in self._fields_}


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        sigs = {
            "segpaged_plan_create": ([ctypes.POINTER(_Spec), ctypes.POINTER(vp),
                                      ctypes.POINTER(Sizes)], ctypes.c_int),
            "segpaged_plan_destroy": ([vp], None),
            "segpaged_plan_sizes": ([vp, ctypes.POINTER(Sizes)], ctypes.c_int),
            "segpaged_plan_table_host": ([vp, _i32p, ctypes.c_int64], ctypes.c_int),
            "segpaged_plan_stats": ([vp, ctypes.c_int32, ctypes.POINTER(Stats)], ctypes.c_int),
            "segpaged_plan_append": ([vp, _i32p], ctypes.c_int),
            "segpaged_build": ([vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "segpaged_export_pages": ([vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "segpaged_import_pages": ([vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "segpaged_select_topp": ([vp, ctypes.c_int32, vp, vp, vp, ctypes.c_float,
                                      ctypes.c_float, vp, vp, vp, ctypes.c_int64, vp],
                                     ctypes.c_int),
            "segpaged_append": ([vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "segpaged_prefill": ([vp, ctypes.c_int32, vp, vp, vp, vp, ctypes.c_float,
                                  vp, vp, vp, ctypes.c_int64, vp], ctypes.c_int),
            "segpaged_decode": ([vp, ctypes.c_int32, vp, vp, vp, vp, ctypes.c_float,
                                 vp, vp, vp, ctypes.c_int64, vp], ctypes.c_int),
            "segpaged_decode_noalloc": ([vp, ctypes.c_int32, vp, vp, vp, vp, ctypes.c_float,
                                         vp, vp, vp], ctypes.c_int),
            "segpaged_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "segpaged_version": ([], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(lib, name, None)
            if fn is None:  # a partial build: calling this entry point raises
                continue
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def _check(rc: int, where: str):
    if rc != 0:
        raise SegPagedError(rc, where)


def _arr32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


class Plan:
    """segpaged_plan: SegmentPageTable plan and work lists (host only).

    Accepts any object with the attributes of workloads.Spec (num_layers,
    num_q_heads, num_kv_heads, head_dim, page_size, seq_len, first_query_pos,
    kind, sink, window, retrieval {(b, l, h): positions}, free_list,
    capacity_pages)."""

    def __init__(self, spec, decode_split_tokens: int = 0, append_capacity: int = 0,
                 append_chunk: int = 0):
        B, L, Hkv = len(spec.seq_len), spec.num_layers, spec.num_kv_heads
        self.num_seqs, self.num_layers = B, L
        self.num_q_heads, self.num_kv_heads = spec.num_q_heads, Hkv
        self.head_dim, self.page_size = spec.head_dim, spec.page_size
        self.append_capacity = append_capacity
        keep = {}
        keep["seq_len"] = _arr32(spec.seq_len)
        keep["q0"] = _arr32(spec.first_query_pos)
        keep["kind"] = _arr32(spec.kind)
        keep["sink"] = _arr32(spec.sink)
        keep["window"] = _arr32(spec.window)
        retr = getattr(spec, "retrieval", None) or {}
        offs = ptr_offs = ptr_pos = None
        if retr:
            U = L * B * Hkv
            counts = np.zeros(U + 1, dtype=np.int64)
            chunks = []
            for l in range(L):
                for b in range(B):
                    for h in range(Hkv):
                        u = (l * B + b) * Hkv + h
                        r = retr.get((b, l, h))
                        if r is not None:
                            counts[u + 1] = len(r)
                            chunks.append(_arr32(r))
            keep["retr_offsets"] = np.cumsum(counts).astype(np.int64)
            keep["retr_pos"] = np.concatenate(chunks) if chunks else np.zeros(1, np.int32)
            if len(keep["retr_pos"]) == 0:
                keep["retr_pos"] = np.zeros(1, np.int32)
            ptr_offs = keep["retr_offsets"].ctypes.data_as(_i64p)
            ptr_pos = keep["retr_pos"].ctypes.data_as(_i32p)
        fl = getattr(spec, "free_list", None)
        ptr_free, fl_len = None, 0
        if fl is not None:
            keep["free"] = _arr32(fl)
            ptr_free, fl_len = keep["free"].ctypes.data_as(_i32p), len(keep["free"])
        dg, dl = getattr(spec, "doc_group", None), getattr(spec, "doc_len", None)
        ptr_dg = ptr_dl = None
        if dg is not None:
            keep["doc_group"] = _arr32(dg)
            ptr_dg = keep["doc_group"].ctypes.data_as(_i32p)
        if dl is not None:
            keep["doc_len"] = _arr32(dl)
            ptr_dl = keep["doc_len"].ctypes.data_as(_i32p)
        c = _Spec(num_seqs=B, num_layers=L, num_q_heads=spec.num_q_heads, num_kv_heads=Hkv,
                  head_dim=spec.head_dim, page_size=spec.page_size,
                  seq_len=keep["seq_len"].ctypes.data_as(_i32p),
                  first_query_pos=keep["q0"].ctypes.data_as(_i32p),
                  kind=keep["kind"].ctypes.data_as(_i32p),
                  sink=keep["sink"].ctypes.data_as(_i32p),
                  window=keep["window"].ctypes.data_as(_i32p),
                  retr_offsets=ptr_offs, retr_pos=ptr_pos, free_list=ptr_free,
                  free_list_len=fl_len, capacity_pages=int(getattr(spec, "capacity_pages", 0) or 0),
                  decode_split_tokens=decode_split_tokens, append_capacity=append_capacity,
                  append_chunk=append_chunk, reserved=0, doc_group=ptr_dg, doc_len=ptr_dl)
        self._h = ctypes.c_void_p()
        self.sizes = Sizes()
        _check(_lib().segpaged_plan_create(ctypes.byref(c), ctypes.byref(self._h),
                                           ctypes.byref(self.sizes)), "segpaged_plan_create")

    @property
    def handle(self):
        return self._h

    def table_host(self) -> np.ndarray:
        out = np.zeros(self.sizes.table_int32s, dtype=np.int32)
        _check(_lib().segpaged_plan_table_host(self._h, out.ctypes.data_as(_i32p), len(out)),
               "segpaged_plan_table_host")
        return out

    def append(self, n_new: Sequence[int]):
        """segpaged_plan_append: every sequence b gains n_new[b] tokens (host only);
        then segpaged_append writes their K/V, layer by layer or all at once."""
        a = _arr32(n_new)
        if len(a) != self.num_seqs:
            raise ValueError("n_new needs one count per sequence")
        _check(_lib().segpaged_plan_append(self._h, a.ctypes.data_as(_i32p)), "segpaged_plan_append")
        self.t_new = int(a.sum())
        _check(_lib().segpaged_plan_sizes(self._h, ctypes.byref(self.sizes)), "segpaged_plan_sizes")

    def stats(self, layer: int = -1) -> Dict[str, int]:
        st = Stats()
        _check(_lib().segpaged_plan_stats(self._h, layer, ctypes.byref(st)), "segpaged_plan_stats")
        return st.as_dict()

    def close(self):
        if self._h:
            _lib().segpaged_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- device buffers (torch only allocates; the library fills them) ----
    def allocate(self, device="cuda", workspace: bool = True):
        """Caller-owned device buffers sized from the plan: table int32, the K and V
        pools (bf16 [pool_pages, P*D]) and the decode workspace (fp32)."""
        import torch
        z = self.sizes
        ppd = self.page_size * self.head_dim
        out = {
            "table": torch.empty(z.table_int32s, dtype=torch.int32, device=device),
            "k_pool": torch.zeros(z.pool_pages, ppd, dtype=torch.bfloat16, device=device),
            "v_pool": torch.zeros(z.pool_pages, ppd, dtype=torch.bfloat16, device=device),
        }
        if workspace:
            out["workspace"] = torch.empty(max(z.decode_workspace_bytes // 4, 4),
                                           dtype=torch.float32, device=device)
        return out


def _ptr(t, name, dtype=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, numel, name):
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


def _pools(plan: Plan, k_pool, v_pool):
    """Both pools bf16 and of the plan's size (NULL allowed when the plan has no pages)."""
    import torch
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        if t is None:
            if plan.sizes.pool_pages > 0:
                raise ValueError(f"{nm} is needed: the plan has {plan.sizes.pool_pages} pages")
            continue
        _ptr(t, nm, torch.bfloat16)
        _need(t, plan.sizes.pool_bytes // 2, nm)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def build(plan: Plan, layer: int, k_dense, v_dense, table, k_pool, v_pool, stream=None):
    """segpaged_build: upload the table slice and scatter dense K/V of `layer`
    (all layers when -1) into the page pools."""
    import torch
    z = plan.sizes
    nl = plan.num_layers if layer < 0 else 1
    dense = nl * z.kv_rows * plan.num_kv_heads * plan.head_dim
    for t, nm in ((k_dense, "k_dense"), (v_dense, "v_dense")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, dense, nm)
    _ptr(table, "table", torch.int32)
    _need(table, z.table_int32s, "table")
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, z.pool_bytes // 2, nm)
    _check(_lib().segpaged_build(plan.handle, layer, _ptr(k_dense, "k"), _ptr(v_dense, "v"),
                                 _ptr(table, "table"), _ptr(k_pool, "kp"), _ptr(v_pool, "vp"),
                                 _stream(stream)), "segpaged_build")


def stream_elems(plan: Plan, layer: int) -> int:
    """bf16 elements per tensor of the page stream of `layer` (all layers when -1)."""
    return plan.stats(layer)["pages"] * plan.page_size * plan.head_dim


def export_pages(plan: Plan, layer: int, table, k_pool, v_pool, k_out, v_out, stream=None):
    """segpaged_export_pages: the pages of `layer` as one stream per tensor."""
    import torch
    z = plan.sizes
    n = stream_elems(plan, layer)
    _ptr(table, "table", torch.int32)
    _need(table, z.table_int32s, "table")
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, z.pool_bytes // 2, nm)
    for t, nm in ((k_out, "k_out"), (v_out, "v_out")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, n, nm)
    _check(_lib().segpaged_export_pages(plan.handle, layer, _ptr(table, "table"),
                                        _ptr(k_pool, "kp"), _ptr(v_pool, "vp"),
                                        _ptr(k_out, "ko"), _ptr(v_out, "vo"), _stream(stream)),
           "segpaged_export_pages")


def import_pages(plan: Plan, layer: int, k_in, v_in, table, k_pool, v_pool, stream=None):
    """segpaged_import_pages: upload the table slice of `layer`, then write the
    streamed pages into this plan's pages."""
    import torch
    z = plan.sizes
    n = stream_elems(plan, layer)
    for t, nm in ((k_in, "k_in"), (v_in, "v_in")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, n, nm)
    _ptr(table, "table", torch.int32)
    _need(table, z.table_int32s, "table")
    for t, nm in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, z.pool_bytes // 2, nm)
    _check(_lib().segpaged_import_pages(plan.handle, layer, _ptr(k_in, "ki"), _ptr(v_in, "vi"),
                                        _ptr(table, "table"), _ptr(k_pool, "kp"),
                                        _ptr(v_pool, "vp"), _stream(stream)),
           "segpaged_import_pages")


def prefill(plan: Plan, layer: int, q, table, k_pool, v_pool, scale: float, o, lse=None,
            workspace=None, stream=None):
    """segpaged_prefill: O (and LSE) for rows q0_b..N_b-1 of every sequence."""
    import torch
    z = plan.sizes
    nl = plan.num_layers if layer < 0 else 1
    rows = nl * z.q_rows * plan.num_q_heads
    for t, nm in ((q, "q"), (o, "o")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, rows * plan.head_dim, nm)
    if lse is not None:
        _ptr(lse, "lse", torch.float32)
        _need(lse, rows, "lse")
    _ptr(table, "table", torch.int32)
    _need(table, z.table_int32s, "table")
    _pools(plan, k_pool, v_pool)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().segpaged_prefill(plan.handle, layer, _ptr(q, "q"), _ptr(table, "t"),
                                   _ptr(k_pool, "kp", torch.bfloat16),
                                   _ptr(v_pool, "vp", torch.bfloat16), float(scale),
                                   _ptr(o, "o"), _ptr(lse, "lse"), _ptr(workspace, "ws"), wsb,
                                   _stream(stream)), "segpaged_prefill")


def append(plan: Plan, layer: int, k_new, v_new, table, k_pool, v_pool, stream=None):
    """segpaged_append: K/V of the tokens the last Plan.append added (bf16
    [T_new][Hkv][D], [L][T_new][Hkv][D] when layer = -1) into their pages."""
    import torch
    t_new = getattr(plan, "t_new", 0)
    nl = plan.num_layers if layer < 0 else 1
    if t_new > 0:
        for t, nm in ((k_new, "k_new"), (v_new, "v_new")):
            _ptr(t, nm, torch.bfloat16)
            _need(t, nl * t_new * plan.num_kv_heads * plan.head_dim, nm)
    _ptr(table, "table", torch.int32)
    _need(table, plan.sizes.table_int32s, "table")
    _pools(plan, k_pool, v_pool)
    _check(_lib().segpaged_append(plan.handle, layer, _ptr(k_new, "k_new"), _ptr(v_new, "v_new"),
                                  _ptr(table, "t"), _ptr(k_pool, "kp", torch.bfloat16),
                                  _ptr(v_pool, "vp", torch.bfloat16), _stream(stream)),
           "segpaged_append")


def select_topp(plan: Plan, layer: int, q, k_dense, table, scale: float, p: float, out_pos,
                out_cnt, workspace, stream=None):
    """segpaged_select_topp: the top-p retrieval set of every (sequence, retrieval
    head) of `layer` from the decode row's attention over the dense history.
    out_pos int32 [Hkv][T_total], out_cnt int32 [B * Hkv]."""
    import torch
    _ptr(q, "q", torch.bfloat16)
    _need(q, plan.num_seqs * plan.num_q_heads * plan.head_dim, "q")
    _ptr(k_dense, "k_dense", torch.bfloat16)
    _need(k_dense, plan.sizes.kv_rows * plan.num_kv_heads * plan.head_dim, "k_dense")
    _ptr(out_pos, "out_pos", torch.int32)
    _need(out_pos, plan.num_kv_heads * plan.sizes.kv_rows, "out_pos")
    _ptr(out_cnt, "out_cnt", torch.int32)
    _need(out_cnt, plan.num_seqs * plan.num_kv_heads, "out_cnt")
    wsb = workspace.numel() * workspace.element_size()
    _check(_lib().segpaged_select_topp(plan.handle, layer, _ptr(q, "q"), _ptr(k_dense, "k_dense"),
                                       _ptr(table, "t", torch.int32), float(scale), float(p),
                                       _ptr(out_pos, "out_pos"), _ptr(out_cnt, "out_cnt"),
                                       _ptr(workspace, "ws"), wsb, _stream(stream)),
           "segpaged_select_topp")


def decode(plan: Plan, layer: int, q, table, k_pool, v_pool, scale: float, o, lse=None,
           workspace=None, stream=None):
    """segpaged_decode: O (and LSE) of the query at position N_b - 1 of each sequence."""
    import torch
    nl = plan.num_layers if layer < 0 else 1
    rows = nl * plan.num_seqs * plan.num_q_heads
    for t, nm in ((q, "q"), (o, "o")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, rows * plan.head_dim, nm)
    if lse is not None:
        _ptr(lse, "lse", torch.float32)
        _need(lse, rows, "lse")
    _ptr(table, "table", torch.int32)
    _need(table, plan.sizes.table_int32s, "table")
    _pools(plan, k_pool, v_pool)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().segpaged_decode(plan.handle, layer, _ptr(q, "q"), _ptr(table, "t"),
                                  _ptr(k_pool, "kp", torch.bfloat16),
                                  _ptr(v_pool, "vp", torch.bfloat16), float(scale),
                                  _ptr(o, "o"), _ptr(lse, "lse"), _ptr(workspace, "ws"), wsb,
                                  _stream(stream)), "segpaged_decode")


NOALLOC_SCRATCH_BYTES = 32 << 20  # SEGPAGED_NOALLOC_SCRATCH_BYTES


def decode_noalloc(plan: Plan, layer: int, q, table, k_pool, v_pool, scale: float, o, lse=None,
                   stream=None):
    """segpaged_decode_noalloc: segpaged_decode with the workspace in the library's
    own device array (no allocation); calls on one GPU must not overlap."""
    import torch
    nl = plan.num_layers if layer < 0 else 1
    rows = nl * plan.num_seqs * plan.num_q_heads
    for t, nm in ((q, "q"), (o, "o")):
        _ptr(t, nm, torch.bfloat16)
        _need(t, rows * plan.head_dim, nm)
    if lse is not None:
        _ptr(lse, "lse", torch.float32)
        _need(lse, rows, "lse")
    _ptr(table, "table", torch.int32)
    _need(table, plan.sizes.table_int32s, "table")
    _pools(plan, k_pool, v_pool)
    _check(_lib().segpaged_decode_noalloc(plan.handle, layer, _ptr(q, "q"), _ptr(table, "t"),
                                          _ptr(k_pool, "kp", torch.bfloat16),
                                          _ptr(v_pool, "vp", torch.bfloat16), float(scale),
                                          _ptr(o, "o"), _ptr(lse, "lse"), _stream(stream)),
           "segpaged_decode_noalloc")
