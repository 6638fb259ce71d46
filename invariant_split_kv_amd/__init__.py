"""Python binding of libisk, the batch-invariant split-KV decode-attention
library for MI355X (gfx950).

Argument marshalling only: every function here maps one-to-one onto an
``isk_*`` entry point of include/isk.h and passes plain pointers and sizes.
Device tensors may be given as torch tensors (their ``data_ptr()`` is passed)
or as integer device addresses.  All computation runs in the HIP kernels of
libisk.so; importing this package fails if the library has not been built
(``python invariant_split_kv_amd/build.py``).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

__all__ = [
    "IskError", "IskDesc", "IskExtraDesc", "IskExtraKv", "IskPlanInfo", "KIND_GQA", "KIND_MLA", "SPLIT_PER_ROW",
    "SPLIT_BATCH_BALANCED", "OUT_BF16", "OUT_F32", "KERNEL_GQA", "KERNEL_MLA_H16", "KERNEL_MLA_H32",
    "KERNEL_MLA_H128", "LIB_PATH", "lib", "plan_create",
    "plan_update", "plan_destroy", "plan_query", "plan_workspace_bytes", "plan_segments",
    "plan_set_timing_events", "plan_create_extra",
    "attn_decode", "attn_decode_extra", "attn_decode_oneshot", "attn_decode_static", "rmsnorm", "linear_bf16", "hbm_read_probe",
    "hbm_gather_probe",
    "last_error", "numerics_id", "Plan",
]

KIND_GQA, KIND_MLA = 0, 1
SPLIT_PER_ROW, SPLIT_BATCH_BALANCED = 0, 1
OUT_BF16, OUT_F32 = 0, 1
# split-kernel families (plan_query()["split_kernel"])
KERNEL_GQA, KERNEL_MLA_H16, KERNEL_MLA_H32, KERNEL_MLA_H128 = 1, 2, 3, 4
STATUS_NAMES = {0: "ISK_OK", -1: "ISK_ERR_INVALID_ARG", -2: "ISK_ERR_UNSUPPORTED",
                -3: "ISK_ERR_WORKSPACE", -4: "ISK_ERR_INDEX", -5: "ISK_ERR_HIP",
                -6: "ISK_ERR_RANGE"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libisk.so")


class IskError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class IskDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_row", ctypes.c_int32),
                ("topk_width", ctypes.c_int32), ("split_mode", ctypes.c_int32), ("split_tokens", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("check_inputs", ctypes.c_int32), ("scale", ctypes.c_float)]


class IskExtraDesc(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_row", ctypes.c_int32), ("topk_width", ctypes.c_int32)]


class IskExtraKv(ctypes.Structure):
    _fields_ = [("kv_pages", ctypes.c_void_p), ("block_table", ctypes.c_void_p), ("lens", ctypes.c_void_p),
                ("topk_idx", ctypes.c_void_p), ("topk_len", ctypes.c_void_p)]


class IskSplitBand(ctypes.Structure):
    _fields_ = [("max_units", ctypes.c_int32), ("split_units", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class IskPlanInfo(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("split_tokens", ctypes.c_int32), ("num_segments", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("num_partials", ctypes.c_int32), ("split_kernel", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python invariant_split_kv_amd/build.py`")
    # One HIP runtime per process: torch ships its own libamdhip64 (same
    # soname), and the device memory handed to libisk comes from it.  Loading
    # torch first makes libisk bind to that runtime instead of pulling in a
    # second copy from /opt/rocm, which on some hosts sees no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P, I32P = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    sig = {
        "isk_plan_create": (ctypes.c_int, [ctypes.POINTER(IskDesc), ctypes.c_int32, I32P, I32P, ctypes.POINTER(P)]),
        "isk_plan_update": (ctypes.c_int, [P, ctypes.c_int32, I32P, I32P]),
        "isk_plan_destroy": (ctypes.c_int, [P]),
        "isk_plan_query": (ctypes.c_int, [P, ctypes.POINTER(IskPlanInfo)]),
        "isk_plan_workspace_bytes": (ctypes.c_size_t, [P]),
        "isk_plan_segments": (ctypes.c_int, [P, I32P, ctypes.c_int32]),
        "isk_attn_decode": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "isk_attn_decode_oneshot": (ctypes.c_int, [ctypes.POINTER(IskDesc), ctypes.c_int32, I32P, I32P,
                                                    P, P, P, P, P, P, P, P, P]),
        "isk_plan_set_timing_events": (ctypes.c_int, [P, P, P, P]),
        "isk_plan_create_extra": (ctypes.c_int, [ctypes.POINTER(IskDesc), ctypes.POINTER(IskExtraDesc), ctypes.c_int32,
                                                  I32P, I32P, I32P, ctypes.POINTER(P)]),
        "isk_plan_create_banded": (ctypes.c_int, [ctypes.POINTER(IskDesc), ctypes.POINTER(IskSplitBand), ctypes.c_int32,
                                                   ctypes.c_int32, I32P, I32P, ctypes.POINTER(P)]),
        "isk_attn_decode_extra": (ctypes.c_int, [P, P, P, P, P, P, P, ctypes.POINTER(IskExtraKv), P, P, P,
                                                  ctypes.c_size_t, P]),
        "isk_rmsnorm": (ctypes.c_int, [P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P]),
        "isk_linear_bf16": (ctypes.c_int, [P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P]),
        "isk_hbm_read_probe": (ctypes.c_int, [P, ctypes.c_size_t, P, ctypes.c_int32, P]),
        "isk_hbm_gather_probe": (ctypes.c_int, [P, ctypes.c_size_t, P, ctypes.c_int32, ctypes.c_int32, P,
                                                ctypes.c_int32, P]),
        "isk_attn_decode_static": (ctypes.c_int, [P, P, P, P, P, P, P, P, P, P]),
        "isk_last_error": (ctypes.c_char_p, []),
        "isk_numerics_id": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


lib = _load()


def _check(status: int) -> None:
    if status != 0:
        raise IskError(status, lib.isk_last_error().decode())


def _i32_host(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr


def _i32p(arr: Optional[np.ndarray]):
    return None if arr is None else arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _ptr(x) -> Optional[int]:
    """Device address of a torch tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def last_error() -> str:
    return lib.isk_last_error().decode()


def numerics_id() -> str:
    return lib.isk_numerics_id().decode()


def plan_create(desc: IskDesc, lens_host, topk_len_host=None) -> int:
    lens = _i32_host(lens_host)
    tl = _i32_host(topk_len_host)
    out = ctypes.c_void_p()
    _check(lib.isk_plan_create(ctypes.byref(desc), len(lens), _i32p(lens), _i32p(tl), ctypes.byref(out)))
    return out.value


def plan_create_extra(desc: IskDesc, extra: IskExtraDesc, lens_host, topk_len_host, extra_topk_len_host) -> int:
    lens = _i32_host(lens_host)
    tl = _i32_host(topk_len_host)
    xtl = _i32_host(extra_topk_len_host)
    out = ctypes.c_void_p()
    _check(lib.isk_plan_create_extra(ctypes.byref(desc), ctypes.byref(extra), len(lens), _i32p(lens), _i32p(tl),
                                     _i32p(xtl), ctypes.byref(out)))
    return out.value


def split_bands(bands) -> ctypes.Array:
    """ctypes array of isk_split_band from (max_units, split_units[, max_splits]) tuples."""
    rows = [tuple(b) + (0,) * (3 - len(b)) for b in bands]
    arr = (IskSplitBand * len(rows))()
    for i, (mu, su, ms) in enumerate(rows):
        arr[i] = IskSplitBand(int(mu), int(su), int(ms), 0)
    return arr


def plan_create_banded(desc: IskDesc, bands, lens_host, topk_len_host=None) -> int:
    arr = bands if isinstance(bands, ctypes.Array) else split_bands(bands)
    lens = _i32_host(lens_host)
    tl = _i32_host(topk_len_host)
    out = ctypes.c_void_p()
    _check(lib.isk_plan_create_banded(ctypes.byref(desc), arr, len(arr), len(lens), _i32p(lens), _i32p(tl),
                                      ctypes.byref(out)))
    return out.value


def plan_update(plan: int, lens_host, topk_len_host=None) -> None:
    lens = _i32_host(lens_host)
    tl = _i32_host(topk_len_host)
    _check(lib.isk_plan_update(plan, len(lens), _i32p(lens), _i32p(tl)))


def plan_destroy(plan: int) -> None:
    _check(lib.isk_plan_destroy(plan))


def plan_query(plan: int) -> dict:
    info = IskPlanInfo()
    _check(lib.isk_plan_query(plan, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in IskPlanInfo._fields_}


def plan_workspace_bytes(plan: int) -> int:
    return int(lib.isk_plan_workspace_bytes(plan))


def plan_segments(plan: int) -> np.ndarray:
    """[n, 5] int32 records (row, begin, end, partial_slot, group), launch order."""
    n = lib.isk_plan_segments(plan, None, 0)
    if n < 0:
        _check(n)
    rec = np.zeros((max(n, 1), 5), dtype=np.int32)
    got = lib.isk_plan_segments(plan, _i32p(rec), n)
    if got < 0:
        _check(got)
    return rec[:n]


def plan_set_timing_events(plan: int, split_begin=None, split_end=None, combine_end=None) -> None:
    """Profiling hook: hipEvent_t handles (ints) recorded around the split
    kernel and after the combine of later attn_decode calls; None disables."""
    _check(lib.isk_plan_set_timing_events(plan, split_begin, split_end, combine_end))


def attn_decode(plan: int, q, kv_pages, block_table, lens, topk_idx, topk_len, out, lse, workspace,
                workspace_bytes: int, stream=None) -> None:
    """Enqueue one decode-attention call on `stream` (torch stream, raw
    hipStream_t int, or None for torch's current stream)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(lib.isk_attn_decode(plan, _ptr(q), _ptr(kv_pages), _ptr(block_table), _ptr(lens), _ptr(topk_idx),
                               _ptr(topk_len), _ptr(out), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                               stream))


def attn_decode_static(plan: int, q, kv_pages, block_table, lens, topk_idx, topk_len, out, lse,
                       stream=None) -> None:
    """attn_decode with the library's fixed device workspace (no workspace
    argument; nothing is allocated)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(lib.isk_attn_decode_static(plan, _ptr(q), _ptr(kv_pages), _ptr(block_table), _ptr(lens), _ptr(topk_idx),
                                      _ptr(topk_len), _ptr(out), _ptr(lse), stream))


def attn_decode_extra(plan: int, q, kv_pages, block_table, lens, topk_idx, topk_len, extra_kv_pages,
                      extra_block_table, extra_lens, extra_topk_idx, extra_topk_len, out, lse, workspace,
                      workspace_bytes: int, stream=None) -> None:
    """attn_decode for a plan with an extra KV source (plan_create_extra)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    x = IskExtraKv(_ptr(extra_kv_pages), _ptr(extra_block_table), _ptr(extra_lens), _ptr(extra_topk_idx),
                   _ptr(extra_topk_len))
    _check(lib.isk_attn_decode_extra(plan, _ptr(q), _ptr(kv_pages), _ptr(block_table), _ptr(lens), _ptr(topk_idx),
                                     _ptr(topk_len), ctypes.byref(x), _ptr(out), _ptr(lse), _ptr(workspace),
                                     int(workspace_bytes), stream))


def attn_decode_oneshot(desc: IskDesc, lens_host, topk_len_host, q, kv_pages, block_table, lens, topk_idx,
                        topk_len, out, lse, stream=None) -> None:
    """Plan, allocate the workspace on `stream` and decode in one call."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    lh = _i32_host(lens_host)
    th = _i32_host(topk_len_host)
    _check(lib.isk_attn_decode_oneshot(ctypes.byref(desc), len(lh), _i32p(lh), _i32p(th), _ptr(q), _ptr(kv_pages),
                                       _ptr(block_table), _ptr(lens), _ptr(topk_idx), _ptr(topk_len), _ptr(out),
                                       _ptr(lse), stream))


def rmsnorm(x, w, y, rows: int, dim: int, eps: float, stream=None) -> None:
    """Enqueue isk_rmsnorm: y = x / sqrt(mean(x^2) + eps) * w per row (bf16)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(lib.isk_rmsnorm(_ptr(x), _ptr(w), _ptr(y), int(rows), int(dim), float(eps), stream))


def linear_bf16(x, w, y, m: int, n: int, k: int, stream=None) -> None:
    """Enqueue isk_linear_bf16: y[m, n] (fp32) = x[m, k] w[n, k]^T (bf16 inputs)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(lib.isk_linear_bf16(_ptr(x), _ptr(w), _ptr(y), int(m), int(n), int(k), stream))


def hbm_read_probe(src, nbytes: int, sink, blocks: int, stream=None) -> None:
    """Enqueue isk_hbm_read_probe: one streaming read of nbytes at src."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(lib.isk_hbm_read_probe(_ptr(src), int(nbytes), _ptr(sink), int(blocks), stream))


def hbm_gather_probe(src, src_bytes: int, rows, n_rows: int, row_bytes: int, sink, blocks: int,
                     stream=None) -> None:
    """Enqueue isk_hbm_gather_probe: one read of the listed rows of src."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    _check(lib.isk_hbm_gather_probe(_ptr(src), int(src_bytes), _ptr(rows), int(n_rows), int(row_bytes), _ptr(sink),
                                    int(blocks), stream))


class Plan:
    """Owning wrapper of an isk_plan handle (destroyed on close/garbage collection)."""

    def __init__(self, desc: IskDesc, lens_host, topk_len_host=None, extra: Optional[IskExtraDesc] = None,
                 extra_topk_len_host=None, bands=None):
        self.desc = desc
        self.extra = extra
        self.handle = None
        if bands is not None:
            if extra is not None:
                raise ValueError("a band table is not combined with an extra KV source")
            self.handle = plan_create_banded(desc, bands, lens_host, topk_len_host)
        elif extra is None:
            self.handle = plan_create(desc, lens_host, topk_len_host)
        else:
            self.handle = plan_create_extra(desc, extra, lens_host, topk_len_host, extra_topk_len_host)

    def update(self, lens_host, topk_len_host=None) -> None:
        plan_update(self.handle, lens_host, topk_len_host)

    def info(self) -> dict:
        return plan_query(self.handle)

    @property
    def workspace_bytes(self) -> int:
        return plan_workspace_bytes(self.handle)

    def segments(self) -> np.ndarray:
        return plan_segments(self.handle)

    def close(self) -> None:
        if self.handle:
            plan_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
