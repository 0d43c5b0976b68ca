"""MI355X (gfx950) FlashAttention-2 forward and backward: a thin ctypes binding of libfa2.so.

The library (``libfa2.so``, built in-tree by ``build_lib``) exports the C ABI
declared in ``include/fa2.h``.  This module only marshals arguments: every
step of the computation runs in the library's HIP kernels.  There is no CPU
fallback -- if the library is missing, every call raises.

Raw entry points (same names and argument order as the C ABI):
    fa2_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream, in_dtype, o_dtype) -> int
    fa2_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, causal, scale, stream,
            in_dtype, o_dtype, grad_dtype) -> int
    fa2_fwd_gqa / fa2_bwd_gqa: the same with H_kv after H (grouped key/value heads)
    fa2_fwd_window / fa2_bwd_window: the *_gqa calls with (window_left, window_right)
        instead of causal (sliding-window mask)
    fa2_plan(B, H, N, d, causal, in_dtype, block_rows=0, block_cols=0, num_units=0) -> dict
    fa2_split_plan(B, H, N, d, window_left, window_right, in_dtype, num_units, max_chunk_tiles=0)
        -> SplitPlan (host schedule; key ranges of heavy query tiles cut into chunks)
    fa2_fwd_split(q, k, v, o, lse, B, H, H_kv, N, d, window_left, window_right, scale, stream,
        in_dtype, o_dtype, items, n_items, n_slots, workspace, workspace_bytes) -> int
    fa2_sparse_plan(N, block_q, block_k, block_mask, causal) -> SparsePlan (host key-tile lists)
    fa2_fwd_sparse(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, stream, in_dtype, o_dtype,
        n_layouts, tile_ptr, entries, n_entries) -> int
    fa2_decode_paged_workspace(B, H, H_kv, n_q, d, max_context, split_keys=0, num_units=0)
        -> (split_keys, workspace_bytes)
    fa2_decode_paged(q, k_cache, v_cache, o, lse, B, H, H_kv, n_q, d, scale, page_table, max_pages,
        context_lens, max_context, page_size, n_pages, split_keys, workspace, workspace_bytes,
        stream, in_dtype, o_dtype) -> int
    fa2_decode_paged_noalloc(... the same without workspace, workspace_bytes ...) -> int
        (partials in a static per-device scratch of FA2_DECODE_SCRATCH_BYTES)
    fa2_fp8_pack_workspace(B, H, N) -> bytes
    fa2_fp8_pack(x, B, H, N, d, signs, codes, scales, workspace, workspace_bytes, stream) -> int
    fa2_fwd_fp8(q8, q_scale, k8, k_scale, v, o, lse, B, H, H_kv, N, d, causal, scale, stream, o_dtype) -> int
    fa2_strerror(status) -> str
    fa2_version() -> int
Convenience wrappers over torch device tensors (k and v may have fewer heads
than q: grouped key/value heads):
    forward(q, k, v, causal=False, scale=None, o_dtype=torch.float32) -> (o, lse)
    backward(q, k, v, o, lse, dout, causal=False, scale=None, grad_dtype=torch.float32)
        -> (dq, dk, dv)
    split_plan(q_shape, causal=False, window=None, num_units=None, max_chunk_tiles=0) -> SplitPlan
    forward_split(q, k, v, plan, causal=False, scale=None, ...) -> (o, lse)
    forward_sparse(q, k, v, plan, scale=None, ...) -> (o, lse)   (plan from fa2_sparse_plan)
    decode_paged(q, k_cache, v_cache, page_table, context_lens, max_context, ...) -> (o, lse)
    fp8_pack(x, signs=None) -> (codes, scales);  forward_fp8(q, k, v, signs, ...) -> (o, lse)
"""

from __future__ import annotations

import ctypes
import math
from pathlib import Path

__all__ = [
    "F32", "BF16",
    "FA2_OK", "FA2_ERR_INVALID_ARG", "FA2_ERR_UNSUPPORTED", "FA2_ERR_NO_DEVICE", "FA2_ERR_LAUNCH",
    "FA2_ERR_SCRATCH", "FA2_DECODE_SCRATCH_BYTES", "Fa2Error", "library_path", "load", "fa2_fwd", "fa2_plan", "fa2_strerror", "fa2_version",
    "fa2_bwd", "fa2_fwd_gqa", "fa2_bwd_gqa", "fa2_fwd_window", "fa2_bwd_window", "forward", "backward",
    "fa2_split_plan", "fa2_fwd_split", "SplitPlan", "split_plan", "forward_split",
    "fa2_sparse_plan", "fa2_fwd_sparse", "SparsePlan", "forward_sparse",
    "fa2_decode_paged_workspace", "fa2_decode_paged", "fa2_decode_paged_noalloc", "decode_paged",
    "fa2_fp8_pack_workspace", "fa2_fp8_pack", "fa2_fwd_fp8", "fp8_pack", "forward_fp8", "fa2_clock_probe", "ClockProbe", "shader_clock_ghz",
    "EXPORTED_SYMBOLS",
]

F32 = 0
BF16 = 1

FA2_OK = 0
FA2_ERR_INVALID_ARG = -1
FA2_ERR_UNSUPPORTED = -2
FA2_ERR_NO_DEVICE = -3
FA2_ERR_LAUNCH = -4
FA2_ERR_SCRATCH = -5

FA2_DECODE_SCRATCH_BYTES = 16 << 20

EXPORTED_SYMBOLS = ("fa2_fwd", "fa2_fwd_gqa", "fa2_fwd_window", "fa2_bwd", "fa2_bwd_gqa",
                    "fa2_bwd_window", "fa2_plan", "fa2_split_plan", "fa2_fwd_split", "fa2_sparse_plan",
                    "fa2_fwd_sparse", "fa2_decode_paged_workspace", "fa2_decode_paged", "fa2_decode_paged_noalloc",
                    "fa2_fp8_pack_workspace", "fa2_fp8_pack", "fa2_fwd_fp8", "fa2_clock_probe", "fa2_strerror", "fa2_version")

_LIB_PATH = Path(__file__).resolve().parent / "libfa2.so"
_lib = None


class Fa2Error(RuntimeError):
    def __init__(self, status: int, where: str = "fa2_fwd"):
        self.status = status
        super().__init__(f"{where} failed with status {status}: {fa2_strerror(status)}")


class _SplitItem(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int) for name in ("tile", "kt_lo", "kt_hi", "slot", "slot0", "n_parts")]


class SplitPlan:
    """A split forward schedule from fa2_split_plan.

    ``items`` is an int32 array [n_items, 6] with the columns of
    fa2_split_item (tile, kt_lo, kt_hi, slot, slot0, n_parts); ``n_slots``
    and ``workspace_bytes`` are what fa2_fwd_split needs.  ``shape`` and
    ``window`` record what the schedule was built for.
    """

    def __init__(self, items, n_slots: int, workspace_bytes: int, shape, window):
        self.items = items
        self.n_slots = int(n_slots)
        self.workspace_bytes = int(workspace_bytes)
        self.shape = tuple(shape)
        self.window = tuple(window)
        self._dev = {}

    @property
    def n_items(self) -> int:
        return int(self.items.shape[0])

    @property
    def splits(self) -> bool:
        return self.n_slots > 0

    def device_items(self, device):
        """The schedule as an int32 device tensor (copied once per device)."""
        import torch

        key = str(device)
        if key not in self._dev:
            self._dev[key] = torch.from_numpy(self.items).to(device)
        return self._dev[key]


class SparsePlan:
    """Key-tile lists of a block-sparse mask from fa2_sparse_plan.

    ``tile_ptr`` (int32 [n_layouts * T + 1]) and ``entries`` (uint32) are the
    host arrays; ``N``, ``causal`` and ``n_layouts`` record what they were
    built for.
    """

    def __init__(self, tile_ptr, entries, N: int, causal: bool, n_layouts: int):
        self.tile_ptr = tile_ptr
        self.entries = entries
        self.N = int(N)
        self.causal = bool(causal)
        self.n_layouts = int(n_layouts)
        self._dev = {}

    @property
    def n_entries(self) -> int:
        return int(self.entries.shape[0])

    def device_arrays(self, device):
        """(tile_ptr, entries) as int32 device tensors (copied once per device)."""
        import torch

        key = str(device)
        if key not in self._dev:
            ptr = torch.from_numpy(self.tile_ptr).to(device)
            ent = torch.from_numpy(self.entries.view("int32")).to(device) if self.n_entries else None
            self._dev[key] = (ptr, ent)
        return self._dev[key]


class _Plan(ctypes.Structure):
    _fields_ = [
        ("block_rows", ctypes.c_int),
        ("block_cols", ctypes.c_int),
        ("waves_per_group", ctypes.c_int),
        ("query_tiles", ctypes.c_int),
        ("workgroups", ctypes.c_longlong),
        ("tile_pairs", ctypes.c_longlong),
        ("normalisations", ctypes.c_longlong),
        ("waves_of_groups", ctypes.c_double),
        ("last_wave_groups", ctypes.c_int),
        ("flops_executed", ctypes.c_double),
        ("flops_credited", ctypes.c_double),
    ]


def library_path() -> Path:
    return _LIB_PATH


def load():
    """Load libfa2.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it first with "
            "`python -m exact_tiled_attention_33_amd.build_lib` (or __graft_entry__.build())"
        )
    lib = ctypes.CDLL(str(_LIB_PATH))
    lib.fa2_fwd.restype = ctypes.c_int
    lib.fa2_fwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_bwd.restype = ctypes.c_int
    lib.fa2_bwd.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_fwd_gqa.restype = ctypes.c_int
    lib.fa2_fwd_gqa.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_fwd_window.restype = ctypes.c_int
    lib.fa2_fwd_window.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_bwd_window.restype = ctypes.c_int
    lib.fa2_bwd_window.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_bwd_gqa.restype = ctypes.c_int
    lib.fa2_bwd_gqa.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_plan.restype = ctypes.c_int
    lib.fa2_plan.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(_Plan),
    ]
    lib.fa2_split_plan.restype = ctypes.c_int
    lib.fa2_split_plan.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_size_t),
    ]
    lib.fa2_fwd_split.restype = ctypes.c_int
    lib.fa2_fwd_split.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
    ]
    lib.fa2_sparse_plan.restype = ctypes.c_int
    lib.fa2_sparse_plan.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
    ]
    lib.fa2_fwd_sparse.restype = ctypes.c_int
    lib.fa2_fwd_sparse.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
    ]
    lib.fa2_decode_paged_workspace.restype = ctypes.c_int
    lib.fa2_decode_paged_workspace.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_size_t),
    ]
    lib.fa2_decode_paged.restype = ctypes.c_int
    lib.fa2_decode_paged.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_decode_paged_noalloc.restype = ctypes.c_int
    lib.fa2_decode_paged_noalloc.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
    ]
    lib.fa2_fp8_pack_workspace.restype = ctypes.c_int
    lib.fa2_fp8_pack_workspace.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
    lib.fa2_fp8_pack.restype = ctypes.c_int
    lib.fa2_fp8_pack.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
    ]
    lib.fa2_fwd_fp8.restype = ctypes.c_int
    lib.fa2_fwd_fp8.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_float, ctypes.c_void_p, ctypes.c_int,
    ]
    lib.fa2_clock_probe.restype = ctypes.c_int
    lib.fa2_clock_probe.argtypes = [ctypes.c_int, ctypes.c_ulonglong, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa2_strerror.restype = ctypes.c_char_p
    lib.fa2_strerror.argtypes = [ctypes.c_int]
    lib.fa2_version.restype = ctypes.c_int
    lib.fa2_version.argtypes = []
    _lib = lib
    return lib


def fa2_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream, in_dtype, o_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_fwd(q, k, v, o, lse, B, H, N, d, int(causal), float(scale),
                              stream, in_dtype, o_dtype))


def fa2_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, causal, scale, stream,
            in_dtype, o_dtype, grad_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, int(causal),
                              float(scale), stream, in_dtype, o_dtype, grad_dtype))


def fa2_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, stream, in_dtype, o_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_fwd_gqa(q, k, v, o, lse, B, H, H_kv, N, d, int(causal), float(scale),
                                  stream, in_dtype, o_dtype))


def fa2_fwd_window(q, k, v, o, lse, B, H, H_kv, N, d, window_left, window_right, scale, stream,
                   in_dtype, o_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_fwd_window(q, k, v, o, lse, B, H, H_kv, N, d, int(window_left),
                                     int(window_right), float(scale), stream, in_dtype, o_dtype))


def fa2_bwd_window(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, window_left, window_right,
                   scale, stream, in_dtype, o_dtype, grad_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_bwd_window(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d,
                                     int(window_left), int(window_right), float(scale), stream, in_dtype,
                                     o_dtype, grad_dtype))


def fa2_bwd_gqa(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, causal, scale, stream,
                in_dtype, o_dtype, grad_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_bwd_gqa(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d,
                                  int(causal), float(scale), stream, in_dtype, o_dtype, grad_dtype))


def fa2_plan(B, H, N, d, causal, in_dtype, block_rows=0, block_cols=0, num_units=0) -> dict:
    out = _Plan()
    st = int(load().fa2_plan(B, H, N, d, int(causal), in_dtype, block_rows, block_cols,
                             num_units, ctypes.byref(out)))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_plan")
    return {name: getattr(out, name) for name, _ in _Plan._fields_}


def fa2_split_plan(B, H, N, d, window_left, window_right, in_dtype, num_units, max_chunk_tiles=0) -> SplitPlan:
    """Raw C call (two passes: count, then fill); raises Fa2Error on a bad status."""
    import numpy as np

    lib = load()
    n_items, n_slots, ws = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_size_t(0)
    args = (B, H, N, d, int(window_left), int(window_right), in_dtype, int(num_units), int(max_chunk_tiles))
    st = int(lib.fa2_split_plan(*args, None, 0, ctypes.byref(n_items), ctypes.byref(n_slots), ctypes.byref(ws)))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_split_plan")
    buf = (_SplitItem * max(1, n_items.value))()
    st = int(lib.fa2_split_plan(*args, ctypes.cast(buf, ctypes.c_void_p), n_items.value, ctypes.byref(n_items),
                                ctypes.byref(n_slots), ctypes.byref(ws)))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_split_plan")
    items = np.frombuffer(buf, dtype=np.int32, count=6 * n_items.value).reshape(n_items.value, 6).copy()
    return SplitPlan(items, n_slots.value, ws.value, (B, H, N, d), (window_left, window_right))


def fa2_fwd_split(q, k, v, o, lse, B, H, H_kv, N, d, window_left, window_right, scale, stream, in_dtype,
                  o_dtype, items, n_items, n_slots, workspace, workspace_bytes) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_fwd_split(q, k, v, o, lse, B, H, H_kv, N, d, int(window_left), int(window_right),
                                    float(scale), stream, in_dtype, o_dtype, items, int(n_items), int(n_slots),
                                    workspace, int(workspace_bytes)))


def fa2_sparse_plan(N, block_q, block_k, block_mask, causal) -> SparsePlan:
    """Raw C call (count, then fill) on a host mask [n_layouts, ceil(N/block_q),
    ceil(N/block_k)] (any array convertible to bool); raises Fa2Error on a bad
    status."""
    import numpy as np

    m = np.ascontiguousarray(np.asarray(block_mask).astype(np.uint8))
    if m.ndim != 3 or m.shape[1] != -(-N // block_q) or m.shape[2] != -(-N // block_k):
        raise ValueError(f"block_mask must be [L, {-(-N // block_q)}, {-(-N // block_k)}], got {m.shape}")
    lib = load()
    n = ctypes.c_int(0)
    args = (N, block_q, block_k, m.shape[0], m.ctypes.data, int(causal))
    st = int(lib.fa2_sparse_plan(*args, None, None, 0, ctypes.byref(n)))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_sparse_plan")
    T = -(-N // 256)
    ptr = np.zeros(m.shape[0] * T + 1, dtype=np.int32)
    ent = np.zeros(max(1, n.value), dtype=np.uint32)
    st = int(lib.fa2_sparse_plan(*args, ptr.ctypes.data, ent.ctypes.data, ent.shape[0], ctypes.byref(n)))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_sparse_plan")
    return SparsePlan(ptr, ent[:n.value].copy(), N, causal, m.shape[0])


def fa2_fwd_sparse(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, stream, in_dtype, o_dtype, n_layouts,
                   tile_ptr, entries, n_entries) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_fwd_sparse(q, k, v, o, lse, B, H, H_kv, N, d, int(causal), float(scale), stream,
                                     in_dtype, o_dtype, int(n_layouts), tile_ptr, entries, int(n_entries)))


def fa2_decode_paged_workspace(B, H, H_kv, n_q, d, max_context, split_keys=0, num_units=0):
    """Raw C call; returns (split_keys, workspace_bytes) or raises Fa2Error."""
    sk, ws = ctypes.c_int(0), ctypes.c_size_t(0)
    st = int(load().fa2_decode_paged_workspace(B, H, H_kv, n_q, d, max_context, split_keys, num_units,
                                               ctypes.byref(sk), ctypes.byref(ws)))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_decode_paged_workspace")
    return sk.value, ws.value


def fa2_decode_paged(q, k_cache, v_cache, o, lse, B, H, H_kv, n_q, d, scale, page_table, max_pages, context_lens,
                     max_context, page_size, n_pages, split_keys, workspace, workspace_bytes, stream, in_dtype,
                     o_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_decode_paged(q, k_cache, v_cache, o, lse, B, H, H_kv, n_q, d, float(scale), page_table,
                                       max_pages, context_lens, max_context, page_size, n_pages, split_keys,
                                       workspace, int(workspace_bytes), stream, in_dtype, o_dtype))


def fa2_decode_paged_noalloc(q, k_cache, v_cache, o, lse, B, H, H_kv, n_q, d, scale, page_table, max_pages,
                             context_lens, max_context, page_size, n_pages, split_keys, stream, in_dtype,
                             o_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_decode_paged_noalloc(q, k_cache, v_cache, o, lse, B, H, H_kv, n_q, d, float(scale),
                                               page_table, max_pages, context_lens, max_context, page_size,
                                               n_pages, split_keys, stream, in_dtype, o_dtype))


def fa2_fp8_pack_workspace(B, H, N) -> int:
    """Raw C call; returns the workspace bytes or raises Fa2Error."""
    ws = ctypes.c_size_t(0)
    st = int(load().fa2_fp8_pack_workspace(B, H, N, ctypes.byref(ws)))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_fp8_pack_workspace")
    return ws.value


def fa2_fp8_pack(x, B, H, N, d, signs, codes, scales, workspace, workspace_bytes, stream) -> int:
    """Raw C call: device pointers as ints; ``signs`` a host float32 array
    of d entries (+-1) or None."""
    import numpy as np

    sg = None
    if signs is not None:
        sg = np.ascontiguousarray(np.asarray(signs, dtype=np.float32))
        if sg.shape != (d,):
            raise ValueError(f"signs must have {d} entries")
    return int(load().fa2_fp8_pack(x, B, H, N, d, sg.ctypes.data if sg is not None else None, codes, scales,
                                   workspace, int(workspace_bytes), stream))


def fa2_fwd_fp8(q8, q_scale, k8, k_scale, v, o, lse, B, H, H_kv, N, d, causal, scale, stream, o_dtype) -> int:
    """Raw C call: pointers and sizes as Python ints; returns the status code."""
    return int(load().fa2_fwd_fp8(q8, q_scale, k8, k_scale, v, o, lse, B, H, H_kv, N, d, int(causal),
                                  float(scale), stream, o_dtype))


def fa2_clock_probe(workgroups, ticks, out, stream) -> int:
    """Raw C call: out is a device pointer (int) to 3 * workgroups uint64."""
    return int(load().fa2_clock_probe(int(workgroups), int(ticks), out, stream))


class ClockProbe:
    """fa2_clock_probe on a stream of its own: ``start(seconds)`` enqueues one
    workgroup that runs for that long beside whatever else runs, ``ghz()``
    waits for it and returns the mean shader clock over its span."""

    def __init__(self, workgroups: int = 1, device=None):
        import torch

        self.dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        self.workgroups = workgroups
        self.out = torch.zeros(3 * workgroups, dtype=torch.int64, device=self.dev)
        self.stream = torch.cuda.Stream(device=self.dev)

    def start(self, seconds: float) -> None:
        ticks = max(1, min(10**9, int(seconds * 1e8)))
        st = fa2_clock_probe(self.workgroups, ticks, self.out.data_ptr(), self.stream.cuda_stream)
        if st != FA2_OK:
            raise Fa2Error(st, "fa2_clock_probe")

    def ghz(self) -> float:
        self.stream.synchronize()
        t = self.out.view(-1, 3).cpu()
        return 0.1 * float(t[:, 0].sum()) / float(t[:, 1].sum())


def shader_clock_ghz(workgroups: int = 256, seconds: float = 50e-6) -> float:
    """Mean shader clock (GHz) of `workgroups` probe workgroups that each run
    for `seconds` on an otherwise idle stream."""
    p = ClockProbe(workgroups)
    p.start(seconds)
    return p.ghz()


def fa2_strerror(status: int) -> str:
    return load().fa2_strerror(int(status)).decode()


def fa2_version() -> int:
    return int(load().fa2_version())


def _dtype_code(dt) -> int:
    import torch

    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {dt} (bf16 or fp32)")


def _check_buffer(t, name, shape, dtype, device):
    """A buffer the kernels read or write through its raw address: it must be
    a contiguous device tensor on ``device`` with exactly this shape and
    dtype.  (A host tensor, a tensor on another device or a shorter one would
    hand the kernel an address it cannot use; the C ABI cannot tell.)"""
    if not getattr(t, "is_cuda", False) or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _check_on_device(device, **tensors):
    """Inputs read through raw addresses: contiguous device tensors on ``device``."""
    for name, t in tensors.items():
        if not getattr(t, "is_cuda", False) or t.device != device:
            raise ValueError(f"{name} must be a device tensor on {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws, name, min_bytes, device):
    """A device workspace of at least ``min_bytes`` bytes on ``device``."""
    if not getattr(ws, "is_cuda", False) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor on {device}")
    if ws.numel() * ws.element_size() < min_bytes:
        raise ValueError(f"{name} holds {ws.numel() * ws.element_size()} bytes, {min_bytes} needed")


def forward(q, k, v, causal: bool = False, scale: float | None = None, o_dtype=None,
            out=None, lse=None, stream=None, window=None):
    """Attention forward on [B, H, N, d] device tensors; returns (o, lse).

    k and v may be [B, H_kv, N, d] with H_kv dividing H (grouped key/value
    heads, fa2_fwd_gqa).  ``window=(left, right)`` selects a sliding-window
    mask (fa2_fwd_window; -1 = unbounded side) and overrides ``causal``.
    ``o_dtype`` defaults to float32.  ``out``/``lse`` may be given to reuse
    buffers.  The kernels are enqueued on ``stream`` (default: torch's
    current stream) and this returns without synchronising.
    """
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError(f"q must be [B, H, N, d] and k, v [B, H_kv, N, d], got {q.shape}, {k.shape}, {v.shape}")
    if k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:] or q.shape[1] % k.shape[1]:
        raise ValueError(f"k, v heads must divide q's and the other dims match, got {q.shape}, {k.shape}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if not getattr(q, "is_cuda", False):
        raise ValueError("q, k, v must be device tensors")
    _check_on_device(q.device, q=q, k=k, v=v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((B, H, N, d), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer(out, "out", q.shape, o_dtype, q.device)
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    wl, wr = (-1, 0 if causal else -1) if window is None else window
    st = fa2_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, k.shape[1], N, d, wl, wr, scale, handle, _dtype_code(q.dtype),
                        _dtype_code(o_dtype))
    if st != FA2_OK:
        raise Fa2Error(st)
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             grad_dtype=None, delta=None, dq=None, dk=None, dv=None, stream=None, window=None):
    """Attention backward on [B, H, N, d] device tensors; returns (dq, dk, dv).

    ``o`` and ``lse`` are what ``forward`` returned for the same q, k, v,
    causal and scale; ``dout`` is the gradient with respect to o (same dtype
    as q).  k and v may have fewer heads than q (grouped key/value heads);
    dk and dv then have k's shape.  ``window=(left, right)`` as in ``forward``
    (it must match the forward call).  ``grad_dtype`` defaults to float32.  ``delta`` ([B, H, N]
    float32) is a workspace, allocated when not given.  The kernels are
    enqueued on ``stream`` (default: torch's current stream) and this
    returns without synchronising.
    """
    import torch

    if q.dim() != 4 or any(t.shape != q.shape for t in (o, dout)) or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q, o, dout must be [B, H, N, d] and k, v [B, H_kv, N, d]")
    if k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:] or q.shape[1] % k.shape[1]:
        raise ValueError(f"k, v heads must divide q's and the other dims match, got {q.shape}, {k.shape}")
    if not (q.dtype == k.dtype == v.dtype == dout.dtype):
        raise TypeError("q, k, v and dout must share a dtype")
    if not getattr(q, "is_cuda", False):
        raise ValueError("all tensors must be device tensors")
    _check_on_device(q.device, q=q, k=k, v=v, o=o, lse=lse, dout=dout)
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    grad_dtype = torch.float32 if grad_dtype is None else grad_dtype
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer(delta, "delta", (B, H, N), torch.float32, q.device)
    outs = []
    for t, name, shape in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape)):
        if t is None:
            t = torch.empty(shape, dtype=grad_dtype, device=q.device)
        _check_buffer(t, name, shape, grad_dtype, q.device)
        outs.append(t)
    dq, dk, dv = outs
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    wl, wr = (-1, 0 if causal else -1) if window is None else window
    st = fa2_bwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                        lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                        B, H, k.shape[1], N, d, wl, wr, scale, handle, _dtype_code(q.dtype),
                        _dtype_code(o.dtype), _dtype_code(grad_dtype))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_bwd")
    return dq, dk, dv


def split_plan(q_shape, causal: bool = False, window=None, num_units: int | None = None,
               max_chunk_tiles: int = 0) -> SplitPlan:
    """fa2_split_plan for a [B, H, N, d] bf16 query; ``num_units`` defaults
    to the current device's compute-unit count."""
    B, H, N, d = q_shape
    wl, wr = (-1, 0 if causal else -1) if window is None else window
    if num_units is None and max_chunk_tiles == 0:
        import torch

        num_units = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    return fa2_split_plan(B, H, N, d, wl, wr, BF16, num_units or 0, max_chunk_tiles)


def forward_split(q, k, v, plan: SplitPlan, causal: bool = False, scale: float | None = None, o_dtype=None,
                  out=None, lse=None, stream=None, window=None, workspace=None):
    """Attention forward over a split schedule (fa2_fwd_split); returns (o, lse).

    Arguments as ``forward``; ``plan`` comes from ``split_plan`` for the same
    shape and mask.  ``workspace`` (a device uint8 tensor of at least
    ``plan.workspace_bytes``) is allocated here when not given.
    """
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError(f"q must be [B, H, N, d] and k, v [B, H_kv, N, d], got {q.shape}, {k.shape}, {v.shape}")
    if not getattr(q, "is_cuda", False):
        raise ValueError("q, k, v must be device tensors")
    _check_on_device(q.device, q=q, k=k, v=v)
    B, H, N, d = q.shape
    wl, wr = (-1, 0 if causal else -1) if window is None else window
    if plan.shape != (B, H, N, d) or plan.window != (wl, wr):
        raise ValueError(f"plan was built for {plan.shape} window {plan.window}, not {tuple(q.shape)} ({wl}, {wr})")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((B, H, N, d), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer(out, "out", q.shape, o_dtype, q.device)
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    if workspace is None and plan.workspace_bytes > 0:
        workspace = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _check_workspace(workspace, "workspace", plan.workspace_bytes, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    items = plan.device_items(q.device)
    st = fa2_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                       k.shape[1], N, d, wl, wr, scale, handle, _dtype_code(q.dtype), _dtype_code(o_dtype),
                       items.data_ptr(), plan.n_items, plan.n_slots, ws_ptr, ws_bytes)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_fwd_split")
    return out, lse


def forward_sparse(q, k, v, plan: SparsePlan, scale: float | None = None, o_dtype=None, out=None, lse=None,
                   stream=None):
    """Attention forward under a block-sparse mask (fa2_fwd_sparse); returns
    (o, lse).  ``plan`` comes from ``fa2_sparse_plan`` for the same N; its
    causal flag applies.  Other arguments as ``forward``."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError(f"q must be [B, H, N, d] and k, v [B, H_kv, N, d], got {q.shape}, {k.shape}, {v.shape}")
    if not getattr(q, "is_cuda", False):
        raise ValueError("q, k, v must be device tensors")
    _check_on_device(q.device, q=q, k=k, v=v)
    B, H, N, d = q.shape
    if plan.N != N:
        raise ValueError(f"plan was built for N = {plan.N}, not {N}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((B, H, N, d), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer(out, "out", q.shape, o_dtype, q.device)
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    ptr, ent = plan.device_arrays(q.device)
    st = fa2_fwd_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                        k.shape[1], N, d, plan.causal, scale, handle, _dtype_code(q.dtype), _dtype_code(o_dtype),
                        plan.n_layouts, ptr.data_ptr(), ent.data_ptr() if ent is not None else None,
                        plan.n_entries)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_fwd_sparse")
    return out, lse


def decode_paged(q, k_cache, v_cache, page_table, context_lens, max_context: int, scale: float | None = None,
                 o_dtype=None, split_keys: int = 0, workspace=None, out=None, lse=None, stream=None):
    """Attention of the newest n_q tokens over a paged cache (fa2_decode_paged);
    returns (o, lse).

    q [B, H, n_q, d] bf16; k_cache, v_cache [n_pages, page_size, H_kv, d]
    bf16; page_table int32 [B, max_pages] and context_lens int32 [B] device
    tensors; ``max_context`` a host bound of context_lens.  ``split_keys`` 0
    lets the library pick the chunk; ``workspace`` (device uint8) is
    allocated here when not given.
    """
    import torch

    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError(f"q must be [B, H, n_q, d], caches [n_pages, page_size, H_kv, d]; got {q.shape}, "
                         f"{k_cache.shape}, {v_cache.shape}")
    if not getattr(q, "is_cuda", False):
        raise ValueError("all tensors must be contiguous device tensors")
    _check_on_device(q.device, q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
                     context_lens=context_lens)
    if page_table.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("page_table and context_lens must be int32")
    B, H, n_q, d = q.shape
    n_pages, page_size, H_kv, _ = k_cache.shape
    if page_table.dim() != 2 or page_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("page_table must be [B, max_pages] and context_lens [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    units = torch.cuda.get_device_properties(q.device).multi_processor_count
    split_keys, ws_bytes = fa2_decode_paged_workspace(B, H, H_kv, n_q, d, max_context, split_keys, units)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, "workspace", ws_bytes, q.device)
    if out is None:
        out = torch.empty((B, H, n_q, d), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, n_q), dtype=torch.float32, device=q.device)
    _check_buffer(out, "out", q.shape, o_dtype, q.device)
    _check_buffer(lse, "lse", (B, H, n_q), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = fa2_decode_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, H_kv, n_q, d, scale, page_table.data_ptr(), page_table.shape[1],
                          context_lens.data_ptr(), max_context, page_size, n_pages, split_keys,
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(), handle,
                          _dtype_code(q.dtype), _dtype_code(o_dtype))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_decode_paged")
    return out, lse


def fp8_pack(x, signs=None, stream=None, workspace=None):
    """fa2_fp8_pack on a contiguous bf16 device tensor [B, H, N, d]; returns
    (codes uint8 [B, H, N, d], scales float32 [B, H]).  ``signs``: d values
    of +-1 (the rotation), or None for no rotation."""
    import torch

    if x.dim() != 4 or x.dtype != torch.bfloat16 or not (x.is_cuda and x.is_contiguous()):
        raise ValueError("x must be a contiguous bf16 device tensor [B, H, N, d]")
    B, H, N, d = x.shape
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H), dtype=torch.float32, device=x.device)
    ws_bytes = fa2_fp8_pack_workspace(B, H, N)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    _check_workspace(workspace, "workspace", ws_bytes, x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    sg = None if signs is None else [float(t) for t in (signs.tolist() if hasattr(signs, "tolist") else signs)]
    st = fa2_fp8_pack(x.data_ptr(), B, H, N, d, sg, codes.data_ptr(), scales.data_ptr(), workspace.data_ptr(),
                      workspace.numel() * workspace.element_size(), handle)
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_fp8_pack")
    return codes, scales


def forward_fp8(q, k, v, signs=None, causal: bool = False, scale: float | None = None, o_dtype=None, out=None,
                lse=None, stream=None, packed=None):
    """FP8 attention forward: pack Q and K (fp8_pack with the same signs),
    then fa2_fwd_fp8; returns (o, lse).  q, k, v bf16 device tensors as for
    ``forward``.  ``packed`` = (q8, q_scale, k8, k_scale) skips the packing."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError(f"q must be [B, H, N, d] and k, v [B, H_kv, N, d], got {q.shape}, {k.shape}, {v.shape}")
    if not getattr(q, "is_cuda", False):
        raise ValueError("q, k, v must be device tensors")
    _check_on_device(q.device, q=q, k=k, v=v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if packed is None:
        q8, qs = fp8_pack(q, signs, stream)
        k8, ks = fp8_pack(k, signs, stream)
    else:
        q8, qs, k8, ks = packed
    _check_buffer(q8, "q8", q.shape, torch.uint8, q.device)
    _check_buffer(qs, "q_scale", (B, H), torch.float32, q.device)
    _check_buffer(k8, "k8", k.shape, torch.uint8, q.device)
    _check_buffer(ks, "k_scale", tuple(k.shape[:2]), torch.float32, q.device)
    o_dtype = torch.float32 if o_dtype is None else o_dtype
    if out is None:
        out = torch.empty((B, H, N, d), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buffer(out, "out", q.shape, o_dtype, q.device)
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    st = fa2_fwd_fp8(q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(), v.data_ptr(), out.data_ptr(),
                     lse.data_ptr(), B, H, k.shape[1], N, d, causal, scale, handle, _dtype_code(o_dtype))
    if st != FA2_OK:
        raise Fa2Error(st, "fa2_fwd_fp8")
    return out, lse
