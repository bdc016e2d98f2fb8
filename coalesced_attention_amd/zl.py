"""Thin Python binding over the C ABI of libzl.so (include/zl.h).

Argument marshalling only: every step of the path runs in libzl.so. PyTorch
provides device memory and the stream. Importing this module loads the
library and raises ImportError if it has not been built; there is no
fallback of any kind.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libzl.so")

ZL_OK = 0
STATUS = {0: "ZL_OK", -1: "ZL_ERR_NULL", -2: "ZL_ERR_SHAPE", -3: "ZL_ERR_RANGE",
          -4: "ZL_ERR_OVERLAP", -5: "ZL_ERR_BUFSIZE", -6: "ZL_ERR_ALIGN",
          -7: "ZL_ERR_WORKLIST", -8: "ZL_ERR_HIP", -9: "ZL_ERR_ARG"}
WORKLIST_MAGIC = 0x31574C5A

# Symbols include/zl.h and include/zl_calib.h declare (checked by the CPU tests).
EXPORTS = ("zl_abi_version", "zl_status_string", "zl_last_error", "zl_build_worklist",
           "zl_coalesced_attn_fwd", "zl_merge_partials", "zl_coalesced_attn_bwd",
           "zl_coalesced_attn_fwd_noalloc", "zl_calib_mfma")
CALIB_OPERANDS = {"random": 0, "constant": 1}
# kv_chunk value that splits only the items with more than 131,072 keys, into
# chunks of at most 65,536 keys (ZL_KV_CHUNK_AUTO)
KV_CHUNK_AUTO = -1
# Device scratch the allocation-free forward holds per GPU (ZL_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


class ZlError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS.get(code, code)} ({detail})")
        self.code = code


class Item(ctypes.Structure):
    _fields_ = [("q_off", ctypes.c_int64), ("kv_off", ctypes.c_int64),
                ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("head_begin", ctypes.c_int32), ("head_cnt", ctypes.c_int32)]


class Problem(ctypes.Structure):
    _fields_ = [("q_rows", ctypes.c_int64), ("kv_rows", ctypes.c_int64),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("kv_chunk", ctypes.c_int32)]


class Tile(ctypes.Structure):
    _fields_ = [("q_row0", ctypes.c_int64), ("kv_row0", ctypes.c_int64),
                ("q_rows", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("head", ctypes.c_int32), ("item", ctypes.c_int32)]


class WorklistHeader(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("abi_version", ctypes.c_uint32),
                ("total_bytes", ctypes.c_uint64), ("q_rows", ctypes.c_int64),
                ("kv_rows", ctypes.c_int64), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("block_m", ctypes.c_int32), ("n_items", ctypes.c_int32),
                ("n_tiles", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("cost_c0", ctypes.c_int32), ("tiles_offset", ctypes.c_uint64),
                ("slots_offset", ctypes.c_uint64), ("total_cost", ctypes.c_int64),
                ("max_slot_cost", ctypes.c_int64), ("block_n_bwd", ctypes.c_int32),
                ("n_bwd_tiles", ctypes.c_int32), ("bwd_tiles_offset", ctypes.c_uint64),
                ("bwd_slots_offset", ctypes.c_uint64), ("bwd_max_slot_cost", ctypes.c_int64),
                ("kv_chunk", ctypes.c_int32), ("n_vitems", ctypes.c_int32),
                ("outmap_offset", ctypes.c_uint64), ("n_merges", ctypes.c_int32),
                ("n_dq_tiles", ctypes.c_int32), ("merges_offset", ctypes.c_uint64),
                ("dq_tiles_offset", ctypes.c_uint64), ("dq_slots_offset", ctypes.c_uint64),
                ("ws_rows", ctypes.c_int64), ("pad", ctypes.c_uint8 * 8)]


TILE_DTYPE = np.dtype([("q_row0", "<i8"), ("kv_row0", "<i8"), ("q_rows", "<i4"),
                       ("kv_len", "<i4"), ("head", "<i4"), ("item", "<i4")])
OUTMAP_DTYPE = np.dtype([("o_shift", "<i8"), ("to_workspace", "<i4"), ("reserved", "<i4")])
MERGE_DTYPE = np.dtype([("q_off", "<i8"), ("ws_row0", "<i8"), ("q_len", "<i4"),
                        ("head_begin", "<i4"), ("head_cnt", "<i4"), ("n_parts", "<i4")])

assert ctypes.sizeof(Item) == 32 and ctypes.sizeof(Tile) == 32
assert ctypes.sizeof(WorklistHeader) == 192 and ctypes.sizeof(Problem) == 32


def _load() -> ctypes.CDLL:
    # One HIP runtime per process: torch ships its own libamdhip64.so.7 and
    # loading torch first makes libzl.so's dependency on that soname resolve
    # to the copy torch already uses (a second runtime in the same process
    # does not see the GPU, and its streams would not be torch's).
    import torch  # noqa: F401
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m coalesced_attention_amd.build` "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, fp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.zl_abi_version.restype = ctypes.c_int
    lib.zl_abi_version.argtypes = []
    lib.zl_status_string.restype = ctypes.c_char_p
    lib.zl_status_string.argtypes = [ctypes.c_int]
    lib.zl_last_error.restype = ctypes.c_char_p
    lib.zl_last_error.argtypes = []
    lib.zl_build_worklist.restype = ctypes.c_int
    lib.zl_build_worklist.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(Item), i32, i32, vp,
                                      ctypes.POINTER(ctypes.c_size_t)]
    lib.zl_coalesced_attn_fwd.restype = ctypes.c_int
    lib.zl_coalesced_attn_fwd.argtypes = [vp, vp, vp, vp, vp, fp, fp, fp, vp]
    lib.zl_merge_partials.restype = ctypes.c_int
    lib.zl_merge_partials.argtypes = [i32, i64, i32, i32, i32, i32, fp, fp, i64, fp, fp, vp]
    lib.zl_coalesced_attn_fwd_noalloc.restype = ctypes.c_int
    lib.zl_coalesced_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, fp, fp, vp]
    lib.zl_coalesced_attn_bwd.restype = ctypes.c_int
    lib.zl_coalesced_attn_bwd.argtypes = [vp, vp, vp, vp, vp, fp, fp, vp, fp, fp, fp, fp, vp]
    lib.zl_calib_mfma.restype = ctypes.c_int
    lib.zl_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double), vp]
    return lib


lib = _load()
ABI_VERSION = lib.zl_abi_version()


def _check(rc: int, where: str) -> None:
    if rc != ZL_OK:
        raise ZlError(rc, where, lib.zl_last_error().decode())


def _items_array(items: Iterable) -> ctypes.Array:
    rows = [it.as_tuple() if hasattr(it, "as_tuple") else tuple(it) for it in items]
    arr = (Item * max(1, len(rows)))()
    for i, (q_off, q_len, kv_off, kv_len, h0, hc) in enumerate(rows):
        arr[i] = Item(q_off, kv_off, q_len, kv_len, h0, hc)
    return arr, len(rows)


class Worklist:
    """A built worklist: host bytes (numpy) and, once uploaded, a device copy."""

    def __init__(self, host: np.ndarray):
        self.host = host
        self.header = WorklistHeader.from_buffer(host)
        self.device = None

    @property
    def n_tiles(self) -> int:
        return self.header.n_tiles

    @property
    def n_slots(self) -> int:
        return self.header.n_slots

    def tiles(self) -> np.ndarray:
        h = self.header
        off = h.tiles_offset
        return self.host[off:off + h.n_tiles * 32].view(TILE_DTYPE)

    def slots(self) -> np.ndarray:
        h = self.header
        if h.n_slots == 0:
            return np.zeros(0, np.int32)
        off = h.slots_offset
        return self.host[off:off + 4 * (h.n_slots + 1)].view(np.int32)

    def bwd_tiles(self) -> np.ndarray:
        h = self.header
        off = h.bwd_tiles_offset
        return self.host[off:off + h.n_bwd_tiles * 32].view(TILE_DTYPE)

    def bwd_slots(self) -> np.ndarray:
        h = self.header
        if h.n_slots == 0:
            return np.zeros(0, np.int32)
        off = h.bwd_slots_offset
        return self.host[off:off + 4 * (h.n_slots + 1)].view(np.int32)

    def dq_tiles(self) -> np.ndarray:
        h = self.header
        off = h.dq_tiles_offset
        return self.host[off:off + h.n_dq_tiles * 32].view(TILE_DTYPE)

    def dq_slots(self) -> np.ndarray:
        h = self.header
        if h.n_slots == 0:
            return np.zeros(0, np.int32)
        off = h.dq_slots_offset
        return self.host[off:off + 4 * (h.n_slots + 1)].view(np.int32)

    def outmap(self) -> np.ndarray:
        h = self.header
        off = h.outmap_offset
        return self.host[off:off + h.n_vitems * 16].view(OUTMAP_DTYPE)

    def merges(self) -> np.ndarray:
        h = self.header
        off = h.merges_offset
        return self.host[off:off + h.n_merges * 32].view(MERGE_DTYPE)

    @property
    def workspace_floats(self) -> int:
        """fp32 elements of the forward workspace (0 when nothing is split)."""
        h = self.header
        return h.ws_rows * h.num_heads * (h.head_dim + 1)

    def to(self, device) -> "Worklist":
        import torch
        self.device = torch.from_numpy(self.host).to(device)
        return self

    def host_ptr(self) -> int:
        return self.host.ctypes.data


def default_slots(device=None) -> int:
    """One static slot per compute unit of the device."""
    import torch
    return torch.cuda.get_device_properties(device if device is not None else 0).multi_processor_count


def build_worklist(items: Iterable, q_rows: int, kv_rows: int, num_heads: int, head_dim: int,
                   softmax_scale: float = 0.0, n_slots: int = 0, device=None,
                   kv_chunk: int = 0) -> Worklist:
    """zl_build_worklist. ``items`` are (q_off, q_len, kv_off, kv_len,
    head_begin, head_cnt) tuples or objects with ``as_tuple()``. With
    ``device`` the worklist is also copied there; ``kv_chunk`` > 0 splits
    items with more keys into key chunks merged inside the forward, and
    ``KV_CHUNK_AUTO`` splits only items with more than 131,072 keys, into
    chunks of at most 65,536."""
    arr, n = _items_array(items)
    prob = Problem(q_rows, kv_rows, num_heads, head_dim, softmax_scale, kv_chunk)
    nbytes = ctypes.c_size_t(0)
    _check(lib.zl_build_worklist(ctypes.byref(prob), arr, n, n_slots, None, ctypes.byref(nbytes)),
           "zl_build_worklist(size)")
    host = np.zeros((nbytes.value + 7) // 8, dtype=np.uint64).view(np.uint8)[:nbytes.value]
    _check(lib.zl_build_worklist(ctypes.byref(prob), arr, n, n_slots, host.ctypes.data,
                                 ctypes.byref(nbytes)), "zl_build_worklist")
    wl = Worklist(host)
    if device is not None:
        wl.to(device)
    return wl


def _stream_handle(stream, device) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check_device(device, **tensors):
    """Every tensor must live on ``device`` (a GPU): a host or foreign-device
    pointer handed to a kernel would fault instead of failing."""
    for name, t in tensors.items():
        if t is not None and (not t.is_cuda or t.device != device):
            raise ValueError(f"{name} must be a CUDA tensor on {device}, got {t.device}")


def _check_qkv(wl: Worklist, q, k, v):
    import torch
    h = wl.header
    for name, t, rows in (("q", q, h.q_rows), ("k", k, h.kv_rows), ("v", v, h.kv_rows)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
        if tuple(t.shape) != (rows, h.num_heads, h.head_dim):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, worklist expects "
                             f"{(rows, h.num_heads, h.head_dim)}")
    _check_device(q.device, k=k, v=v)
    if wl.device is not None:
        _check_device(q.device, worklist=wl.device)


def coalesced_attn_fwd(wl: Worklist, q, k, v, o=None, lse=None, stream=None, workspace=None):
    """zl_coalesced_attn_fwd. Returns (o [q_rows, H, d] fp32, lse [q_rows, H] fp32).
    Rows no item covers are left as they were in ``o``/``lse``. A worklist
    that splits items needs a workspace of ``wl.workspace_floats`` fp32
    (allocated here when not given)."""
    import torch
    _check_qkv(wl, q, k, v)
    h = wl.header
    if wl.device is None:
        wl.to(q.device)
    if o is None:
        o = torch.empty((h.q_rows, h.num_heads, h.head_dim), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((h.q_rows, h.num_heads), dtype=torch.float32, device=q.device)
    if o.dtype != torch.float32 or lse.dtype != torch.float32 or not o.is_contiguous() \
            or not lse.is_contiguous():
        raise ValueError("o and lse must be contiguous fp32")
    if tuple(o.shape) != (h.q_rows, h.num_heads, h.head_dim) or tuple(lse.shape) != (h.q_rows, h.num_heads):
        raise ValueError("o / lse shape does not match the worklist")
    _check_device(q.device, o=o, lse=lse, workspace=workspace)
    ws_ptr = None
    if wl.workspace_floats > 0:
        if workspace is None:
            workspace = torch.empty(wl.workspace_floats, dtype=torch.float32, device=q.device)
        if workspace.dtype != torch.float32 or not workspace.is_contiguous() \
                or workspace.numel() < wl.workspace_floats:
            raise ValueError(f"workspace must be contiguous fp32 with >= {wl.workspace_floats} elements")
        ws_ptr = workspace.data_ptr()
    _check(lib.zl_coalesced_attn_fwd(wl.host_ptr(), wl.device.data_ptr(), q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), o.data_ptr(), lse.data_ptr(), ws_ptr,
                                     _stream_handle(stream, q.device)), "zl_coalesced_attn_fwd")
    return o, lse


def coalesced_attn_fwd_noalloc(wl: Worklist, q, k, v, o, lse, stream=None):
    """zl_coalesced_attn_fwd_noalloc: the forward into caller-provided ``o``
    and ``lse`` with the key-chunk partials in the library's own device
    scratch (no allocation here or in the library). The worklist must
    already be on the device."""
    import torch
    _check_qkv(wl, q, k, v)
    h = wl.header
    if wl.device is None:
        raise ValueError("the worklist must already be on the device (Worklist.to)")
    if o.dtype != torch.float32 or lse.dtype != torch.float32 or not o.is_contiguous() \
            or not lse.is_contiguous():
        raise ValueError("o and lse must be contiguous fp32")
    if tuple(o.shape) != (h.q_rows, h.num_heads, h.head_dim) or tuple(lse.shape) != (h.q_rows, h.num_heads):
        raise ValueError("o / lse shape does not match the worklist")
    _check_device(q.device, o=o, lse=lse)
    _check(lib.zl_coalesced_attn_fwd_noalloc(wl.host_ptr(), wl.device.data_ptr(), q.data_ptr(),
                                             k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                             _stream_handle(stream, q.device)),
           "zl_coalesced_attn_fwd_noalloc")
    return o, lse


def coalesced_attn_bwd(wl: Worklist, q, k, v, o, lse, dout, dq=None, dk=None, dv=None, ws=None,
                       stream=None):
    """zl_coalesced_attn_bwd. Gradients ACCUMULATE into dq/dk/dv (fresh zero
    tensors when not given). Returns (dq, dk, dv)."""
    import torch
    _check_qkv(wl, q, k, v)
    h = wl.header
    if wl.device is None:
        wl.to(q.device)
    if dout.dtype != torch.bfloat16 or not dout.is_contiguous() or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("dout must be a contiguous bf16 tensor shaped like q")
    if o.dtype != torch.float32 or tuple(o.shape) != tuple(q.shape) or not o.is_contiguous():
        raise ValueError("o must be the forward's fp32 output")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (h.q_rows, h.num_heads) or not lse.is_contiguous():
        raise ValueError("lse must be the forward's fp32 [q_rows, H] output")
    z = lambda shape: torch.zeros(shape, dtype=torch.float32, device=q.device)
    dq = z(q.shape) if dq is None else dq
    dk = z(k.shape) if dk is None else dk
    dv = z(v.shape) if dv is None else dv
    ws = torch.empty((h.q_rows, h.num_heads), dtype=torch.float32, device=q.device) if ws is None else ws
    for name, t, shape in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, v.shape),
                           ("ws", ws, (h.q_rows, h.num_heads))):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous fp32 of shape {tuple(shape)}")
    _check_device(q.device, o=o, lse=lse, dout=dout, dq=dq, dk=dk, dv=dv, ws=ws)
    _check(lib.zl_coalesced_attn_bwd(wl.host_ptr(), wl.device.data_ptr(), q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                                     _stream_handle(stream, q.device)), "zl_coalesced_attn_bwd")
    return dq, dk, dv


def merge_partials(o, lse, row0: int, n_parts: int, rows: int, part_row_stride: int,
                   head_begin: int, head_cnt: int, o_out=None, lse_out=None, stream=None):
    """zl_merge_partials over parts stored in ``o`` [T, H, d] / ``lse`` [T, H]
    starting at ``row0``. Returns (o_out [rows, H, d], lse_out [rows, H])."""
    import torch
    T, H, d = o.shape
    if o.dtype != torch.float32 or lse.dtype != torch.float32 or not o.is_contiguous() \
            or not lse.is_contiguous() or tuple(lse.shape) != (T, H):
        raise ValueError("o [T,H,d] and lse [T,H] must be contiguous fp32")
    if row0 < 0 or row0 + (n_parts - 1) * part_row_stride + rows > T:
        raise ValueError("parts exceed the buffers")
    if o_out is None:
        o_out = torch.empty((rows, H, d), dtype=torch.float32, device=o.device)
    if lse_out is None:
        lse_out = torch.empty((rows, H), dtype=torch.float32, device=o.device)
    if tuple(o_out.shape) != (rows, H, d) or tuple(lse_out.shape) != (rows, H) \
            or not o_out.is_contiguous() or not lse_out.is_contiguous() \
            or o_out.dtype != torch.float32 or lse_out.dtype != torch.float32:
        raise ValueError("o_out / lse_out must be contiguous fp32 of shapes [rows, H, d] / [rows, H]")
    _check_device(o.device, o=o, lse=lse, o_out=o_out, lse_out=lse_out)
    _check(lib.zl_merge_partials(n_parts, rows, H, head_begin, head_cnt, d,
                                 o.data_ptr() + row0 * H * d * 4, lse.data_ptr() + row0 * H * 4,
                                 part_row_stride, o_out.data_ptr(), lse_out.data_ptr(),
                                 _stream_handle(stream, o.device)), "zl_merge_partials")
    return o_out, lse_out


def calibrate_mfma(operands: str = "random", iters: int = 400_000, stream=None) -> float:
    """TFLOP/s of a register-only stream of bf16 32x32x16 MFMAs on the current
    GPU with the given operand kind ("random" or "constant"): the rate this
    GPU attains under its power limit, for context beside a kernel's rate.
    Synchronous."""
    import torch
    if operands not in CALIB_OPERANDS:
        raise ValueError(f"operands must be one of {sorted(CALIB_OPERANDS)}")
    dev = torch.device("cuda", torch.cuda.current_device())
    out = ctypes.c_double(0.0)
    _check(lib.zl_calib_mfma(CALIB_OPERANDS[operands], int(iters), ctypes.byref(out),
                             _stream_handle(stream, dev)), "zl_calib_mfma")
    return out.value
