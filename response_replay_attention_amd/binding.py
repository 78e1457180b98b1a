"""Thin Python binding of libls_replay.so (include/ls_replay.h).

Argument marshalling only: every step of the replay path runs in the HIP
library.  PyTorch provides device memory and the stream.  The functions carry
the C names and raise :class:`LsError` on a non-zero status.  There is no
fallback: if the library is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libls_replay.so")

LS_OK = 0
LS_SPLIT_CONTIGUOUS = 0
LS_SPLIT_BLOCK_CYCLIC = 1
LS_SPLIT_EXPLICIT = 2
LS_ACCUMULATE_KV = 1
PAGE_SIZE = 256
LS_NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol include/ls_replay.h declares
EXPORTS = (
    "ls_status_string", "ls_version", "ls_kv_page_table",
    "ls_replay_attn_fwd_workspace", "ls_replay_attn_bwd_workspace",
    "ls_replay_attn_fwd", "ls_replay_attn_fwd_members", "ls_replay_attn_fwd_noalloc",
    "ls_kv_page_append", "ls_lse_merge",
    "ls_replay_attn_bwd",
    "ls_timing_enable", "ls_timing_reset", "ls_timing_read", "ls_calib_mfma",
)


class LsError(RuntimeError):
    def __init__(self, func: str, status: int, text: str):
        super().__init__(f"{func} failed: status {status} ({text})")
        self.status = status


class AttnShape(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("prompt_len", ctypes.c_int64),
        ("resp_len", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q_offset", ctypes.c_int32),
        ("kv_rows", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class PageTable(ctypes.Structure):
    _fields_ = [
        ("l2p", ctypes.c_void_p),
        ("order", ctypes.c_void_p),
        ("split_offsets", ctypes.c_void_p),
        ("split_offsets_host", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
    ]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m response_replay_attention_amd.build`")
    h = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "ls_status_string": (ctypes.c_char_p, [I32]),
        "ls_version": (I32, []),
        "ls_kv_page_table": (I32, [I32, I32, I64, P, I32, I32, I32, I32, P, P, P]),
        "ls_replay_attn_fwd_workspace": (SZ, [P, P]),
        "ls_replay_attn_bwd_workspace": (SZ, [P, P]),
        "ls_replay_attn_fwd": (I32, [P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "ls_replay_attn_fwd_members": (I32, [P, P, I32, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "ls_replay_attn_fwd_noalloc": (I32, [P, P, P, P, P, P, P, P, P, P, P]),
        "ls_kv_page_append": (I32, [I32, I32, I32, P, P, P, P, P, P, I32, P]),
        "ls_lse_merge": (I32, [I32, I64, I32, P, P, P, P, P, P]),
        "ls_replay_attn_bwd": (I32, [P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]),
        "ls_timing_enable": (I32, [I32]),
        "ls_timing_reset": (I32, []),
        "ls_timing_read": (I32, [ctypes.c_char_p, ctypes.POINTER(I32), ctypes.POINTER(ctypes.c_double)]),
        "ls_calib_mfma": (I32, [I32, I32, I32, P, ctypes.POINTER(ctypes.c_double), P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(h, name)
        fn.restype = res
        fn.argtypes = args
    _lib_handle = h
    return h


def _check(func: str, status: int) -> None:
    if status != LS_OK:
        text = lib().ls_status_string(status).decode()
        raise LsError(func, status, text)


def _ptr(t: Optional[torch.Tensor], dtype: Optional[torch.dtype] = None, name: str = "") -> int:
    if t is None:
        return 0
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensor must be contiguous")
    return t.data_ptr()


def _expect(t, shape, name: str) -> None:
    """The kernels trust the sizes in the shape struct: a tensor that does not
    match them would be read or written out of bounds, so refuse it here."""
    if t is None:
        raise ValueError(f"{name}: missing")
    if tuple(int(x) for x in t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _expect_at_least(t, numel: int, name: str) -> None:
    if t is None or t.numel() < numel:
        raise ValueError(f"{name}: needs at least {numel} elements")


def _check_attn_tensors(shape: "AttnShape", pt: "PageTable", q, k_pool, v_pool, k_resp, v_resp,
                        nparts: Optional[int] = None) -> None:
    hq, hkv, d, R = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.resp_len
    kvr = shape.kv_rows if shape.kv_rows else shape.q_offset + R
    _expect(q, (hq, R, d), "q")
    _expect(k_resp, (hkv, kvr, d), "k_resp")
    _expect(v_resp, (hkv, kvr, d), "v_resp")
    if pt.num_pages > 0:
        _expect(k_pool, (pt.num_phys_pages, hkv, shape.page_size, d), "k_pool")
        _expect(v_pool, (pt.num_phys_pages, hkv, shape.page_size, d), "v_pool")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(hq: int, hkv: int, head_dim: int, prompt_len: int, resp_len: int,
               scale: float, page_size: int = PAGE_SIZE, q_offset: int = 0, kv_rows: int = 0,
               flags: int = 0) -> AttnShape:
    return AttnShape(hq, hkv, head_dim, page_size, prompt_len, resp_len, scale, q_offset, kv_rows,
                     flags)


# ----------------------------------------------------------------- C calls

def ls_version() -> int:
    return int(lib().ls_version())


def ls_status_string(status: int) -> str:
    return lib().ls_status_string(status).decode()


def ls_kv_page_table(num_pages: int, page_size: int, prompt_len: int, l2p, num_phys_pages: int,
                     num_splits: int, policy: int, block_pages: int = 1,
                     owner=None) -> Tuple[np.ndarray, np.ndarray]:
    """Host page split.  ``l2p``/``owner``: int32 sequences or None.
    Returns ``(order [num_pages], split_offsets [num_splits+1])`` (int32)."""
    l2p_a = None if l2p is None else np.ascontiguousarray(np.asarray(l2p, dtype=np.int32))
    own_a = None if owner is None else np.ascontiguousarray(np.asarray(owner, dtype=np.int32))
    order = np.zeros(max(num_pages, 1), dtype=np.int32)
    offs = np.zeros(max(num_splits, 0) + 1, dtype=np.int32)
    st = lib().ls_kv_page_table(
        num_pages, page_size, prompt_len,
        None if l2p_a is None else l2p_a.ctypes.data, num_phys_pages, num_splits, policy,
        block_pages, None if own_a is None else own_a.ctypes.data,
        order.ctypes.data, offs.ctypes.data)
    _check("ls_kv_page_table", st)
    return order[:num_pages], offs


def ls_replay_attn_fwd_workspace(shape: AttnShape, pt: PageTable) -> int:
    return int(lib().ls_replay_attn_fwd_workspace(ctypes.byref(shape), ctypes.byref(pt)))


def ls_replay_attn_bwd_workspace(shape: AttnShape, pt: PageTable) -> int:
    return int(lib().ls_replay_attn_bwd_workspace(ctypes.byref(shape), ctypes.byref(pt)))


def ls_replay_attn_fwd(shape: AttnShape, pt: PageTable, q, k_pool, v_pool, k_resp, v_resp,
                       part_o, part_m, part_l, workspace=None, stream=None) -> None:
    bf, f32 = torch.bfloat16, torch.float32
    _check_attn_tensors(shape, pt, q, k_pool, v_pool, k_resp, v_resp)
    rows = (pt.num_splits + 1) * shape.num_q_heads * shape.resp_len
    _expect_at_least(part_o, rows * shape.head_dim, "part_o")
    _expect_at_least(part_m, rows, "part_m")
    _expect_at_least(part_l, rows, "part_l")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ls_replay_attn_fwd(
        ctypes.byref(shape), ctypes.byref(pt), _ptr(q, bf, "q"), _ptr(k_pool, bf, "k_pool"),
        _ptr(v_pool, bf, "v_pool"), _ptr(k_resp, bf, "k_resp"), _ptr(v_resp, bf, "v_resp"),
        _ptr(part_o, f32, "part_o"), _ptr(part_m, f32, "part_m"), _ptr(part_l, f32, "part_l"),
        _ptr(workspace), ws_bytes, _stream(stream))
    _check("ls_replay_attn_fwd", st)


def ls_replay_attn_fwd_noalloc(shape: AttnShape, pt: PageTable, q, k_pool, v_pool, k_resp, v_resp,
                               part_o, part_m, part_l, stream=None) -> None:
    """The forward with the library's own device scratch as its workspace:
    no device memory is allocated by this call or by the library."""
    bf, f32 = torch.bfloat16, torch.float32
    _check_attn_tensors(shape, pt, q, k_pool, v_pool, k_resp, v_resp)
    rows = (pt.num_splits + 1) * shape.num_q_heads * shape.resp_len
    _expect_at_least(part_o, rows * shape.head_dim, "part_o")
    _expect_at_least(part_m, rows, "part_m")
    _expect_at_least(part_l, rows, "part_l")
    st = lib().ls_replay_attn_fwd_noalloc(
        ctypes.byref(shape), ctypes.byref(pt), _ptr(q, bf, "q"), _ptr(k_pool, bf, "k_pool"),
        _ptr(v_pool, bf, "v_pool"), _ptr(k_resp, bf, "k_resp"), _ptr(v_resp, bf, "v_resp"),
        _ptr(part_o, f32, "part_o"), _ptr(part_m, f32, "part_m"), _ptr(part_l, f32, "part_l"),
        _stream(stream))
    _check("ls_replay_attn_fwd_noalloc", st)


def ls_replay_attn_fwd_members(shape: AttnShape, pt: PageTable, member_offsets, member_offsets_dev,
                               q, k_pool, v_pool, k_resp, v_resp, part_o, part_m, part_l,
                               workspace=None, stream=None) -> None:
    """``member_offsets``: host int32 numpy array [G+1]; ``member_offsets_dev``: its device copy
    (an int32 tensor), or None for one member."""
    bf, f32 = torch.bfloat16, torch.float32
    _check_attn_tensors(shape, pt, q, k_pool, v_pool, k_resp, v_resp)
    rows = (pt.num_splits + 1) * shape.num_q_heads * shape.resp_len
    _expect_at_least(part_o, rows * shape.head_dim, "part_o")
    _expect_at_least(part_m, rows, "part_m")
    _expect_at_least(part_l, rows, "part_l")
    offs = np.ascontiguousarray(member_offsets, dtype=np.int32)
    if member_offsets_dev is not None:
        _expect(member_offsets_dev, (offs.size,), "member_offsets_dev")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dev_ptr = 0 if member_offsets_dev is None else _ptr(member_offsets_dev, torch.int32, "member_offsets_dev")
    st = lib().ls_replay_attn_fwd_members(
        ctypes.byref(shape), ctypes.byref(pt), int(offs.size - 1), offs.ctypes.data, dev_ptr,
        _ptr(q, bf, "q"), _ptr(k_pool, bf, "k_pool"), _ptr(v_pool, bf, "v_pool"),
        _ptr(k_resp, bf, "k_resp"), _ptr(v_resp, bf, "v_resp"), _ptr(part_o, f32, "part_o"),
        _ptr(part_m, f32, "part_m"), _ptr(part_l, f32, "part_l"), _ptr(workspace), ws_bytes,
        _stream(stream))
    _check("ls_replay_attn_fwd_members", st)


def ls_kv_page_append(k_chunk, v_chunk, slots, slots_dev, k_pool, v_pool, stream=None) -> None:
    """``k_chunk``/``v_chunk``: bf16 [Hkv, T, d]; ``slots``: host int32 [ceil(T/256)];
    ``slots_dev``: its device copy (int32 tensor); pools bf16 [num_phys, Hkv, 256, d]."""
    bf = torch.bfloat16
    hkv, tokens, d = (int(x) for x in k_chunk.shape)
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    if sl.size != (tokens + PAGE_SIZE - 1) // PAGE_SIZE:
        raise ValueError(f"slots: expected {(tokens + PAGE_SIZE - 1) // PAGE_SIZE} entries, got {sl.size}")
    _expect(v_chunk, (hkv, tokens, d), "v_chunk")
    _expect(slots_dev, (sl.size,), "slots_dev")
    _expect(k_pool, (int(k_pool.shape[0]), hkv, PAGE_SIZE, d), "k_pool")
    _expect(v_pool, tuple(k_pool.shape), "v_pool")
    st = lib().ls_kv_page_append(
        hkv, d, tokens, _ptr(k_chunk, bf, "k_chunk"), _ptr(v_chunk, bf, "v_chunk"),
        sl.ctypes.data, _ptr(slots_dev, torch.int32, "slots_dev"), _ptr(k_pool, bf, "k_pool"),
        _ptr(v_pool, bf, "v_pool"), int(k_pool.shape[0]), _stream(stream))
    _check("ls_kv_page_append", st)


def ls_lse_merge(num_parts: int, rows: int, head_dim: int, part_o, part_m, part_l, o_bf16, lse,
                 stream=None) -> None:
    f32 = torch.float32
    _expect_at_least(part_o, num_parts * rows * head_dim, "part_o")
    _expect_at_least(part_m, num_parts * rows, "part_m")
    _expect_at_least(part_l, num_parts * rows, "part_l")
    _expect_at_least(o_bf16, rows * head_dim, "o")
    _expect_at_least(lse, rows, "lse")
    st = lib().ls_lse_merge(num_parts, rows, head_dim, _ptr(part_o, f32, "part_o"),
                            _ptr(part_m, f32, "part_m"), _ptr(part_l, f32, "part_l"),
                            _ptr(o_bf16, torch.bfloat16, "o"), _ptr(lse, f32, "lse"),
                            _stream(stream))
    _check("ls_lse_merge", st)


def ls_replay_attn_bwd(shape: AttnShape, pt: PageTable, q, k_pool, v_pool, k_resp, v_resp, o, lse,
                       d_o, dq, dk_resp, dv_resp, workspace, stream=None) -> None:
    bf, f32 = torch.bfloat16, torch.float32
    _check_attn_tensors(shape, pt, q, k_pool, v_pool, k_resp, v_resp)
    hq, hkv, d, R = shape.num_q_heads, shape.num_kv_heads, shape.head_dim, shape.resp_len
    kvr = shape.kv_rows if shape.kv_rows else shape.q_offset + R
    for t, name in ((o, "o"), (d_o, "d_o"), (dq, "dq")):
        _expect(t, (hq, R, d), name)
    _expect_at_least(lse, hq * R, "lse")
    _expect(dk_resp, (hkv, kvr, d), "dk_resp")
    _expect(dv_resp, (hkv, kvr, d), "dv_resp")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ls_replay_attn_bwd(
        ctypes.byref(shape), ctypes.byref(pt), _ptr(q, bf, "q"), _ptr(k_pool, bf, "k_pool"),
        _ptr(v_pool, bf, "v_pool"), _ptr(k_resp, bf, "k_resp"), _ptr(v_resp, bf, "v_resp"),
        _ptr(o, bf, "o"), _ptr(lse, f32, "lse"), _ptr(d_o, bf, "d_o"), _ptr(dq, f32, "dq"),
        _ptr(dk_resp, f32, "dk_resp"), _ptr(dv_resp, f32, "dv_resp"), _ptr(workspace), ws_bytes,
        _stream(stream))
    _check("ls_replay_attn_bwd", st)


def ls_timing_enable(on: bool) -> None:
    _check("ls_timing_enable", lib().ls_timing_enable(1 if on else 0))


def ls_timing_reset() -> None:
    _check("ls_timing_reset", lib().ls_timing_reset())


def ls_timing_read(kernel: str) -> Tuple[int, float]:
    n = ctypes.c_int32(0)
    ms = ctypes.c_double(0.0)
    _check("ls_timing_read", lib().ls_timing_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)


def ls_calib_mfma(mode: int, workgroups: int, iters: int, out: torch.Tensor, stream=None) -> float:
    """Launch the MFMA calibration probe; returns the launch's flops.  `out`
    is a float32 device tensor of at least workgroups * 512 elements."""
    _expect_at_least(out, int(workgroups) * 512, "out")
    flops = ctypes.c_double(0.0)
    _check("ls_calib_mfma", lib().ls_calib_mfma(int(mode), int(workgroups), int(iters),
                                                _ptr(out, torch.float32, "out"),
                                                ctypes.byref(flops), _stream(stream)))
    return float(flops.value)
