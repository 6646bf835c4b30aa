"""Torch-facing helpers over the C ABI: PyTorch supplies device memory and the
current stream; the computation is entirely the library's HIP kernels."""
from __future__ import annotations

import numpy as np

from . import _lib

FMT = {"q8_0": _lib.QG_FMT_Q8_0, "q4_0": _lib.QG_FMT_Q4_0, "bf16": _lib.QG_FMT_BF16}
_ENTRY = {_lib.QG_FMT_Q8_0: _lib.qgemv_q8_0, _lib.QG_FMT_Q4_0: _lib.qgemv_q4_0, _lib.QG_FMT_BF16: _lib.qgemv_bf16}


def _fmt(fmt):
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def _stream(torch, device):
    return torch.cuda.current_stream(device).cuda_stream


def _require_device(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# Shapes, dtypes and sizes are checked before anything touches the device, so a
# wrong buffer is refused before the kernels could read or write past its end.
def _check_x(torch, x, name="x"):
    if x.dtype != torch.float32 or x.dim() != 2:
        raise ValueError(f"{name} must be fp32 [T][cols]")


def _check_ids(torch, ids, dims, what):
    if ids.dtype != torch.int32 or ids.dim() != dims:
        raise ValueError(f"ids must be int32 {what}")


def _check_weights(W, need, what="the shape"):
    have = W.numel() * W.element_size()
    if need == 0 or have < need:
        raise ValueError(f"W holds {have} bytes, {what} needs {need}")


def _check_out(torch, out, numel, name="out", dtype=None):
    dtype = torch.float32 if dtype is None else dtype
    if out.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {out.dtype}")
    if out.numel() < numel:
        raise ValueError(f"{name} holds {out.numel()} elements, the call writes {numel}")


def _same_device(x, *others):
    for t, name in others:
        if t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")


def gemv(fmt, W, x, rows: int, out=None):
    """y[T][rows] = W . x[t] for packed weights W (uint8 device tensor) and x fp32 [T][cols]."""
    import torch
    f = _fmt(fmt)
    _check_x(torch, x)
    T, cols = x.shape
    _check_weights(W, _lib.qg_packed_bytes(f, rows, cols))
    if out is not None:
        _check_out(torch, out, T * rows)
    _require_device(W, "W")
    _require_device(x, "x")
    if out is None:
        out = torch.empty((T, rows), dtype=torch.float32, device=x.device)
    _require_device(out, "out")
    _same_device(x, (W, "W"), (out, "out"))
    st = _ENTRY[f](rows, cols, T, W.data_ptr(), x.data_ptr(), out.data_ptr(), _stream(torch, x.device))
    _lib.check(st, "qgemv")
    return out


def gemv_rows(fmt, W, x, rows: int, ids, out=None):
    """y[T][len(ids)] = W[ids[i]] . x[t]: the mat-vec over a subset of W's rows
    (ids int32 on the device; an id outside [0, rows) gives a NaN column)."""
    import torch
    f = _fmt(fmt)
    _check_x(torch, x)
    _check_ids(torch, ids, 1, "[n_sel]")
    T, cols = x.shape
    _check_weights(W, _lib.qg_packed_bytes(f, rows, cols))
    if out is not None:
        _check_out(torch, out, T * ids.numel())
    for t, n in ((W, "W"), (x, "x"), (ids, "ids")):
        _require_device(t, n)
    if out is None:
        out = torch.empty((T, ids.numel()), dtype=torch.float32, device=x.device)
    _require_device(out, "out")
    _same_device(x, (W, "W"), (ids, "ids"), (out, "out"))
    st = _lib.qgemv_rows(f, rows, cols, ids.numel(), ids.data_ptr(), T, W.data_ptr(), x.data_ptr(), out.data_ptr(),
                         _stream(torch, x.device))
    _lib.check(st, "qgemv_rows")
    return out


def argmax(fmt, W, x, rows: int, work=None):
    """(idx int32 [T], val fp32 [T]): per token, the row with the largest W . x[t]
    (lowest row on ties) and its value, without writing the [T][rows] product."""
    import torch
    f = _fmt(fmt)
    _check_x(torch, x)
    T, cols = x.shape
    _check_weights(W, _lib.qg_packed_bytes(f, rows, cols))
    if work is not None:
        _check_out(torch, work, T, "work", torch.int64)
    _require_device(W, "W")
    _require_device(x, "x")
    if work is None:
        work = torch.empty(T, dtype=torch.int64, device=x.device)
    _require_device(work, "work")
    _same_device(x, (W, "W"), (work, "work"))
    idx = torch.empty(T, dtype=torch.int32, device=x.device)
    val = torch.empty(T, dtype=torch.float32, device=x.device)
    st = _lib.qgemv_argmax(f, rows, cols, T, W.data_ptr(), x.data_ptr(), work.data_ptr(), idx.data_ptr(), val.data_ptr(),
                           _stream(torch, x.device))
    _lib.check(st, "qgemv_argmax")
    return idx, val


def grouped_experts(fmt, W, x, ids, n_experts: int, rows: int, out=None):
    """y[T][topk][rows] = W_{ids[t][j]} . x[t]; ids int32 [T][topk] on the device."""
    import torch
    f = _fmt(fmt)
    _check_x(torch, x)
    _check_ids(torch, ids, 2, "[T][topk]")
    T, cols = x.shape
    topk = ids.shape[1]
    if ids.shape[0] != T:
        raise ValueError("ids and x disagree on T")
    _check_weights(W, _lib.qg_packed_bytes(f, rows * n_experts, cols), "the experts")
    if out is not None:
        _check_out(torch, out, T * topk * rows)
    for t, n in ((W, "W"), (x, "x"), (ids, "ids")):
        _require_device(t, n)
    if out is None:
        out = torch.empty((T, topk, rows), dtype=torch.float32, device=x.device)
    _require_device(out, "out")
    _same_device(x, (W, "W"), (ids, "ids"), (out, "out"))
    st = _lib.qgemv_grouped_experts(f, n_experts, rows, cols, T, topk, ids.data_ptr(), W.data_ptr(), x.data_ptr(),
                                    out.data_ptr(), _stream(torch, x.device))
    _lib.check(st, "qgemv_grouped_experts")
    return out


def quantize(fmt, src, method: str = "absmax", out=None):
    """Packed Q8_0 / Q4_0 bytes (uint8 device tensor) of fp32 [rows][cols] values
    on the device; Q4_0 takes method "absmax" or "lloyd"."""
    import torch
    f = _fmt(fmt)
    if src.dtype != torch.float32 or src.dim() != 2:
        raise ValueError("src must be fp32 [rows][cols]")
    rows, cols = src.shape
    need = _lib.qg_packed_bytes(f, rows, cols)
    if f not in (_lib.QG_FMT_Q8_0, _lib.QG_FMT_Q4_0) or need == 0:
        raise ValueError("quantizers exist for q8_0 and q4_0 with cols a multiple of 32")
    if out is not None and out.numel() * out.element_size() < need:
        raise ValueError(f"out holds {out.numel() * out.element_size()} bytes, the shape needs {need}")
    _require_device(src, "src")
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=src.device)
    _require_device(out, "out")
    _same_device(src, (out, "out"))
    s = _stream(torch, src.device)
    if f == _lib.QG_FMT_Q8_0:
        if method != "absmax":
            raise ValueError("q8_0 has the absmax quantizer only")
        st = _lib.qg_quantize_q8_0(rows, cols, src.data_ptr(), out.data_ptr(), s)
    else:
        m = {"absmax": _lib.QG_Q4_ABSMAX, "lloyd": _lib.QG_Q4_LLOYD}[method]
        st = _lib.qg_quantize_q4_0(rows, cols, m, src.data_ptr(), out.data_ptr(), s)
    _lib.check(st, "qg_quantize")
    return out


def _experts_checks(torch, f, tables, ids, n_experts, rows, cols):
    _check_ids(torch, ids, 2, "[T][topk]")
    need = _lib.qg_packed_bytes(f, rows * n_experts, cols)
    for W in tables:
        _check_weights(W, need, "the experts")


def experts_gate_up(fmt, Wg, Wu, x, ids, n_experts: int, rows: int):
    """(yg, yu), each [T][topk][rows]: the gate and up projections of the experts
    each token picked (ids int32 [T][topk]), both tables streamed by one launch."""
    import torch
    f = _fmt(fmt)
    _check_x(torch, x)
    T, cols = x.shape
    _experts_checks(torch, f, (Wg, Wu), ids, n_experts, rows, cols)
    if ids.shape[0] != T:
        raise ValueError("ids and x disagree on T")
    for t, n in ((Wg, "Wg"), (Wu, "Wu"), (x, "x"), (ids, "ids")):
        _require_device(t, n)
    _same_device(x, (Wg, "Wg"), (Wu, "Wu"), (ids, "ids"))
    topk = ids.shape[1]
    yg = torch.empty((T, topk, rows), dtype=torch.float32, device=x.device)
    yu = torch.empty_like(yg)
    st = _lib.qgemv_experts_gate_up(f, n_experts, rows, cols, T, topk, ids.data_ptr(), Wg.data_ptr(), Wu.data_ptr(),
                                    x.data_ptr(), yg.data_ptr(), yu.data_ptr(), _stream(torch, x.device))
    _lib.check(st, "qgemv_experts_gate_up")
    return yg, yu


def experts_down(fmt, W, h, ids, n_experts: int, rows: int):
    """y[T][topk][rows] = W_{ids[t][j]} . h[t][j] for the per-pair inputs h [T][topk][cols]."""
    import torch
    f = _fmt(fmt)
    if h.dtype != torch.float32 or h.dim() != 3 or tuple(h.shape[:2]) != tuple(ids.shape):
        raise ValueError("h must be fp32 [T][topk][cols] matching ids")
    T, topk, cols = h.shape
    _experts_checks(torch, f, (W,), ids, n_experts, rows, cols)
    for t, n in ((W, "W"), (h, "h"), (ids, "ids")):
        _require_device(t, n)
    _same_device(h, (W, "W"), (ids, "ids"))
    y = torch.empty((T, topk, rows), dtype=torch.float32, device=h.device)
    st = _lib.qgemv_experts_down(f, n_experts, rows, cols, T, topk, ids.data_ptr(), W.data_ptr(), h.data_ptr(),
                                 y.data_ptr(), _stream(torch, h.device))
    _lib.check(st, "qgemv_experts_down")
    return y


def pack_q8_0(d_bits: np.ndarray, codes: np.ndarray) -> np.ndarray:
    rows, cols = codes.shape
    d = np.ascontiguousarray(d_bits, dtype=np.uint16)
    c = np.ascontiguousarray(codes, dtype=np.int8)
    out = np.empty(_lib.qg_packed_bytes(_lib.QG_FMT_Q8_0, rows, cols), dtype=np.uint8)
    _lib.check(_lib.qg_pack_q8_0(rows, cols, d.ctypes.data, c.ctypes.data, out.ctypes.data), "qg_pack_q8_0")
    return out


def unpack_q8_0(packed: np.ndarray, rows: int, cols: int):
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    d = np.empty((rows, cols // 32), dtype=np.uint16)
    c = np.empty((rows, cols), dtype=np.int8)
    _lib.check(_lib.qg_unpack_q8_0(rows, cols, p.ctypes.data, d.ctypes.data, c.ctypes.data), "qg_unpack_q8_0")
    return d, c


def pack_q4_0(d_bits: np.ndarray, codes: np.ndarray) -> np.ndarray:
    rows, cols = codes.shape
    d = np.ascontiguousarray(d_bits, dtype=np.uint16)
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(_lib.qg_packed_bytes(_lib.QG_FMT_Q4_0, rows, cols), dtype=np.uint8)
    _lib.check(_lib.qg_pack_q4_0(rows, cols, d.ctypes.data, c.ctypes.data, out.ctypes.data), "qg_pack_q4_0")
    return out


def unpack_q4_0(packed: np.ndarray, rows: int, cols: int):
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    d = np.empty((rows, cols // 32), dtype=np.uint16)
    c = np.empty((rows, cols), dtype=np.uint8)
    _lib.check(_lib.qg_unpack_q4_0(rows, cols, p.ctypes.data, d.ctypes.data, c.ctypes.data), "qg_unpack_q4_0")
    return d, c


def query_tile(fmt, rows: int, cols: int, T: int) -> dict:
    st, t = _lib.qg_query_tile(_fmt(fmt), rows, cols, T)
    _lib.check(st, "qg_query_tile")
    keys = ("lanes_per_row", "rows_per_batch", "waves_per_wg", "k_slice", "rows_per_wg", "mfma", "kind", "depth")
    return dict(zip(keys, t))
