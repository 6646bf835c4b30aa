"""ctypes binding of libqgemv.so: the C-ABI names, argument marshalling only.

Every compute step runs in the HIP kernels behind the C ABI; this module never
computes a result itself and fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemv.so")

QG_OK, QG_EINVAL, QG_EALIGN, QG_EUNSUPPORTED, QG_EHIP = 0, 1, 2, 3, 4
QG_FMT_Q8_0, QG_FMT_Q4_0, QG_FMT_BF16 = 0, 1, 2
QG_MAX_T = 4
QG_TILE_FIELDS = 8

EXPORTS = (
    "qgemv_q8_0", "qgemv_q4_0", "qgemv_bf16", "qgemv_grouped_experts", "qgemv_argmax", "qgemv_rows", "qg_packed_bytes",
    "qg_pack_q8_0", "qg_unpack_q8_0", "qg_pack_q4_0", "qg_unpack_q4_0", "qg_query_tile",
    "qg_status_string", "qg_last_error", "qg_quantize_q8_0", "qg_quantize_q4_0", "qgemv_experts_gate_up",
    "qgemv_experts_down", "qg_read_probe", "qgemv_argmax_noalloc",
)
QG_Q4_ABSMAX, QG_Q4_LLOYD = 0, 1


class QGError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({status_string(status)}): {detail}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libqgemv.so (built in-tree by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    for name in ("qgemv_q8_0", "qgemv_q4_0", "qgemv_bf16"):
        f = getattr(L, name)
        f.restype = i32
        f.argtypes = [i64, i64, i32, vp, vp, vp, vp]
    L.qgemv_grouped_experts.restype = i32
    L.qgemv_grouped_experts.argtypes = [i32, i64, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    L.qgemv_experts_gate_up.restype = i32
    L.qgemv_experts_gate_up.argtypes = [i32, i64, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.qgemv_experts_down.restype = i32
    L.qgemv_experts_down.argtypes = [i32, i64, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    L.qgemv_rows.restype = i32
    L.qgemv_rows.argtypes = [i32, i64, i64, i64, vp, i32, vp, vp, vp, vp]
    L.qgemv_argmax.restype = i32
    L.qgemv_argmax.argtypes = [i32, i64, i64, i32, vp, vp, vp, vp, vp, vp]
    L.qgemv_argmax_noalloc.restype = i32
    L.qgemv_argmax_noalloc.argtypes = [i32, i64, i64, i32, vp, vp, vp, vp, vp]
    L.qg_packed_bytes.restype = sz
    L.qg_packed_bytes.argtypes = [i32, i64, i64]
    for name in ("qg_pack_q8_0", "qg_unpack_q8_0", "qg_pack_q4_0", "qg_unpack_q4_0"):
        f = getattr(L, name)
        f.restype = i32
        f.argtypes = [i64, i64, vp, vp, vp]
    L.qg_quantize_q8_0.restype = i32
    L.qg_quantize_q8_0.argtypes = [i64, i64, vp, vp, vp]
    L.qg_quantize_q4_0.restype = i32
    L.qg_quantize_q4_0.argtypes = [i64, i64, i32, vp, vp, vp]
    L.qg_read_probe.restype = i32
    L.qg_read_probe.argtypes = [vp, i64, i64, ctypes.c_uint32, vp, vp]
    L.qg_query_tile.restype = i32
    L.qg_query_tile.argtypes = [i32, i64, i64, i32, ctypes.POINTER(ctypes.c_int)]
    L.qg_status_string.restype = ctypes.c_char_p
    L.qg_status_string.argtypes = [i32]
    L.qg_last_error.restype = ctypes.c_char_p
    L.qg_last_error.argtypes = []
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().qg_status_string(status).decode()


def last_error() -> str:
    return load().qg_last_error().decode()


def check(status: int, where: str) -> None:
    if status != QG_OK:
        raise QGError(status, where, last_error())


# --- the C-ABI entry points, same names, raw pointers / integers -------------
def qgemv_q8_0(rows, cols, T, W, x, y, stream=None) -> int:
    return load().qgemv_q8_0(rows, cols, T, W, x, y, stream)


def qgemv_q4_0(rows, cols, T, W, x, y, stream=None) -> int:
    return load().qgemv_q4_0(rows, cols, T, W, x, y, stream)


def qgemv_bf16(rows, cols, T, W, x, y, stream=None) -> int:
    return load().qgemv_bf16(rows, cols, T, W, x, y, stream)


def qgemv_grouped_experts(fmt, n_experts, rows, cols, T, topk, ids, W, x, y, stream=None) -> int:
    return load().qgemv_grouped_experts(fmt, n_experts, rows, cols, T, topk, ids, W, x, y, stream)


def qgemv_experts_gate_up(fmt, n_experts, rows, cols, T, topk, ids, Wg, Wu, x, yg, yu, stream=None) -> int:
    return load().qgemv_experts_gate_up(fmt, n_experts, rows, cols, T, topk, ids, Wg, Wu, x, yg, yu, stream)


def qgemv_experts_down(fmt, n_experts, rows, cols, T, topk, ids, W, h, y, stream=None) -> int:
    return load().qgemv_experts_down(fmt, n_experts, rows, cols, T, topk, ids, W, h, y, stream)


def qgemv_rows(fmt, rows, cols, n_sel, ids, T, W, x, y, stream=None) -> int:
    return load().qgemv_rows(fmt, rows, cols, n_sel, ids, T, W, x, y, stream)


def qgemv_argmax(fmt, rows, cols, T, W, x, work, idx, val, stream=None) -> int:
    return load().qgemv_argmax(fmt, rows, cols, T, W, x, work, idx, val, stream)


def qgemv_argmax_noalloc(fmt, rows, cols, T, W, x, idx, val, stream=None) -> int:
    return load().qgemv_argmax_noalloc(fmt, rows, cols, T, W, x, idx, val, stream)


def qg_packed_bytes(fmt, rows, cols) -> int:
    return load().qg_packed_bytes(fmt, rows, cols)


def qg_pack_q8_0(rows, cols, d_bits, codes, out) -> int:
    return load().qg_pack_q8_0(rows, cols, d_bits, codes, out)


def qg_unpack_q8_0(rows, cols, packed, d_bits, codes) -> int:
    return load().qg_unpack_q8_0(rows, cols, packed, d_bits, codes)


def qg_pack_q4_0(rows, cols, d_bits, codes, out) -> int:
    return load().qg_pack_q4_0(rows, cols, d_bits, codes, out)


def qg_unpack_q4_0(rows, cols, packed, d_bits, codes) -> int:
    return load().qg_unpack_q4_0(rows, cols, packed, d_bits, codes)


def qg_quantize_q8_0(rows, cols, src, dst, stream=None) -> int:
    return load().qg_quantize_q8_0(rows, cols, src, dst, stream)


def qg_quantize_q4_0(rows, cols, method, src, dst, stream=None) -> int:
    return load().qg_quantize_q4_0(rows, cols, method, src, dst, stream)


def qg_read_probe(src, nbytes, max_groups, magic, out, stream=None) -> int:
    return load().qg_read_probe(src, nbytes, max_groups, magic, out, stream)


def qg_query_tile(fmt, rows, cols, T):
    out = (ctypes.c_int * QG_TILE_FIELDS)()
    st = load().qg_query_tile(fmt, rows, cols, T, out)
    return st, list(out)
