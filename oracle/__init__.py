"""CPU oracle for the multi-token block-quantized mat-vec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it.

The arithmetic lives in ``qgemv_oracle.c`` (plain C, fp64); this module only
builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qgemv_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

FMT_Q8_0, FMT_Q4_0, FMT_BF16 = 0, 1, 2


def build(out: str = LIB, mutant: int = 0) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", "-Werror", "-o", out, SRC, "-lm"]
    if mutant:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    tmp = out + f".tmp{os.getpid()}"
    cmd[cmd.index(out)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes front of one compiled oracle library (the real one or a mutant)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(path)
        L = ctypes.CDLL(path)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_fp16_to_f64.restype = ctypes.c_double
        L.oracle_fp16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_row_bytes.restype = i64
        L.oracle_row_bytes.argtypes = [i32, i64]
        L.oracle_packed_bytes.restype = i64
        L.oracle_packed_bytes.argtypes = [i32, i64, i64]
        L.oracle_dequant.restype = i32
        L.oracle_dequant.argtypes = [i32, i64, i64, vp, vp]
        L.oracle_unpack.restype = i32
        L.oracle_unpack.argtypes = [i32, i64, i64, vp, vp, vp]
        L.oracle_gemv.restype = i32
        L.oracle_gemv.argtypes = [i32, i64, i64, i32, vp, vp, i64, vp, vp, vp]
        L.oracle_grouped.restype = i32
        L.oracle_grouped.argtypes = [i32, i64, i64, i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_grouped_per_slot.restype = i32
        L.oracle_grouped_per_slot.argtypes = [i32, i64, i64, i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_f32_to_fp16_array.restype = None
        L.oracle_f32_to_fp16_array.argtypes = [i64, vp, vp]
        L.oracle_quantize_q8_0.restype = i32
        L.oracle_quantize_q8_0.argtypes = [i64, i64, vp, vp]
        L.oracle_quantize_q4_0.restype = i32
        L.oracle_quantize_q4_0.argtypes = [i64, i64, i32, vp, vp]
        self.L = L

    # scalars -----------------------------------------------------------
    def fp16(self, bits: int) -> float:
        return self.L.oracle_fp16_to_f64(int(bits))

    def bf16(self, bits: int) -> float:
        return self.L.oracle_bf16_to_f64(int(bits))

    def row_bytes(self, fmt: int, cols: int) -> int:
        return self.L.oracle_row_bytes(fmt, cols)

    def packed_bytes(self, fmt: int, rows: int, cols: int) -> int:
        return self.L.oracle_packed_bytes(fmt, rows, cols)

    def num_threads(self) -> int:
        return self.L.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        """Threads of the following calls (timing only; results do not depend on it)."""
        self.L.oracle_set_num_threads(int(n))

    # arrays ------------------------------------------------------------
    @staticmethod
    def _u8(W):
        W = np.ascontiguousarray(W)
        return W.view(np.uint8).reshape(-1)

    def dequant(self, fmt: int, rows: int, cols: int, W) -> np.ndarray:
        W = self._u8(W)
        assert W.size >= self.packed_bytes(fmt, rows, cols)
        out = np.empty((rows, cols), dtype=np.float64)
        rc = self.L.oracle_dequant(fmt, rows, cols, W.ctypes.data, out.ctypes.data)
        if rc:
            raise ValueError(f"oracle_dequant rc={rc}")
        return out

    def unpack(self, fmt: int, rows: int, cols: int, W):
        W = self._u8(W)
        d = np.empty((rows, cols // 32), dtype=np.uint16)
        c = np.empty((rows, cols), dtype=np.int32)
        rc = self.L.oracle_unpack(fmt, rows, cols, W.ctypes.data, d.ctypes.data, c.ctypes.data)
        if rc:
            raise ValueError(f"oracle_unpack rc={rc}")
        return d, c

    def gemv(self, fmt: int, rows: int, cols: int, W, x, sel=None):
        """Returns (y, bound), each fp64 [T][rows] (or [T][len(sel)])."""
        W = self._u8(W)
        x = np.ascontiguousarray(x, dtype=np.float32)
        T = x.shape[0]
        assert x.shape == (T, cols)
        assert W.size >= self.packed_bytes(fmt, rows, cols)
        if sel is None:
            nsel, sp = rows, None
        else:
            sel = np.ascontiguousarray(sel, dtype=np.int64)
            nsel, sp = sel.size, sel.ctypes.data
        y = np.empty((T, nsel), dtype=np.float64)
        b = np.empty((T, nsel), dtype=np.float64)
        rc = self.L.oracle_gemv(fmt, rows, cols, T, W.ctypes.data, x.ctypes.data, nsel, sp,
                                y.ctypes.data, b.ctypes.data)
        if rc:
            raise ValueError(f"oracle_gemv rc={rc}")
        return y, b

    def argmax(self, fmt: int, rows: int, cols: int, W, x):
        """The fused LM-head step written out: per token, the row with the largest
        y (the lowest such row on ties) and that y, from the fp64 mat-vec above.
        Returns (idx int64 [T], val fp64 [T], y, bound); y and bound are what the
        acceptance test needs to tell near-ties apart."""
        y, bound = self.gemv(fmt, rows, cols, W, x)
        idx = np.argmax(y, axis=1)  # numpy returns the first (lowest) index of the maximum
        return idx, y[np.arange(y.shape[0]), idx], y, bound

    def gate_up(self, fmt: int, n_experts: int, rows: int, cols: int, ids, Wg, Wu, x):
        """The gate and up projections of the routed experts: the grouped product of
        each table with the tokens' x.  Returns ((yg, bound_g), (yu, bound_u))."""
        return self.grouped(fmt, n_experts, rows, cols, ids, Wg, x), self.grouped(fmt, n_experts, rows, cols, ids, Wu, x)

    def down(self, fmt: int, n_experts: int, rows: int, cols: int, ids, W, h):
        """y[t][j] = W_{ids[t][j]} . h[t][j] for per-slot inputs h [T][topk][cols].
        Returns (y, bound), each fp64 [T][topk][rows]."""
        W = self._u8(W)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        h = np.ascontiguousarray(h, dtype=np.float32)
        T, topk = ids.shape
        assert h.shape == (T, topk, cols)
        assert W.size >= self.packed_bytes(fmt, n_experts * rows, cols)
        y = np.empty((T, topk, rows), dtype=np.float64)
        b = np.empty((T, topk, rows), dtype=np.float64)
        rc = self.L.oracle_grouped_per_slot(fmt, n_experts, rows, cols, T, topk, ids.ctypes.data, W.ctypes.data,
                                            h.ctypes.data, y.ctypes.data, b.ctypes.data)
        if rc:
            raise ValueError(f"oracle_grouped_per_slot rc={rc}")
        return y, b

    def to_fp16_bits(self, v) -> np.ndarray:
        """fp32 values -> binary16 bit patterns (nearest, ties to even)."""
        v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
        out = np.empty(v.size, dtype=np.uint16)
        self.L.oracle_f32_to_fp16_array(v.size, v.ctypes.data, out.ctypes.data)
        return out

    def quantize(self, fmt: int, rows: int, cols: int, src, method: int = 0) -> np.ndarray:
        """fp32 [rows][cols] -> packed Q8_0 (method 0) or Q4_0 (method 0 absmax, 1 Lloyd) bytes."""
        src = np.ascontiguousarray(src, dtype=np.float32)
        assert src.size == rows * cols
        out = np.empty(self.packed_bytes(fmt, rows, cols), dtype=np.uint8)
        if fmt == FMT_Q8_0:
            assert method == 0
            rc = self.L.oracle_quantize_q8_0(rows, cols, src.ctypes.data, out.ctypes.data)
        elif fmt == FMT_Q4_0:
            rc = self.L.oracle_quantize_q4_0(rows, cols, method, src.ctypes.data, out.ctypes.data)
        else:
            raise ValueError("quantizers exist for Q8_0 and Q4_0")
        if rc:
            raise ValueError(f"oracle_quantize rc={rc}")
        return out

    def grouped(self, fmt: int, n_experts: int, rows: int, cols: int, ids, W, x):
        """Returns (y, bound), each fp64 [T][topk][rows]."""
        W = self._u8(W)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        x = np.ascontiguousarray(x, dtype=np.float32)
        T, topk = ids.shape
        assert x.shape == (T, cols)
        assert W.size >= self.packed_bytes(fmt, n_experts * rows, cols)
        y = np.empty((T, topk, rows), dtype=np.float64)
        b = np.empty((T, topk, rows), dtype=np.float64)
        rc = self.L.oracle_grouped(fmt, n_experts, rows, cols, T, topk, ids.ctypes.data, W.ctypes.data,
                                   x.ctypes.data, y.ctypes.data, b.ctypes.data)
        if rc:
            raise ValueError(f"oracle_grouped rc={rc}")
        return y, b


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
