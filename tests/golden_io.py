"""Reader for the hand-written fixtures in tests/golden/ (no arithmetic)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FMTS = {"q8_0": 0, "q4_0": 1, "bf16": 2}


def load(name):
    fmt = rows = cols = None
    W, xs, ys = None, [], []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "fmt":
                fmt = FMTS[vals[0]]
            elif key == "rows":
                rows = int(vals[0])
            elif key == "cols":
                cols = int(vals[0])
            elif key == "W":
                W = np.array([int(v, 16) for v in vals], dtype=np.uint8)
            elif key == "x":
                xs.append([float(v) for v in vals])
            elif key == "y":
                ys.append([float(v) for v in vals])
    x = np.array(xs, dtype=np.float32)
    y = np.array(ys, dtype=np.float64)
    return dict(fmt=fmt, rows=rows, cols=cols, W=W, x=x, y=y)


def hand_vectors():
    return sorted(n for n in os.listdir(GOLDEN) if n.startswith("e") and n.endswith(".txt"))


def bandwidth_rows():
    out = []
    with open(os.path.join(GOLDEN, "m5_tile_sweep_bandwidth.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                fmt, n_in, n_out, ntok, ous, ogbs, nus, ngbs = line.split()
                out.append((FMTS[fmt], int(n_in), int(n_out), int(ntok), float(ous), float(ogbs),
                            float(nus), float(ngbs)))
    return out


def quant_vectors():
    return sorted(n for n in os.listdir(GOLDEN) if n.startswith("q") and n.endswith(".txt"))


def load_quant(name):
    """A hand-quantized block: fmt, method (0 absmax, 1 Lloyd), v fp32[32], d bits, codes."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "fmt":
                out["fmt"] = FMTS[vals[0]]
            elif key == "method":
                out["method"] = {"absmax": 0, "lloyd": 1}[vals[0]]
            elif key == "v":
                out["v"] = np.array([float(v) for v in vals], dtype=np.float32)
            elif key == "d":
                out["d"] = int(vals[0], 16)
            elif key == "codes":
                out["codes"] = np.array([int(v) for v in vals], dtype=np.int64)
    return out
