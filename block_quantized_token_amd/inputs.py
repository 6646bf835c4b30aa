"""Seeded synthetic inputs for the multi-token block-quantized mat-vec.

This module is shared by the CPU oracle's tests, the GPU parity tests, the
smoke check and the benchmark.  It only draws random values and lays them out
as bytes; it holds none of the method's arithmetic (no dequantisation, no dot
products), so neither side of a parity check borrows the other's maths from it.

Byte layouts (read from the format names the pages use -- Q8_0, Q4_0, BF16 --
in the ggml family's convention; both the M5 multi-token audit, section 2.1
table, and the M2 Max "Where the time goes" page's mat-vec table quote Q8_0 at
34 bytes per 32 weights and Q4_0 at 18 bytes per 32):

* Q8_0 block (34 B): little-endian fp16 scale ``d`` then 32 signed int8 codes.
* Q4_0 block (18 B): little-endian fp16 scale ``d`` then 16 bytes; byte ``j``
  holds code ``j`` in its low nibble and code ``j + 16`` in its high nibble.
* BF16: one little-endian bfloat16 per weight.

Rows are stored one after another; inside a row the blocks run along k.

Value recipe (one generator per call, numpy PCG64, fixed draw order: scales,
then codes, then activations, then expert ids):

* Q8_0: ``d = fp16(|N(0,1)| * 0.01)`` (round to nearest even), codes uniform
  integers in [-127, 127].
* Q4_0: ``d = fp16(|N(0,1)| * 0.02)``, codes uniform integers in [0, 15].
* BF16: ``bf16(N(0,1) * 0.02)`` (fp64 -> fp32 -> bf16, round to nearest even).
* activations: fp32 N(0,1), drawn as ``[4][cols]``; a T-token input is the
  first T rows, so lower T is a prefix of T = 4.
* grouped experts: ``ids = permutation(n_experts)[:T*topk]`` reshaped
  ``[T][topk]`` -- distinct experts, none shared across tokens.
"""
from __future__ import annotations

import numpy as np

FMT_Q8_0 = 0
FMT_Q4_0 = 1
FMT_BF16 = 2
FMT_NAMES = {FMT_Q8_0: "q8_0", FMT_Q4_0: "q4_0", FMT_BF16: "bf16"}

Q8_0_BLOCK = np.dtype([("d", "<u2"), ("qs", "i1", (32,))])
Q4_0_BLOCK = np.dtype([("d", "<u2"), ("qs", "u1", (16,))])
assert Q8_0_BLOCK.itemsize == 34 and Q4_0_BLOCK.itemsize == 18

MAX_T = 4


def rng_for(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- raw fields
def fp16_bits(values: np.ndarray) -> np.ndarray:
    """fp64 values -> IEEE binary16 bit patterns, round to nearest even."""
    return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(values: np.ndarray) -> np.ndarray:
    """fp64 values -> fp32 -> bfloat16 bit patterns, round to nearest even."""
    b = np.asarray(values, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def q8_0_fields(rng: np.random.Generator, rows: int, cols: int, scale_sigma: float = 0.01):
    assert cols % 32 == 0
    d = fp16_bits(np.abs(rng.standard_normal((rows, cols // 32))) * scale_sigma)
    codes = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    return d, codes


def q4_0_fields(rng: np.random.Generator, rows: int, cols: int, scale_sigma: float = 0.02):
    assert cols % 32 == 0
    d = fp16_bits(np.abs(rng.standard_normal((rows, cols // 32))) * scale_sigma)
    codes = rng.integers(0, 16, size=(rows, cols), dtype=np.uint8)
    return d, codes


def bf16_fields(rng: np.random.Generator, rows: int, cols: int, sigma: float = 0.02):
    return bf16_bits(rng.standard_normal((rows, cols)) * sigma)


def activations(rng: np.random.Generator, cols: int, T: int = MAX_T) -> np.ndarray:
    x = rng.standard_normal((MAX_T, cols)).astype(np.float32)
    return np.ascontiguousarray(x[:T])


def dense_fp32(rng: np.random.Generator, rows: int, cols: int, sigma: float = 0.02) -> np.ndarray:
    """fp32 [rows][cols] values to quantize: N(0,1) * sigma, as a weight matrix is
    initialised; one block in 16 has one element 20x larger (an outlier), one in
    64 is all zero and one in 64 is scaled by 1e-6 (its fp16 scale underflows)."""
    v = rng.standard_normal((rows, cols)) * sigma
    blocks = v.reshape(rows * (cols // 32), 32)
    kind = rng.random(blocks.shape[0])
    pos = rng.integers(0, 32, blocks.shape[0])
    out = kind < 1 / 16
    blocks[out, pos[out]] *= 20
    blocks[(kind >= 1 / 16) & (kind < 1 / 16 + 1 / 64)] = 0
    blocks[kind >= 1 - 1 / 64] *= 1e-6
    return blocks.reshape(rows, cols).astype(np.float32)


def expert_ids(rng: np.random.Generator, n_experts: int, T: int, topk: int) -> np.ndarray:
    assert T * topk <= n_experts
    return rng.permutation(n_experts)[: T * topk].astype(np.int32).reshape(T, topk)


# Distinct experts over the T tokens of a verify pass at the M5 audit's expert
# overlap (share 0.65: 18.1 distinct at T = 3 and 21.3 at T = 4 in its section
# 2.2; T = 2 taken as 10 + 0.35 * 10, rounded); share 0 is T * topk.
UNIQUE_AT_SHARE_065 = {1: 10, 2: 14, 3: 18, 4: 21}


def expert_ids_shared(rng: np.random.Generator, n_experts: int, T: int, topk: int, unique: int) -> np.ndarray:
    """[T][topk] ids naming exactly ``unique`` distinct experts, each token's topk
    distinct.  Token 0 takes topk new experts; the other new experts are dealt to
    tokens 1..T-1 in turn; each token fills its other slots with experts that
    earlier tokens use, drawn at random; each row is shuffled."""
    assert topk <= unique <= min(T * topk, n_experts) and (T > 1 or unique == topk)
    pool = rng.permutation(n_experts)[:unique]
    ids = np.empty((T, topk), dtype=np.int32)
    ids[0] = pool[:topk]
    new = pool[topk:]
    share = [0] * T
    for i in range(len(new)):
        share[1 + i % (T - 1)] += 1
    assert max(share) <= topk
    used, k = list(pool[:topk]), 0
    for t in range(1, T):
        mine = list(new[k:k + share[t]])
        k += share[t]
        pick = list(rng.choice(np.array(used), topk - len(mine), replace=False))
        row = np.array(mine + pick, dtype=np.int32)
        rng.shuffle(row)
        ids[t] = row
        used += mine
    return ids


# ------------------------------------------------------------- byte layout
def pack_q8_0(d: np.ndarray, codes: np.ndarray) -> np.ndarray:
    rows, nb = d.shape
    blk = np.empty((rows, nb), dtype=Q8_0_BLOCK)
    blk["d"] = d
    blk["qs"] = codes.reshape(rows, nb, 32)
    return blk.reshape(-1).view(np.uint8)


def pack_q4_0(d: np.ndarray, codes: np.ndarray) -> np.ndarray:
    rows, nb = d.shape
    c = codes.reshape(rows, nb, 32).astype(np.uint8)
    blk = np.empty((rows, nb), dtype=Q4_0_BLOCK)
    blk["d"] = d
    blk["qs"] = c[:, :, :16] | (c[:, :, 16:] << 4)
    return blk.reshape(-1).view(np.uint8)


def pack_bf16(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits.astype("<u2")).reshape(-1).view(np.uint8)


def packed_row_bytes(fmt: int, cols: int) -> int:
    if fmt == FMT_Q8_0:
        return cols // 32 * 34
    if fmt == FMT_Q4_0:
        return cols // 32 * 18
    if fmt == FMT_BF16:
        return cols * 2
    raise ValueError(fmt)


def weights(rng: np.random.Generator, fmt: int, rows: int, cols: int) -> np.ndarray:
    """Draw and pack one weight matrix; returns the packed bytes (uint8, 1-D)."""
    if fmt == FMT_Q8_0:
        return pack_q8_0(*q8_0_fields(rng, rows, cols))
    if fmt == FMT_Q4_0:
        return pack_q4_0(*q4_0_fields(rng, rows, cols))
    if fmt == FMT_BF16:
        return pack_bf16(bf16_fields(rng, rows, cols))
    raise ValueError(fmt)


def weights_chunked(seed: int, fmt: int, rows: int, cols: int, chunk_rows: int = 16384) -> np.ndarray:
    """Large matrices drawn chunk by chunk (one child generator per chunk, from
    ``SeedSequence(seed).spawn``) so the LM-head case never holds fp64
    temporaries for all 1.27 G codes at once."""
    out = np.empty(rows * packed_row_bytes(fmt, cols), dtype=np.uint8)
    nchunks = (rows + chunk_rows - 1) // chunk_rows
    children = np.random.SeedSequence(seed).spawn(nchunks)
    rb = packed_row_bytes(fmt, cols)
    for i, ss in enumerate(children):
        r0 = i * chunk_rows
        r1 = min(rows, r0 + chunk_rows)
        out[r0 * rb:r1 * rb] = weights(np.random.default_rng(ss), fmt, r1 - r0, cols)
    return out


# ------------------------------------------------------------ the workloads
# name -> (fmt, rows, cols, T values).  Shapes follow the pages' tensors:
# 2560 hidden, the 10240-row attn_qkv, 6144 n_in, the 8192x2560 mat-vec of the
# M2 Max table and the 248,320 x 5,120 LM head.
CONFIGS = {
    "c1_q8_0_2560x2560": (FMT_Q8_0, 2560, 2560, (1, 2, 3, 4)),
    "c2a_q8_0_10240x2560": (FMT_Q8_0, 10240, 2560, (1, 2, 3, 4)),
    "c2b_q8_0_2560x6144": (FMT_Q8_0, 2560, 6144, (1, 2, 3, 4)),
    "c3_q4_0_8192x2560": (FMT_Q4_0, 8192, 2560, (1, 2, 3, 4)),
    "c3_bf16_8192x2560": (FMT_BF16, 8192, 2560, (1, 2, 3, 4)),
    "c4_q8_0_248320x5120": (FMT_Q8_0, 248320, 5120, (1, 2, 3, 4)),
}
GROUPED = {"c5_q4_0_experts": dict(fmt=FMT_Q4_0, n_experts=256, rows=512, cols=2560, T=4, topk=10)}
# The routed-experts layer around it: gate and up of [512][2560] each, down of
# [2560][512], 256 experts, Q4_0 (the C5 expert shape, the down projection its
# transpose).
EXPERT_LAYER = dict(fmt=FMT_Q4_0, n_experts=256, n_ff=512, n_embd=2560, topk=10)


def dense_case(name: str, seed: int = 0):
    """Packed weights and x[4][cols] for one dense workload."""
    fmt, rows, cols, _ = CONFIGS[name]
    if rows * packed_row_bytes(fmt, cols) > (1 << 28):
        W = weights_chunked(seed, fmt, rows, cols)
        rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(1 + (rows + 16383) // 16384)[-1])
    else:
        rng = rng_for(seed)
        W = weights(rng, fmt, rows, cols)
    x = activations(rng, cols)
    return dict(fmt=fmt, rows=rows, cols=cols, W=W, x=x)


def grouped_case(name: str = "c5_q4_0_experts", seed: int = 0):
    g = GROUPED[name]
    rng = rng_for(seed)
    W = weights(rng, g["fmt"], g["n_experts"] * g["rows"], g["cols"])
    x = activations(rng, g["cols"], g["T"])
    ids = expert_ids(rng, g["n_experts"], g["T"], g["topk"])
    return dict(g, W=W, x=x, ids=ids)


def expert_layer_case(T: int, unique: int, seed: int = 0):
    """Gate, up and down tables, x [T][n_embd], per-slot inputs h [T][topk][n_ff]
    and ids with ``unique`` distinct experts, for the routed-experts layer."""
    g = EXPERT_LAYER
    rng = rng_for(seed)
    E, ff, emb = g["n_experts"], g["n_ff"], g["n_embd"]
    Wg = weights(rng, g["fmt"], E * ff, emb)
    Wu = weights(rng, g["fmt"], E * ff, emb)
    Wd = weights(rng, g["fmt"], E * emb, ff)
    x = activations(rng, emb, T)
    h = rng.standard_normal((T, g["topk"], ff)).astype(np.float32)
    ids = expert_ids_shared(rng, E, T, g["topk"], unique)
    return dict(g, T=T, Wg=Wg, Wu=Wu, Wd=Wd, x=x, h=h, ids=ids)
