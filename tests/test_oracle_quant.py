"""Pins of the oracle's quantizers (fp32 -> packed Q8_0 / Q4_0) against things
other than themselves:

* the fp32 -> binary16 encoder against numpy's own conversion (every finite
  binary16 value, every midpoint between neighbours and its fp32 neighbours,
  random values over the whole range, overflow edges);
* hand-quantized blocks (tests/golden/q*.txt), including exact ties;
* properties that the definitions fix: the extreme element's code, every
  other code the nearest level away from near-ties, the scale the nearest
  binary16 to its exact value, zero blocks, round trips of values already on
  the grid, scale and sign symmetry, and for the Lloyd refinement that it is
  never worse than its absmax start and that its scale is the least-squares
  scale of its own codes;
* mutants: the oracle rebuilt with one planted mistake in a quantizer or the
  encoder must fail at least one of these pins.

The packed bytes are decoded here with numpy byte slicing, independently of
the oracle's own decoder.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle as oracle_pkg
from block_quantized_token_amd import inputs as I
from tests import golden_io

Q8, Q4 = I.FMT_Q8_0, I.FMT_Q4_0


def split_blocks(fmt, packed, nblk):
    """(d bits uint16 [nblk], d value fp64 [nblk], codes int64 [nblk][32]) by byte slicing."""
    size = 34 if fmt == Q8 else 18
    b = np.asarray(packed, dtype=np.uint8).reshape(nblk, size)
    dbits = b[:, 0].astype(np.uint16) | (b[:, 1].astype(np.uint16) << 8)
    dval = dbits.view(np.float16).astype(np.float64)
    if fmt == Q8:
        codes = b[:, 2:].view(np.int8).astype(np.int64)
    else:
        lo, hi = b[:, 2:] & 15, b[:, 2:] >> 4
        codes = np.concatenate([lo, hi], axis=1).astype(np.int64)
    return dbits, dval, codes


def half_ulp16(x):
    """Half the binary16 spacing at |x| (subnormal spacing below 2^-14)."""
    a = np.maximum(np.abs(x), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(a)) - 10) / 2


def quantize_blocks(o, fmt, v, method=0):
    v = np.ascontiguousarray(v, dtype=np.float32)
    nblk = v.size // 32
    return split_blocks(fmt, o.quantize(fmt, 1, v.size, v, method), nblk)


def quant_inputs(seed=5):
    """Blocks of several distributions: normal, heavy tails, uniform, one outlier, zeros, tiny."""
    rng = np.random.default_rng(seed)
    parts = [rng.standard_normal((64, 32)),
             rng.standard_t(2, (64, 32)),
             rng.uniform(-3, 3, (64, 32)),
             np.where(rng.random((64, 32)) < 1 / 32, 40.0, 1.0) * rng.standard_normal((64, 32)),
             np.zeros((2, 32)),
             rng.standard_normal((4, 32)) * 1e-8,
             rng.standard_normal((8, 32)) * 1e-5]
    return np.concatenate(parts).astype(np.float32)


# ---------------------------------------------------------------- the pins
def encoder_failures(o):
    fails = []
    finite = np.arange(0x7C00, dtype=np.uint16)
    vals = np.concatenate([finite, finite | 0x8000]).view(np.float16).astype(np.float32)
    if not np.array_equal(o.to_fp16_bits(vals), vals.astype(np.float16).view(np.uint16)):
        fails.append("fp16 encoder: finite binary16 values do not round-trip")
    pos = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact: 12 significant bits
    probe = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))])
    rng = np.random.default_rng(1)
    rand = (np.exp2(rng.uniform(-30, 17, 200000)) * rng.choice([-1, 1], 200000)).astype(np.float32)
    edges = np.array([65504, 65519.996, 65520, 65536, 1e30, np.inf, -np.inf, 2.0 ** -25, 2.0 ** -26,
                      np.nextafter(np.float32(2.0 ** -25), np.float32(1)), 0.0, -0.0], dtype=np.float32)
    probe = np.concatenate([probe, -probe, rand, edges]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = probe.astype(np.float16).view(np.uint16)
    got = o.to_fp16_bits(probe)
    if not np.array_equal(got, ref):
        fails.append(f"fp16 encoder differs from numpy on {(got != ref).sum()} values")
    return fails


def golden_failures(o):
    fails = []
    for name in golden_io.quant_vectors():
        g = golden_io.load_quant(name)
        dbits, _, codes = quantize_blocks(o, g["fmt"], g["v"], g["method"])
        if dbits[0] != g["d"] or not np.array_equal(codes[0], g["codes"]):
            fails.append(f"{name}: d {dbits[0]:#06x} codes {codes[0].tolist()}")
    return fails


def q8_failures(o):
    fails = []
    v = quant_inputs()
    nb = v.shape[0]
    dbits, d, codes = quantize_blocks(o, Q8, v)
    v64 = v.astype(np.float64)
    amax = np.abs(v64).max(axis=1)
    exact = amax / 127
    zero = d == 0
    # the scale is the binary16 nearest to max|v| / 127, and a zero scale means the zero block
    if np.any(np.abs(d - exact) > half_ulp16(exact) * (1 + 1e-6)):
        fails.append("q8_0: scale is not the nearest binary16 of max|v|/127")
    if np.any(codes[zero] != 0) or np.any(exact[zero] > 2.0 ** -24):
        fails.append("q8_0: zero-scale blocks")
    nz = ~zero
    e = np.zeros_like(v64)
    e[nz] = v64[nz] * 127 / amax[nz, None]
    ext = np.abs(v64).argmax(axis=1)
    if np.any(codes[nz, ext[nz]] != np.sign(v64[nz, ext[nz]]) * 127):
        fails.append("q8_0: the extreme is not coded +-127")
    frac = np.abs(e) - np.floor(np.abs(e))
    clear = nz[:, None] & (np.abs(frac - 0.5) > 1e-4)
    want = np.sign(e) * np.floor(np.abs(e) + 0.5)  # nearest, halves away from zero
    if np.any(codes[clear] != want[clear]) or np.any(np.abs(codes - e)[nz] > 0.5 + 1e-4):
        fails.append("q8_0: codes are not the nearest levels")
    # values already on the grid come back exactly
    rng = np.random.default_rng(2)
    c = rng.integers(-127, 128, (nb, 32))
    c[np.arange(nb), rng.integers(0, 32, nb)] = rng.choice([-127, 127], nb)
    k = rng.integers(3, 13, nb)
    vg = (c * np.exp2(-k)[:, None]).astype(np.float32)
    db2, _, c2 = quantize_blocks(o, Q8, vg)
    if not (np.array_equal(c2, c) and np.array_equal(db2, ((15 - k) << 10).astype(np.uint16))):
        fails.append("q8_0: grid values do not round-trip")
    # scale by 2^3 and negate: the same codes (negated), the scale times 2^3
    big = nz & (d > 2.0 ** -10) & (d < 2.0 ** 10)
    _, d3, c3 = quantize_blocks(o, Q8, (-8 * v[big]).astype(np.float32))
    if not (np.array_equal(c3, -codes[big]) and np.array_equal(d3, 8 * d[big])):
        fails.append("q8_0: scale / sign symmetry")
    return fails


def q4_failures(o):
    fails = []
    v = quant_inputs(6)
    nb = v.shape[0]
    dbits, d, codes = quantize_blocks(o, Q4, v, 0)
    v64 = v.astype(np.float64)
    ext = np.abs(v64).argmax(axis=1)  # numpy: the first index of the largest magnitude
    vmax = v64[np.arange(nb), ext]
    exact = vmax / -8
    zero = d == 0
    if np.any(np.abs(d - exact) > half_ulp16(exact) * (1 + 1e-6)):
        fails.append("q4_0: scale is not the nearest binary16 of (signed extreme)/-8")
    if np.any(codes[zero] != 8) or np.any(np.abs(exact[zero]) > 2.0 ** -24):
        fails.append("q4_0: zero-scale blocks")
    nz = ~zero
    if np.any(codes[nz, ext[nz]] != 0):
        fails.append("q4_0: the first extreme is not code 0")
    e = np.zeros_like(v64)
    e[nz] = v64[nz] * -8 / vmax[nz, None] + 8.5
    frac = e - np.floor(e)
    clear = nz[:, None] & (np.minimum(frac, 1 - frac) > 1e-4)
    want = np.minimum(15, np.floor(e))
    if np.any(codes[clear] != want[clear]) or codes.min() < 0 or codes.max() > 15:
        fails.append("q4_0: codes are not min(15, floor(v/d + 8.5))")
    # grid values (q in -8..7 with -8 present, d a power of two) come back exactly
    rng = np.random.default_rng(3)
    q = rng.integers(-7, 8, (nb, 32))
    q[np.arange(nb), rng.integers(0, 32, nb)] = -8
    sgn = rng.choice([-1, 1], nb)
    k = rng.integers(3, 13, nb)
    d0 = sgn * np.exp2(-k)
    vg = (q * d0[:, None]).astype(np.float32)
    for method in (0, 1):
        db2, dv2, c2 = quantize_blocks(o, Q4, vg, method)
        if not (np.array_equal(c2, q + 8) and np.array_equal(dv2, d0)):
            fails.append(f"q4_0 method {method}: grid values do not round-trip")
    # Lloyd: never worse than its absmax start; its scale the least-squares scale of its codes
    _, dl, cl = quantize_blocks(o, Q4, v, 1)
    sse_a = ((v64 - d[:, None] * (codes - 8)) ** 2).sum(axis=1)
    sse_l = ((v64 - dl[:, None] * (cl - 8)) ** 2).sum(axis=1)
    if np.any(sse_l > sse_a * (1 + 2e-3) + 1e-30):
        fails.append("q4_0 lloyd: worse than the absmax start")
    if not np.sum(sse_l < sse_a * (1 - 1e-3)) > nb // 4:
        fails.append("q4_0 lloyd: hardly ever better than the absmax start")
    ql = cl - 8
    s2 = (ql * ql).sum(axis=1)
    ls = np.where(s2 > 0, (v64 * ql).sum(axis=1) / np.maximum(s2, 1), 0.0)
    if np.any(np.abs(dl - ls) > 2 * half_ulp16(ls) * (1 + 1e-6)):
        fails.append("q4_0 lloyd: scale is not the least-squares scale of its codes")
    return fails


def quant_pin_failures(o):
    return encoder_failures(o) + golden_failures(o) + q8_failures(o) + q4_failures(o)


# ---------------------------------------------------------------- the tests
def test_quantizer_pins_hold(orc):
    assert quant_pin_failures(orc) == []


@pytest.mark.parametrize("name", golden_io.quant_vectors())
def test_hand_quantized_block(orc, name):
    g = golden_io.load_quant(name)
    dbits, _, codes = quantize_blocks(orc, g["fmt"], g["v"], g["method"])
    assert dbits[0] == g["d"], hex(dbits[0])
    assert codes[0].tolist() == g["codes"].tolist()


def test_quantizer_argument_errors(orc):
    v = np.zeros((2, 64), np.float32)
    with pytest.raises(ValueError):
        orc.quantize(Q4, 2, 64, v, method=2)
    bad = v.copy()
    bad[1, 3] = np.inf
    for fmt in (Q8, Q4):
        with pytest.raises(ValueError):
            orc.quantize(fmt, 2, 64, bad)
        bad[1, 3] = np.nan


def test_lloyd_converges_on_most_blocks(orc):
    """With the round cap, a few blocks may stop before the codes settle; the pins
    above do not need convergence, but a cap that bites often would be a bad reading."""
    v = quant_inputs(9)
    _, dl, cl = quantize_blocks(orc, Q4, v, 1)
    # converged blocks: every code is the nearest level for the stored scale (up to its fp16 rounding)
    nz = dl != 0
    r = v[nz].astype(np.float64) / dl[nz, None]
    q = cl[nz] - 8
    near = (np.abs(r - q) <= 0.5 + 8 * 2.0 ** -11) | ((q == -8) & (r < -8)) | ((q == 7) & (r > 7))
    assert near.all(axis=1).mean() > 0.95


QUANT_MUTANTS = {
    8: "Q8_0 scale max|v| / 128",
    9: "Q8_0 codes truncated instead of rounded",
    10: "Q4_0 scale from |extreme| (sign dropped)",
    11: "Q4_0 Lloyd without refinement",
    12: "fp16 encoder truncates",
}


@pytest.mark.parametrize("mutant", sorted(QUANT_MUTANTS))
def test_quantizer_pins_catch_planted_mistake(mutant):
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, f"liboracle_m{mutant}.so")
        oracle_pkg.build(path, mutant=mutant)
        fails = quant_pin_failures(oracle_pkg.Oracle(path))
    assert fails, f"mutant {mutant} ({QUANT_MUTANTS[mutant]}) passed every pin"
