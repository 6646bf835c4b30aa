"""Pins of the CPU oracle against things other than itself.

* the IEEE-754 binary16 / bfloat16 decoders against numpy's own conversions,
  for every one of the 65,536 bit patterns;
* hand-written blocks with closed-form results (tests/golden/e*.txt);
* identity-like and all-equal matrices (closed forms);
* a second, independent dequantisation written with numpy byte slicing and
  numpy's float16 view, followed by an fp64 matmul (brute force);
* dyadic inputs, where every partial sum is exact, so the result is unique;
* the bandwidth rows of the M5 multi-token audit's section 2.1 table, which
  fix the bytes per Q8_0 / BF16 row that the oracle walks;
* mutants: the oracle rebuilt with one planted mistake each must fail at least
  one of the pins above.
"""
import os
import tempfile

import numpy as np
import pytest

import oracle as oracle_pkg
from block_quantized_token_amd import inputs as I
from tests import golden_io

Q8, Q4, BF = I.FMT_Q8_0, I.FMT_Q4_0, I.FMT_BF16


# ------------------------------------------------------------ independent decode
def numpy_dequant(fmt, rows, cols, W):
    """Second implementation of the dequantisation: byte slicing + numpy float16/bf16 views."""
    W = np.ascontiguousarray(W).view(np.uint8)
    if fmt == BF:
        b = W[: rows * cols * 2].reshape(rows, cols, 2)
        bits = b[..., 0].astype(np.uint32) | (b[..., 1].astype(np.uint32) << 8)
        return (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    nb = cols // 32
    bb = 34 if fmt == Q8 else 18
    blk = W[: rows * nb * bb].reshape(rows, nb, bb)
    d = np.ascontiguousarray(blk[:, :, 0:2]).view("<f2")[..., 0].astype(np.float64)
    if fmt == Q8:
        c = np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).astype(np.float64)
    else:
        qs = blk[:, :, 2:]
        c = np.concatenate([qs & 15, qs >> 4], axis=-1).astype(np.float64) - 8.0
    return (d[:, :, None] * c).reshape(rows, cols)


def numpy_gemv(fmt, rows, cols, W, x):
    w = numpy_dequant(fmt, rows, cols, W)
    xd = x.astype(np.float64)
    return xd @ w.T, np.abs(xd) @ np.abs(w).T


# ------------------------------------------------------------ the pin battery
BRUTE_SHAPES = [(1, 32), (3, 64), (17, 96), (67, 288), (130, 640), (64, 2560)]


def pin_failures(o):
    """Run every pin against oracle instance ``o``; return a list of failure strings."""
    fails = []
    # scalar decoders, every bit pattern
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref16 = bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        refbf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got16 = np.array([o.fp16(int(b)) for b in bits])
    gotbf = np.array([o.bf16(int(b)) for b in bits])
    for name, got, ref in (("fp16", got16, ref16), ("bf16", gotbf, refbf)):
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        if not same.all():
            fails.append(f"{name} decoder differs on {(~same).sum()} patterns")
    # hand vectors with closed forms
    for name in golden_io.hand_vectors():
        g = golden_io.load(name)
        y, _ = o.gemv(g["fmt"], g["rows"], g["cols"], g["W"], g["x"])
        if not np.array_equal(y.reshape(g["y"].shape), g["y"]):
            fails.append(f"{name}: {y.ravel()} != {g['y'].ravel()}")
    # identity-like matrices: y == x exactly
    for fmt, n in ((Q8, 64), (Q8, 256), (Q4, 64), (Q4, 256)):
        rng = np.random.default_rng(n + fmt)
        perm = rng.permutation(n)
        d = np.full((n, n // 32), 0x3C00, dtype=np.uint16)
        if fmt == Q8:
            codes = np.zeros((n, n), dtype=np.int8)
            codes[np.arange(n), perm] = 1
            W = I.pack_q8_0(d, codes)
        else:
            codes = np.full((n, n), 8, dtype=np.uint8)
            codes[np.arange(n), perm] = 9
            W = I.pack_q4_0(d, codes)
        x = rng.standard_normal((4, n)).astype(np.float32)
        y, _ = o.gemv(fmt, n, n, W, x)
        if not np.array_equal(y, x[:, perm].astype(np.float64)):
            fails.append(f"identity fmt={fmt} n={n}")
    # all-equal matrices: y = cols * c * s (Q4_0: cols * (c - 8) * s)
    for fmt, c, sbits, s in ((Q8, -7, 0x3800, 0.5), (Q8, 127, 0x2E66, 0.0999755859375),
                             (Q4, 3, 0x3C00, 1.0), (Q4, 15, 0x0200, 2.0 ** -15)):
        rows, cols = 3, 96
        d = np.full((rows, cols // 32), sbits, dtype=np.uint16)
        if fmt == Q8:
            W = I.pack_q8_0(d, np.full((rows, cols), c, dtype=np.int8))
            expect = cols * c * s
        else:
            W = I.pack_q4_0(d, np.full((rows, cols), c, dtype=np.uint8))
            expect = cols * (c - 8) * s
        y, _ = o.gemv(fmt, rows, cols, W, np.ones((1, cols), np.float32))
        if not np.all(y == expect):
            fails.append(f"all-equal fmt={fmt} c={c}: {y.ravel()[0]} != {expect}")
    # brute force against the independent numpy decode + fp64 matmul
    for fmt in (Q8, Q4, BF):
        for rows, cols in BRUTE_SHAPES:
            rng = np.random.default_rng(rows * 7919 + cols + fmt)
            W = I.weights(rng, fmt, rows, cols)
            x = I.activations(rng, cols)
            y, b = o.gemv(fmt, rows, cols, W, x)
            ry, rb = numpy_gemv(fmt, rows, cols, W, x)
            if not (np.all(np.abs(y - ry) <= 1e-12 * rb + 1e-300) and np.allclose(b, rb, rtol=1e-12, atol=0)):
                fails.append(f"brute force fmt={fmt} {rows}x{cols}")
    # down projection (per-slot inputs): with every input of token t equal to x[t]
    # it is the grouped product; each slot is the brute force of its expert's rows
    E, rows, cols = 6, 40, 96
    rng = np.random.default_rng(21)
    W = I.weights(rng, Q8, E * rows, cols)
    ids = np.array([[1, 4, 1], [5, 0, 2]], dtype=np.int32)  # an expert twice in one token too
    x = I.activations(rng, cols, 2)
    yd, _ = o.down(Q8, E, rows, cols, ids, W, np.repeat(x[:, None, :], 3, axis=1))
    if not np.array_equal(yd, o.grouped(Q8, E, rows, cols, ids, W, x)[0]):
        fails.append("down with per-token inputs != grouped")
    h = rng.standard_normal((2, 3, cols)).astype(np.float32)
    yd, _ = o.down(Q8, E, rows, cols, ids, W, h)
    erb = rows * I.packed_row_bytes(Q8, cols)
    for t in range(2):
        for j in range(3):
            e = int(ids[t, j])
            ry, rb = numpy_gemv(Q8, rows, cols, W[e * erb:(e + 1) * erb], h[t, j][None])
            if not np.all(np.abs(yd[t, j] - ry[0]) <= 1e-12 * rb[0] + 1e-300):
                fails.append(f"down slot ({t},{j}) != brute force")
    # dyadic: every partial sum exact, so equality with the brute force is exact
    for fmt in (Q8, Q4):
        rows, cols = 33, 640
        rng = np.random.default_rng(11 + fmt)
        d = rng.choice(np.array([0x3400, 0x3800, 0x3C00], dtype=np.uint16), size=(rows, cols // 32))
        if fmt == Q8:
            W = I.pack_q8_0(d, rng.integers(-128, 128, (rows, cols), dtype=np.int8))
        else:
            W = I.pack_q4_0(d, rng.integers(0, 16, (rows, cols), dtype=np.uint8))
        x = (rng.integers(-4, 5, (4, cols)) / 4.0).astype(np.float32)
        y, _ = o.gemv(fmt, rows, cols, W, x)
        if not np.array_equal(y, numpy_gemv(fmt, rows, cols, W, x)[0]):
            fails.append(f"dyadic fmt={fmt}")
    return fails


def test_pins_hold(orc):
    assert pin_failures(orc) == []


@pytest.mark.parametrize("name", golden_io.hand_vectors())
def test_hand_vector(orc, name):
    g = golden_io.load(name)
    y, b = orc.gemv(g["fmt"], g["rows"], g["cols"], g["W"], g["x"])
    assert np.array_equal(y.reshape(g["y"].shape), g["y"])
    assert np.all(b >= np.abs(y))


def test_q4_0_nibble_order_distinguishes_orders(orc):
    """E4: under the adopted order y = 56; the pairwise (2j, 2j+1) order would give -4."""
    g = golden_io.load("e4_q4_0_nibble_order.txt")
    y, _ = orc.gemv(g["fmt"], 1, 32, g["W"], g["x"][:1])
    assert y[0, 0] == 56.0


def test_unpack_reads_generator_fields(orc):
    rng = np.random.default_rng(5)
    d, c = I.q8_0_fields(rng, 7, 96)
    gd, gc = orc.unpack(Q8, 7, 96, I.pack_q8_0(d, c))
    assert np.array_equal(gd, d) and np.array_equal(gc, c.astype(np.int32))
    d, c = I.q4_0_fields(rng, 5, 64)
    gd, gc = orc.unpack(Q4, 5, 64, I.pack_q4_0(d, c))
    assert np.array_equal(gd, d) and np.array_equal(gc, c.astype(np.int32))


def test_grouped_equals_plain_per_slot(orc):
    rng = np.random.default_rng(3)
    n_experts, rows, cols, T, topk = 9, 40, 256, 4, 3
    for fmt in (Q8, Q4, BF):
        W = I.weights(rng, fmt, n_experts * rows, cols)
        x = I.activations(rng, cols)
        ids = np.array([[1, 4, 1], [4, 0, 8], [8, 8, 2], [3, 4, 5]], dtype=np.int32)
        y, b = orc.grouped(fmt, n_experts, rows, cols, ids, W, x)
        rb = I.packed_row_bytes(fmt, cols)
        for t in range(T):
            for j in range(topk):
                e = ids[t, j]
                Wp = W[e * rows * rb:(e + 1) * rows * rb]
                py, pb = orc.gemv(fmt, rows, cols, Wp, x[t:t + 1])
                assert np.array_equal(y[t, j], py[0]) and np.array_equal(b[t, j], pb[0])


def test_grouped_rejects_bad_ids(orc):
    W = I.weights(np.random.default_rng(0), Q8, 2 * 4, 32)
    with pytest.raises(ValueError):
        orc.grouped(Q8, 2, 4, 32, np.array([[0, 2]], np.int32), W, np.ones((1, 32), np.float32))


def test_token_prefix_invariance(orc):
    """Each token's result does not depend on T (exact in the oracle)."""
    rng = np.random.default_rng(9)
    for fmt in (Q8, Q4, BF):
        W = I.weights(rng, fmt, 50, 512)
        x = I.activations(rng, 512)
        y4, _ = orc.gemv(fmt, 50, 512, W, x)
        for T in (1, 2, 3):
            yT, _ = orc.gemv(fmt, 50, 512, W, x[:T])
            assert np.array_equal(yT, y4[:T])


def test_row_selection_matches_full(orc):
    rng = np.random.default_rng(2)
    W = I.weights(rng, Q8, 100, 256)
    x = I.activations(rng, 256)
    y, b = orc.gemv(Q8, 100, 256, W, x)
    sel = np.array([99, 0, 17, 17, 63])
    ys, bs = orc.gemv(Q8, 100, 256, W, x, sel=sel)
    assert np.array_equal(ys, y[:, sel]) and np.array_equal(bs, b[:, sel])


def test_page_bandwidth_rows(orc):
    """Every Q8_0 / BF16 row of the M5 audit's section 2.1 table: bytes / us reproduces its GB/s.

    The table prints us to 0.01 and GB/s to 0.1, so the printed GB/s must lie within
    [bytes / (us + 0.005), bytes / (us - 0.005)] widened by the 0.05 display rounding."""
    def consistent(nbytes, us, gbs):
        lo, hi = nbytes / ((us + 0.005) * 1e3), nbytes / ((us - 0.005) * 1e3)
        return lo - 0.05 <= gbs <= hi + 0.05

    for fmt, n_in, n_out, _ntok, ous, ogbs, nus, ngbs in golden_io.bandwidth_rows():
        nbytes = orc.packed_bytes(fmt, n_out, n_in)
        assert consistent(nbytes, ous, ogbs), (n_in, n_out, ous)
        assert consistent(nbytes, nus, ngbs), (n_in, n_out, nus)
        # a 32-byte Q8_0 block (no scale) or a 36-byte one would not fit
        if fmt == Q8:
            for bb in (32, 36):
                alt = n_out * n_in // 32 * bb
                assert not (consistent(alt, ous, ogbs) and consistent(alt, nus, ngbs))


def test_bits_per_weight(orc):
    """Q4_0 is 4.5 bits per weight (opus-mtp-turbo report, finding 3); Q8_0 8.5; BF16 16.
    The same report sizes a 640 x 2560 Q8_0 matrix at 1.74 MB and the 40525 x 2560 Q8_0
    head at about 110 MB."""
    assert orc.packed_bytes(Q4, 1, 32) * 8 / 32 == 4.5
    assert orc.packed_bytes(Q8, 1, 32) * 8 / 32 == 8.5
    assert orc.packed_bytes(BF, 1, 32) * 8 / 32 == 16
    assert round(orc.packed_bytes(Q8, 640, 2560) / 1e6, 2) == 1.74
    assert round(orc.packed_bytes(Q8, 40525, 2560) / 1e6) == 110
    assert orc.row_bytes(Q8, 33) == -1 and orc.row_bytes(Q4, 48) == -1


MUTANTS = {
    1: "drops the last block of each row",
    2: "Q4_0 offset sign flipped (c + 8)",
    3: "Q4_0 pairwise nibble order",
    4: "Q8_0 scale taken from block 0",
    5: "token index reversed",
    6: "fp16 subnormal scales flushed to zero",
    7: "fp16 / bf16 read big-endian",
    13: "down projection reads the token's first input for every slot",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant):
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, f"liboracle_m{mutant}.so")
        oracle_pkg.build(path, mutant=mutant)
        fails = pin_failures(oracle_pkg.Oracle(path))
    assert fails, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"


# ---------------------------------------------------------------- argmax
def test_argmax_ties_take_the_lowest_row(orc):
    """Rows 3 and 6 are the same largest row; rows 1 and 4 equal but smaller."""
    rows, cols = 8, 64
    d = np.full((rows, cols // 32), 0x3C00, dtype=np.uint16)           # scale 1
    codes = np.zeros((rows, cols), dtype=np.int8)
    codes[1, :] = 2
    codes[3, :] = 5
    codes[4, :] = 2
    codes[6, :] = 5
    W = I.pack_q8_0(d, codes)
    x = np.ones((2, cols), dtype=np.float32)
    x[1] = -1.0                                                         # token 1: every y <= 0, max is 0
    idx, val, _, _ = orc.argmax(I.FMT_Q8_0, rows, cols, W, x)
    assert idx.tolist() == [3, 0] and val.tolist() == [5.0 * cols, 0.0]


def test_argmax_all_negative(orc):
    rows, cols = 5, 32
    d = np.full((rows, 1), 0x3C00, dtype=np.uint16)
    codes = np.array([[-9] * 32, [-2] * 32, [-7] * 32, [-2] * 32, [-3] * 32], dtype=np.int8)
    idx, val, _, _ = orc.argmax(I.FMT_Q8_0, rows, cols, I.pack_q8_0(d, codes), np.ones((1, cols), np.float32))
    assert idx.tolist() == [1] and val.tolist() == [-64.0]


def test_argmax_matches_brute_force(orc):
    rng = np.random.default_rng(77)
    rows, cols = 300, 512
    W = I.weights(rng, I.FMT_Q4_0, rows, cols)
    x = I.activations(rng, cols)
    idx, val, _, _ = orc.argmax(I.FMT_Q4_0, rows, cols, W, x)
    y = x.astype(np.float64) @ numpy_dequant(I.FMT_Q4_0, rows, cols, W).T
    assert idx.tolist() == np.argmax(y, axis=1).tolist()
    assert np.allclose(val, y.max(axis=1), rtol=0, atol=1e-9 * np.abs(y).max())
