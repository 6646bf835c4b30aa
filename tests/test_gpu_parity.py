"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Bar (per output): |y_gpu - y_oracle| <= 1e-4 * sum_k |w_k x_k| + 1e-6.
Dyadic and identity inputs, whose exact result is representable, must match
bit for bit; so must repeated calls, a token's outputs at different T, and the
grouped kernel against the plain one.
"""
import os
import sys

import numpy as np
import pytest

from block_quantized_token_amd import _lib, inputs as I, ops

pytestmark = pytest.mark.gpu

Q8, Q4, BF = I.FMT_Q8_0, I.FMT_Q4_0, I.FMT_BF16
NAMES = {Q8: "q8_0", Q4: "q4_0", BF: "bf16"}


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    _lib.load()
    return _t


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(torch, arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def gpu_gemv(torch, fmt, W_dev, x, rows):
    y = ops.gemv(NAMES[fmt], W_dev, dev(torch, x), rows)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_parity(y, ref, bound, what):
    err = np.abs(y.astype(np.float64) - ref)
    tol = 1e-4 * bound + 1e-6
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} outputs out of tolerance; worst err {err.max():.3e}, "
                           f"worst err/tol {(err / tol).max():.3f}")
    assert np.isfinite(y).all(), what


def check_dense(torch, orc, fmt, rows, cols, W, x, what, sel=None, same_bits=((1, 2, 3, 4),)):
    """Every T against the oracle; within each group of ``same_bits`` (T values whose
    default kernels share their arithmetic) a token's outputs agree bit for bit."""
    Wd = dev(torch, W)
    ys = {}
    for T in range(x.shape[0], 0, -1):
        say(f"[{what}] fmt={NAMES[fmt]} rows={rows} cols={cols} T={T}")
        y = gpu_gemv(torch, fmt, Wd, x[:T], rows)
        ref, bound = orc.gemv(fmt, rows, cols, W, x[:T], sel=sel)
        assert_parity(y if sel is None else y[:, sel], ref, bound, f"{what} T={T}")
        ys[T] = y
    for group in same_bits:
        Ts = [T for T in group if T in ys]
        for T in Ts[:-1]:  # a token's outputs do not depend on T
            assert np.array_equal(ys[T], ys[Ts[-1]][:T]), f"{what}: token results differ between T={T} and T={Ts[-1]}"
    return ys[x.shape[0]]


# ------------------------------------------------------------- hand vectors
def test_hand_vectors_bitwise(torch, orc):
    from tests import golden_io
    for name in golden_io.hand_vectors():
        g = golden_io.load(name)
        say(f"[hand] {name}")
        y = gpu_gemv(torch, g["fmt"], dev(torch, g["W"]), g["x"], g["rows"])
        assert np.array_equal(y.astype(np.float64).reshape(g["y"].shape), g["y"]), (name, y, g["y"])


def test_identity_bitwise(torch):
    for fmt, n in ((Q8, 64), (Q8, 1024), (Q4, 64), (Q4, 1024)):
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
        say(f"[identity] fmt={NAMES[fmt]} n={n}")
        y = gpu_gemv(torch, fmt, dev(torch, W), x, n)
        assert np.array_equal(y, x[:, perm])


def dyadic_weights(rng, fmt, rows, cols):
    d = rng.choice(np.array([0x3400, 0x3800, 0x3C00], dtype=np.uint16), size=(rows, cols // 32))
    if fmt == Q8:
        return I.pack_q8_0(d, rng.integers(-128, 128, (rows, cols), dtype=np.int8))
    return I.pack_q4_0(d, rng.integers(0, 16, (rows, cols), dtype=np.uint8))


@pytest.mark.parametrize("fmt,rows,cols", [(Q8, 10240, 2560), (Q8, 2560, 6144), (Q4, 8192, 2560), (Q8, 333, 736)])
def test_dyadic_bitwise(torch, orc, fmt, rows, cols):
    """Every partial sum is a multiple of 2^-6 below 2^20: exact in fp32 in any order."""
    rng = np.random.default_rng(rows + cols)
    W = dyadic_weights(rng, fmt, rows, cols)
    x = (rng.integers(-4, 5, (4, cols)) / 4.0).astype(np.float32)
    say(f"[dyadic] fmt={NAMES[fmt]} {rows}x{cols}")
    y = gpu_gemv(torch, fmt, dev(torch, W), x, rows)
    ref, _ = orc.gemv(fmt, rows, cols, W, x)
    assert np.array_equal(y.astype(np.float64), ref)


def test_bf16_dyadic_bitwise(torch, orc):
    rng = np.random.default_rng(4)
    rows, cols = 777, 1032
    vals = rng.integers(-64, 65, (rows, cols)) / 16.0
    W = I.pack_bf16(I.bf16_bits(vals))
    x = (rng.integers(-4, 5, (4, cols)) / 4.0).astype(np.float32)
    y = gpu_gemv(torch, BF, dev(torch, W), x, rows)
    ref, _ = orc.gemv(BF, rows, cols, W, x)
    assert np.array_equal(y.astype(np.float64), ref)


# --------------------------------------------------------- ragged and tiny
TINY_ROWS = (1, 2, 3, 5, 17, 33, 67)
TINY_COLS = tuple(32 * i for i in range(1, 10)) + (256, 544, 640, 768, 1056, 1280, 4096, 6144)


@pytest.mark.parametrize("fmt", [Q8, Q4])
def test_tiny_shapes(torch, orc, fmt):
    for rows in TINY_ROWS:
        for cols in TINY_COLS:
            rng = np.random.default_rng(rows * 1000 + cols)
            W = I.weights(rng, fmt, rows, cols)
            x = I.activations(rng, cols)
            check_dense(torch, orc, fmt, rows, cols, W, x, "tiny")


def test_tiny_shapes_bf16(torch, orc):
    for rows in TINY_ROWS:
        for cols in (8, 16, 24, 40, 56, 504, 520, 1000, 1032):
            rng = np.random.default_rng(rows * 1000 + cols)
            W = I.weights(rng, BF, rows, cols)
            x = I.activations(rng, cols)
            check_dense(torch, orc, BF, rows, cols, W, x, "tiny")


@pytest.mark.parametrize("fmt,rows,cols", [(Q8, 64, 65536), (Q4, 48, 6656), (BF, 40, 7000), (Q8, 1000, 4608),
                                           (BF, 37, 6152)])
def test_many_slices(torch, orc, fmt, rows, cols):
    """More k slices than waves per workgroup: waves loop over several slices."""
    rng = np.random.default_rng(cols)
    W = I.weights(rng, fmt, rows, cols)
    x = I.activations(rng, cols)
    check_dense(torch, orc, fmt, rows, cols, W, x, "many-slices")


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("name", ["c1_q8_0_2560x2560", "c2a_q8_0_10240x2560", "c2b_q8_0_2560x6144",
                                  "c3_q4_0_8192x2560", "c3_bf16_8192x2560"])
def test_config_full(torch, orc, name):
    c = I.dense_case(name)
    check_dense(torch, orc, c["fmt"], c["rows"], c["cols"], c["W"], c["x"], name)


def test_repeat_calls_bitwise(torch):
    c = I.dense_case("c2a_q8_0_10240x2560")
    Wd, xd = dev(torch, c["W"]), dev(torch, c["x"])
    ys = [ops.gemv("q8_0", Wd, xd, c["rows"]).cpu().numpy() for _ in range(3)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])


def test_tile_override_keeps_bits(torch, monkeypatch):
    """Different row tilings with the same k split (512-wide slices) give identical bits."""
    c = I.dense_case("c2a_q8_0_10240x2560")
    Wd, xd = dev(torch, c["W"]), dev(torch, c["x"])
    monkeypatch.setenv("QGEMV_TILE", "q8_0:4,5,40,L2")
    base = ops.gemv("q8_0", Wd, xd, c["rows"]).cpu().numpy()
    for tile in ("q8_0:1,5,2", "q8_0:2,5,8", "q8_0:1,5,64", "q8_0:2,5,100"):
        monkeypatch.setenv("QGEMV_TILE", tile)
        say(f"[tile] {tile}")
        assert np.array_equal(ops.gemv("q8_0", Wd, xd, c["rows"]).cpu().numpy(), base), tile


@pytest.mark.parametrize("name", ["c2a_q8_0_10240x2560", "c2b_q8_0_2560x6144", "c3_q4_0_8192x2560",
                                  "c3_bf16_8192x2560"])
def test_direct_and_streamed_kernels_agree_bitwise(torch, monkeypatch, name):
    """Both kernel kinds split k the same way, so their outputs must be identical."""
    c = I.dense_case(name)
    fmt = NAMES[c["fmt"]]
    Wd = dev(torch, c["W"])
    nw = min(12, -(-c["cols"] // 512))
    for T in (1, 2, 3, 4):
        xd = dev(torch, c["x"][:T])
        outs = {}
        for tile in (f"{fmt}:2,{nw},4,d", f"{fmt}:4,{nw},8,d", f"{fmt}:4,{nw},16,s", f"{fmt}:4,{nw},40,s",
                     f"{fmt}:8,{nw},32,s", f"{fmt}:4,{nw},32,l4"):
            monkeypatch.setenv("QGEMV_TILE", tile)
            st, t = _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], T)
            if st != 0:
                continue  # not in the compiled set for this T
            say(f"[kinds] {name} T={T} tile={tile}")
            outs[tile] = ops.gemv(fmt, Wd, xd, c["rows"]).cpu().numpy()
        ref = next(iter(outs.values()))
        for tile, y in outs.items():
            assert np.array_equal(y, ref), (name, T, tile)
        assert any(t.endswith(",d") for t in outs)
        assert any(t.endswith(",s") for t in outs) or (fmt == "bf16" and T >= 3)  # no streamed bf16 at T>=3


@pytest.mark.parametrize("name", ["c1_q8_0_2560x2560", "c2a_q8_0_10240x2560", "c2b_q8_0_2560x6144",
                                  "c3_q4_0_8192x2560", "c3_bf16_8192x2560"])
def test_dma_ring_depths_agree_bitwise(torch, monkeypatch, name):
    """The LDS-DMA kind at every compiled ring depth and several row tilings
    (partial rings, more tiles than slots, a ragged last tile) gives the bits of
    the register-streamed and direct kinds."""
    c = I.dense_case(name)
    fmt = NAMES[c["fmt"]]
    Wd = dev(torch, c["W"])
    nw = -(-c["cols"] // 512)
    for T in (1, 2, 3, 4):
        xd = dev(torch, c["x"][:T])
        monkeypatch.setenv("QGEMV_TILE", f"{fmt}:2,{nw},4,d")
        ref = ops.gemv(fmt, Wd, xd, c["rows"]).cpu().numpy()
        ran = 0
        for d in (2, 3, 4, 6):
            for rw, k in ((8, "l"), (40, "l"), (48, "L"), (120, "l"), (16, "L"), (120, "L")):
                tile = f"{fmt}:4,{nw},{rw},{k}{d}"
                monkeypatch.setenv("QGEMV_TILE", tile)
                st, _t = _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], T)
                if st != 0:
                    continue  # x does not leave a slot, or the ring does not fit the LDS
                say(f"[dma] {name} T={T} tile={tile}")
                y = ops.gemv(fmt, Wd, xd, c["rows"]).cpu().numpy()
                assert np.array_equal(y, ref), (name, T, tile)
                ran += 1
        for d in (2, 3, 4):  # unit-balanced kind: any number of waves
            for nwu, rw in ((4, 40), (8, 16), (3, 120), (4, 8)):
                tile = f"{fmt}:4,{nwu},{rw},u{d}"
                monkeypatch.setenv("QGEMV_TILE", tile)
                st, _t = _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], T)
                if st != 0:
                    continue  # x and the rings do not fit the LDS
                say(f"[units] {name} T={T} tile={tile}")
                y = ops.gemv(fmt, Wd, xd, c["rows"]).cpu().numpy()
                assert np.array_equal(y, ref), (name, T, tile)
                ran += 1
        # 12 slices: a ring of 3 slots per wave, which x needs at T >= 3, passes the LDS
        assert ran >= 3 or (name == "c2b_q8_0_2560x6144" and T >= 3), (name, T, ran)


# ------------------------------------- 256-wide k slices, 16 lanes per row (h<depth>)
def half_tile(cols, rw=40, depth=2, rg=1, fmt="q8_0"):
    return f"{fmt}:4,{(cols // 256) * rg},{rw},h{depth}"


@pytest.mark.parametrize("name,rw,depth", [("c2a_q8_0_10240x2560", 40, 2), ("c2a_q8_0_10240x2560", 40, 3),
                                           ("c1_q8_0_2560x2560", 16, 2), ("c3_q4_0_8192x2560", 32, 2),
                                           ("c3_bf16_8192x2560", 32, 2), ("c3_q4_0_8192x2560", 40, 3)])
def test_half_slice_config_full(torch, orc, monkeypatch, name, rw, depth):
    """The half-slice kernel on the workloads: parity at every T, a token's bits equal across T."""
    c = I.dense_case(name)
    monkeypatch.setenv("QGEMV_TILE", half_tile(c["cols"], rw, depth, fmt=NAMES[c["fmt"]]))
    st, t = _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], 4)
    assert st == 0 and t[6] == 7 and t[7] == depth, (st, t)
    check_dense(torch, orc, c["fmt"], c["rows"], c["cols"], c["W"], c["x"], f"half {name} rw={rw} d={depth}")


def test_half_slice_tiny_and_dyadic(torch, orc, monkeypatch):
    """Ragged rows (partial tiles, fewer tiles than the ring), one to twelve slices,
    two row groups; dyadic inputs bitwise."""
    for fmt in (Q8, Q4, BF):
        for rows in TINY_ROWS:
            for cols in (256, 512, 768, 1280, 2304, 3072):
                for rw, depth, rg in ((8, 2, 1), (24, 3, 1), (16, 2, 2)):
                    monkeypatch.setenv("QGEMV_TILE", half_tile(cols, rw, depth, rg, NAMES[fmt]))
                    if _lib.qg_query_tile(fmt, rows, cols, 4)[0]:
                        continue  # more than twelve waves, or past the LDS
                    rng = np.random.default_rng(rows * 1000 + cols + rw + fmt)
                    W = I.weights(rng, fmt, rows, cols)
                    x = I.activations(rng, cols)
                    check_dense(torch, orc, fmt, rows, cols, W, x, f"half tiny rw={rw} d={depth} rg={rg}")
    rng = np.random.default_rng(97)
    rows, cols = 1000, 2816
    W = dyadic_weights(rng, Q8, rows, cols)
    x = (rng.integers(-4, 5, (4, cols)) / 4.0).astype(np.float32)
    monkeypatch.setenv("QGEMV_TILE", half_tile(cols, 40, 2))
    y = gpu_gemv(torch, Q8, dev(torch, W), x, rows)
    ref, _ = orc.gemv(Q8, rows, cols, W, x)
    assert np.array_equal(y.astype(np.float64), ref)


# ------------------------------------ matrix cores on 256-wide slices (kind x)
def mx_tile(cols, rw=40, rg=1, fmt="q8_0", r=1):
    return f"{fmt}:4,{(cols // 256) * rg},{rw},x" + ("2" if r == 2 else "")


@pytest.mark.parametrize("name,rw,r", [("c2a_q8_0_10240x2560", 40, 1), ("c2a_q8_0_10240x2560", 32, 1),
                                       ("c1_q8_0_2560x2560", 16, 1), ("c3_q4_0_8192x2560", 32, 1),
                                       ("c3_bf16_8192x2560", 32, 1), ("c3_bf16_8192x2560", 40, 1),
                                       ("c2a_q8_0_10240x2560", 64, 2), ("c3_q4_0_8192x2560", 32, 2),
                                       ("c3_q4_0_8192x2560", 48, 2), ("c1_q8_0_2560x2560", 32, 2)])
def test_mx_config_full(torch, orc, monkeypatch, name, rw, r):
    """Matrix cores on 256-wide slices on the workloads, tiles of 16 or 32 rows:
    parity at every T, a token's bits equal across T."""
    c = I.dense_case(name)
    monkeypatch.setenv("QGEMV_TILE", mx_tile(c["cols"], rw, fmt=NAMES[c["fmt"]], r=r))
    st, t = _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], 4)
    assert st == 0 and t[6] == 8 and t[3] == 256 and t[7] == r, (st, t)
    check_dense(torch, orc, c["fmt"], c["rows"], c["cols"], c["W"], c["x"], f"mx {name} rw={rw} r={r}")


@pytest.mark.parametrize("name,rw", [("c2b_q8_0_2560x6144", 16), ("c2b_q8_0_2560x6144", 48),
                                     ("c2a_q8_0_10240x2560", 48), ("c3_q4_0_8192x2560", 32),
                                     ("c3_bf16_8192x2560", 16)])
def test_mx512_config_full(torch, orc, monkeypatch, name, rw):
    """Matrix cores on 512-wide slices (kind X) on the workloads: parity at every T,
    a token's bits equal across T, and the persistent kind's bits (the same arithmetic)."""
    c = I.dense_case(name)
    fmt = NAMES[c["fmt"]]
    nsl = c["cols"] // 512
    monkeypatch.setenv("QGEMV_TILE", f"{fmt}:4,{nsl},{rw},X")
    st, t = _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], 4)
    assert st == 0 and t[6] == 11 and t[3] == 512, (st, t)
    y = check_dense(torch, orc, c["fmt"], c["rows"], c["cols"], c["W"], c["x"], f"mx512 {name} rw={rw}")
    monkeypatch.setenv("QGEMV_TILE", f"{fmt}:4,{nsl},32,P")
    if _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], 4)[0] == 0:
        yp = gpu_gemv(torch, c["fmt"], dev(torch, c["W"]), c["x"], c["rows"])
        assert np.array_equal(yp, y), name


def test_mx_row_tilings_keep_bits(torch, monkeypatch):
    """The same 256-wide k split at any rows per workgroup, row groups and tile
    height (16 or 32 rows): identical bits."""
    c = I.dense_case("c2a_q8_0_10240x2560")
    Wd, xd = dev(torch, c["W"]), dev(torch, c["x"])
    monkeypatch.setenv("QGEMV_TILE", mx_tile(c["cols"], 48))
    base = ops.gemv("q8_0", Wd, xd, c["rows"]).cpu().numpy()
    for rw, r in ((16, 1), (24, 1), (40, 1), (64, 1), (200, 1), (32, 2), (48, 2), (64, 2), (96, 2)):
        monkeypatch.setenv("QGEMV_TILE", mx_tile(c["cols"], rw, r=r))
        say(f"[mx tiling] rw={rw} r={r}")
        assert np.array_equal(ops.gemv("q8_0", Wd, xd, c["rows"]).cpu().numpy(), base), (rw, r)


def test_mx_tiny_ragged_and_row_groups(torch, orc, monkeypatch):
    """Ragged rows (a partial last tile, waves with no tile), one to twelve
    slices, two and three row groups, tiles of 16 and 32 rows, every format."""
    for fmt in (Q8, Q4, BF):
        for rows in TINY_ROWS + (40, 100):
            for cols in (256, 512, 768, 1280, 2304, 3072):
                for rw, rg, r in ((16, 1, 1), (40, 1, 1), (24, 2, 1), (48, 3, 1), (32, 1, 2), (40, 2, 2),
                                  (16, 1, "X"), (48, 2, "X")):
                    if r == "X":
                        if cols % 512:
                            continue
                        monkeypatch.setenv("QGEMV_TILE", f"{NAMES[fmt]}:4,{cols // 512 * rg},{rw},X")
                    else:
                        monkeypatch.setenv("QGEMV_TILE", mx_tile(cols, rw, rg, NAMES[fmt], r))
                    if _lib.qg_query_tile(fmt, rows, cols, 4)[0]:
                        continue  # more than twelve waves, or past the LDS
                    rng = np.random.default_rng(rows * 1000 + cols + rw + fmt)
                    W = I.weights(rng, fmt, rows, cols)
                    x = I.activations(rng, cols)
                    check_dense(torch, orc, fmt, rows, cols, W, x, f"mx tiny rw={rw} rg={rg} r={r}")


def test_mx_exact_inputs_bitwise(torch, orc, monkeypatch):
    """Inputs whose exact result is representable: dyadic weights and x (every partial
    sum a multiple of 2^-6 below 2^20), and identity-like matrices (y = a permutation
    of x, whose 24-bit significands the three bf16 pieces carry exactly)."""
    rng = np.random.default_rng(97)
    for fmt, rows, cols in ((Q8, 1000, 2816), (Q4, 777, 2560), (Q8, 10240, 2560)):
        W = dyadic_weights(rng, fmt, rows, cols)
        x = (rng.integers(-4, 5, (4, cols)) / 4.0).astype(np.float32)
        monkeypatch.setenv("QGEMV_TILE", mx_tile(cols, 40, fmt=NAMES[fmt]))
        y = gpu_gemv(torch, fmt, dev(torch, W), x, rows)
        ref, _ = orc.gemv(fmt, rows, cols, W, x)
        assert np.array_equal(y.astype(np.float64), ref), (fmt, rows, cols)
    for fmt, n in ((Q8, 256), (Q8, 1024), (Q4, 1024)):
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
        mant = rng.integers(1 << 23, 1 << 24, (4, n)).astype(np.float64)
        x = (mant * 2.0 ** rng.integers(-60, 20, (4, n)) * rng.choice([-1, 1], (4, n))).astype(np.float32)
        monkeypatch.setenv("QGEMV_TILE", mx_tile(n, 16, fmt=NAMES[fmt]))
        y = gpu_gemv(torch, fmt, dev(torch, W), x, n)
        assert np.array_equal(y, x[:, perm]), (fmt, n)
    n = 512  # BF16 identity
    perm = rng.permutation(n)
    dense = np.zeros((n, n), dtype=np.float32)
    dense[np.arange(n), perm] = 1.0
    W = (dense.view(np.uint32) >> 16).astype(np.uint16).view(np.uint8).reshape(-1)
    mant = rng.integers(1 << 23, 1 << 24, (4, n)).astype(np.float64)
    x = (mant * 2.0 ** rng.integers(-60, 20, (4, n)) * rng.choice([-1, 1], (4, n))).astype(np.float32)
    monkeypatch.setenv("QGEMV_TILE", mx_tile(n, 16, fmt="bf16"))
    y = gpu_gemv(torch, BF, dev(torch, W), x, n)
    assert np.array_equal(y, x[:, perm])


# ----------------- persistent matrix cores on 512-wide slices fed by the ring (kind P)
def mxp_tile(cols, chunk=4, fmt="q8_0"):
    return f"{fmt}:4,{cols // 512},{16 * chunk},P"


@pytest.mark.parametrize("name,chunk", [("c2a_q8_0_10240x2560", 4), ("c1_q8_0_2560x2560", 2),
                                        ("c3_q4_0_8192x2560", 4), ("c3_bf16_8192x2560", 2)])
def test_mxp_config_full(torch, orc, monkeypatch, name, chunk):
    """The persistent ring kind on the workloads: parity at every T, a token's bits equal across T."""
    c = I.dense_case(name)
    monkeypatch.setenv("QGEMV_TILE", mxp_tile(c["cols"], chunk, NAMES[c["fmt"]]))
    st, t = _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], 4)
    assert st == 0 and t[6] == 9 and t[3] == 512, (st, t)
    check_dense(torch, orc, c["fmt"], c["rows"], c["cols"], c["W"], c["x"], f"mxp {name} chunk={chunk}")


def test_mxp_ragged_chunks_and_formats(torch, orc, monkeypatch):
    """Ragged rows (a partial last tile; fewer tiles than workgroups; several tiles
    and chunks per workgroup, so both chunk buffers are reused), one to eleven
    slices (a twelfth would leave no wave to sum the chunks: refused), chunks of one
    to eight tiles, every format."""
    for fmt in (Q8, Q4, BF):
        for rows, cols in ((1, 512), (3, 1024), (17, 512), (67, 2560), (1000, 1536), (4096 + 37, 512),
                           (20480 + 9, 1024), (777, 5632), (777, 6144)):
            for chunk in (1, 2, 8):
                monkeypatch.setenv("QGEMV_TILE", mxp_tile(cols, chunk, NAMES[fmt]))
                nw = cols // 512  # slots of max(tile, 8 KB), chunk buffers of 16 rows x pad(4) fp32 per slice
                lds = nw * {Q8: 8704, Q4: 8192, BF: 16384}[fmt] + 2 * chunk * nw * 16 * 4 * 4 + 16
                st = _lib.qg_query_tile(fmt, rows, cols, 4)[0]
                assert (st == 0) == (lds <= 160 * 1024 and nw <= 11), (fmt, rows, cols, chunk, st)
                if st:
                    continue
                rng = np.random.default_rng(rows * 1000 + cols + chunk + fmt)
                W = I.weights(rng, fmt, rows, cols)
                x = I.activations(rng, cols)
                check_dense(torch, orc, fmt, rows, cols, W, x, f"mxp {rows}x{cols} chunk={chunk}")


def test_mxp_chunks_keep_bits(torch, monkeypatch):
    """The same 512-wide k split at any chunk size: identical bits."""
    c = I.dense_case("c2a_q8_0_10240x2560")
    Wd, xd = dev(torch, c["W"]), dev(torch, c["x"])
    monkeypatch.setenv("QGEMV_TILE", mxp_tile(c["cols"], 4))
    base = ops.gemv("q8_0", Wd, xd, c["rows"]).cpu().numpy()
    for chunk in (1, 2, 3, 8):
        monkeypatch.setenv("QGEMV_TILE", mxp_tile(c["cols"], chunk))
        say(f"[mxp chunk] {chunk}")
        assert np.array_equal(ops.gemv("q8_0", Wd, xd, c["rows"]).cpu().numpy(), base), chunk


def test_mxp_direct_stores_keep_bits(torch, orc, monkeypatch):
    """Kind P holds a workgroup's outputs in LDS and writes them at its end when they fit
    (every shape here); the direct stores it falls back to on taller matrices, forced by
    QGEMV_P_DIRECT_STORES, give the same bits and pass the oracle too."""
    for fmt, rows, cols, chunk in ((Q8, 10240, 2560, 3), (Q4, 4096 + 37, 1024, 1), (BF, 333, 1536, 2)):
        rng = np.random.default_rng(rows + cols + fmt)
        W = I.weights(rng, fmt, rows, cols)
        x = I.activations(rng, cols)
        monkeypatch.setenv("QGEMV_TILE", mxp_tile(cols, chunk, NAMES[fmt]))
        monkeypatch.delenv("QGEMV_P_DIRECT_STORES", raising=False)
        held = check_dense(torch, orc, fmt, rows, cols, W, x, f"mxp held {rows}x{cols}")
        monkeypatch.setenv("QGEMV_P_DIRECT_STORES", "1")
        direct = check_dense(torch, orc, fmt, rows, cols, W, x, f"mxp direct {rows}x{cols}")
        assert np.array_equal(held, direct), (fmt, rows, cols)


def test_mxp_exact_inputs_bitwise(torch, orc, monkeypatch):
    """Dyadic inputs (exact result representable) and identity-like matrices (y = a
    permutation of x, carried exactly by the three bf16 pieces)."""
    rng = np.random.default_rng(98)
    for fmt, rows, cols in ((Q8, 1000, 3072), (Q4, 777, 2560), (Q8, 10240, 2560)):
        W = dyadic_weights(rng, fmt, rows, cols)
        x = (rng.integers(-4, 5, (4, cols)) / 4.0).astype(np.float32)
        monkeypatch.setenv("QGEMV_TILE", mxp_tile(cols, 2, NAMES[fmt]))
        y = gpu_gemv(torch, fmt, dev(torch, W), x, rows)
        ref, _ = orc.gemv(fmt, rows, cols, W, x)
        assert np.array_equal(y.astype(np.float64), ref), (fmt, rows, cols)
    for fmt, n in ((Q8, 512), (Q8, 1024), (Q4, 1024)):
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
        mant = rng.integers(1 << 23, 1 << 24, (4, n)).astype(np.float64)
        x = (mant * 2.0 ** rng.integers(-60, 20, (4, n)) * rng.choice([-1, 1], (4, n))).astype(np.float32)
        monkeypatch.setenv("QGEMV_TILE", mxp_tile(n, 1, NAMES[fmt]))
        y = gpu_gemv(torch, fmt, dev(torch, W), x, n)
        assert np.array_equal(y, x[:, perm]), (fmt, n)


def test_tile_override_other_k_split(torch, orc, monkeypatch):
    c = I.dense_case("c2b_q8_0_2560x6144")
    monkeypatch.setenv("QGEMV_TILE", "q8_0:2,4,16")  # 12 slices over 4 waves
    y = gpu_gemv(torch, Q8, dev(torch, c["W"]), c["x"], c["rows"])
    ref, bound = orc.gemv(Q8, c["rows"], c["cols"], c["W"], c["x"])
    assert_parity(y, ref, bound, "c2b nw=4")


# ------------------------------------------------- matrix-core (MFMA) kernel
def mfma_tile(cols, rw=32, rg=1):
    nsl = -(-cols // 512)
    return f"q8_0:8,{nsl * rg},{rw},m"


@pytest.mark.parametrize("name,rw,rg", [("c1_q8_0_2560x2560", 16, 1), ("c2a_q8_0_10240x2560", 32, 2),
                                        ("c2b_q8_0_2560x6144", 16, 1), ("c2a_q8_0_10240x2560", 48, 1)])
def test_mfma_config_full(torch, orc, monkeypatch, name, rw, rg):
    """The matrix-core kernel on the workloads: parity, and a token's bits do not depend on T."""
    c = I.dense_case(name)
    monkeypatch.setenv("QGEMV_TILE", mfma_tile(c["cols"], rw, rg))
    st, t = _lib.qg_query_tile(c["fmt"], c["rows"], c["cols"], 4)
    assert st == 0 and t[5] == 1 and t[6] == 1, (st, t)
    check_dense(torch, orc, c["fmt"], c["rows"], c["cols"], c["W"], c["x"], f"mfma {name}")


def test_mfma_tiny_shapes(torch, orc, monkeypatch):
    """Ragged rows (partial 16-row tiles) and short last k slices (streamed rows
    must be a multiple of 16 bytes: cols a multiple of 256)."""
    for rows in TINY_ROWS:
        for cols in (256, 512, 768, 1280, 1792, 2304, 4096, 6144):
            monkeypatch.setenv("QGEMV_TILE", mfma_tile(cols, 16 if rows < 40 else 48))
            rng = np.random.default_rng(rows * 1000 + cols)
            W = I.weights(rng, Q8, rows, cols)
            x = I.activations(rng, cols)
            check_dense(torch, orc, Q8, rows, cols, W, x, "mfma tiny")


def test_mfma_dyadic_bitwise(torch, orc, monkeypatch):
    """Dyadic x splits into one exact bf16 piece and every partial sum is exact: bitwise."""
    rng = np.random.default_rng(99)
    rows, cols = 1000, 2816
    W = dyadic_weights(rng, Q8, rows, cols)
    x = (rng.integers(-4, 5, (4, cols)) / 4.0).astype(np.float32)
    monkeypatch.setenv("QGEMV_TILE", mfma_tile(cols, 32))
    y = gpu_gemv(torch, Q8, dev(torch, W), x, rows)
    ref, _ = orc.gemv(Q8, rows, cols, W, x)
    assert np.array_equal(y.astype(np.float64), ref)


def test_mfma_x_pieces_full_range(torch, orc, monkeypatch):
    """x with full 24-bit significands over a wide exponent range (the kernel
    splits each x into three bf16 pieces)."""
    rng = np.random.default_rng(5)
    rows, cols = 96, 1024
    W = I.weights(rng, Q8, rows, cols)
    mant = rng.integers(1 << 23, 1 << 24, (4, cols)).astype(np.float64)
    x = (mant * 2.0 ** rng.integers(-40, -10, (4, cols)) * rng.choice([-1, 1], (4, cols))).astype(np.float32)
    monkeypatch.setenv("QGEMV_TILE", mfma_tile(cols, 32))
    y = gpu_gemv(torch, Q8, dev(torch, W), x, rows)
    ref, bound = orc.gemv(Q8, rows, cols, W, x)
    assert_parity(y, ref, bound, "mfma x pieces")


def test_mfma_persistent_agrees_bitwise(torch, orc, monkeypatch):
    """The persistent matrix-core kernel (one workgroup per CU, chunked partial
    sums summed by the last-arriving wave) gives the bits of the per-workgroup
    matrix-core kernel, and matches the oracle, on ragged and small shapes."""
    shapes = [(1, 256), (17, 768), (67, 2560), (300, 1024), (2560, 2560), (10240, 2560), (2560, 6144), (4099, 512)]
    for rows, cols in shapes:
        rng = np.random.default_rng(rows + 7 * cols)
        W = I.weights(rng, Q8, rows, cols)
        x = I.activations(rng, cols)
        Wd = dev(torch, W)
        for chunk in (16, 128):
            monkeypatch.setenv("QGEMV_TILE", mfma_tile(cols, 32))
            ref = gpu_gemv(torch, Q8, Wd, x, rows)
            nsl = -(-cols // 512)
            monkeypatch.setenv("QGEMV_TILE", f"q8_0:8,{nsl},{chunk},p")
            say(f"[persist] {rows}x{cols} chunk={chunk}")
            y = check_dense(torch, orc, Q8, rows, cols, W, x, f"persist {rows}x{cols} chunk={chunk}")
            assert np.array_equal(y, ref), (rows, cols, chunk)


# ------------------------------------------------------------- fused argmax
def argmax_check(torch, orc, fmt, rows, cols, W, x, what, sel_oracle=True):
    """Fused argmax against (a) the argmax of the dense call's own output, bit for
    bit (same per-row arithmetic, lowest row on ties), and (b) the oracle: the
    chosen row's exact y is within the error bounds of the true maximum."""
    Wd, xd = dev(torch, W), dev(torch, x)
    idx, val = ops.argmax(NAMES[fmt], Wd, xd, rows)
    torch.cuda.synchronize()
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    y = ops.gemv(NAMES[fmt], Wd, xd, rows).cpu().numpy()
    assert idx.tolist() == np.argmax(y, axis=1).tolist(), what
    assert np.array_equal(val, y[np.arange(y.shape[0]), idx]), what
    if sel_oracle:
        oi, ov, yo, bo = orc.argmax(fmt, rows, cols, W, x)
        tol = 1e-4 * bo + 1e-6
        for t in range(x.shape[0]):
            assert yo[t, idx[t]] >= ov[t] - (tol[t, idx[t]] + tol[t, oi[t]]), (what, t, idx[t], oi[t])
            assert abs(val[t] - yo[t, idx[t]]) <= tol[t, idx[t]], (what, t)
    return idx, val


@pytest.mark.parametrize("name", ["c1_q8_0_2560x2560", "c2a_q8_0_10240x2560", "c2b_q8_0_2560x6144",
                                  "c3_q4_0_8192x2560", "c3_bf16_8192x2560"])
def test_argmax_configs(torch, orc, name):
    c = I.dense_case(name)
    for T in (1, 2, 3, 4):
        say(f"[argmax] {name} T={T}")
        argmax_check(torch, orc, c["fmt"], c["rows"], c["cols"], c["W"], c["x"][:T], f"{name} T={T}")


def test_argmax_ties_negatives_and_kinds(torch, orc, monkeypatch):
    """Exact ties (duplicated largest rows: the lowest wins), all-negative outputs,
    ragged row counts, and every kernel kind the fused argmax runs on."""
    rng = np.random.default_rng(31)
    for rows, cols in ((1, 256), (67, 512), (1000, 2560), (333, 736)):
        W = I.weights(rng, Q8, rows, cols)
        x = I.activations(rng, cols)
        if rows > 10:  # copy the largest row of token 0 over two later rows and an earlier one
            y0, _ = orc.gemv(Q8, rows, cols, W, x[:1])
            best = int(np.argmax(y0[0]))
            rb = I.packed_row_bytes(Q8, cols)
            W = W.copy()
            for r in (rows // 3, rows - 1, 2):
                W[r * rb:(r + 1) * rb] = W[best * rb:(best + 1) * rb]
        neg = -np.abs(x)  # a second activation pattern
        for kind_tile in (None, "q8_0:4,{nsl},40,l3", "q8_0:4,{nsl},48,L2", "q8_0:4,{nsl},16,s", "q8_0:2,{nsl},4,d",
                          "q8_0:8,{nsl},64,p", "q8_0:4,{nsl256},40,x", "q8_0:4,{nsl256},64,x2",
                          "q8_0:4,{nsl256},24,h2", "q8_0:4,{nsl},32,P", "q8_0:4,{nsl},48,X"):
            nsl, nsl256 = -(-cols // 512), cols // 256
            if "{nsl256}" in (kind_tile or "") and cols % 256:
                continue  # 256-wide slices
            if (kind_tile or "").endswith((",P", ",X")) and cols % 512:
                continue  # 512-wide slices
            if kind_tile:
                kind_tile = kind_tile.format(nsl=nsl, nsl256=nsl256)
            if kind_tile:
                monkeypatch.setenv("QGEMV_TILE", kind_tile)
            else:
                monkeypatch.delenv("QGEMV_TILE", raising=False)
            if kind_tile and cols % 256 and not kind_tile.endswith(",d"):
                continue  # streamed kinds need 16-byte rows
            what = f"{rows}x{cols} tile={kind_tile}"
            say(f"[argmax] {what}")
            idx, _ = argmax_check(torch, orc, Q8, rows, cols, W, x, what)
            if rows > 10:
                assert idx[0] == min(2, best), what
            argmax_check(torch, orc, Q8, rows, cols, W, neg, what + " neg-x")


# ------------------------------------------------------------- row subset
def rows_tile(fmt, rows, cols, T):
    """The dense tile with the row subset's default arithmetic: the matrix cores on
    256-wide slices up to 12 of them, else on 512-wide slices up to 12, where the LDS
    fits; else the vector-ALU kinds on 512-wide slices."""
    for n, kind in ((cols // 256, "x"), (cols // 512, "X")):
        width = 256 if kind == "x" else 512
        if cols % width == 0 and 1 <= n <= 12:
            spec = f"{NAMES[fmt]}:4,{n},16,{kind}"
            os.environ["QGEMV_TILE"] = spec
            ok = _lib.qg_query_tile(fmt, rows, cols, T)[0] == 0
            del os.environ["QGEMV_TILE"]
            if ok:
                return spec
            break
    nsl = -(-cols // 512)
    for spec in (f"{NAMES[fmt]}:4,{nsl},16,L2", f"{NAMES[fmt]}:4,{nsl},8,d"):
        os.environ["QGEMV_TILE"] = spec
        ok = _lib.qg_query_tile(fmt, rows, cols, T)[0] == 0
        del os.environ["QGEMV_TILE"]
        if ok:
            return spec
    raise AssertionError("no tile")


def rows_check(torch, orc, monkeypatch, fmt, rows, cols, W, x, ids, what, pin=None):
    """Row subset against the oracle on the selected rows and, bit for bit, against
    the dense call's own output at those rows with the same arithmetic (the same
    matrix-core kind, or a vector-ALU kind on 512-wide slices)."""
    Wd, xd = dev(torch, W), dev(torch, x)
    if pin:
        monkeypatch.setenv("QGEMV_TILE", pin)
    y = ops.gemv_rows(NAMES[fmt], Wd, xd, rows, dev(torch, ids.astype(np.int32))).cpu().numpy()
    monkeypatch.delenv("QGEMV_TILE", raising=False)
    ok = (ids >= 0) & (ids < rows)
    assert np.isnan(y[:, ~ok]).all(), what
    if ok.any():
        ref, bound = orc.gemv(fmt, rows, cols, W, x, sel=ids[ok])
        assert_parity(y[:, ok], ref, bound, what)
        monkeypatch.setenv("QGEMV_TILE", rows_tile(fmt, rows, cols, x.shape[0]))
        full = ops.gemv(NAMES[fmt], Wd, xd, rows).cpu().numpy()
        monkeypatch.delenv("QGEMV_TILE")
        assert np.array_equal(y[:, ok], full[:, ids[ok]]), what


@pytest.mark.parametrize("fmt", [Q8, Q4, BF])
def test_rows_subset_shapes(torch, orc, monkeypatch, fmt):
    rng = np.random.default_rng(40 + fmt)
    for rows, cols in ((100, 256), (333, 2560), (70, 6144 if fmt != BF else 4608)):
        W = I.weights(rng, fmt, rows, cols)
        x = I.activations(rng, cols)
        for n_sel in (1, 7, 65, 130):
            ids = rng.integers(0, rows, n_sel)          # unsorted, with repeats
            for T in (1, 4):
                say(f"[rows] fmt={NAMES[fmt]} {rows}x{cols} n_sel={n_sel} T={T}")
                rows_check(torch, orc, monkeypatch, fmt, rows, cols, W, x[:T], ids, f"{rows}x{cols} n={n_sel} T={T}")
                spec = rows_tile(fmt, rows, cols, T)
                pin = spec.replace(",16,", ",32,")
                monkeypatch.setenv("QGEMV_TILE", pin)
                fits = _lib.qg_query_tile(fmt, rows, cols, T)[0] == 0
                monkeypatch.delenv("QGEMV_TILE")
                if spec.endswith(("x", "X")) and fits:  # the same kind pinned, 32 ids per workgroup
                    rows_check(torch, orc, monkeypatch, fmt, rows, cols, W, x[:T], ids,
                               f"{rows}x{cols} n={n_sel} T={T} pin={pin}", pin=pin)


@pytest.mark.parametrize("fmt", [Q8, Q4, BF])
def test_rows_subset_wide_workgroups(torch, orc, monkeypatch, fmt):
    """Subsets long enough for 80 and 128 ids per workgroup (ids 64.. held in a
    second register), each with a short last workgroup."""
    rng = np.random.default_rng(50 + fmt)
    rows, cols = 333, 2560
    W = I.weights(rng, fmt, rows, cols)
    x = I.activations(rng, cols)
    for n_sel in (20001, 32768 + 77):
        ids = rng.integers(0, rows, n_sel)
        ids[rng.choice(n_sel, 9, replace=False)] = -5  # a few bad ids spread over the range
        for T in (1, 4):
            say(f"[rows] fmt={NAMES[fmt]} {rows}x{cols} n_sel={n_sel} T={T}")
            rows_check(torch, orc, monkeypatch, fmt, rows, cols, W, x[:T], ids, f"{rows}x{cols} n={n_sel} T={T}")


def test_rows_subset_bad_ids(torch, orc, monkeypatch):
    rng = np.random.default_rng(3)
    rows, cols = 50, 512
    W = I.weights(rng, Q8, rows, cols)
    x = I.activations(rng, cols)
    ids = np.array([3, -1, 49, 50, 7, 1 << 30, 0], dtype=np.int64)
    rows_check(torch, orc, monkeypatch, Q8, rows, cols, W, x, ids, "bad ids")


# ---------------------------------------------------------- grouped experts
def grouped_check(torch, orc, fmt, n_experts, rows, cols, ids, W, x, what):
    say(f"[{what}] fmt={NAMES[fmt]} experts={n_experts} rows={rows} cols={cols} ids={ids.tolist()}")
    y = ops.grouped_experts(NAMES[fmt], dev(torch, W), dev(torch, x), dev(torch, ids), n_experts, rows)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    ref, bound = orc.grouped(fmt, n_experts, rows, cols, ids, W, x)
    assert_parity(y, ref, bound, what)
    return y


def test_grouped_config(torch, orc, monkeypatch):
    g = I.grouped_case()
    y = grouped_check(torch, orc, g["fmt"], g["n_experts"], g["rows"], g["cols"], g["ids"], g["W"], g["x"], "c5")
    # equals the plain call on each selected expert bit for bit, run on the kind the
    # grouped kernel shares its arithmetic with (matrix cores on 256-wide k slices)
    st, t = _lib.qg_query_tile(g["fmt"], g["rows"], g["cols"], g["T"])
    assert st == 0 and t[6] == 8, t
    rb = I.packed_row_bytes(g["fmt"], g["cols"])
    Wd = dev(torch, g["W"])
    monkeypatch.setenv("QGEMV_TILE", f"{NAMES[g['fmt']]}:4,{g['cols'] // 256},32,x")
    for t in range(g["T"]):
        for j in (0, g["topk"] - 1):
            e = int(g["ids"][t, j])
            We = Wd[e * g["rows"] * rb:(e + 1) * g["rows"] * rb]
            yp = gpu_gemv(torch, g["fmt"], We, g["x"][t:t + 1], g["rows"])
            assert np.array_equal(yp[0], y[t, j])


@pytest.mark.parametrize("fmt", [Q4, Q8, BF])
def test_grouped_sharing(torch, orc, monkeypatch, fmt):
    """Shared and duplicated experts on the default (matrix-core) path, on the
    LDS-DMA vector-ALU and direct paths (tile overrides), pinned matrix-core tiles
    with row groups, and at a width whose rows are not 16-byte aligned."""
    cases = [
        np.array([[3, 5], [3, 7], [3, 5], [3, 9]], np.int32),   # expert 3 shared by 4 tokens, 5 by 2
        np.array([[1, 1, 2], [2, 2, 1], [0, 11, 2], [11, 0, 4]], np.int32),  # duplicates inside a token
        np.array([[7, 8, 9, 10]], np.int32),                    # T = 1
        np.array([[4, 6], [6, 4], [4, 6]], np.int32),           # T = 3, ne = 3
    ]
    n_experts, rows = 12, 200
    for cols, tile in ((1024, None), (1024, f"{NAMES[fmt]}:4,2,8,d"), (1024, f"{NAMES[fmt]}:4,2,24,L2"),
                       (1024, f"{NAMES[fmt]}:4,8,64,x"), (768, f"{NAMES[fmt]}:4,3,16,x"),
                       (1024, f"{NAMES[fmt]}:4,4,64,x2"), (768, f"{NAMES[fmt]}:4,6,32,x2"),
                       (1056 if fmt != BF else 1048, None)):
        if tile:
            monkeypatch.setenv("QGEMV_TILE", tile)
        else:
            monkeypatch.delenv("QGEMV_TILE", raising=False)
        rng = np.random.default_rng(10 + fmt + cols)
        W = I.weights(rng, fmt, n_experts * rows, cols)
        x = I.activations(rng, cols)
        for ids in cases:
            T = ids.shape[0]
            grouped_check(torch, orc, fmt, n_experts, rows, cols, ids, W, x[:T], f"sharing cols={cols} tile={tile}")


def test_grouped_bad_id_gives_nan_rows(torch, orc):
    rng = np.random.default_rng(77)
    n_experts, rows, cols = 6, 100, 512
    W = I.weights(rng, Q8, n_experts * rows, cols)
    x = I.activations(rng, cols, 2)
    ids = np.array([[0, 6], [-1, 2]], np.int32)
    y = ops.grouped_experts("q8_0", dev(torch, W), dev(torch, x), dev(torch, ids), n_experts, rows)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    assert np.isnan(y[0, 1]).all() and np.isnan(y[1, 0]).all()
    good = np.array([[0, 0], [2, 2]], np.int32)
    ref, bound = orc.grouped(Q8, n_experts, rows, cols, good, W, x)
    assert_parity(y[0, 0], ref[0, 0], bound[0, 0], "good slot 0,0")
    assert_parity(y[1, 1], ref[1, 1], bound[1, 1], "good slot 1,1")
