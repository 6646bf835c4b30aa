"""The C-ABI library on the CPU: it loads, exports every function include/qgemv.h
declares, packs and unpacks bit-exactly, and rejects bad arguments with the
documented status before touching the GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from block_quantized_token_amd import _lib, inputs as I, ops
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qgemv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from block_quantized_token_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(q\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in range(5):
        assert _lib.status_string(st).startswith(("QG_OK", "QG_E"))
    assert "unknown" in _lib.status_string(99)


def test_packed_bytes(lib, orc):
    for fmt in (0, 1, 2):
        for rows, cols in ((1, 32), (10240, 2560), (2560, 6144), (248320, 5120), (7, 640)):
            assert _lib.qg_packed_bytes(fmt, rows, cols) == orc.packed_bytes(fmt, rows, cols)
    assert _lib.qg_packed_bytes(0, 4, 33) == 0 and _lib.qg_packed_bytes(1, 4, 48) == 0
    assert _lib.qg_packed_bytes(7, 4, 32) == 0 and _lib.qg_packed_bytes(0, -1, 32) == 0


def test_pack_matches_generator_and_oracle(lib, orc):
    rng = np.random.default_rng(1)
    d, c = I.q8_0_fields(rng, 9, 320)
    packed = ops.pack_q8_0(d, c)
    assert np.array_equal(packed, I.pack_q8_0(d, c))
    od, oc = orc.unpack(0, 9, 320, packed)
    assert np.array_equal(od, d) and np.array_equal(oc, c.astype(np.int32))
    d4, c4 = I.q4_0_fields(rng, 9, 320)
    packed4 = ops.pack_q4_0(d4, c4)
    assert np.array_equal(packed4, I.pack_q4_0(d4, c4))
    od, oc = orc.unpack(1, 9, 320, packed4)
    assert np.array_equal(od, d4) and np.array_equal(oc, c4.astype(np.int32))


def test_pack_unpack_every_field_value(lib):
    """All 65,536 scale patterns, every int8 code and every nibble round-trip bit-exactly."""
    rows, cols = 2048, 1024  # 65,536 blocks
    d = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(rows, cols // 32)
    c8 = (np.arange(rows * cols) % 256 - 128).astype(np.int8).reshape(rows, cols)
    gd, gc = ops.unpack_q8_0(ops.pack_q8_0(d, c8), rows, cols)
    assert np.array_equal(gd, d) and np.array_equal(gc, c8)
    c4 = (np.arange(rows * cols) * 7 % 16).astype(np.uint8).reshape(rows, cols)
    gd, gc = ops.unpack_q4_0(ops.pack_q4_0(d, c4), rows, cols)
    assert np.array_equal(gd, d) and np.array_equal(gc, c4)


def test_unpack_pack_random_bytes(lib):
    rng = np.random.default_rng(2)
    for rows, cols, fmt in ((13, 96, 0), (13, 96, 1)):
        raw = rng.integers(0, 256, size=_lib.qg_packed_bytes(fmt, rows, cols), dtype=np.uint8)
        if fmt == 0:
            assert np.array_equal(ops.pack_q8_0(*ops.unpack_q8_0(raw, rows, cols)), raw)
        else:
            assert np.array_equal(ops.pack_q4_0(*ops.unpack_q4_0(raw, rows, cols)), raw)


def test_pack_q4_0_rejects_wide_codes(lib):
    d = np.zeros((1, 1), np.uint16)
    c = np.full((1, 32), 16, np.uint8)
    with pytest.raises(_lib.QGError) as e:
        ops.pack_q4_0(d, c)
    assert e.value.status == _lib.QG_EINVAL


# ------------------------------------------------------------ argument checks
# Fake but aligned device addresses: every call below must be refused on the
# host, so nothing is ever dereferenced or launched.
W0, X0, Y0, I0 = 0x10000000, 0x20000000, 0x30000000, 0x40000000


@pytest.mark.parametrize("args, status", [
    ((64, 256, 1, W0, X0, 0), _lib.QG_EINVAL),          # null y
    ((64, 256, 1, 0, X0, Y0), _lib.QG_EINVAL),          # null W
    ((64, 256, 1, W0, 0, Y0), _lib.QG_EINVAL),          # null x
    ((0, 256, 1, W0, X0, Y0), _lib.QG_EINVAL),          # rows 0
    ((64, 0, 1, W0, X0, Y0), _lib.QG_EINVAL),           # cols 0
    ((64, 256, 0, W0, X0, Y0), _lib.QG_EINVAL),         # T 0
    ((64, 256, 5, W0, X0, Y0), _lib.QG_EINVAL),         # T 5
    ((64, 250, 1, W0, X0, Y0), _lib.QG_EINVAL),         # not whole blocks
    ((64, 256, 1, W0 + 2, X0, Y0), _lib.QG_EALIGN),     # W misaligned
    ((64, 256, 1, W0, X0 + 4, Y0), _lib.QG_EALIGN),     # x misaligned
    ((64, 256, 1, W0, X0, Y0 + 2), _lib.QG_EALIGN),     # y misaligned
    ((64, 256, 1, W0, X0, W0 + 64), _lib.QG_EINVAL),    # y inside W
    ((64, 256, 2, W0, X0, X0 + 256), _lib.QG_EINVAL),   # y overlaps x
    ((1 << 31, 256, 1, W0, X0, Y0), _lib.QG_EUNSUPPORTED),
])
def test_dense_argument_errors(lib, args, status):
    for entry in (_lib.qgemv_q8_0, _lib.qgemv_q4_0):
        assert entry(*args) == status, _lib.last_error()
        assert _lib.last_error()


def test_bf16_cols(lib):
    assert _lib.qgemv_bf16(64, 250, 1, W0, X0, Y0) == _lib.QG_EUNSUPPORTED
    assert _lib.qgemv_bf16(64, 256, 1, W0 + 8, X0, Y0) == _lib.QG_EALIGN


@pytest.mark.parametrize("args, status", [
    ((3, 4, 64, 256, 1, 2, I0, W0, X0, Y0), _lib.QG_EINVAL),    # bad fmt
    ((0, 0, 64, 256, 1, 2, I0, W0, X0, Y0), _lib.QG_EINVAL),    # no experts
    ((0, 4, 64, 256, 1, 0, I0, W0, X0, Y0), _lib.QG_EINVAL),    # topk 0
    ((0, 4, 64, 256, 1, 2, 0, W0, X0, Y0), _lib.QG_EINVAL),     # null ids
    ((0, 4, 64, 256, 1, 2, I0 + 2, W0, X0, Y0), _lib.QG_EALIGN),
    ((0, 4, 64, 256, 5, 2, I0, W0, X0, Y0), _lib.QG_EINVAL),    # T 5
    ((0, 4, 64, 256, 1, 2, I0, W0, X0, I0), _lib.QG_EINVAL),    # y overlaps ids
])
def test_grouped_argument_errors(lib, args, status):
    assert _lib.qgemv_grouped_experts(*args) == status, _lib.last_error()


V0, K0 = 0x50000000, 0x60000000


@pytest.mark.parametrize("args, status", [
    ((0, 64, 256, 1, W0, X0, 0, I0, V0), _lib.QG_EINVAL),          # null work
    ((0, 64, 256, 1, W0, X0, K0, 0, V0), _lib.QG_EINVAL),          # null idx
    ((0, 64, 256, 1, W0, X0, K0, I0, 0), _lib.QG_EINVAL),          # null val
    ((0, 64, 256, 5, W0, X0, K0, I0, V0), _lib.QG_EINVAL),         # T 5
    ((7, 64, 256, 1, W0, X0, K0, I0, V0), _lib.QG_EINVAL),         # bad fmt
    ((0, 64, 256, 1, W0, X0, K0 + 4, I0, V0), _lib.QG_EALIGN),     # work not 8-byte aligned
    ((0, 64, 256, 1, W0, X0, K0, I0 + 2, V0), _lib.QG_EALIGN),     # idx misaligned
    ((0, 64, 256, 2, W0, X0, K0, I0, I0 + 4), _lib.QG_EINVAL),     # val overlaps idx
    ((0, 64, 256, 1, W0, X0, W0 + 8, I0, V0), _lib.QG_EINVAL),     # work inside W
    ((0, 64, 256, 1, W0, X0, K0, X0, V0), _lib.QG_EINVAL),         # idx overlaps x
])
def test_argmax_argument_errors(lib, args, status):
    assert _lib.qgemv_argmax(*args) == status, _lib.last_error()
    assert _lib.last_error()



def test_tile_query_and_override(lib, monkeypatch):
    monkeypatch.delenv("QGEMV_TILE", raising=False)
    t = ops.query_tile("q8_0", 10240, 2560, 1)
    # matrix cores on 256-wide k slices, one wave per slice (a row's block spread over 4 lanes)
    assert (t["kind"], t["lanes_per_row"], t["k_slice"], t["waves_per_wg"]) == (8, 4, 256, 10)
    # the k split must not depend on T (bit-identical tokens across T): waves
    # that each reduce one slice (streamed kinds; direct with waves >= slices)
    # or the same number of slice-looping waves
    def k_split(t, cols):
        nsl = -(-cols // t["k_slice"])
        return (t["k_slice"], nsl if t["kind"] in (1, 7, 8, 9, 11) else min(t["waves_per_wg"], nsl))
    for fmt in ("q8_0", "q4_0", "bf16"):
        for rows, cols in ((10240, 2560), (2560, 6144), (248320, 5120), (8192, 2560), (7, 65536),
                           (151936, 3584), (65536, 5120)):
            tiles = [ops.query_tile(fmt, rows, cols, T) for T in (1, 2, 3, 4)]
            assert len({k_split(t, cols) for t in tiles}) == 1, (fmt, rows, cols, tiles)
            # the vector-ALU kinds share their arithmetic per k slice; of the matrix-core
            # kinds only X and P (the same 512-wide slices) do
            arith = {(t["mfma"], {8: 8, 9: 11}.get(t["kind"], t["kind"]) if t["kind"] in (8, 9, 11) else -1)
                     for t in tiles}
            assert len(arith) == 1, (fmt, rows, cols, tiles)
    # the LM head and other Q8_0 matrices of 224 MiB or more with at least seven 512-wide
    # slices, or of 512 MiB or more: the persistent matrix cores on 512-wide slices
    for rows, cols in ((248320, 5120), (151936, 3584), (65536, 5120), (49152, 5120)):
        t = ops.query_tile("q8_0", rows, cols, 4)
        assert (t["kind"], t["k_slice"], t["waves_per_wg"], t["lanes_per_row"]) == (9, 512, cols // 512, 4), t
    assert ops.query_tile("q8_0", 32768, 5120, 4)["kind"] != 9  # 170 MiB
    assert ops.query_tile("q8_0", 100000, 2560, 4)["kind"] != 9  # 259 MiB, five slices
    assert ops.query_tile("q8_0", 220000, 2560, 4)["kind"] == 9  # 571 MiB
    # more than twelve 256-wide slices: the matrix cores on 512-wide slices
    t = ops.query_tile("q8_0", 2560, 6144, 1)
    assert (t["kind"], t["k_slice"], t["waves_per_wg"], t["lanes_per_row"]) == (11, 512, 12, 4), t
    # Q4_0 at the LM head's shape: kind X while its rows fit one workgroup per CU (T <= 2),
    # the persistent kind on the same slices (the same bits) when they do not (T >= 3)
    assert [ops.query_tile("q4_0", 248320, 5120, T)["kind"] for T in (1, 2, 3, 4)] == [11, 11, 9, 9]
    assert ops.query_tile("q4_0", 163840, 5120, 4)["kind"] == 11  # 256 workgroups at every T
    monkeypatch.setenv("QGEMV_TILE", "q8_0:2,5,8")
    t = ops.query_tile("q8_0", 10240, 2560, 4)
    assert (t["rows_per_batch"], t["waves_per_wg"], t["rows_per_wg"]) == (2, 5, 8)
    q4 = ops.query_tile("q4_0", 10240, 2560, 4)  # other formats keep their default
    assert (q4["rows_per_batch"], q4["rows_per_wg"]) != (2, 8)
    # LDS-DMA kind: depth after 'l'
    monkeypatch.setenv("QGEMV_TILE", "q8_0:4,5,48,l6")
    t = ops.query_tile("q8_0", 10240, 2560, 4)
    assert (t["kind"], t["depth"], t["rows_per_wg"]) == (2, 6, 48)
    monkeypatch.setenv("QGEMV_TILE", "q8_0:4,5,48,l2")  # T=1: x takes one slot of two
    assert ops.query_tile("q8_0", 10240, 2560, 1)["depth"] == 2
    # malformed, outside the set, or not compiled (16 rows x 4 tokens; pipelined RB=8 at T=4;
    # DMA depth 5; DMA depth 2 at T=4, where x takes two slots; DMA with rb 2; a DMA ring
    # past the LDS)
    for bad in ("q8_0:3,5,8", "q8_0:2,13,8", "q8_0:2,5,6", "q9:2,5,8", "q8_0:2,5", "q8_0:16,5,32", "q8_0:8,5,32",
                "q8_0:4,5,48,l5", "q8_0:4,5,48,l2", "q8_0:2,5,48,l4", "q8_0:4,10,48,l6", "q8_0:4,5,48,l", "q8_0:4,5,48,l6x",
                "q8_0:4,10,48,P", "q8_0:4,5,40,P", "q8_0:4,5,1024,P",  # P: nw != slices, rw % 16, LDS
                "q8_0:4,10,48,x3", "q8_0:4,10,48,x0x", "q8_0:4,4,48,X", "q8_0:4,5,2048,X"):
        monkeypatch.setenv("QGEMV_TILE", bad)
        st, _ = _lib.qg_query_tile(0, 10240, 2560, 4)
        assert st == _lib.QG_EINVAL, bad
        assert _lib.qgemv_q8_0(10240, 2560, 4, W0, X0, Y0) == _lib.QG_EINVAL
    # P runs one more wave than it has slices, which sums the chunks: twelve 512-wide
    # slices (6144 columns) leave no room for it and are refused; eleven are accepted
    monkeypatch.setenv("QGEMV_TILE", "q8_0:4,12,48,P")
    assert _lib.qg_query_tile(0, 2560, 6144, 4)[0] == _lib.QG_EINVAL
    assert "at most 11" in _lib.last_error()
    monkeypatch.setenv("QGEMV_TILE", "q8_0:4,11,48,P")
    assert _lib.qg_query_tile(0, 2560, 5632, 4)[0] == 0


def test_header_names_every_tile_kind(lib, monkeypatch):
    """Every kind letter QGEMV_TILE accepts is documented in the header, and every
    documented letter is accepted for some tile."""
    text = open(HEADER).read()
    start = text.index("QGEMV_TILE=")
    para = text[start:text.index("QG_EINVAL.\n", start)]
    documented = set(re.findall(r"^ \*   ([a-zA-Z])(?:<D>)?\s", para, flags=re.M))
    # (kind, spec suffix, shape) that the compiled set accepts
    probes = {"d": ("d", 10240, 2560, "2,5,8"), "s": ("s", 10240, 2560, "4,5,16"),
              "l": ("l2", 10240, 2560, "4,5,40"), "L": ("L2", 10240, 2560, "4,5,40"),
              "u": ("u2", 10240, 2560, "4,4,40"), "h": ("h2", 10240, 2560, "4,10,40"),
              "m": ("m", 10240, 2560, "8,5,32"), "p": ("p", 248320, 5120, "8,10,64"),
              "x": ("x", 10240, 2560, "4,10,40"), "P": ("P", 10240, 2560, "4,5,48"),
              "X": ("X", 10240, 2560, "4,5,48")}
    accepted = set()
    for letter in "abcdefghijklmnopqrstuvwxyzABCDEFGHIJKLMNOPQRSTUVWXYZ":
        suffix, rows, cols, head = probes.get(letter, (letter, 10240, 2560, "4,10,40"))
        for spec in (f"{head},{suffix}", f"{head},{letter}2", f"{head},{letter}"):
            monkeypatch.setenv("QGEMV_TILE", "q8_0:" + spec)
            st, _ = _lib.qg_query_tile(0, rows, cols, 1)
            if st == _lib.QG_OK:
                accepted.add(letter)
                break
    monkeypatch.delenv("QGEMV_TILE")
    assert accepted == documented == set(probes), (accepted, documented)


def test_binding_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    W = torch.zeros(34 * 4, dtype=torch.uint8)
    x = torch.zeros(1, 32)
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.gemv("q8_0", W, x, rows=4)


def _binding_cases(torch):
    """(call, message) pairs: each call passes one buffer of the wrong dtype, rank or
    size, which the binding must refuse before any kernel could run past its end."""
    f32, i32, i64 = torch.float32, torch.int32, torch.int64
    rows, cols, E = 8, 256, 4
    W = torch.zeros(rows * cols // 32 * 34, dtype=torch.uint8)
    WE = torch.zeros(E * rows * cols // 32 * 18, dtype=torch.uint8)
    x = torch.zeros(2, cols)
    ids1 = torch.zeros(5, dtype=i32)
    ids2 = torch.zeros(2, 3, dtype=i32)
    h = torch.zeros(2, 3, cols)
    return [
        (lambda: ops.gemv("q8_0", W, x.half(), rows), "x must be fp32"),
        (lambda: ops.gemv("q8_0", W, x[0], rows), "x must be fp32"),
        (lambda: ops.gemv("q8_0", W[:-1], x, rows), "W holds"),
        (lambda: ops.gemv("q8_0", W, x, rows, out=torch.zeros(2, rows, dtype=torch.float16)), "out must be"),
        (lambda: ops.gemv("q8_0", W, x, rows, out=torch.zeros(2 * rows - 1)), "out holds"),
        (lambda: ops.gemv_rows("q8_0", W, x.bfloat16(), rows, ids1), "x must be fp32"),
        (lambda: ops.gemv_rows("q8_0", W, x, rows, ids1.long()), "ids must be int32"),
        (lambda: ops.gemv_rows("q8_0", W, x, rows, ids1, out=torch.zeros(2 * 5 - 1)), "out holds"),
        (lambda: ops.gemv_rows("q8_0", W, x, rows, ids1, out=torch.zeros(2, 5, dtype=i32)), "out must be"),
        (lambda: ops.argmax("q8_0", W, x.double(), rows), "x must be fp32"),
        (lambda: ops.argmax("q8_0", W, x, rows, work=torch.zeros(2, dtype=i32)), "work must be"),
        (lambda: ops.argmax("q8_0", W, x, rows, work=torch.zeros(1, dtype=i64)), "work holds"),
        (lambda: ops.grouped_experts("q4_0", WE, x.half(), ids2, E, rows), "x must be fp32"),
        (lambda: ops.grouped_experts("q4_0", WE, x.reshape(2, 1, cols), ids2, E, rows), "x must be fp32"),
        (lambda: ops.grouped_experts("q4_0", WE[:-1], x, ids2, E, rows), "W holds"),
        (lambda: ops.grouped_experts("q4_0", WE, x, ids2, E, rows, out=torch.zeros(2 * 3 * rows - 1)), "out holds"),
        (lambda: ops.grouped_experts("q4_0", WE, x, ids2, E, rows, out=torch.zeros(2, 3, rows, dtype=f32).half()),
         "out must be"),
        (lambda: ops.grouped_experts("q4_0", WE, x, ids2[:1], E, rows), "disagree on T"),
        (lambda: ops.experts_gate_up("q4_0", WE, WE, x.half(), ids2, E, rows), "x must be fp32"),
        (lambda: ops.experts_gate_up("q4_0", WE, WE[:-1], x, ids2, E, rows), "W holds"),
        (lambda: ops.experts_gate_up("q4_0", WE, WE, x, ids2.long(), E, rows), "ids must be int32"),
        (lambda: ops.experts_down("q4_0", WE, h.half(), ids2, E, rows), "h must be fp32"),
        (lambda: ops.experts_down("q4_0", WE[:-1], h, ids2, E, rows), "W holds"),
        (lambda: ops.quantize("q8_0", x.half()), "src must be fp32"),
        (lambda: ops.quantize("q8_0", x, out=torch.zeros(10, dtype=torch.uint8)), "out holds"),
    ]


def test_binding_refuses_wrong_dtypes_ranks_and_sizes(lib):
    torch = pytest.importorskip("torch")
    for call, msg in _binding_cases(torch):
        with pytest.raises(ValueError, match=msg):
            call()


@pytest.mark.parametrize("args, status", [
    ((0, 64, 256, 8, 0, 1, W0, X0, Y0), _lib.QG_EINVAL),            # null ids
    ((0, 64, 256, 0, I0, 1, W0, X0, Y0), _lib.QG_EINVAL),           # no rows selected
    ((0, 64, 256, 8, I0 + 2, 1, W0, X0, Y0), _lib.QG_EALIGN),       # ids misaligned
    ((0, 64, 256, 8, I0, 1, W0, X0, I0 + 4), _lib.QG_EINVAL),       # y overlaps ids
    ((0, 64, 256, 8, I0, 5, W0, X0, Y0), _lib.QG_EINVAL),           # T 5
    ((0, 64, 32, 8, I0, 1, W0, X0, Y0), _lib.QG_EUNSUPPORTED),      # 34-byte rows
    ((0, 64, 8192, 8, I0, 1, W0, X0, Y0), _lib.QG_EUNSUPPORTED),    # 16 k slices
    ((0, 1 << 20, 2560, 8, I0, 1, W0, X0, Y0), _lib.QG_EUNSUPPORTED),  # W of 2.85 GB
    ((2, 64, 5120, 8, I0, 1, W0, X0, Y0), _lib.QG_EUNSUPPORTED),    # BF16 rings of 10 slices
])
def test_rows_subset_argument_errors(lib, args, status):
    assert _lib.qgemv_rows(*args) == status, _lib.last_error()
    assert _lib.last_error()


@pytest.mark.parametrize("call, status", [
    (lambda: _lib.qg_quantize_q8_0(4, 64, 0, Y0), _lib.QG_EINVAL),              # null src
    (lambda: _lib.qg_quantize_q8_0(4, 64, X0, 0), _lib.QG_EINVAL),              # null dst
    (lambda: _lib.qg_quantize_q8_0(0, 64, X0, Y0), _lib.QG_EINVAL),             # no rows
    (lambda: _lib.qg_quantize_q8_0(4, 48, X0, Y0), _lib.QG_EINVAL),             # partial block
    (lambda: _lib.qg_quantize_q8_0(4, 64, X0 + 4, Y0), _lib.QG_EALIGN),         # src misaligned
    (lambda: _lib.qg_quantize_q4_0(4, 64, 0, X0, Y0 + 2, None), _lib.QG_EALIGN),  # dst misaligned
    (lambda: _lib.qg_quantize_q4_0(4, 64, 2, X0, Y0, None), _lib.QG_EINVAL),    # unknown method
    (lambda: _lib.qg_quantize_q4_0(4, 64, 1, X0, X0 + 256, None), _lib.QG_EINVAL),  # dst overlaps src
    (lambda: _lib.qg_quantize_q8_0(1, 1 << 25, X0, Y0), _lib.QG_EUNSUPPORTED),  # cols beyond range
])
def test_quantizer_argument_errors(lib, call, status):
    assert call() == status, _lib.last_error()
    assert _lib.last_error()


@pytest.mark.parametrize("call, status", [
    (lambda: _lib.qgemv_experts_gate_up(0, 8, 64, 256, 1, 2, I0, W0, 0, X0, Y0, Y0 + 4096), _lib.QG_EINVAL),  # null Wu
    (lambda: _lib.qgemv_experts_gate_up(0, 8, 64, 256, 1, 2, I0, W0, W0, X0, Y0, 0), _lib.QG_EINVAL),         # null yu
    (lambda: _lib.qgemv_experts_gate_up(0, 8, 64, 256, 1, 2, I0, W0, W0 + 8, X0, Y0, Y0 + 4096),
     _lib.QG_EALIGN),                                                                                          # Wu misaligned
    (lambda: _lib.qgemv_experts_gate_up(0, 8, 64, 256, 1, 2, I0, W0, W0, X0, Y0, Y0 + 4), _lib.QG_EINVAL),     # yg, yu overlap
    (lambda: _lib.qgemv_experts_gate_up(0, 8, 64, 256, 1, 2, I0, W0, 0x50000000, X0, Y0, 0x50000000),
     _lib.QG_EINVAL),                                                                                          # yu overlaps Wu
    (lambda: _lib.qgemv_experts_down(0, 8, 64, 256, 2, 2, I0, W0, X0, X0 + 2048), _lib.QG_EINVAL),           # y overlaps h
    (lambda: _lib.qgemv_experts_down(0, 8, 64, 256, 5, 2, I0, W0, X0, Y0), _lib.QG_EINVAL),                   # T 5
])
def test_expert_projection_argument_errors(lib, call, status):
    assert call() == status, _lib.last_error()
    assert _lib.last_error()


def test_read_probe_rejects_bad_arguments(lib):
    """The probe's argument checks run before any HIP call (no GPU needed)."""
    buf = ctypes.create_string_buffer(64 + 16)
    src = (ctypes.addressof(buf) + 15) & ~15
    out = src + 48  # inside src when bytes >= 52
    cases = [
        ((None, 32, 1, 0, src + 32), _lib.QG_EINVAL),
        ((src, 32, 1, 0, None), _lib.QG_EINVAL),
        ((src, 0, 1, 0, src + 32), _lib.QG_EINVAL),
        ((src, 24, 1, 0, src + 32), _lib.QG_EINVAL),
        ((src, 32, 0, 0, src + 32), _lib.QG_EINVAL),
        ((src + 4, 32, 1, 0, src + 48), _lib.QG_EALIGN),
        ((src, 32, 1, 0, src + 34), _lib.QG_EALIGN),
        ((src, 64, 1, 0, out), _lib.QG_EINVAL),
    ]
    for args, status in cases:
        assert _lib.qg_read_probe(*args) == status, (args, _lib.last_error())
        assert _lib.last_error()

