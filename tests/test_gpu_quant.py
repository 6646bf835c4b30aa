"""GPU parity of the on-device quantizers (fp32 -> packed Q8_0 / Q4_0 blocks)
against the CPU oracle: the packed bytes must be identical, since every code is
an integer decided in fp32 by both sides."""
import sys

import numpy as np
import pytest

from block_quantized_token_amd import _lib, inputs as I, ops
from tests import golden_io

pytestmark = pytest.mark.gpu

Q8, Q4 = I.FMT_Q8_0, I.FMT_Q4_0
CASES = [(Q8, "absmax", 0), (Q4, "absmax", 0), (Q4, "lloyd", 1)]


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    _lib.load()
    return _t


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu_quantize(torch, fmt, v, method):
    src = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda()
    out = ops.quantize("q8_0" if fmt == Q8 else "q4_0", src, method)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(torch, orc, fmt, method, m, v, what):
    rows, cols = v.shape
    say(f"[quantize] fmt={fmt} method={method} {rows}x{cols} {what}")
    got = gpu_quantize(torch, fmt, v, method)
    ref = orc.quantize(fmt, rows, cols, v, m)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at block {bad[0] // (34 if fmt == Q8 else 18)}"


@pytest.mark.parametrize("fmt, method, m", CASES)
def test_quantize_shapes(torch, orc, fmt, method, m):
    """Ragged workgroup tails (1, 3, 514 blocks ...), several tiles, the bench shape."""
    rng = np.random.default_rng(50 + fmt + m)
    for rows, cols in ((1, 32), (3, 96), (257, 64), (100, 2560), (333, 6144), (10240, 2560)):
        check(torch, orc, fmt, method, m, I.dense_fp32(rng, rows, cols), f"{rows}x{cols}")


@pytest.mark.parametrize("fmt, method, m", CASES)
def test_quantize_distributions_and_ties(torch, orc, fmt, method, m):
    """Heavy tails, uniform values, huge and tiny magnitudes (fp16 scale overflow and
    underflow, subnormal scales), the hand-quantized blocks, and blocks of exact ties."""
    rng = np.random.default_rng(60 + fmt + m)
    parts = [rng.standard_t(2, (256, 32)), rng.uniform(-1, 1, (256, 32)),
             rng.standard_normal((64, 32)) * 1e4, rng.standard_normal((64, 32)) * 1e-5,
             rng.standard_normal((64, 32)) * 1e-3, np.zeros((3, 32))]
    for name in golden_io.quant_vectors():
        parts.append(golden_io.load_quant(name)["v"][None, :].astype(np.float64))
    # exact ties: d a power of two, values on half levels
    k = rng.integers(-3, 4, (128, 32))
    half = (k + 0.5) * 2.0 ** -5
    half[:, 0] = 127 * 2.0 ** -5 if fmt == Q8 else 8 * 2.0 ** -5
    parts.append(half)
    v = np.concatenate(parts).astype(np.float32)
    check(torch, orc, fmt, method, m, v, "distributions")


def test_quantize_feeds_the_gemv(torch, orc):
    """Quantized on the device, multiplied on the device: the result is the oracle's
    mat-vec of the oracle's bytes (the bytes are identical, so the usual bound holds)."""
    rng = np.random.default_rng(70)
    rows, cols = 1000, 2560
    v = I.dense_fp32(rng, rows, cols)
    x = I.activations(rng, cols)
    for fmt, method, m in CASES:
        src = torch.from_numpy(v).cuda()
        Wd = ops.quantize("q8_0" if fmt == Q8 else "q4_0", src, method)
        y = ops.gemv("q8_0" if fmt == Q8 else "q4_0", Wd, torch.from_numpy(x).cuda(), rows).cpu().numpy()
        ref, bound = orc.gemv(fmt, rows, cols, orc.quantize(fmt, rows, cols, v, m), x)
        assert np.all(np.abs(y - ref) <= 1e-4 * bound + 1e-6), (fmt, method)
        # and the quantization error itself is small for these weights
        rel = np.linalg.norm(y - x.astype(np.float64) @ v.T.astype(np.float64)) / np.linalg.norm(ref)
        assert rel < (0.02 if fmt == Q8 else 0.2), (fmt, method, rel)
