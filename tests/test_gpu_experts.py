"""GPU parity of the routed-experts layer's projections: gate/up (two tables in
one launch) and down (one input per (token, expert) pair), against the oracle,
at the audit's expert overlap (share 0.65) and with no overlap."""
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


def within(y, ref, bound, what):
    bad = ~(np.abs(y - ref) <= 1e-4 * bound + 1e-6)
    assert not bad.any(), f"{what}: {bad.sum()} outputs outside the bound, first at {np.argwhere(bad)[0]}"


@pytest.mark.parametrize("T", [1, 2, 3, 4])
@pytest.mark.parametrize("share", ["0.65", "0"])
def test_expert_layer(torch, orc, T, share):
    unique = I.UNIQUE_AT_SHARE_065[T] if share == "0.65" else 10 * T
    c = I.expert_layer_case(T, unique, seed=T)
    fmt, E, ff, emb, ids = c["fmt"], c["n_experts"], c["n_ff"], c["n_embd"], c["ids"]
    say(f"[experts] T={T} share={share} unique={len(np.unique(ids))}")
    idd = dev(torch, ids)
    Wg, Wu, Wd = dev(torch, c["Wg"]), dev(torch, c["Wu"]), dev(torch, c["Wd"])
    xd = dev(torch, c["x"])
    yg, yu = ops.experts_gate_up(NAMES[fmt], Wg, Wu, xd, idd, E, ff)
    (rg, bg), (ru, bu) = orc.gate_up(fmt, E, ff, emb, ids, c["Wg"], c["Wu"], c["x"])
    within(yg.cpu().numpy(), rg, bg, "gate")
    within(yu.cpu().numpy(), ru, bu, "up")
    # the same bits as the one-table grouped call on each table
    assert np.array_equal(yg.cpu().numpy(), ops.grouped_experts(NAMES[fmt], Wg, xd, idd, E, ff).cpu().numpy())
    assert np.array_equal(yu.cpu().numpy(), ops.grouped_experts(NAMES[fmt], Wu, xd, idd, E, ff).cpu().numpy())
    y = ops.experts_down(NAMES[fmt], Wd, dev(torch, c["h"]), idd, E, emb).cpu().numpy()
    rd, bd = orc.down(fmt, E, emb, ff, ids, c["Wd"], c["h"])
    within(y, rd, bd, "down")


@pytest.mark.parametrize("fmt", [Q8, Q4, BF])
def test_down_equals_grouped_with_token_inputs(torch, fmt):
    """With h[t][j] = x[t] for every j the down call is the grouped call, bit for bit."""
    rng = np.random.default_rng(80 + fmt)
    E, rows, cols, T, topk = 12, 300, 512, 4, 3
    W = I.weights(rng, fmt, E * rows, cols)
    x = I.activations(rng, cols, T)
    ids = I.expert_ids_shared(rng, E, T, topk, 6)
    Wd, idd = dev(torch, W), dev(torch, ids)
    y = ops.experts_down(NAMES[fmt], Wd, dev(torch, np.repeat(x[:, None, :], topk, axis=1)), idd, E, rows)
    ref = ops.grouped_experts(NAMES[fmt], Wd, dev(torch, x), idd, E, rows)
    assert np.array_equal(y.cpu().numpy(), ref.cpu().numpy())


@pytest.mark.parametrize("fmt", [Q8, Q4, BF])
def test_experts_ragged_and_repeats(torch, orc, fmt):
    """Short and unaligned rows (the direct kernel), ragged row tiles, several
    k slices, an expert named twice by one token (down: two groups), bad ids."""
    rng = np.random.default_rng(90 + fmt)
    for rows, cols in ((37, 96), (70, 1024), (130, 3000 if fmt == BF else 2976)):
        E, T, topk = 5, 3, 2
        Wg = I.weights(rng, fmt, E * rows, cols)
        Wu = I.weights(rng, fmt, E * rows, cols)
        x = I.activations(rng, cols, T)
        ids = np.array([[4, 1], [1, 1], [0, 4]], dtype=np.int32)[:T]
        say(f"[experts] fmt={NAMES[fmt]} {rows}x{cols}")
        idd = dev(torch, ids)
        yg, yu = ops.experts_gate_up(NAMES[fmt], dev(torch, Wg), dev(torch, Wu), dev(torch, x), idd, E, rows)
        (rg, bg), (ru, bu) = orc.gate_up(fmt, E, rows, cols, ids, Wg, Wu, x)
        within(yg.cpu().numpy(), rg, bg, f"gate {rows}x{cols}")
        within(yu.cpu().numpy(), ru, bu, f"up {rows}x{cols}")
        h = rng.standard_normal((T, topk, cols)).astype(np.float32)
        y = ops.experts_down(NAMES[fmt], dev(torch, Wg), dev(torch, h), idd, E, rows).cpu().numpy()
        rd, bd = orc.down(fmt, E, rows, cols, ids, Wg, h)
        within(y, rd, bd, f"down {rows}x{cols}")
    # bad ids: those slots' rows are NaN in every output, the others are right
    bad = np.array([[1, 9], [-1, 2]], dtype=np.int32)
    rows, cols, E = 50, 512, 4
    Wg = I.weights(rng, fmt, E * rows, cols)
    x = I.activations(rng, cols, 2)
    yg, yu = ops.experts_gate_up(NAMES[fmt], dev(torch, Wg), dev(torch, Wg), dev(torch, x), dev(torch, bad), E, rows)
    h = rng.standard_normal((2, 2, cols)).astype(np.float32)
    yd = ops.experts_down(NAMES[fmt], dev(torch, Wg), dev(torch, h), dev(torch, bad), E, rows)
    for y in (yg.cpu().numpy(), yu.cpu().numpy(), yd.cpu().numpy()):
        assert np.isnan(y[0, 1]).all() and np.isnan(y[1, 0]).all()
        assert np.isfinite(y[0, 0]).all() and np.isfinite(y[1, 1]).all()
