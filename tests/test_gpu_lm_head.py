"""The 248,320 x 5,120 Q8_0 LM head (the drafter-cost issue, "perf(speculative): cut
the MTP drafter's per-step cost...": the LM head the drafter and the verify pass
read) against the fp64 oracle on EVERY output.

The oracle runs once, at T = 4, over all rows: a token's oracle result does not
depend on T (pinned on the CPU by test_oracle's T-prefix check), so y[:T] of that
one run is the reference for every T.  Each kernel kind that can serve the head
(the default tiles, the LDS-DMA vector-ALU ring, the register-streamed kernel, the
per-workgroup and persistent matrix-core kernels, the persistent matrix-core
kernel fed by the LDS-DMA ring) is compared output by output at
T = 1..4, and the fused argmax against the tolerance-aware oracle rule at T = 1..4.
"""
import sys

import numpy as np
import pytest

from block_quantized_token_amd import _lib, inputs as I, ops

pytestmark = pytest.mark.gpu

NAME = "c4_q8_0_248320x5120"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    _lib.load()
    return _t


@pytest.fixture(scope="module")
def head(torch, orc):
    say(f"[{NAME}] generating 1.35 GB of packed weights")
    c = I.dense_case(NAME)
    say(f"[{NAME}] oracle over all {c['rows']} rows at T=4")
    ref, bound = orc.gemv(c["fmt"], c["rows"], c["cols"], c["W"], c["x"])
    W_dev = torch.from_numpy(c["W"]).cuda()
    x_dev = torch.from_numpy(c["x"]).cuda()
    return dict(c, ref=ref, bound=bound, W_dev=W_dev, x_dev=x_dev)


def run(torch, head, T):
    y = ops.gemv("q8_0", head["W_dev"], head["x_dev"][:T].contiguous(), head["rows"])
    torch.cuda.synchronize()
    return y.cpu().numpy()


def assert_all_rows(head, y, T, what):
    ref, bound = head["ref"][:T], head["bound"][:T]
    assert y.shape == ref.shape, what
    err = np.abs(y.astype(np.float64) - ref)
    tol = 1e-4 * bound + 1e-6
    bad = err > tol
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outputs out of tolerance; worst err/tol "
                           f"{(err / tol).max():.3f} at {np.unravel_index(np.argmax(err / tol), err.shape)}")
    assert np.isfinite(y).all(), what


def check_kind(torch, head, monkeypatch, tile, what):
    """Every output at T = 4, 3, 2, 1; a token's bits agree across T for one kind."""
    if tile is None:
        monkeypatch.delenv("QGEMV_TILE", raising=False)
    else:
        monkeypatch.setenv("QGEMV_TILE", "q8_0:" + tile)
    ys = {}
    for T in (4, 3, 2, 1):
        say(f"[{NAME}] {what} T={T} tile={ops.query_tile('q8_0', head['rows'], head['cols'], T)}")
        ys[T] = run(torch, head, T)
        assert_all_rows(head, ys[T], T, f"{what} T={T}")
    return ys


def test_default_tiles_every_output(torch, head, monkeypatch):
    ys = check_kind(torch, head, monkeypatch, None, "default")
    # the default kind is the same within each group: a token's bits do not depend on T there
    groups = {}
    for T in (1, 2, 3, 4):
        t = ops.query_tile("q8_0", head["rows"], head["cols"], T)
        groups.setdefault((t["kind"], t["mfma"], t["k_slice"]), []).append(T)
    for Ts in groups.values():
        for T in Ts[:-1]:
            assert np.array_equal(ys[T], ys[Ts[-1]][:T]), f"default: bits differ between T={T} and T={Ts[-1]}"


@pytest.mark.parametrize("tile,what", [
    ("4,10,64,l3", "LDS-DMA vector-ALU ring"),
    ("4,10,32,s", "register-streamed"),
    ("8,10,192,m", "matrix cores per workgroup"),
    ("8,10,64,p", "persistent matrix cores"),
    ("4,10,64,P", "persistent matrix cores on the LDS-DMA ring"),
])
def test_kind_every_output_and_t_invariant(torch, head, monkeypatch, tile, what):
    ys = check_kind(torch, head, monkeypatch, tile, what)
    for T in (1, 2, 3):
        assert np.array_equal(ys[T], ys[4][:T]), f"{what}: bits differ between T={T} and T=4"


def test_fused_argmax_every_t(torch, head, monkeypatch):
    """idx/val equal the argmax of the dense call's own output bit for bit, and the
    chosen row's exact value is within the two rows' error bounds of the oracle's
    maximum (ties within rounding cannot be decided by an fp32 kernel)."""
    monkeypatch.delenv("QGEMV_TILE", raising=False)
    ref, bound = head["ref"], head["bound"]
    tol = 1e-4 * bound + 1e-6
    for T in (1, 2, 3, 4):
        say(f"[{NAME}] fused argmax T={T}")
        xd = head["x_dev"][:T].contiguous()
        idx, val = ops.argmax("q8_0", head["W_dev"], xd, head["rows"])
        torch.cuda.synchronize()
        idx, val = idx.cpu().numpy(), val.cpu().numpy()
        y = run(torch, head, T)
        assert idx.tolist() == np.argmax(y, axis=1).tolist(), T
        assert np.array_equal(val, y[np.arange(T), idx]), T
        for t in range(T):
            oi = int(np.argmax(ref[t]))
            assert ref[t, idx[t]] >= ref[t, oi] - (tol[t, idx[t]] + tol[t, oi]), (T, t, idx[t], oi)
            assert abs(val[t] - ref[t, idx[t]]) <= tol[t, idx[t]], (T, t)


def test_rows_subset_draft_vocabulary(torch, head, monkeypatch):
    """32,768 of the head's rows (a draft vocabulary: the drafter-cost issue's
    draft-vocabulary item), T = 1..4: each selected row equals the dense call's row
    bit for bit (the matrix cores on 512-wide slices, the default's arithmetic) and
    the oracle's row within the bound."""
    rows = head["rows"]
    rng = np.random.default_rng(8)
    ids = np.sort(rng.choice(rows, 32768, replace=False))
    monkeypatch.delenv("QGEMV_TILE", raising=False)
    full = run(torch, head, 4)
    idd = torch.from_numpy(ids.astype(np.int32)).cuda()
    for T in (1, 2, 3, 4):
        say(f"[{NAME}] draft vocabulary T={T}")
        y = ops.gemv_rows("q8_0", head["W_dev"], head["x_dev"][:T].contiguous(), rows, idd)
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        assert np.array_equal(y, full[:T, ids]), T
        err = np.abs(y.astype(np.float64) - head["ref"][:T, ids])
        assert (err <= 1e-4 * head["bound"][:T, ids] + 1e-6).all(), T


def test_q4_0_head_kinds_share_bits(torch, orc, monkeypatch):
    """The head's shape in Q4_0 (715 MB): the default runs the matrix cores on 512-wide
    slices per workgroup (kind X) while one workgroup per CU holds their partial sums
    (T <= 2) and the persistent kind on the same slices from T = 3 on.  The two share
    their arithmetic, so a token's bits must not change with T; every output is checked
    against the oracle (one T = 4 run serves every T)."""
    monkeypatch.delenv("QGEMV_TILE", raising=False)
    rows, cols = 248320, 5120
    kinds = [ops.query_tile("q4_0", rows, cols, T)["kind"] for T in (1, 2, 3, 4)]
    assert kinds == [11, 11, 9, 9], kinds
    say("[q4_0 head] generating 715 MB of packed weights")
    W = I.weights_chunked(77, I.FMT_Q4_0, rows, cols)
    x = I.activations(I.rng_for(78), cols)
    say("[q4_0 head] oracle over all rows at T=4")
    ref, bound = orc.gemv(I.FMT_Q4_0, rows, cols, W, x)
    Wd, xd = torch.from_numpy(W).cuda(), torch.from_numpy(x).cuda()
    ys = {}
    for T in (4, 3, 2, 1):
        say(f"[q4_0 head] T={T} kind={kinds[T - 1]}")
        ys[T] = ops.gemv("q4_0", Wd, xd[:T].contiguous(), rows).cpu().numpy()
        err = np.abs(ys[T].astype(np.float64) - ref[:T])
        assert (err <= 1e-4 * bound[:T] + 1e-6).all(), T
    for T in (1, 2, 3):
        assert np.array_equal(ys[T], ys[4][:T]), f"a token's bits differ between T={T} and T=4"
