"""The allocation-free fused argmax (qgemv_argmax_noalloc) against the entry point
with a caller-owned workspace (qgemv_argmax), through the C ABI: the same rows and
values bit for bit on two calls in a row, the second with a smaller input (fewer
rows, fewer tokens), so the library's device keys are reused and re-cleared."""
import sys

import numpy as np
import pytest

from block_quantized_token_amd import _lib, inputs as I

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    _lib.load()
    return _t


def _both(torch, fmt, rows, cols, T, seed):
    rng = I.rng_for(seed)
    W = torch.from_numpy(I.weights(rng, fmt, rows, cols)).cuda()
    x = torch.from_numpy(I.activations(rng, cols, T)).cuda()
    sp = torch.cuda.current_stream().cuda_stream
    work = torch.empty(T, dtype=torch.int64, device="cuda")
    res = []
    for noalloc in (False, True):
        idx = torch.full((T,), -7, dtype=torch.int32, device="cuda")
        val = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = _lib.qgemv_argmax_noalloc(fmt, rows, cols, T, W.data_ptr(), x.data_ptr(), idx.data_ptr(),
                                           val.data_ptr(), sp)
        else:
            st = _lib.qgemv_argmax(fmt, rows, cols, T, W.data_ptr(), x.data_ptr(), work.data_ptr(), idx.data_ptr(),
                                   val.data_ptr(), sp)
        _lib.check(st, "argmax")
        torch.cuda.synchronize()
        res.append((idx.cpu().numpy(), val.cpu().numpy()))
    return res


@pytest.mark.parametrize("fmt", [I.FMT_Q8_0, I.FMT_Q4_0, I.FMT_BF16])
def test_noalloc_argmax_equals_workspace_argmax(torch, fmt):
    # a large call (four tokens, the 10240 x 2560 shape), then a smaller one
    for rows, cols, T, seed in ((10240, 2560, 4, 11), (777, 1024, 2, 12)):
        say(f"[noalloc] fmt={fmt} rows={rows} cols={cols} T={T}")
        (i0, v0), (i1, v1) = _both(torch, fmt, rows, cols, T, seed)
        assert np.array_equal(i0, i1), (fmt, rows, T, i0, i1)
        assert np.array_equal(v0.view(np.uint32), v1.view(np.uint32)), (fmt, rows, T, v0, v1)
        assert ((i1 >= 0) & (i1 < rows)).all() and np.isfinite(v1).all()


def test_noalloc_rejects_bad_arguments(torch):
    x = torch.zeros(4, 256, device="cuda")
    W = torch.zeros(8 * 8 * 34, dtype=torch.uint8, device="cuda")
    idx = torch.zeros(8, dtype=torch.int32, device="cuda")
    val = torch.zeros(8, device="cuda")
    for T in (0, 5):  # T past the keys the library holds
        assert _lib.qgemv_argmax_noalloc(0, 8, 256, T, W.data_ptr(), x.data_ptr(), idx.data_ptr(), val.data_ptr(),
                                         None) == _lib.QG_EINVAL
    assert _lib.qgemv_argmax_noalloc(0, 8, 256, 1, W.data_ptr(), x.data_ptr(), 0, val.data_ptr(), None) == _lib.QG_EINVAL
    assert _lib.qgemv_argmax_noalloc(0, 8, 256, 1, W.data_ptr(), x.data_ptr(), idx.data_ptr() + 2, val.data_ptr(),
                                     None) == _lib.QG_EALIGN
