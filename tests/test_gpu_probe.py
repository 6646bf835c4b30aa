"""GPU: the HBM read probe reads every 16-byte chunk of its buffer once, whatever
the size and the workgroup limit (a single nonzero word, wherever it is, reaches
the wave that reads it; that wave's XOR equals the word and is stored)."""
import sys

import numpy as np
import pytest

from block_quantized_token_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    if not _t.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    _lib.load()
    return _t


def probe(torch, buf, nbytes, groups, magic, out):
    st = _lib.qg_read_probe(buf.data_ptr(), nbytes, groups, magic, out.data_ptr())
    _lib.check(st, "qg_read_probe")
    torch.cuda.synchronize()
    return int(out.item()) & 0xFFFFFFFF


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, 27852800])
def test_probe_reads_every_chunk(torch, nbytes):
    words = nbytes // 4
    for groups in (1, 3, 2048):
        for pos in (0, words - 1, words // 2, min(words - 1, 4097)):
            print(f"[probe] bytes={nbytes} groups={groups} word={pos}", file=sys.stderr, flush=True)
            buf = torch.zeros(words, dtype=torch.int32, device="cuda")
            w = 0x5A5A0000 | (pos & 0xFFFF) | 1
            buf[pos] = np.int32(np.uint32(w).view(np.int32))
            out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            assert probe(torch, buf, nbytes, groups, w, out) == w, (nbytes, groups, pos)
            # any other magic: nothing is stored
            out.fill_(7)
            assert probe(torch, buf, nbytes, groups, w ^ 0x100, out) == 7
