"""The measurement probes do the work they claim: hbm_read_probe's sink words are the XOR of every
word it was asked to read (contiguous and scattered blocks), and hbm_copy_probe writes the XOR fold
of each 32 bytes it reads into 16 bytes."""
import numpy as np
import pytest
import torch

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu


def _xor_all(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(a.view(np.uint32).ravel()))


@pytest.mark.parametrize("scattered", [False, True])
def test_read_probe_reads_every_block(scattered):
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    blk, nblk = 2048, 4096
    buf = torch.randint(0, 256, (blk * nblk,), dtype=torch.uint8, device="cuda", generator=g)
    ids = torch.randperm(nblk, generator=g, device="cuda")[: nblk // 3].to(torch.int32) if scattered else None
    sink = dapf8.hbm_read_probe(buf, blk, ids, workgroups=64)
    torch.cuda.synchronize()
    host = buf.cpu().numpy().reshape(nblk, blk)
    sel = host if ids is None else host[ids.cpu().numpy()]
    assert _xor_all(sink.cpu().numpy()) == _xor_all(np.ascontiguousarray(sel))


def test_copy_probe_writes_the_xor_fold():
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    n = 16 * 100003
    src = torch.randint(0, 256, (2 * n,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dapf8.hbm_copy_probe(src, dst, workgroups=37)
    torch.cuda.synchronize()
    s = src.cpu().numpy().reshape(-1, 2, 16)
    assert (dst.cpu().numpy().reshape(-1, 16) == (s[:, 0] ^ s[:, 1])).all()
