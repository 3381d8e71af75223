"""GPU parity of the INT4 weight-only GEMV: the packer bit-exact against a packer written here from
the layout the header states, and w4a16_gemv against the oracle (fp32 output within a bound derived
from fp32 accumulation of the offset weights; bf16 output within 1e-2 * max|ref|)."""
import numpy as np
import pytest
import torch

import oracle
import synth

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu


def pack_reference(q, s):
    """The packed layout, from its definition: tile (n // 16, k // 128), column c = n % 16, group
    g, dword j, element e -> nibble e // 2 (even e) or 4 + e // 2 (odd e), value q + 8."""
    N, K = q.shape
    KB = K // 128
    u = (np.clip(q.astype(np.int32), -8, 7) + 8).astype(np.uint32)
    u = u.reshape(N // 16, 16, KB, 4, 4, 8)           # [t][c][kb][g][j][e]
    pos = np.array([0, 4, 1, 5, 2, 6, 3, 7])           # nibble of element e
    words = (u << (4 * pos).astype(np.uint32)).sum(axis=-1).astype(np.uint32)  # [t][c][kb][g][j]
    words = words.transpose(0, 2, 1, 3, 4)             # [t][kb][c][g][j]
    packed = np.ascontiguousarray(words).view(np.uint8).reshape(-1)
    ps = np.ascontiguousarray(s.T)                     # [K/128][N]
    return packed, ps


def _case(rng, M, N, K):
    xb = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    q[0, :8] = [-8, 7, 0, -1, 1, -7, 6, -2]
    s = (rng.random((N, K // 128)) * 0.02 + 0.001).astype(np.float32)
    return xb, q, s


@pytest.mark.parametrize("shape", [(1, 64, 128), (3, 64, 640), (1, 64, 512), (5, 192, 1024), (16, 64, 1536),
                                   (16, 256, 2048),
                                   # several 16-column tiles per workgroup: 2 (260 tiles), 7 (1792 tiles, one
                                   # workgroup per compute unit), 8 with a last workgroup of 4 (1796 tiles)
                                   (2, 4160, 384), (1, 28672, 256), (3, 28736, 256)])
def test_pack_and_gemv(shape):
    M, N, K = shape
    print(f"\n[case] w4 M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(M * 1000 + N + K)
    xb, q, s = _case(rng, M, N, K)
    tq, ts = torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda()
    packed, ps = dapf8.w4_pack(tq, ts)
    ref_packed, ref_ps = pack_reference(q, s)
    torch.cuda.synchronize()
    assert (packed.cpu().numpy() == ref_packed).all()
    assert (ps.cpu().numpy() == ref_ps).all()
    tx = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    y32 = dapf8.w4a16_gemv(tx, packed, ps, N, out_dtype=torch.float32)
    y16 = dapf8.w4a16_gemv(tx, packed, ps, N, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.w4a16_gemv(xb, q, s)
    x = synth.bf16_bits_to_f32(xb).astype(np.float64)
    # fp32 accumulation of (1.5 + q/16) * x per 128-k group, then the offset's correction (1.5 sum x)
    # and the factor 16: about 2^-24 sum |x| (48 + |q|) s per group, with room for the sums' order
    bound = 1e-5 * (np.abs(x) @ ((48.0 + np.abs(q.astype(np.float64))) * np.repeat(s, 128, axis=1)).T) + 1e-30
    err = np.abs(y32.cpu().numpy().astype(np.float64) - ref)
    assert (err <= bound).all(), float((err / bound).max())
    e16 = np.abs(y16.float().cpu().numpy().astype(np.float64) - ref)
    assert e16.max() <= 1e-2 * np.abs(ref).max()


def test_saturating_pack_and_zero_rows():
    rng = np.random.default_rng(9)
    N, K = 64, 512
    q = rng.integers(-20, 20, size=(N, K)).astype(np.int8)
    s = np.ones((N, K // 128), np.float32)
    packed, ps = dapf8.w4_pack(torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda())
    ref_packed, _ = pack_reference(q, s)
    torch.cuda.synchronize()
    assert (packed.cpu().numpy() == ref_packed).all()
    x = torch.zeros((0, K), dtype=torch.bfloat16, device="cuda")
    y = dapf8.w4a16_gemv(x, packed, ps, N)
    assert y.shape == (0, N)
