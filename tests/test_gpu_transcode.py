"""GPU parity of kv_transcode_pages (BF16 pool pages -> FP8 pool pages) against the oracle: the
whole destination pools bit-exact, including untouched pages, skipped out-of-range pairs and the
format's special values (saturation, NaN, signed zero, subnormals)."""
import numpy as np
import pytest
import torch

import oracle
import synth

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu

SHAPES = [
    # (Hkv, P, Dk, Dv, shared)
    (8, 16, 128, 128, False),
    (1, 64, 576, 512, True),
    (2, 3, 64, 16, False),
    (3, 17, 192, 48, False),
    # more page shapes: power-of-two block sizes (the shift split of a unit) and not (the division)
    (2, 16, 64, 16, False),
    (3, 32, 192, 48, False),
    (2, 48, 128, 80, False),
]


def _source(rng, n, H, P, D, chunked):
    x = (rng.standard_normal((n, H, P, D)) * 4).astype(np.float32)
    special = rng.random(x.shape) < 0.02
    pick = rng.integers(0, 8, size=x.shape)
    table = np.array([np.inf, -np.inf, np.nan, 1e6, -0.0, 3e-4, -2e-3, 0.0], np.float32)
    x = np.where(special, table[pick], x)
    bits = synth.to_bf16_bits(x)
    if chunked:  # [n][H][P][D] -> [n][H][D/32][P][32]
        return np.ascontiguousarray(bits.reshape(n, H, P, D // 32, 32).transpose(0, 1, 3, 2, 4))
    return np.ascontiguousarray(bits.transpose(0, 1, 3, 2))  # V: [n][H][D][P]


@pytest.mark.parametrize("shape", SHAPES)
def test_transcode_bit_exact(shape):
    H, P, Dk, Dv, shared = shape
    print(f"\n[case] transcode H={H} P={P} Dk={Dk} Dv={Dv} shared={shared}", flush=True)
    rng = np.random.default_rng(hash(shape) % (2 ** 32))
    ns, nd = 40, 50
    k_src = _source(rng, ns, H, P, Dk, True)
    v_src = None if shared else _source(rng, ns, H, P, Dv, False)
    k_dst = rng.integers(0, 256, size=(nd, H, Dk // 64, P, 64), dtype=np.uint8)
    v_dst = None if shared else rng.integers(0, 256, size=(nd, H, Dv, P), dtype=np.uint8)
    n = 30
    src = rng.integers(0, ns, size=n).astype(np.int32)
    dst = rng.permutation(nd)[:n].astype(np.int32)
    src[3], dst[7], src[11], dst[12] = -1, nd, ns + 5, -3  # skipped pairs
    ks = (rng.random(H) * 0.05 + 0.005).astype(np.float32)
    vs = (rng.random(H) * 0.05 + 0.005).astype(np.float32)

    dev = "cuda"
    t_k_src = torch.from_numpy(k_src.view(np.int16)).to(dev).view(torch.bfloat16)
    t_v_src = None if shared else torch.from_numpy(v_src.view(np.int16)).to(dev).view(torch.bfloat16)
    t_k_dst = torch.from_numpy(k_dst.copy()).to(dev)
    t_v_dst = None if shared else torch.from_numpy(v_dst.copy()).to(dev)
    dapf8.kv_transcode_pages(t_k_src, t_v_src, t_k_dst, t_v_dst, torch.from_numpy(src).to(dev),
                             torch.from_numpy(dst).to(dev), torch.from_numpy(ks).to(dev),
                             None if shared else torch.from_numpy(vs).to(dev))
    torch.cuda.synchronize()

    oracle.kv_transcode_pages(k_src, v_src, k_dst, v_dst, src, dst, ks, None if shared else vs, page_size=P)
    assert (t_k_dst.cpu().numpy() == k_dst).all()
    if not shared:
        assert (t_v_dst.cpu().numpy() == v_dst).all()


def test_transcode_zero_pages_is_noop():
    k = torch.zeros((2, 1, 2, 4, 32), dtype=torch.bfloat16, device="cuda")
    kd = torch.full((2, 1, 1, 4, 64), 7, dtype=torch.uint8, device="cuda")
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    dapf8.kv_transcode_pages(k, None, kd, None, e, e, torch.ones(1, device="cuda"))
    torch.cuda.synchronize()
    assert (kd == 7).all()


def test_transcode_every_bf16_value():
    # every bf16 bit pattern (NaNs, infinities, subnormals, both zeros) under several scales, one
    # scale per head: 65536 values per (page, head) block, K-only pool
    H, P, Dk = 5, 64, 1024
    print(f"\n[case] transcode exhaustive bf16 H={H} P={P} Dk={Dk}", flush=True)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    logical = np.broadcast_to(bits.reshape(1, 1, P, Dk), (1, H, P, Dk))
    k_src = np.ascontiguousarray(logical.reshape(1, H, P, Dk // 32, 32).transpose(0, 1, 3, 2, 4))
    ks = np.array([1.0, 0.5, np.float32(1.0) / np.float32(3.0), 0.0137, np.float32(7.3) / np.float32(448.0)],
                  np.float32)
    k_dst = np.zeros((1, H, Dk // 64, P, 64), np.uint8)
    t_k_src = torch.from_numpy(k_src.view(np.int16)).cuda().view(torch.bfloat16)
    t_k_dst = torch.zeros(k_dst.shape, dtype=torch.uint8, device="cuda")
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    dapf8.kv_transcode_pages(t_k_src, None, t_k_dst, None, z, z, torch.from_numpy(ks).cuda())
    torch.cuda.synchronize()
    oracle.kv_transcode_pages(k_src, None, k_dst, None, np.zeros(1, np.int32), np.zeros(1, np.int32), ks,
                              page_size=P)
    got = t_k_dst.cpu().numpy()
    bad = np.argwhere(got != k_dst)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"


def test_transcode_scales_across_fp32_range():
    # ~10^7 values, one scale per head, from subnormal scales (whose reciprocal overflows) through
    # the edges of the reciprocal's normal range to scales near the fp32 maximum; the values are
    # drawn so that the quotients cover e4m3's subnormals, normals and saturation, with bf16 rounding
    H, P, Dk, n = 24, 64, 1024, 7
    print(f"\n[case] transcode scale sweep H={H} P={P} Dk={Dk} pages={n}", flush=True)
    rng = np.random.default_rng(11)
    fixed = np.array([2.0 ** -149, 2.0 ** -130, 2.0 ** -126, np.nextafter(np.float32(2.0 ** -126), np.float32(0)),
                      2.0 ** -100, 1e-3, 0.0137, 1.0, 2.0 ** 100, np.nextafter(np.float32(2.0 ** 126), np.float32(0)),
                      2.0 ** 126, 2.0 ** 127, 3.0e38], np.float32)
    ks = np.concatenate([fixed, np.exp(rng.uniform(-80, 80, H - fixed.size))]).astype(np.float32)
    mag = np.exp(rng.uniform(-12, 7, size=(n, H, P, Dk)))  # |x / s| from ~6e-6 to ~1100
    x = (rng.choice([-1.0, 1.0], size=mag.shape) * mag * ks.reshape(1, H, 1, 1).astype(np.float64))
    with np.errstate(over="ignore"):  # the largest scales overflow some values to infinity, as intended
        bits = synth.to_bf16_bits(x.astype(np.float32))
    k_src = np.ascontiguousarray(bits.reshape(n, H, P, Dk // 32, 32).transpose(0, 1, 3, 2, 4))
    k_dst = np.zeros((n, H, Dk // 64, P, 64), np.uint8)
    pages = np.arange(n, dtype=np.int32)
    t_k_src = torch.from_numpy(k_src.view(np.int16)).cuda().view(torch.bfloat16)
    t_k_dst = torch.zeros(k_dst.shape, dtype=torch.uint8, device="cuda")
    tp = torch.from_numpy(pages).cuda()
    dapf8.kv_transcode_pages(t_k_src, None, t_k_dst, None, tp, tp, torch.from_numpy(ks).cuda())
    torch.cuda.synchronize()
    oracle.kv_transcode_pages(k_src, None, k_dst, None, pages, pages, ks, page_size=P)
    got = t_k_dst.cpu().numpy()
    bad = np.argwhere(got != k_dst)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:4].tolist()}"
    # the draw reaches every class of code: zeros, subnormals, normals, saturated
    mags = k_dst & 0x7F
    assert (mags == 0).any() and ((mags > 0) & (mags < 8)).any() and (mags == 0x7E).any()
