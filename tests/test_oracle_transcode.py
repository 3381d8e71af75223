"""Pins of the oracle's BF16 -> FP8 page transcode (prefill BF16 cache -> decode FP8 cache;
Cloudflare, "Smaller, faster, safer", section 量化 KV cache: BF16 kept for prefill, FP8 for decode).

Pinned by (1) a closed form: values 2^e with per-head scales 2^k have the e4m3 code
((e - k + 7) << 3) by the format's definition, so every (page, head, slot, dim) position is checked
against a value that does not involve the oracle's encoder, through the logical [page][h][t][d]
order of tests/layout.py; (2) the special values of the format written out from its definition
(saturation at 448, NaN, signed zero, subnormals and their ties); (3) an invariant: transcoding
pages filled by a BF16 append equals appending the same rows straight into an FP8 pool.
"""
import numpy as np

import synth
from layout import k_to_logical, k_to_phys

FP8, BF16 = 0, 1


def _phys_v(v_logical):
    # logical [n][H][P][Dv] -> physical [n][H][Dv][P]
    return np.ascontiguousarray(v_logical.transpose(0, 1, 3, 2))


def test_closed_form_powers_of_two(orc):
    rng = np.random.default_rng(3)
    ns, nd, H, P, Dk, Dv = 5, 7, 3, 4, 128, 32
    # exponent per logical position, and per-head scale exponents
    ek = rng.integers(-4, 7, size=(ns, H, P, Dk))
    ev = rng.integers(-4, 7, size=(ns, H, P, Dv))
    sk = np.array([0, 1, -2], np.int64)
    sv = np.array([2, -1, 0], np.int64)
    sign_k = rng.integers(0, 2, size=ek.shape)
    sign_v = rng.integers(0, 2, size=ev.shape)
    k_val = np.where(sign_k == 1, -1.0, 1.0) * np.exp2(ek.astype(np.float64))
    v_val = np.where(sign_v == 1, -1.0, 1.0) * np.exp2(ev.astype(np.float64))
    k_src = k_to_phys(synth.to_bf16_bits(k_val.astype(np.float32)), BF16)
    v_src = _phys_v(synth.to_bf16_bits(v_val.astype(np.float32)))
    k_dst = np.full((nd, H, Dk // 64, P, 64), 0x55, np.uint8)
    v_dst = np.full((nd, H, Dv, P), 0x55, np.uint8)
    src = np.array([4, 0, 2], np.int32)
    dst = np.array([1, 6, 3], np.int32)
    orc.kv_transcode_pages(k_src, v_src, k_dst, v_dst, src, dst, np.exp2(sk).astype(np.float32),
                           np.exp2(sv).astype(np.float32), page_size=P)
    kd = k_to_logical(k_dst)
    vd = v_dst.transpose(0, 1, 3, 2)
    for s_, d_ in zip(src, dst):
        want_k = (((ek[s_] - sk[:, None, None] + 7) << 3) | (sign_k[s_] << 7)).astype(np.uint8)
        want_v = (((ev[s_] - sv[:, None, None] + 7) << 3) | (sign_v[s_] << 7)).astype(np.uint8)
        assert (kd[d_] == want_k).all()
        assert (vd[d_] == want_v).all()
    untouched = [p for p in range(nd) if p not in set(dst.tolist())]
    assert (k_dst[untouched] == 0x55).all() and (v_dst[untouched] == 0x55).all()


def test_special_values(orc):
    # (bf16 value, scale, expected code) from the E4M3FN definition: bias 7, 3 mantissa bits,
    # largest finite 448 = 0x7E, NaN = S.1111.111, subnormals m * 2^-9, ties to even mantissa
    cases = [
        (448.0, 1.0, 0x7E), (1000.0, 1.0, 0x7E), (-1e30, 1.0, 0xFE), (float("inf"), 1.0, 0x7E),
        (float("nan"), 1.0, 0x7F), (0.0, 1.0, 0x00), (-0.0, 1.0, 0x80), (2.0 ** -9, 1.0, 0x01),
        (2.0 ** -10, 1.0, 0x00), (3 * 2.0 ** -10, 1.0, 0x02), (2.0 ** -6, 1.0, 0x08), (1.0, 1.0, 0x38),
        (-1.5, 1.0, 0xBC), (1.0625, 1.0, 0x38), (1.1875, 1.0, 0x3A), (896.0, 2.0, 0x7E), (3.0, 0.5, 0x4C),
        (464.0, 1.0, 0x7E), (480.0, 1.0, 0x7E),
    ]
    n = len(cases)
    H, P, Dk = 1, n, 64
    vals = np.zeros((1, H, P, Dk), np.float32)
    for t, (x, _, _) in enumerate(cases):
        vals[0, 0, t, :] = x
    bits = synth.to_bf16_bits(vals)
    for t, (x, _, _) in enumerate(cases):
        if np.isnan(x):
            bits[0, 0, t, :] = 0x7FC0  # positive quiet NaN
    k_src = k_to_phys(bits, BF16)
    for t, (x, s, want) in enumerate(cases):
        k_dst = np.zeros((1, H, 1, P, 64), np.uint8)
        orc.kv_transcode_pages(k_src, None, k_dst, None, np.array([0], np.int32), np.array([0], np.int32),
                               np.array([s], np.float32), page_size=P)
        got = k_to_logical(k_dst)[0, 0, t]
        assert (got == want).all(), (x, s, hex(int(got[0])), hex(want))


def test_transcode_equals_direct_fp8_append(orc):
    rng = np.random.default_rng(11)
    B, H, P, Dk, Dv, npg = 3, 2, 16, 128, 64, 12
    lens = [37, 16, 5]
    pt = np.full((B, 4), -1, np.int32)
    perm = rng.permutation(npg).astype(np.int32)
    off = 0
    for b, L in enumerate(lens):
        n = (L + P - 1) // P
        pt[b, :n] = perm[off:off + n]
        off += n
    T = sum(lens)
    seq = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    k = synth.to_bf16_bits((rng.standard_normal((T, H, Dk)) * 3).astype(np.float32))
    v = synth.to_bf16_bits((rng.standard_normal((T, H, Dv)) * 0.5).astype(np.float32))
    ks = np.array([0.01, 0.02], np.float32)
    vs = np.array([0.003, 0.004], np.float32)
    kb = np.zeros((npg, H, Dk // 32, P, 32), np.uint16)
    vb = np.zeros((npg, H, Dv, P), np.uint16)
    orc.kv_append(k, v, kb, vb, BF16, pt, seq, pos, None, None, page_size=P, num_pages=npg)
    kf = np.zeros((npg, H, Dk // 64, P, 64), np.uint8)
    vf = np.zeros((npg, H, Dv, P), np.uint8)
    orc.kv_append(k, v, kf, vf, FP8, pt, seq, pos, ks, vs, page_size=P, num_pages=npg)
    kt = np.zeros_like(kf)
    vt = np.zeros_like(vf)
    used = perm[:off]
    orc.kv_transcode_pages(kb, vb, kt, vt, used, used, ks, vs, page_size=P)
    # empty slots hold zero in both (zero bf16 -> code 0)
    assert (kt == kf).all() and (vt == vf).all()


def test_out_of_range_pairs_are_skipped(orc):
    H, P, Dk = 1, 2, 64
    k_src = np.full((2, H, Dk // 32, P, 32), 0x3F80, np.uint16)  # 1.0
    k_dst = np.full((3, H, 1, P, 64), 0x11, np.uint8)
    src = np.array([0, -1, 2, 1], np.int32)
    dst = np.array([5, 0, 1, 2], np.int32)
    orc.kv_transcode_pages(k_src, None, k_dst, None, src, dst, np.array([1.0], np.float32), page_size=P)
    assert (k_dst[0] == 0x11).all() and (k_dst[1] == 0x11).all()
    assert (k_dst[2] == 0x38).all()
