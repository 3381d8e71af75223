"""Pins of the oracle's tag check, quantize-on-append and scale setup.

Tag check (Cloudflare, "Smaller, faster, safer", section 保护共享 KV cache; siami.tw digest,
section on the shared KV-cache integrity check): every physical page carries a tag that changes
on reallocation, each request records the (page, tag) pairs it expects, a mismatch aborts the
request.  Pinned here by brute force over explicit Python loops, and by injected stale tags whose
affected requests are known by construction.

Append and scales are pinned through torch's float8_e4m3fn / bfloat16 casts and numpy views of the
pool layout (K in 64-byte dimension chunks, read back in [page][Hkv][P][Dk] order through
layout.k_to_logical; V [page][Hkv][Dv][P]).
"""
import numpy as np
import pytest
import torch

import synth
from layout import k_shape, k_to_logical

FP8, BF16 = 0, 1


def brute_verify(pt, exp, lens, live, P):
    out = []
    for b in range(pt.shape[0]):
        L = int(lens[b])
        if L < 0 or L > pt.shape[1] * P:
            out.append(1)
            continue
        bad = 0
        for j in range((L + P - 1) // P):
            p = int(pt[b, j])
            if p < 0 or p >= len(live) or int(live[p]) != int(exp[b, j]):
                bad = 1
        out.append(bad)
    return np.array(out, np.uint8)


def test_verify_brute_force_random(orc):
    rng = np.random.default_rng(0)
    for trial in range(200):
        B, P, npg = int(rng.integers(1, 9)), int(rng.choice([1, 4, 16])), int(rng.integers(1, 40))
        stride = int(rng.integers(1, 8))
        pt = rng.integers(-2, npg + 2, size=(B, stride)).astype(np.int32)
        live = rng.integers(0, 4, size=npg).astype(np.uint32)
        exp = np.where(pt >= 0, live[np.clip(pt, 0, npg - 1)], 0).astype(np.uint32)
        flip = rng.random((B, stride)) < 0.1
        exp[flip] ^= 1
        lens = rng.integers(-1, stride * P + 3, size=B).astype(np.int32)
        got = orc.kv_tag_verify(pt, exp, lens, live, page_size=P)
        assert (got == brute_verify(pt, exp, lens, live, P)).all(), trial


def test_verify_edge_cases(orc):
    P = 4
    live = np.array([10, 11, 0xFFFFFFFF, 0], np.uint32)
    pt = np.array([[0, 1, -1], [2, 3, 1], [3, 0, 0], [5, 0, 0], [0, 1, 2]], np.int32)
    exp = np.array([[10, 11, 99], [0xFFFFFFFF, 0, 11], [0, 10, 7], [0, 10, 10], [10, 11, 0xFFFFFFFF]], np.uint32)
    lens = np.array([8, 12, 5, 1, 13], np.int32)
    got = orc.kv_tag_verify(pt, exp, lens, live, page_size=P)
    # 0: entries past ceil(8/4)=2 are ignored (stale tag 99 in slot 2) -> ok
    # 1: wrapped generation 0xFFFFFFFF and 0 compare by equality -> ok
    # 2: ceil(5/4)=2 entries checked: both match; the stale third entry is ignored -> ok
    # 3: page id 5 is out of range -> abort
    # 4: needs 4 pages with a stride of 3 -> abort
    assert list(got) == [0, 0, 0, 1, 1]
    assert list(orc.kv_tag_verify(pt, exp, np.zeros(5, np.int32), live, page_size=P)) == [0] * 5


def test_verify_tiny_workload_one_stale_request(orc):
    w = synth.make("tiny_mha", seed=1)
    got = orc.kv_tag_verify(w.page_table, w.expected_tags, w.seq_lens, w.live_tags, page_size=16)
    assert got.sum() == 1 and (got == w.expected_abort).all()
    clean = w.expected_tags.copy()
    for b, j in w.stale_refs:
        clean[b, j] = w.live_tags[w.page_table[b, j]]
    assert orc.kv_tag_verify(w.page_table, clean, w.seq_lens, w.live_tags, page_size=16).sum() == 0


def test_verify_capacity_churn_injections(orc):
    # capacity workload at reduced batch, higher stale rate so several requests are hit
    w = synth.make("capacity", seed=2, B=16, stale_rate=2e-3)
    assert w.alloc_generations.max() >= 2                   # pages really were reused
    got = orc.kv_tag_verify(w.page_table, w.expected_tags, w.seq_lens, w.live_tags, page_size=16)
    assert (got == w.expected_abort).all() and got.sum() >= 1


def _pool_views(kp, vp, npg, H, P, Dk, Dv, kv_dt):
    return (k_to_logical(kp.reshape(k_shape(npg, H, P, Dk, kv_dt))),
            None if vp is None else vp.reshape(npg, H, Dv, P))


@pytest.mark.parametrize("in_dt", ["f32", "bf16"])
def test_append_fp8_codes_layout_and_untouched_bytes(orc, in_dt):
    rng = np.random.default_rng(1)
    npg, H, P, Dk, Dv, B = 12, 3, 4, 128, 16, 3
    pt = rng.permutation(npg)[: B * 3].reshape(B, 3).astype(np.int32)
    T = 7
    seq_ids = rng.integers(0, B, T).astype(np.int32)
    positions = rng.integers(0, 3 * P, T).astype(np.int32)
    # distinct (seq, pos) so no slot is written twice
    seen = set()
    keep = [i for i in range(T) if (seq_ids[i], positions[i]) not in seen and not seen.add((seq_ids[i], positions[i]))]
    seq_ids, positions = seq_ids[keep], positions[keep]
    T = len(keep)
    k = (rng.standard_normal((T, H, Dk)) * 3).astype(np.float32)
    v = (rng.standard_normal((T, H, Dv)) * 3).astype(np.float32)
    k[0, 0, 0] = 1e6                                           # saturates
    if in_dt == "bf16":
        k, v = synth.to_bf16_bits(k), synth.to_bf16_bits(v)
    ks = np.array([0.01, 0.02, 0.005], np.float32)
    vs = np.array([0.03, 0.004, 0.01], np.float32)
    kp = np.full(npg * H * P * Dk, 0x5A, np.uint8)
    vp = np.full(npg * H * Dv * P, 0x5A, np.uint8)
    orc.kv_append(k, v, kp, vp, FP8, pt, seq_ids, positions, ks, vs, page_size=P, num_pages=npg)
    K, V = _pool_views(kp, vp, npg, H, P, Dk, Dv, FP8)
    kf = synth.bf16_bits_to_f32(k) if in_dt == "bf16" else k
    vf = synth.bf16_bits_to_f32(v) if in_dt == "bf16" else v
    touched_k = np.zeros(K.shape, bool)
    touched_v = np.zeros(V.shape, bool)
    for i in range(T):
        page, slot = pt[seq_ids[i], positions[i] // P], positions[i] % P
        for h in range(H):
            t = (kf[i, h].astype(np.float64) / ks[h]).astype(np.float32)
            ref = torch.from_numpy(np.clip(t, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert (K[page, h, slot] == ref).all()
            t = (vf[i, h].astype(np.float64) / vs[h]).astype(np.float32)
            ref = torch.from_numpy(np.clip(t, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert (V[page, h, :, slot] == ref).all()
            touched_k[page, h, slot] = True
            touched_v[page, h, :, slot] = True
    assert (K[~touched_k] == 0x5A).all() and (V[~touched_v] == 0x5A).all()
    assert K[pt[seq_ids[0], positions[0] // P], 0, positions[0] % P, 0] == 0x7E


def test_append_bf16_abort_and_bounds(orc):
    rng = np.random.default_rng(2)
    npg, H, P, D, B = 6, 2, 4, 64, 3
    pt = np.array([[0, 1], [2, 3], [4, -1]], np.int32)
    k = rng.standard_normal((5, H, D)).astype(np.float32)
    v = rng.standard_normal((5, H, D)).astype(np.float32)
    seq_ids = np.array([0, 1, 2, 2, 0], np.int32)
    positions = np.array([5, 0, 6, 1, 8], np.int32)      # (2,6) hits page id -1; (0,8) is past the table
    # two more tokens whose sequence ids lie outside the batch: no slot, nothing written
    k = np.concatenate([k, rng.standard_normal((2, H, D)).astype(np.float32)])
    v = np.concatenate([v, rng.standard_normal((2, H, D)).astype(np.float32)])
    seq_ids = np.concatenate([seq_ids, np.array([B, -1], np.int32)])
    positions = np.concatenate([positions, np.array([1, 2], np.int32)])
    kp = np.zeros(npg * H * P * D, np.uint16)
    vp = np.zeros(npg * H * D * P, np.uint16)
    abort = np.array([0, 1, 0], np.uint8)                 # request 1 aborted: not written
    orc.kv_append(k, v, kp, vp, BF16, pt, seq_ids, positions, None, None, abort, page_size=P, num_pages=npg)
    K, V = _pool_views(kp, vp, npg, H, P, D, D, BF16)
    ref = lambda x: torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (K[1, :, 1] == ref(k[0])).all() and (V[1, :, :, 1] == ref(v[0])).all()
    assert (K[4, :, 1] == ref(k[3])).all()
    written = np.zeros(K.shape, bool)
    written[1, :, 1] = True
    written[4, :, 1] = True
    assert (K[~written] == 0).all()


def test_scales_amax_over_448(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((50, 4, 16)) * np.array([1, 10, 0.1, 0])[None, :, None]).astype(np.float32)
    s = orc.kv_scales(x)
    assert s[3] == 1.0                                      # all-zero head -> scale 1
    for h in range(3):
        amax = np.abs(x[:, h]).max()
        assert s[h] == np.float32(np.float64(amax) / 448.0)  # fp32 of the exact quotient
        codes = orc.quantize_fp8(x[:, h].ravel(), s[h])
        assert (codes & 0x7F).max() == 0x7E                 # the largest |x| lands on 448
    # chunked accumulation gives the same scales
    amax = np.zeros(4, np.float32)
    for c in range(0, 50, 7):
        orc.kv_absmax_update(x[c:c + 7], amax)
    assert (orc.scale_from_absmax(amax) == s).all()
