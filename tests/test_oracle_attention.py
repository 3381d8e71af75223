"""Pins of the oracle's decode attention against closed forms, invariants and an independent
dense implementation -- none of which re-types the oracle's own loops.

The attention the pages run is ordinary softmax attention of one new query per sequence over
the sequence's cached K/V (Cloudflare, "Smaller, faster, safer", section 量化 KV cache: the FP8
kernel converts the stored values on read); the oracle evaluates it in fp64 over the exactly
dequantised values.  The tests reason in the logical order K [page][Hkv][P][Dk] and hand the
oracle the boundary's physical K order (64-byte dimension chunks, see layout.py); V is
[page][Hkv][Dv][P].
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

from layout import k_to_phys

FP8, BF16 = 0, 1


def dec_table():
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def finite_codes(rng, shape):
    """Random finite e4m3 codes (never 0x7F / 0xFF)."""
    c = rng.integers(0, 254, size=shape).astype(np.uint8)
    c[c >= 0x7F] += 1          # skip 0x7F; 0xFE stays below 0xFF
    return c


class Problem:
    """A small paged problem built by hand: contiguous logical tokens scattered over pages."""

    def __init__(self, rng, B, Hq, Hkv, Dk, Dv, P, lens, kv_dt=FP8, shared=False, num_pages=None):
        self.B, self.Hq, self.Hkv, self.Dk, self.Dv, self.P = B, Hq, Hkv, Dk, Dv, P
        self.lens = np.array(lens, np.int32)
        need = [-(-int(L) // P) for L in lens]
        self.num_pages = num_pages or sum(need) + 3
        self.pt = np.full((B, max(need + [1])), -1, np.int32)
        perm = rng.permutation(self.num_pages).astype(np.int32)
        off = 0
        for b, n in enumerate(need):
            self.pt[b, :n] = perm[off:off + n]
            off += n
        self.kv_dt = kv_dt
        self.shared = shared
        if kv_dt == FP8:
            self.k = finite_codes(rng, (self.num_pages, Hkv, P, Dk))
            self.v = None if shared else finite_codes(rng, (self.num_pages, Hkv, Dv, P))
        else:
            f = rng.standard_normal((self.num_pages, Hkv, P, Dk)).astype(np.float32)
            self.k = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
            if shared:
                self.v = None
            else:
                f = rng.standard_normal((self.num_pages, Hkv, Dv, P)).astype(np.float32)
                self.v = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
        self.ks = (rng.uniform(0.5, 2.0, Hkv) / 448).astype(np.float32)
        self.vs = (rng.uniform(0.5, 2.0, Hkv) / 448).astype(np.float32)
        self.q = rng.standard_normal((B, Hq, Dk)).astype(np.float32)
        self.sm = 1.0 / math.sqrt(Dk)

    def kvals(self):
        if self.kv_dt == FP8:
            return dec_table()[self.k] * self.ks[None, :, None, None].astype(np.float64)
        return (self.k.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def vvals(self):
        """V values as [page][Hkv][P][Dv] (token-major) for the dense reference."""
        if self.shared:
            return self.kvals()[..., :self.Dv]
        if self.kv_dt == FP8:
            v = dec_table()[self.v] * self.vs[None, :, None, None].astype(np.float64)
        else:
            v = (self.v.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return np.swapaxes(v, 2, 3)

    def run(self, orc, **kw):
        args = dict(sm_scale=self.sm, Hkv=self.Hkv, Dk=self.Dk, Dv=self.Dv, page_size=self.P)
        args.update(kw)
        return orc.paged_decode_attn(self.q, k_to_phys(self.k, self.kv_dt), self.v, self.kv_dt, self.pt, self.lens,
                                     self.ks, self.vs, **args)

    def dense(self, b, g):
        """Gather sequence b's K/V rows of KV head g into dense [L][D] arrays (plain loops)."""
        kv, vv = self.kvals(), self.vvals()
        K = np.array([kv[self.pt[b, t // self.P], g, t % self.P] for t in range(self.lens[b])])
        V = np.array([vv[self.pt[b, t // self.P], g, t % self.P] for t in range(self.lens[b])])
        return K, V


@pytest.mark.parametrize("kv_dt", [FP8, BF16])
def test_matches_independent_dense_softmax(orc, kv_dt):
    rng = np.random.default_rng(1)
    p = Problem(rng, B=3, Hq=8, Hkv=2, Dk=64, Dv=16, P=4, lens=[1, 7, 23], kv_dt=kv_dt)
    out = p.run(orc)
    G = p.Hq // p.Hkv
    for b in range(p.B):
        for h in range(p.Hq):
            K, V = p.dense(b, h // G)
            w = softmax(p.sm * (K @ p.q[b, h].astype(np.float64)))
            np.testing.assert_allclose(out[b, h], w @ V, rtol=1e-12, atol=1e-13)


def test_zero_query_gives_mean_of_v(orc):
    rng = np.random.default_rng(2)
    p = Problem(rng, B=2, Hq=4, Hkv=4, Dk=64, Dv=16, P=8, lens=[37, 64])
    p.q[:] = 0
    out = p.run(orc)
    for b in range(p.B):
        for h in range(p.Hq):
            _, V = p.dense(b, h)
            np.testing.assert_allclose(out[b, h], V.mean(0), rtol=1e-13, atol=1e-15)


def test_one_hot_score_selects_one_row(orc):
    rng = np.random.default_rng(3)
    D, L = 64, 13
    p = Problem(rng, B=1, Hq=1, Hkv=1, Dk=D, Dv=D, P=4, lens=[L])
    # K_t = e_t (code 0x38 = 1.0 on dim t), so the scores are alpha*sm*s_K on token j and 0 elsewhere
    p.k[:] = 0
    for t in range(L):
        p.k[p.pt[0, t // p.P], 0, t % p.P, t] = 0x38
    j = 9
    p.q[:] = 0
    p.q[0, 0, j] = 1e7          # alpha*sm*s_K > 700, so exp(-score gap) underflows to 0
    out = p.run(orc)
    _, V = p.dense(0, 0)
    assert (out[0, 0] == V[j]).all()


def test_single_token_returns_its_value(orc):
    rng = np.random.default_rng(4)
    p = Problem(rng, B=2, Hq=2, Hkv=1, Dk=64, Dv=32, P=16, lens=[1, 1])
    out = p.run(orc)
    for b in range(2):
        _, V = p.dense(b, 0)
        assert (out[b, 0] == V[0]).all() and (out[b, 1] == V[0]).all()


def test_two_tokens_sigmoid_closed_form(orc):
    rng = np.random.default_rng(5)
    p = Problem(rng, B=1, Hq=1, Hkv=1, Dk=64, Dv=8, P=16, lens=[2])
    p.k[:] = 0
    page = p.pt[0, 0]
    p.k[page, 0, 0, 0] = 0x38      # K_0 = e_0 * s_K
    p.k[page, 0, 1, 1] = 0x40      # K_1 = 2 e_1 * s_K  (0x40 = 2.0)
    p.q[:] = 0
    p.q[0, 0, 0], p.q[0, 0, 1] = 300.0, 100.0
    out = p.run(orc)
    sk = float(p.ks[0])
    s0, s1 = p.sm * 300.0 * sk, p.sm * 200.0 * sk
    _, V = p.dense(0, 0)
    exp = expit(s0 - s1) * V[0] + expit(s1 - s0) * V[1]
    np.testing.assert_allclose(out[0, 0], exp, rtol=1e-14, atol=1e-16)


def test_gqa_equals_replicated_mha(orc):
    rng = np.random.default_rng(6)
    G = 4
    p = Problem(rng, B=2, Hq=8, Hkv=2, Dk=64, Dv=16, P=4, lens=[9, 30])
    out = p.run(orc)
    # MHA problem whose KV head h is a copy of GQA head h // G
    k = np.repeat(p.k, G, axis=1)
    v = np.repeat(p.v, G, axis=1)
    ks, vs = np.repeat(p.ks, G), np.repeat(p.vs, G)
    mha = orc.paged_decode_attn(p.q, k_to_phys(k, FP8), v, FP8, p.pt, p.lens, ks, vs, sm_scale=p.sm, Hkv=8, Dk=64,
                                Dv=16, page_size=4)
    assert (out == mha).all()


def test_physical_page_permutation_invariance(orc):
    rng = np.random.default_rng(7)
    p = Problem(rng, B=3, Hq=4, Hkv=2, Dk=64, Dv=8, P=4, lens=[5, 16, 27])
    out = p.run(orc)
    perm = rng.permutation(p.num_pages)          # physical page i moves to slot perm[i]
    k2 = np.empty_like(p.k)
    v2 = np.empty_like(p.v)
    k2[perm] = p.k
    v2[perm] = p.v
    pt2 = np.where(p.pt >= 0, perm[np.maximum(p.pt, 0)], -1).astype(np.int32)
    out2 = orc.paged_decode_attn(p.q, k_to_phys(k2, FP8), v2, FP8, pt2, p.lens, p.ks, p.vs, sm_scale=p.sm, Hkv=2,
                                 Dk=64, Dv=8, page_size=4)
    assert (out == out2).all()


@pytest.mark.parametrize("split", [1, 4, 7, 64, 1000])
def test_split_merge_equals_single_pass(orc, split):
    rng = np.random.default_rng(8)
    p = Problem(rng, B=3, Hq=4, Hkv=2, Dk=64, Dv=16, P=8, lens=[1, 63, 200])
    p.q *= 3.0
    out = p.run(orc)
    rows = [(b, h) for b in range(3) for h in range(4)]
    sp = p.run(orc, rows=rows, split=split).reshape(3, 4, 16)
    np.testing.assert_allclose(sp, out, rtol=1e-12, atol=1e-14)


def test_aborted_rows_and_empty_sequences_are_zero(orc):
    rng = np.random.default_rng(9)
    p = Problem(rng, B=3, Hq=2, Hkv=1, Dk=64, Dv=8, P=4, lens=[5, 6, 7])
    p.lens[2] = 0
    out = p.run(orc, abort_mask=np.array([0, 1, 0], np.uint8))
    assert (out[1] == 0).all() and (out[2] == 0).all() and (out[0] != 0).any()


def test_shared_kv_equals_explicit_value_pool(orc):
    rng = np.random.default_rng(10)
    Dk, Dv = 128, 80
    p = Problem(rng, B=2, Hq=8, Hkv=1, Dk=Dk, Dv=Dv, P=8, lens=[11, 40], shared=True)
    out = p.run(orc)
    v = np.ascontiguousarray(np.swapaxes(p.k[..., :Dv], 2, 3))   # [page][1][Dv][P]
    exp = orc.paged_decode_attn(p.q, k_to_phys(p.k, FP8), v, FP8, p.pt, p.lens, p.ks, p.ks, sm_scale=p.sm, Hkv=1,
                                Dk=Dk, Dv=Dv, page_size=8)
    assert (out == exp).all()


def test_bf16_query_is_read_exactly(orc):
    rng = np.random.default_rng(11)
    p = Problem(rng, B=1, Hq=2, Hkv=1, Dk=64, Dv=16, P=4, lens=[9])
    qb = torch.from_numpy(p.q).to(torch.bfloat16)
    p.q = qb.float().numpy()
    out32 = p.run(orc)
    p.q = qb.view(torch.int16).numpy().view(np.uint16)
    outb = p.run(orc)
    assert (out32 == outb).all()
