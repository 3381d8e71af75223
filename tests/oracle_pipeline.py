"""The oracle's end-to-end decode step on a synthetic workload (test infrastructure).

Step order, as the pages describe it (Cloudflare, "Smaller, faster, safer", section
保护共享 KV cache): the batched tag check runs first and yields the abort mask; then the new
token's K/V is quantised into its page slot (aborted requests skipped); then attention reads the
cache (aborted requests produce zero rows).  Scales are set up once from the initial fill.
"""
from __future__ import annotations

import numpy as np

import oracle
from layout import k_shape

FP8, BF16 = oracle.KV_FP8, oracle.KV_BF16


def kv_code(kv: str) -> int:
    return FP8 if kv == "fp8" else BF16


def pool_shapes(w, kv="fp8", num_pages=None):
    s = w.spec
    n = w.num_pages if num_pages is None else num_pages
    k = k_shape(n, s.Hkv, s.page_size, s.Dk, kv_code(kv))
    v = None if s.shared_kv else (n, s.Hkv, s.Dv, s.page_size)
    return k, v


def oracle_scales(w, layer=0):
    s = w.spec
    ak = np.zeros(s.Hkv, np.float32)
    av = np.zeros(s.Hkv, np.float32)
    for b in range(w.B):
        k, v = w.fill_tokens(b, layer)
        oracle.kv_absmax_update(k, ak)
        if v is not None:
            oracle.kv_absmax_update(v, av)
    ks = oracle.scale_from_absmax(ak)
    vs = None if s.shared_kv else oracle.scale_from_absmax(av)
    return ks, vs


def oracle_fill(w, kv="fp8", layer=0, scales=None):
    """Pools holding the initial fill (tokens [0, ctx_len) of every sequence)."""
    s = w.spec
    kd = kv_code(kv)
    el = np.uint8 if kd == FP8 else np.uint16
    kshape, vshape = pool_shapes(w, kv)
    kp = np.zeros(kshape, el)
    vp = None if vshape is None else np.zeros(vshape, el)
    ks, vs = scales if scales is not None else (oracle_scales(w, layer) if kd == FP8 else (None, None))
    for b in range(w.B):
        k, v = w.fill_tokens(b, layer)
        n = k.shape[0]
        oracle.kv_append(k, v, kp, vp, kd, w.page_table, np.full(n, b, np.int32), np.arange(n, dtype=np.int32),
                         ks, vs, page_size=s.page_size, num_pages=w.num_pages)
    return kp, vp, ks, vs


def oracle_step(w, kv="fp8", layer=0, verify=True, rows=None):
    """Full step: verify -> append -> attention.  Returns a dict of every intermediate."""
    s = w.spec
    kd = kv_code(kv)
    kp, vp, ks, vs = oracle_fill(w, kv, layer)
    abort = (oracle.kv_tag_verify(w.page_table, w.expected_tags, w.seq_lens, w.live_tags, page_size=s.page_size)
             if verify else None)
    if s.append:
        k_new, v_new, ids, pos = w.step_tokens(layer)
        oracle.kv_append(k_new, v_new, kp, vp, kd, w.page_table, ids, pos, ks, vs, abort,
                         page_size=s.page_size, num_pages=w.num_pages)
    out = oracle.paged_decode_attn(w.q, kp, vp, kd, w.page_table, w.seq_lens, ks, vs, abort, sm_scale=s.scale(),
                                   Hkv=s.Hkv, Dk=s.Dk, Dv=s.Dv, page_size=s.page_size, rows=rows)
    return dict(k_pool=kp, v_pool=vp, k_scale=ks, v_scale=vs, abort=abort, out=out)


def oracle_subproblem(w, b, kv, k_scale, v_scale, abort_b=0, layer=0, heads=None, seed=7919):
    """The oracle's step for request b alone, in a compact pool of its own pages.

    Request b's logical page j is placed in physical page compact[j] of a pool with exactly
    n_b pages (a seeded permutation, so page indirection is still exercised).  Attention of b
    depends only on its own pages, so its output rows equal those of the full batch.  The scales
    are passed in (the caller computes them with the oracle over the whole fill).
    Returns (k_pool, v_pool, compact, out[len(heads)][Dv])."""
    s = w.spec
    kd = kv_code(kv)
    el = np.uint8 if kd == FP8 else np.uint16
    P = s.page_size
    n = w.n_pages(b)
    compact = np.random.default_rng(seed + b).permutation(n).astype(np.int32)
    pt = compact.reshape(1, n)
    kp = np.zeros(k_shape(n, s.Hkv, P, s.Dk, kd), el)
    vp = None if s.shared_kv else np.zeros((n, s.Hkv, s.Dv, P), el)
    ab = np.array([abort_b], np.uint8)
    k, v = w.fill_tokens(b, layer)
    c = k.shape[0]
    oracle.kv_append(k, v, kp, vp, kd, pt, np.zeros(c, np.int32), np.arange(c, dtype=np.int32), k_scale, v_scale,
                     page_size=P, num_pages=n)
    del k, v
    if s.append:
        ctx = int(w.ctx_lens[b])
        kn, vn = w.kv_tokens(b, layer, ctx, ctx + 1)
        oracle.kv_append(kn, vn, kp, vp, kd, pt, np.zeros(1, np.int32), np.array([ctx], np.int32), k_scale,
                         v_scale, ab, page_size=P, num_pages=n)
    heads = list(range(s.Hq)) if heads is None else list(heads)
    out = oracle.paged_decode_attn(w.q[b:b + 1], kp, vp, kd, pt, w.seq_lens[b:b + 1], k_scale, v_scale, ab,
                                   sm_scale=s.scale(), Hkv=s.Hkv, Dk=s.Dk, Dv=s.Dv, page_size=P,
                                   rows=[(0, h) for h in heads])
    return kp, vp, compact, out
