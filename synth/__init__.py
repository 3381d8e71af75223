"""synth -- seeded synthetic decode workloads for paged KV-cache attention.

This module only *draws* inputs.  It holds none of the method's arithmetic: no quantisation,
no scale rule, no tag check, no attention.  Both the HIP library's tests/benchmark and the CPU
oracle take their inputs from here, so the two sides see identical data.

What it draws, per workload (shapes follow the workloads the pages discuss -- decode over a
paged KV cache with FP8 or BF16 storage, per-page tags, pages reused after being freed):
  * query heads q : [B][Hq][Dk]  (fp32, or bf16 bit patterns = round-to-nearest-even of fp32 draws)
  * per-sequence K/V token rows  (fp32 or bf16 draws, N(0,1); optional x20 outlier channels)
  * context lengths (explicit list or uniform integers, inclusive bounds)
  * the physical page assignment (seeded permutation of the pool, or a free-list churn
    simulation in which freed pages are handed out again with their tag bumped)
  * live per-page tags and each request's expected tags, with seeded stale-tag injections
    whose affected requests are known by construction.

Every stream comes from numpy's PCG64 seeded through SeedSequence([seed, workload id, stream
id, ...]), so the data of one sequence can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = ["Spec", "Workload", "SPECS", "make", "to_bf16_bits", "bf16_bits_to_f32"]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 draws, rounded to nearest even (torch's CPU cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class Spec:
    name: str
    wid: int                      # workload id mixed into every seed
    B: int
    Hq: int
    Hkv: int
    Dk: int
    Dv: int
    page_size: int
    lens: Optional[tuple] = None  # explicit attention lengths
    len_range: tuple = (1, 1)     # inclusive range of context lengths before the step
    append: bool = False          # the step appends one token per sequence at position ctx_len
    q_dt: str = "bf16"            # "f32" | "bf16"
    kv_dt_src: str = "bf16"       # dtype of the drawn K/V rows: "f32" | "bf16"
    out_dt: str = "bf16"
    shared_kv: bool = False       # V = first Dv dims of the K row, no separate V pool
    sm_scale: Optional[float] = None  # None -> 1/sqrt(Dk)
    split_tokens: int = 0         # 0 = library's choice
    num_pages: Optional[int] = None   # None -> just enough pages (plus 1/16 spare)
    alloc: str = "perm"           # "perm" (random permutation) | "churn" (free-list reuse, tag bumps)
    stale: str = "none"           # "none" | "one" (one request, one page) | "bernoulli"
    stale_rate: float = 0.0
    outlier_frac: float = 0.0     # fraction of (head, dim) channels scaled by outlier_mult
    outlier_mult: float = 20.0
    layers: int = 1
    budget_bytes: Optional[int] = None  # HBM budget for K+V of all layers (capacity workload)
    kv_dt: str = "fp8"            # storage dtype used for budget sizing

    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.Dk)


# The five workloads.  Lengths are attention lengths after the step's append (if any).
SPECS = {
    # tiny MHA, one layer, 64-page pool by seeded permutation, one stale request, fp32 end to end
    "tiny_mha": Spec("tiny_mha", 1, B=4, Hq=8, Hkv=8, Dk=64, Dv=64, page_size=16, lens=(17, 64, 129, 200),
                     q_dt="f32", kv_dt_src="f32", out_dt="f32", num_pages=64, stale="one"),
    # GQA decode, one layer, 1% outlier channels x20, one appended token per sequence
    "gqa": Spec("gqa", 2, B=32, Hq=32, Hkv=8, Dk=128, Dv=128, page_size=16, len_range=(1024, 8192),
                append=True, q_dt="bf16", kv_dt_src="bf16", out_dt="bf16", outlier_frac=0.01),
    # long-context split-KV decode, 4096-token partitions
    "long": Spec("long", 3, B=8, Hq=64, Hkv=8, Dk=128, Dv=128, page_size=16, len_range=(131072, 262144),
                 q_dt="bf16", kv_dt_src="f32", out_dt="bf16", split_tokens=4096),
    # high-concurrency capacity case: 8192 prompt + decode position U[1,1000], 61 layers, 80 GB budget,
    # free-list reuse with tag bumps, stale tags on 1e-4 of page references
    "capacity": Spec("capacity", 4, B=64, Hq=32, Hkv=8, Dk=128, Dv=128, page_size=16, len_range=(8192, 9191),
                     append=True, q_dt="bf16", kv_dt_src="bf16", out_dt="bf16", alloc="churn",
                     stale="bernoulli", stale_rate=1e-4, layers=61, budget_bytes=80 * 10**9),
    # shared-KV latent-style decode: 128 query heads on one KV head of dim 576 (V = first 512 dims)
    "shared_kv": Spec("shared_kv", 5, B=64, Hq=128, Hkv=1, Dk=576, Dv=512, page_size=64,
                      len_range=(4096, 32768), q_dt="bf16", kv_dt_src="f32", out_dt="bf16", shared_kv=True,
                      sm_scale=1.0 / 24.0),
}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def pages_per_layer(spec: Spec, kv_dt: str) -> int:
    """Pages of one layer that the HBM budget holds (K and V of all layers share the budget)."""
    el = 1 if kv_dt == "fp8" else 2
    per_page = spec.page_size * spec.Hkv * (spec.Dk + (0 if spec.shared_kv else spec.Dv)) * el
    return spec.budget_bytes // (spec.layers * per_page)


@dataclass
class Workload:
    spec: Spec
    seed: int
    q: np.ndarray                 # [B][Hq][Dk] float32 or uint16 (bf16 bits)
    ctx_lens: np.ndarray          # [B] tokens already in the cache before the step
    seq_lens: np.ndarray          # [B] attention length (ctx + appended)
    page_table: np.ndarray        # [B][pt_stride] int32, -1 past the end of a sequence
    num_pages: int
    live_tags: np.ndarray         # [num_pages] uint32
    expected_tags: np.ndarray     # [B][pt_stride] uint32
    expected_abort: np.ndarray    # [B] uint8 -- requests given a stale tag, known by construction
    stale_refs: list = field(default_factory=list)     # injected (b, j) page references
    k_outliers: tuple = ()        # (head idx array, dim idx array)
    v_outliers: tuple = ()
    alloc_generations: Optional[np.ndarray] = None     # times each page was handed out (churn)

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def B(self) -> int:
        return self.spec.B

    def kv_tokens(self, b: int, layer: int = 0, t0: int = 0, t1: Optional[int] = None):
        """Drawn K (and V) rows of tokens [t0, t1) of sequence b: ([n][Hkv][Dk], [n][Hkv][Dv] | None).

        Rows are drawn for the whole sequence from one stream, so any sub-range is consistent."""
        s = self.spec
        L = int(self.seq_lens[b])
        t1 = L if t1 is None else t1
        g = _rng(self.seed, s.wid, 100, layer, b)
        k = g.standard_normal((L, s.Hkv, s.Dk), dtype=np.float32)[t0:t1]
        v = None if s.shared_kv else g.standard_normal((L, s.Hkv, s.Dv), dtype=np.float32)[t0:t1]
        if len(self.k_outliers):
            k = k.copy()
            k[:, self.k_outliers[0], self.k_outliers[1]] *= np.float32(s.outlier_mult)
        if v is not None and len(self.v_outliers):
            v = v.copy()
            v[:, self.v_outliers[0], self.v_outliers[1]] *= np.float32(s.outlier_mult)
        if s.kv_dt_src == "bf16":
            k = to_bf16_bits(k)
            v = None if v is None else to_bf16_bits(v)
        return np.ascontiguousarray(k), (None if v is None else np.ascontiguousarray(v))

    def fill_tokens(self, b: int, layer: int = 0):
        """Rows already in the cache before the step: tokens [0, ctx_len)."""
        return self.kv_tokens(b, layer, 0, int(self.ctx_lens[b]))

    def step_tokens(self, layer: int = 0):
        """The step's appended rows: (k_new [B][Hkv][Dk], v_new | None, seq_ids, positions)."""
        assert self.spec.append
        ks, vs = [], []
        for b in range(self.B):
            c = int(self.ctx_lens[b])
            k, v = self.kv_tokens(b, layer, c, c + 1)
            ks.append(k)
            vs.append(v)
        k_new = np.concatenate(ks, 0)
        v_new = None if self.spec.shared_kv else np.concatenate(vs, 0)
        return k_new, v_new, np.arange(self.B, dtype=np.int32), self.ctx_lens.astype(np.int32).copy()

    def n_pages(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // self.spec.page_size)


def _alloc_perm(rng, need, num_pages):
    perm = rng.permutation(num_pages).astype(np.int32)
    out, off = [], 0
    for n in need:
        out.append(perm[off:off + n])
        off += n
    return out, None


def _alloc_churn(rng, need, num_pages, tags):
    """Free-list simulation: earlier sequences take pages, some finish and return them, the free
    list is reshuffled, and every hand-out bumps the page's tag (+1 mod 2^32).  Then the live
    sequences take their pages.  Returns per-sequence page lists and per-page hand-out counts."""
    gens = np.zeros(num_pages, np.int64)
    free = list(rng.permutation(num_pages))
    held = []
    for _round in range(6):
        # allocate history sequences until ~90% of the pool is in use
        while len(free) > num_pages // 10:
            n = int(rng.integers(1, 600))
            n = min(n, len(free) - num_pages // 10)
            if n <= 0:
                break
            pages = free[:n]
            del free[:n]
            for p in pages:
                tags[p] = np.uint32((int(tags[p]) + 1) & 0xFFFFFFFF)
                gens[p] += 1
            held.append(pages)
        # a random ~60% of the sequences finish and return their pages
        keep = []
        for pages in held:
            if rng.random() < 0.6:
                free.extend(pages)
            else:
                keep.append(pages)
        held = keep
        order = rng.permutation(len(free))
        free = [free[i] for i in order]
    # everything still held finishes too, then the live batch is admitted
    for pages in held:
        free.extend(pages)
    order = rng.permutation(len(free))
    free = [free[i] for i in order]
    out = []
    for n in need:
        if n > len(free):
            raise ValueError("pool too small for the live batch")
        pages = free[:n]
        del free[:n]
        for p in pages:
            tags[p] = np.uint32((int(tags[p]) + 1) & 0xFFFFFFFF)
            gens[p] += 1
        out.append(np.array(pages, np.int32))
    return out, gens


def make(spec, seed: int = 1, **overrides) -> Workload:
    """Draw a workload.  `spec` is a Spec or a name in SPECS; keyword overrides replace Spec fields
    (used for reduced-size parity cases)."""
    if isinstance(spec, str):
        spec = SPECS[spec]
    if overrides:
        spec = dataclasses.replace(spec, **overrides)
    s = spec
    # lengths
    if s.lens is not None:
        seq_lens = np.array(s.lens, np.int32)
        assert seq_lens.size == s.B
        ctx = seq_lens - (1 if s.append else 0)
    else:
        lo, hi = s.len_range
        ctx = _rng(seed, s.wid, 2).integers(lo, hi, size=s.B, endpoint=True).astype(np.int32)
        seq_lens = ctx + (1 if s.append else 0)
    seq_lens = seq_lens.astype(np.int32)
    ctx = ctx.astype(np.int32)
    P = s.page_size
    need = [-(-int(L) // P) for L in seq_lens]
    pt_stride = max(1, max(need))
    # pool
    if s.budget_bytes is not None:
        num_pages = pages_per_layer(s, s.kv_dt)
    elif s.num_pages is not None:
        num_pages = s.num_pages
    else:
        num_pages = sum(need) + max(1, sum(need) // 16)
    trng = _rng(seed, s.wid, 4)
    live = trng.integers(0, 2**32, size=num_pages, dtype=np.uint64).astype(np.uint32)
    # a few pages start at the top of the tag range so their next hand-out wraps to 0
    live[trng.choice(num_pages, size=min(8, num_pages), replace=False)] = np.uint32(0xFFFFFFFF)
    arng = _rng(seed, s.wid, 3)
    if s.alloc == "perm":
        pages, gens = _alloc_perm(arng, need, num_pages)
    else:
        pages, gens = _alloc_churn(arng, need, num_pages, live)
    page_table = np.full((s.B, pt_stride), -1, np.int32)
    expected = np.zeros((s.B, pt_stride), np.uint32)
    for b, pg in enumerate(pages):
        page_table[b, :len(pg)] = pg
        expected[b, :len(pg)] = live[pg]
    # stale-tag injection: the expected tag of a chosen reference is one generation behind
    srng = _rng(seed, s.wid, 5)
    stale_refs = []
    if s.stale == "one":
        b = int(srng.integers(0, s.B))
        j = int(srng.integers(0, need[b]))
        stale_refs.append((b, j))
    elif s.stale == "bernoulli":
        for b in range(s.B):
            hits = np.nonzero(srng.random(need[b]) < s.stale_rate)[0]
            stale_refs.extend((b, int(j)) for j in hits)
        if not stale_refs:
            b = int(srng.integers(0, s.B))
            stale_refs.append((b, int(srng.integers(0, need[b]))))
    abort = np.zeros(s.B, np.uint8)
    for b, j in stale_refs:
        expected[b, j] = np.uint32((int(expected[b, j]) - 1) & 0xFFFFFFFF)
        abort[b] = 1
    # queries
    q = _rng(seed, s.wid, 1).standard_normal((s.B, s.Hq, s.Dk), dtype=np.float32)
    if s.q_dt == "bf16":
        q = to_bf16_bits(q)
    # outlier channels: round(frac * Hkv * D) distinct (head, dim) pairs, separately for K and V
    ko = vo = ()
    if s.outlier_frac > 0:
        orng = _rng(seed, s.wid, 6)
        nk = int(round(s.outlier_frac * s.Hkv * s.Dk))
        idx = orng.choice(s.Hkv * s.Dk, size=nk, replace=False)
        ko = (idx // s.Dk, idx % s.Dk)
        if not s.shared_kv:
            nv = int(round(s.outlier_frac * s.Hkv * s.Dv))
            idx = orng.choice(s.Hkv * s.Dv, size=nv, replace=False)
            vo = (idx // s.Dv, idx % s.Dv)
    return Workload(spec=s, seed=seed, q=q, ctx_lens=ctx, seq_lens=seq_lens, page_table=page_table,
                    num_pages=int(num_pages), live_tags=live, expected_tags=expected, expected_abort=abort,
                    stale_refs=stale_refs, k_outliers=ko, v_outliers=vo, alloc_generations=gens)
