#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X: FP8 vs BF16 KV, GQA decode workload.

Workload (one layer): batch 32, 32 query heads / 8 KV heads, head dim 128, page 16, context
lengths uniform in [1024, 8192], bf16 queries, K/V drawn bf16 N(0,1) with 1% outlier channels
x20, one new token appended per sequence per step.  Inputs are seeded synthetic data.

One step = the whole hot path on that batch:
  the batched page-tag check and the guarded append of the new token (quantised into its slot),
  issued as one launch (kv_tag_verify_append) -> paged_decode_attn (dequantise on read, online
  softmax, split-KV merge).  The same step as three calls (kv_tag_verify, kv_append,
  paged_decode_attn) is timed beside it (fp8.separate_step_ms).
Two copies of the pools are used alternately so the 256 MB last-level cache cannot serve a
step from the previous one.  Timing uses HIP events on the stream the library launches on.
The step is timed replayed from a HIP graph (one captured step per pool copy; --no-graph times
eager launches).  The roofline's denominator is the attention call alone: 20 calls (pool copies
alternating) captured back to back in a HIP graph and replayed, the elapsed time divided by the
number of calls; events around single eager calls are reported beside it.

The default line also carries: the read ceiling of the library's plain streaming kernel
(hbm_read_probe), the long-context leg (attention on 3 GB of FP8 KV), the capacity leg's tag
check against 61 layers of attention, and the oracle timed on the host (one thread, and one
thread per sequence up to 16).  --no-legs and --no-cpu-baseline skip them.

Prints one JSON line.  value = decode tokens/s of the FP8 step (B tokens per step).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "decode_attention_paged_fp8_amd", "csrc")
ATTN_KERNELS = ("attn_sk_kernel", "merge_sk_kernel", "attn_mfma_kernel", "attn_generic_kernel", "merge_kernel")


# the sources each workload's attention call is built from (kernels, shared headers, launch plan)
_COMMON = ("api.hip", "common.hpp", "mfma_util.hpp")
ATTN_SOURCES = {
    "gqa": _COMMON + ("attn_mfma.hip",),
    "long": _COMMON + ("attn_mfma.hip",),
    "shared_kv": _COMMON + ("attn_latent.hip", "attn_mfma.hip"),  # the merge kernel lives in attn_mfma.hip
    "all_attention": _COMMON + ("attn_generic.hip", "attn_latent.hip", "attn_mfma.hip"),
    "transcode": ("api.hip", "common.hpp", "kv_ops.hip"),
    "w4gemv": ("api.hip", "common.hpp", "w4_gemv.hip"),
}
# the file a workload's traffic summary lives in
TRAFFIC_FILES = {"transcode": "traffic_kv_transcode_pages.md", "w4gemv": "traffic_w4a16_gemv.md"}


def kernel_source_hash(workload: str | None = "all_attention") -> str:
    """sha256 over the sources a workload's attention call is built from (None: every library
    source): a traffic figure measured on other sources is void."""
    import hashlib

    files = ATTN_SOURCES.get(workload, ATTN_SOURCES["all_attention"]) if workload is not None else None
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if (f in files) if files is not None else f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kv: str):
    """HBM bytes per attention call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of
    this workload, or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, TRAFFIC_FILES.get(workload, f"traffic_paged_decode_attn_{workload}.md"))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            m = line.strip().strip("`").split(": ", 1)
            if len(m) == 2:
                vals[m[0].strip()] = m[1].strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash(workload):
        return None
    v = vals.get(f"hbm_bytes_per_call[{kv}]")
    return int(v) if v else None


def algorithmic_bytes(w, kv: str) -> dict:
    """Bytes one attention call must move at minimum: every attended token's K and V of every KV
    head once, the queries, the outputs, the page-table entries read and the scales."""
    s = w.spec
    el = 1 if kv == "fp8" else 2
    tokens = int(w.seq_lens.sum())
    kv_bytes = tokens * s.Hkv * (s.Dk + (0 if s.shared_kv else s.Dv)) * el
    q_bytes = s.B * s.Hq * s.Dk * (4 if s.q_dt == "f32" else 2)
    o_bytes = s.B * s.Hq * s.Dv * (4 if s.out_dt == "f32" else 2)
    pt_bytes = sum(w.n_pages(b) for b in range(s.B)) * 4
    sc_bytes = (2 * s.Hkv * 4) if kv == "fp8" else 0
    return dict(kv=kv_bytes, total=kv_bytes + q_bytes + o_bytes + pt_bytes + sc_bytes, tokens=tokens)


def run_kv(w, kv, steps, warmup, split_tokens=0, use_graph=True, no_tag_check=False):
    import torch

    import decode_attention_paged_fp8_amd as dapf8
    from gpu_pipeline import GpuState

    s = w.spec
    st = GpuState(w, kv)
    # second copy of the pools (same page table) for cache rotation
    pools = [(st.k_pool, st.v_pool), (st.k_pool.clone(), st.v_pool.clone())]
    step_in = st.step_inputs()
    ws = dapf8.make_workspace(st.q, st.k_pool, st.v_pool, st.page_table, s.Dv, split_tokens)
    out = torch.empty((s.B, s.Hq, s.Dv), dtype=torch.bfloat16, device="cuda")
    abort = st.abort
    k_new, v_new, ids, pos = step_in

    # The step as three calls: the tag check, the guarded append, the attention.
    def step_separate(i, ev=None):
        kp, vp = pools[i % 2]
        dapf8.kv_tag_verify(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, abort, s.page_size)
        dapf8.kv_append(k_new, v_new, kp, vp, st.page_table, ids, pos, st.k_scale, st.v_scale, abort)
        if ev is not None:
            ev[0].record()
        dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale, abort, out=out,
                                sm_scale=s.scale(), split_tokens=split_tokens, workspace=ws)
        if ev is not None:
            ev[1].record()

    # The pages' default no-op tracker: checking disabled, so no tag check is launched and neither
    # the append nor the attention takes an abort mask.
    def step_untracked(i, ev=None):
        kp, vp = pools[i % 2]
        dapf8.kv_append(k_new, v_new, kp, vp, st.page_table, ids, pos, st.k_scale, st.v_scale)
        if ev is not None:
            ev[0].record()
        dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale, out=out,
                                sm_scale=s.scale(), split_tokens=split_tokens, workspace=ws)
        if ev is not None:
            ev[1].record()

    # The measured step: the same work with the check and the append in one launch
    # (kv_tag_verify_append: each request's workgroup checks its tags, then writes its own token).
    def step(i, ev=None):
        kp, vp = pools[i % 2]
        dapf8.kv_tag_verify_append(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, abort, k_new, v_new,
                                   kp, vp, ids, pos, st.k_scale, st.v_scale)
        if ev is not None:
            ev[0].record()
        dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale, abort, out=out,
                                sm_scale=s.scale(), split_tokens=split_tokens, workspace=ws)
        if ev is not None:
            ev[1].record()

    if no_tag_check:
        step = step_untracked

    # Ablation: the tag check inside attention's page walk (no separate pass; the append is then
    # unguarded) -- the alternative the pages weigh against their separate batched check.
    cmask = torch.zeros(s.B, dtype=torch.uint8, device="cuda")

    def step_checked(i, ev=None):
        kp, vp = pools[i % 2]
        dapf8.kv_append(k_new, v_new, kp, vp, st.page_table, ids, pos, st.k_scale, st.v_scale)
        if ev is not None:
            ev[0].record()
        dapf8.paged_decode_attn_checked(st.q, kp, vp, st.page_table, st.seq_lens, st.expected_tags, st.live_tags,
                                        cmask, st.k_scale, st.v_scale, out=out, sm_scale=s.scale(), workspace=ws)
        if ev is not None:
            ev[1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(steps):
        step(i, evs[i])
    t_end.record()
    torch.cuda.synchronize()
    eager_step_ms = t_start.elapsed_time(t_end) / steps
    attn_ms = [a.elapsed_time(b) for a, b in evs]

    checked = None
    if s.Dk == 128 and s.Dv == 128 and s.page_size == 16 and not no_tag_check:
        for i in range(warmup):
            step_checked(i)
        cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for i in range(steps):
            step_checked(i, cevs[i])
        torch.cuda.synchronize()
        def checked_call(c):
            kp, vp = pools[c % 2]
            return lambda: dapf8.paged_decode_attn_checked(st.q, kp, vp, st.page_table, st.seq_lens, st.expected_tags,
                                                           st.live_tags, cmask, st.k_scale, st.v_scale, out=out,
                                                           sm_scale=s.scale(), workspace=ws)

        checked = dict(attn_ms=graph_calls_ms([checked_call(c) for c in range(20)], reps=max(2, steps // 20)),
                       attn_eager_event_ms=sum(a.elapsed_time(b) for a, b in cevs) / steps, graph_step_ms=None)

    # The same step captured as a HIP graph (one per pool copy) and replayed: no host launch gaps.
    def graph_time(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(0)
            fn(1)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for c in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(c)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % 2].replay()
        torch.cuda.synchronize()
        t_start.record()
        for i in range(steps):
            graphs[i % 2].replay()
        t_end.record()
        torch.cuda.synchronize()
        ms = t_start.elapsed_time(t_end) / steps
        del graphs
        return ms

    # The attention call alone, back to back, replayed from a HIP graph (20 calls alternating the
    # pool copies): the per-call time that the roofline uses.
    def attn_call(c):
        kp, vp = pools[c % 2]
        return lambda: dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale,
                                               abort, out=out, sm_scale=s.scale(), split_tokens=split_tokens,
                                               workspace=ws)

    attn_graph_ms = graph_calls_ms([attn_call(c) for c in range(20)], reps=max(2, steps // 20))

    graph_step_ms = untracked_step_ms = separate_step_ms = None
    if use_graph:
        graph_step_ms = graph_time(step)
        untracked_step_ms = graph_step_ms if no_tag_check else graph_time(step_untracked)
        separate_step_ms = None if no_tag_check else graph_time(step_separate)
        if checked is not None:
            checked["graph_step_ms"] = graph_time(step_checked)
    step_ms = graph_step_ms if graph_step_ms is not None else eager_step_ms

    # the tag check and the append on their own (same stream, events around each launch)
    def timed(fn, n=50):
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            e[i][0].record()
            fn(i)
            e[i][1].record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in e) / n

    verify_ms = None if no_tag_check else graph_calls_ms(
        [lambda: dapf8.kv_tag_verify(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, abort,
                                     s.page_size)] * 20, reps=5)
    verify_append_ms = None if no_tag_check else graph_calls_ms(
        [lambda c=c: dapf8.kv_tag_verify_append(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, abort,
                                                k_new, v_new, *pools[c % 2], ids, pos, st.k_scale, st.v_scale)
         for c in range(20)], reps=5)
    append_ms = timed(lambda i: dapf8.kv_append(k_new, v_new, *pools[i % 2], st.page_table, ids, pos, st.k_scale,
                                                st.v_scale, None if no_tag_check else abort))
    variant, split = dapf8.paged_decode_attn_variant(s.B, s.Hq, s.Hkv, s.Dk, s.Dv, s.page_size, w.pt_stride,
                                                     split_tokens, 0 if kv == "fp8" else 1)
    # the attention output of one plain step (pool copy 0), for the FP8-vs-BF16 comparison
    step(0)
    torch.cuda.synchronize()
    out_copy = out.float().cpu()
    del pools, st, ws
    torch.cuda.empty_cache()
    return dict(out=out_copy, step_ms=step_ms, eager_step_ms=eager_step_ms, graph_step_ms=graph_step_ms,
                attn_ms=attn_graph_ms, attn_eager_event_ms=sum(attn_ms) / len(attn_ms),
                attn_ms_min=min(attn_ms), verify_ms=verify_ms,
                append_ms=append_ms, variant=variant, split=split, checked=checked,
                untracked_step_ms=untracked_step_ms, separate_step_ms=separate_step_ms,
                verify_append_ms=verify_append_ms)


def graph_calls_ms(calls, reps=5, warm=2):
    """Per-call time of `calls` (each launches library work on the current stream), captured once in a
    HIP graph and replayed `reps` times back to back; HIP events on the replay stream bracket the
    replays."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * len(calls))
    del g
    return ms


class DevPools:
    """A workload's page table, lengths, tags and queries (from the seeded generator) with K/V pools
    filled on the device: every attended token's rows drawn N(0,1) by torch's seeded GPU generator
    (same shapes and distribution as the generator's host draws, which would take minutes to
    produce at these sizes), per-head scales from the fill (kv_absmax_update / kv_scale_from_absmax)
    and kv_append into `copies` pool copies."""

    def __init__(self, w, kv="fp8", copies=1, seed=11):
        import torch

        import decode_attention_paged_fp8_amd as dapf8
        from gpu_pipeline import t_act, t_int

        s = w.spec
        self.w, self.kv = w, kv
        self.page_table = t_int(w.page_table)
        self.seq_lens = t_int(w.seq_lens)
        self.live_tags = t_int(w.live_tags, torch.uint32)
        self.expected_tags = t_int(w.expected_tags, torch.uint32)
        self.q = t_act(w.q)
        self.abort = torch.zeros(w.B, dtype=torch.uint8, device="cuda")
        self.pools = [dapf8.alloc_pools(w.num_pages, s.Hkv, s.page_size, s.Dk, s.Dv, kv, s.shared_kv)
                      for _ in range(copies)]
        g = torch.Generator(device="cuda")

        def rows(b):
            g.manual_seed(seed * 100003 + b)
            L = int(w.seq_lens[b])
            k = torch.randn((L, s.Hkv, s.Dk), generator=g, device="cuda")
            v = None if s.shared_kv else torch.randn((L, s.Hkv, s.Dv), generator=g, device="cuda")
            return k, v

        self.k_scale = self.v_scale = None
        if kv == "fp8":
            ak = torch.zeros(s.Hkv, dtype=torch.float32, device="cuda")
            av = torch.zeros(s.Hkv, dtype=torch.float32, device="cuda")
            for b in range(w.B):
                k, v = rows(b)
                dapf8.kv_absmax_update(k, ak)
                if v is not None:
                    dapf8.kv_absmax_update(v, av)
            self.k_scale = dapf8.kv_scale_from_absmax(ak)
            self.v_scale = None if s.shared_kv else dapf8.kv_scale_from_absmax(av)
        for b in range(w.B):
            k, v = rows(b)
            n = k.shape[0]
            ids = torch.full((n,), b, dtype=torch.int32, device="cuda")
            pos = torch.arange(n, dtype=torch.int32, device="cuda")
            for kp, vp in self.pools:
                dapf8.kv_append(k, v, kp, vp, self.page_table, ids, pos, self.k_scale, self.v_scale)
            del k, v
        torch.cuda.synchronize()


def stream_ceiling(call_bytes: int, reps: int = 5) -> dict:
    """hbm_read_probe, the library's plain read-only streaming kernel: the attainable read rate over a
    2 GiB buffer, read front to back and as randomly scattered 2 KiB blocks (the page-block pattern),
    and the scattered read of exactly one GQA attention call's byte count, launched back to back from
    a graph like the attention calls (its fixed per-launch costs included)."""
    import torch

    import decode_attention_paged_fp8_amd as dapf8

    blk = 2048
    buf = torch.zeros(2 << 30, dtype=torch.uint8, device="cuda")
    nblk = buf.numel() // blk
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    ids = torch.randperm(nblk, generator=gen, device="cuda").to(torch.int32)
    sink = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    res = {}
    ms = graph_calls_ms([lambda: dapf8.hbm_read_probe(buf, blk, sink=sink)] * 4, reps=reps)
    res["contiguous_2GiB_gbs"] = round(buf.numel() / (ms * 1e-3) / 1e9, 1)
    ms = graph_calls_ms([lambda: dapf8.hbm_read_probe(buf, blk, ids, sink=sink)] * 4, reps=reps)
    res["scattered_2KiB_blocks_2GiB_gbs"] = round(buf.numel() / (ms * 1e-3) / 1e9, 1)
    n = call_bytes // blk
    sets = [ids[:n].contiguous(), ids[n:2 * n].contiguous()]
    ms = graph_calls_ms([lambda i=i: dapf8.hbm_read_probe(buf, blk, sets[i % 2], sink=sink) for i in range(20)],
                        reps=reps)
    res["scattered_call_size"] = {"bytes": n * blk, "us_per_launch": round(ms * 1e3, 2),
                                  "gbs": round(n * blk / (ms * 1e-3) / 1e9, 1)}
    res["kernel"] = "hbm_read_probe (16-byte non-temporal loads, 2048 workgroups x 256 threads)"
    del buf, ids, sets, sink
    torch.cuda.empty_cache()
    return res


def long_context_leg(reps: int = 3) -> dict:
    """Long-context split-KV workload (B8, 64/8 heads, D128, P16, lengths U[131072, 262144], FP8):
    attention calls back to back from a graph on a device-filled pool (3.0 GB of KV per call)."""
    import torch

    import decode_attention_paged_fp8_amd as dapf8
    import synth

    w = synth.make("long", seed=1)
    s = w.spec
    st = DevPools(w, "fp8")
    kp, vp = st.pools[0]
    ws = dapf8.make_workspace(st.q, kp, vp, st.page_table, s.Dv, s.split_tokens)
    out = torch.empty((s.B, s.Hq, s.Dv), dtype=torch.bfloat16, device="cuda")
    call = lambda: dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale,
                                           out=out, sm_scale=s.scale(), split_tokens=s.split_tokens, workspace=ws)
    ms = graph_calls_ms([call] * 6, reps=reps)
    verify_ms = graph_calls_ms([lambda: dapf8.kv_tag_verify(st.page_table, st.expected_tags, st.seq_lens,
                                                             st.live_tags, st.abort, s.page_size)] * 20, reps=reps)
    by = algorithmic_bytes(w, "fp8")
    gbs = by["total"] / (ms * 1e-3) / 1e9
    variant, split = dapf8.paged_decode_attn_variant(s.B, s.Hq, s.Hkv, s.Dk, s.Dv, s.page_size, w.pt_stride,
                                                     s.split_tokens, 0)
    del st, ws, out
    torch.cuda.empty_cache()
    return {"workload": "long_b8_h64kv8_d128_p16_len131072-262144", "attended_tokens": by["tokens"],
            "algorithmic_bytes_per_call": by["total"], "call_ms": round(ms, 5),
            "decode_tokens_per_s": round(s.B / (ms * 1e-3), 1), "achieved_gbs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("long", "fp8"),
            "verify_ms": round(verify_ms, 5), "verify_over_attention": round(verify_ms / ms, 5),
            "variant": variant, "split_tokens": split,
            "data": "device-filled N(0,1) K/V (seeded torch GPU generator), generator page table and queries"}


def tiny_mha_leg(reps: int = 20) -> dict:
    """The tiny MHA workload (B4, lengths 17/64/129/200, 8/8 heads, D64, P16, fp32 q/K/V/out): far
    too small for a bandwidth figure, so only the latency of one attention call and of the whole step
    (tag check and attention; this workload appends no token), replayed from a graph."""
    import torch

    import decode_attention_paged_fp8_amd as dapf8
    import synth
    from gpu_pipeline import GpuState

    w = synth.make("tiny_mha", seed=1)
    s = w.spec
    st = GpuState(w, "fp8")
    ws = dapf8.make_workspace(st.q, st.k_pool, st.v_pool, st.page_table, s.Dv)
    out = torch.empty((s.B, s.Hq, s.Dv), dtype=torch.float32, device="cuda")
    attn = lambda: dapf8.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, st.k_scale,
                                           st.v_scale, st.abort, out=out, sm_scale=s.scale(), workspace=ws)

    def step():
        dapf8.kv_tag_verify(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, st.abort, s.page_size)
        attn()

    attn_ms = graph_calls_ms([attn] * 20, reps=reps)
    step_ms = graph_calls_ms([step] * 20, reps=reps)
    variant, _ = dapf8.paged_decode_attn_variant(s.B, s.Hq, s.Hkv, s.Dk, s.Dv, s.page_size, w.pt_stride, 0, 0)
    del st, ws, out
    torch.cuda.empty_cache()
    return {"workload": "tiny_mha_b4_h8kv8_d64_p16", "attn_us": round(attn_ms * 1e3, 2),
            "step_us": round(step_ms * 1e3, 2), "variant": variant}


def capacity_tag_check_leg(reps: int = 5) -> dict:
    """The capacity workload's tag check (B64, churned page table, stale tags on 1e-4 of references)
    against 61 layers of attention: one layer's FP8 pool (1.3 GB, beyond the 256 MB last-level cache;
    two copies alternate) is timed back to back from a graph and taken 61 times, the check likewise,
    once per decode step.  Also the admission arithmetic of the 80 GB budget."""
    import torch

    import decode_attention_paged_fp8_amd as dapf8
    import synth

    w = synth.make("capacity", seed=1)
    s = w.spec
    st = DevPools(w, "fp8", copies=2)
    ws = dapf8.make_workspace(st.q, st.pools[0][0], st.pools[0][1], st.page_table, s.Dv)
    out = torch.empty((s.B, s.Hq, s.Dv), dtype=torch.bfloat16, device="cuda")
    verify = lambda: dapf8.kv_tag_verify(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, st.abort,
                                         s.page_size)
    verify()
    torch.cuda.synchronize()
    n_abort = int(st.abort.sum().item())

    def attn(c):
        kp, vp = st.pools[c % 2]
        return lambda: dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale,
                                               st.abort, out=out, sm_scale=s.scale(), workspace=ws)

    verify_ms = graph_calls_ms([verify] * 20, reps=reps)
    attn_ms = graph_calls_ms([attn(c) for c in range(10)], reps=reps)
    by = algorithmic_bytes(w, "fp8")
    gbs = by["total"] / (attn_ms * 1e-3) / 1e9
    worst = -(-(s.len_range[1] + 1) // s.page_size)
    del st, ws, out
    torch.cuda.empty_cache()
    return {"workload": "capacity_b64_h32kv8_d128_p16_61layers_80GB_budget", "verify_ms": round(verify_ms, 5),
            "attention_ms_per_layer": round(attn_ms, 5), "layers": s.layers,
            "verify_over_61_layers_attention": round(verify_ms / (s.layers * attn_ms), 6),
            "attention_layer_gbs": round(gbs, 1), "attention_layer_frac": round(gbs / HBM_PEAK_GBS, 4),
            "page_references": int(sum(w.n_pages(b) for b in range(w.B))), "aborted_requests": n_abort,
            "expected_aborted": int(w.expected_abort.sum()),
            "admission": {"budget_bytes": s.budget_bytes, "worst_case_pages_per_sequence": worst,
                          "fp8_pages_per_layer": synth.pages_per_layer(s, "fp8"),
                          "bf16_pages_per_layer": synth.pages_per_layer(s, "bf16"),
                          "fp8_admits_sequences": synth.pages_per_layer(s, "fp8") // worst,
                          "bf16_admits_sequences": synth.pages_per_layer(s, "bf16") // worst}}


def _host_cpu() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count()}


def cpu_baseline(w) -> dict:
    """The oracle (plain C, fp64) timed on the host on the same GQA decode step: (i) single-threaded
    over the first 8 sequences, scaled to the batch by attended tokens; (ii) the whole batch with the
    oracle's attention dispatched per sequence over a thread pool (the C calls release Python's
    lock), at most 16 threads (the host cores a single-GPU machine gives one GPU).  The tag check and the append
    are single calls in both.  Pools are filled by the oracle once, before timing."""
    import concurrent.futures as cf

    import oracle
    from oracle_pipeline import oracle_fill

    s = w.spec
    kp, vp, ks, vs = oracle_fill(w, "fp8")
    k_new, v_new, ids, pos = w.step_tokens()
    kw = dict(sm_scale=s.scale(), Hkv=s.Hkv, Dk=s.Dk, Dv=s.Dv, page_size=s.page_size)

    def head(b_list):
        ab = oracle.kv_tag_verify(w.page_table, w.expected_tags, w.seq_lens, w.live_tags, page_size=s.page_size)
        oracle.kv_append(k_new, v_new, kp, vp, oracle.KV_FP8, w.page_table, ids, pos, ks, vs, ab,
                         page_size=s.page_size, num_pages=w.num_pages)
        return ab

    def attn(b, ab):
        return oracle.paged_decode_attn(w.q, kp, vp, oracle.KV_FP8, w.page_table, w.seq_lens, ks, vs, ab,
                                        rows=[(b, h) for h in range(s.Hq)], **kw)

    n1 = 8
    t0 = time.perf_counter()
    ab = head(range(n1))
    for b in range(n1):
        attn(b, ab)
    t1 = time.perf_counter() - t0
    frac = float(w.seq_lens[:n1].sum()) / float(w.seq_lens.sum())
    single = s.B / (t1 / frac)
    threads = max(1, min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    ab = head(range(s.B))
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda b: attn(b, ab), range(s.B)))
    tn = time.perf_counter() - t0
    host = _host_cpu()
    return dict(value=round(s.B / tn, 3), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"the whole GQA step (tag check, append, attention of all {s.B} sequences, "
                       f"{int(w.seq_lens.sum())} attended tokens) with attention dispatched per sequence over "
                       f"{threads} threads: {tn:.2f} s",
                single_thread={"value": round(single, 3), "unit": "tokens/s", "cores": 1,
                               "sample": f"first {n1} of {s.B} sequences ({int(w.seq_lens[:n1].sum())} tokens), "
                                         f"{t1:.2f} s, scaled to the batch by attended tokens"},
                host=host)


def _events(n):
    import torch

    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def bench_attention_only(name, steps, warmup, kv="fp8"):
    """Long-context and latent-style workloads: time paged_decode_attn calls on a filled pool."""
    import torch

    import decode_attention_paged_fp8_amd as dapf8
    import synth

    w = synth.make(name, seed=1)
    s = w.spec
    # pools filled on the device (same shapes and distribution as the generator's draws, which would
    # take minutes on the host at these sizes)
    st = DevPools(w, kv)
    kp, vp = st.pools[0]
    ws = dapf8.make_workspace(st.q, kp, vp, st.page_table, s.Dv, s.split_tokens)
    out = torch.empty((s.B, s.Hq, s.Dv), dtype=torch.bfloat16, device="cuda")

    def call():
        dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale,
                                out=out, sm_scale=s.scale(), Dv=s.Dv, split_tokens=s.split_tokens, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = _events(steps)
    for i in range(steps):
        evs[i][0].record()
        call()
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    by = algorithmic_bytes(w, kv)
    variant, split = dapf8.paged_decode_attn_variant(s.B, s.Hq, s.Hkv, s.Dk, s.Dv, s.page_size, w.pt_stride,
                                                     s.split_tokens, 0 if kv == "fp8" else 1, s.shared_kv)
    flops = 2.0 * by["tokens"] * s.Hq * (s.Dk + s.Dv)
    gbs = by["total"] / (ms * 1e-3) / 1e9
    return {"metric": "decode-attn tokens/s + effective KV GB/s (% HBM peak), FP8 vs BF16 KV",
            "value": round(s.B / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": f"{kv} KV, bf16 q/out", "data": "synthetic",
            "config": {"workload": name, "batch": s.B, "q_heads": s.Hq, "kv_heads": s.Hkv, "head_dim_k": s.Dk,
                       "head_dim_v": s.Dv, "page_size": s.page_size, "attended_tokens": by["tokens"],
                       "split_tokens": split, "variant": variant, "parallelism": "single-gpu"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, kv),
                         "algorithmic_bytes_per_launch": by["total"], "avg_launch_ms": round(ms, 5)},
            "mfma_view": {"flops_per_launch": flops, "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                          "bf16_dense_peak_tflops": 2500.0}}


def bench_transcode(steps, warmup):
    """Prefill -> decode handoff: every page the GQA workload's requests use, copied from a BF16
    cache into an FP8 cache by kv_transcode_pages (HBM-bound: 2 bytes read, 1 written per value)."""
    import numpy as np
    import torch

    import decode_attention_paged_fp8_amd as dapf8
    import synth
    from gpu_pipeline import GpuState, t_act

    w = synth.make("gqa", seed=1)
    s = w.spec
    ak = torch.zeros(s.Hkv, dtype=torch.float32, device="cuda")
    av = torch.zeros(s.Hkv, dtype=torch.float32, device="cuda")

    def amax(b, k, v):
        if k.shape[0]:
            dapf8.kv_absmax_update(t_act(k), ak)
            dapf8.kv_absmax_update(t_act(v), av)

    st = GpuState(w, "bf16", on_rows=amax)
    ks, vs = dapf8.kv_scale_from_absmax(ak), dapf8.kv_scale_from_absmax(av)
    used = np.concatenate([w.page_table[b, :(int(w.seq_lens[b]) + s.page_size - 1) // s.page_size]
                           for b in range(w.B)]).astype(np.int32)
    n = int(used.size)
    src = torch.from_numpy(used).cuda()
    dst = torch.from_numpy(np.random.default_rng(5).permutation(n).astype(np.int32)).cuda()
    kd, vd = dapf8.alloc_pools(n, s.Hkv, s.page_size, s.Dk, s.Dv, "fp8")

    def call():
        dapf8.kv_transcode_pages(st.k_pool, st.v_pool, kd, vd, src, dst, ks, vs)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = _events(steps)
    for i in range(steps):
        evs[i][0].record()
        call()
        evs[i][1].record()
    torch.cuda.synchronize()
    eager_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    # the roofline time: calls back to back replayed from a HIP graph (no host launch gaps)
    ms = graph_calls_ms([call] * 10, reps=max(2, steps // 10))
    nbytes = n * s.Hkv * s.page_size * (s.Dk + s.Dv) * 3
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the attainable rate of the same byte mix: hbm_copy_probe reads 2 bytes per byte written,
    # contiguous, over the same byte counts (its own buffers, two copies alternating)
    wbytes = nbytes // 3
    bufs = [(torch.empty(2 * wbytes, dtype=torch.uint8, device="cuda"),
             torch.empty(wbytes, dtype=torch.uint8, device="cuda")) for _ in range(2)]
    pms = graph_calls_ms([lambda i=i: dapf8.hbm_copy_probe(*bufs[i % 2]) for i in range(10)],
                         reps=max(2, steps // 10))
    del bufs
    ceiling = {"kernel": "hbm_copy_probe (2 bytes read per byte written, 16-byte non-temporal loads and stores)",
               "bytes": 3 * wbytes, "us_per_launch": round(pms * 1e3, 2),
               "gbs": round(3 * wbytes / (pms * 1e-3) / 1e9, 1)}
    return {"metric": "kv_transcode_pages GB/s (% HBM peak)", "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16 -> fp8-e4m3", "data": "synthetic",
            "config": {"workload": "transcode_gqa_pages_b32_kv8_d128_p16", "pages": n, "kv_heads": s.Hkv,
                       "head_dim": s.Dk, "page_size": s.page_size, "parallelism": "single-gpu"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("transcode", "transcode"),
                         "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 5),
                         "kernel": "transcode_kernel, calls back to back replayed from a HIP graph"},
            "eager_event_ms": round(eager_ms, 5), "read_write_ceiling": ceiling,
            "frac_of_ceiling": round(gbs / ceiling["gbs"], 4)}


def bench_pages(steps, warmup):
    """Device page allocator: an allocation and the release of the same pages, for the growth a
    decode step makes (one page for each of 64 requests) and for a bulk admission (64 requests x
    512 pages).  The pair is captured ten times in a HIP graph and replayed, so host launch costs
    are not counted."""
    import torch

    import decode_attention_paged_fp8_amd as dapf8

    N, B, reps = 80000, 64, 10
    fl, fc, lt = dapf8.alloc_page_allocator(N)
    pt = torch.full((B, 1024), -1, dtype=torch.int32, device="cuda")
    et = torch.zeros_like(pt)
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    res = {}
    for name, k in (("decode_step_64x1", 1), ("admission_64x512", 512)):
        cnt = torch.full((B,), k, dtype=torch.int32, device="cuda")
        pages = torch.empty(B * k, dtype=torch.int32, device="cuda")
        status = torch.empty(4, dtype=torch.int32, device="cuda")
        granted = torch.empty(B, dtype=torch.uint8, device="cuda")

        def pair():
            dapf8.kv_pages_alloc(fl, fc, lt, cnt, zero, pt, et, granted=granted)
            pages.view(B, k).copy_(pt[:, :k])
            dapf8.kv_pages_free(fl, fc, pages, status=status)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            pair()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                pair()
        for _ in range(max(1, warmup // reps)):
            g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(1, steps // reps)
        t0.record()
        for _ in range(n):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / (n * reps) * 1e3
        ok = int(granted.sum().item()) == B and int(status[1].item()) == 0
        res[name] = {"pages": B * k, "alloc_plus_free_us": round(us, 2), "pages_per_s": round(B * k / (us * 1e-6), 1),
                     "all_granted_and_freed": ok}
        del g
    return {"metric": "device page allocator latency (allocation + release of the same pages)",
            "value": res["decode_step_64x1"]["alloc_plus_free_us"], "unit": "us", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
            "data": "synthetic", "config": {"workload": "page_alloc_pool80000_b64", "parallelism": "single-gpu"},
            "roofline": {"bound": "latency",
                         "note": "single-workgroup kernels: a few dependent memory round trips each"},
            "cases": res}


def bench_w4gemv(steps, warmup):
    """INT4 weight-only decode GEMV on synthetic weights: N = 28672, K = 8192 (117 MB of packed
    weights), decode batches M = 1, 4, 16.  Three weight copies rotate so the 256 MB last-level
    cache cannot serve a call from the previous one; 30 calls per replayed HIP graph."""
    import numpy as np
    import torch

    import decode_attention_paged_fp8_amd as dapf8

    N, K, copies, per_graph = 28672, 8192, 3, 30
    rng = np.random.default_rng(3)
    weights = []
    for _ in range(copies):
        q = torch.from_numpy(rng.integers(-8, 8, size=(N, K)).astype(np.int8)).cuda()
        sc = torch.from_numpy((rng.random((N, K // 128)) * 0.02 + 0.001).astype(np.float32)).cuda()
        weights.append(dapf8.w4_pack(q, sc))
        del q, sc
    res = {}
    for M in (1, 4, 16):
        x = torch.randn((M, K), device="cuda").to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

        def calls():
            for i in range(per_graph):
                pk, ps = weights[i % copies]
                dapf8.w4a16_gemv(x, pk, ps, N, out=y)

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            calls()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        for _ in range(max(1, warmup // per_graph)):
            g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(1, steps // per_graph)
        t0.record()
        for _ in range(n):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / (n * per_graph) * 1e3
        nbytes = N * K // 2 + N * (K // 128) * 4 + M * K * 2 + M * N * 2
        gbs = nbytes / (us * 1e-6) / 1e9
        res[f"M{M}"] = {"us": round(us, 2), "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "bytes": nbytes}
        del g
    # the read probe over the same weight bytes (copies rotating as above): what a kernel that only
    # streams the packed weights reaches at this size, launch and ramp included
    sink = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    flat = [pk.view(torch.uint8).reshape(-1) for pk, _ in weights]
    ms = graph_calls_ms([lambda i=i: dapf8.hbm_read_probe(flat[i % copies], 2048, sink=sink)
                         for i in range(per_graph)], reps=5)
    wbytes = flat[0].numel()
    ceiling = {"kernel": "hbm_read_probe over the packed weights (16-byte non-temporal loads)", "bytes": wbytes,
               "us_per_launch": round(ms * 1e3, 2), "gbs": round(wbytes / (ms * 1e-3) / 1e9, 1)}
    del sink, flat
    best = res["M1"]
    return {"metric": "INT4 weight-only decode GEMV GB/s (% HBM peak)", "value": best["gbs"], "unit": "GB/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(best["us"] * 1e-3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int4 weights, bf16 x",
            "data": "synthetic (uniform int4, random scales)",
            "config": {"workload": "w4a16_gemv_n28672_k8192", "N": N, "K": K, "parallelism": "single-gpu"},
            "roofline": {"bound": "hbm", "achieved": best["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": best["frac"], "traffic": measured_traffic("w4gemv", "w4gemv"), "algorithmic_bytes_per_launch": best["bytes"],
                         "avg_launch_ms": round(best["us"] * 1e-3, 5)},
            "batches": res, "read_ceiling": ceiling,
            "m1_time_over_ceiling": round(ceiling["us_per_launch"] / best["us"], 4)}


def bench_capacity(steps, warmup):
    """61-layer capacity workload: one tag check per step, then per layer append + attention.

    The FP8 pools of all 61 layers live in HBM at once (80 GB budget for K+V); layer 0 is filled
    from the drawn rows and the other layers hold copies of it (the data does not change the
    work; each layer's attention reads its own pool)."""
    import torch

    import decode_attention_paged_fp8_amd as dapf8
    import synth
    from gpu_pipeline import GpuState

    w = synth.make("capacity", seed=1)
    s = w.spec
    st = GpuState(w, "fp8")
    layers = [(st.k_pool, st.v_pool)]
    for _ in range(1, s.layers):
        layers.append((st.k_pool.clone(), st.v_pool.clone()))
    k_new, v_new, ids, pos = st.step_inputs()
    ws = dapf8.make_workspace(st.q, st.k_pool, st.v_pool, st.page_table, s.Dv)
    out = torch.empty((s.B, s.Hq, s.Dv), dtype=torch.bfloat16, device="cuda")
    abort = st.abort

    def verify():
        dapf8.kv_tag_verify(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, abort, s.page_size)

    def layer(kp, vp):
        dapf8.kv_append(k_new, v_new, kp, vp, st.page_table, ids, pos, st.k_scale, st.v_scale, abort)
        dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale, abort, out=out,
                                sm_scale=s.scale(), workspace=ws)

    def step():
        verify()
        for kp, vp in layers:
            layer(kp, vp)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    n_abort = int(abort.sum().item())
    e0, e1 = _events(1)[0]
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    # the check and one layer's attention on their own
    ev = _events(20)
    for i in range(20):
        ev[i][0].record()
        verify()
        ev[i][1].record()
    torch.cuda.synchronize()
    verify_ms = sum(a.elapsed_time(b) for a, b in ev) / 20
    ev = _events(61)
    for i, (kp, vp) in enumerate(layers):
        ev[i][0].record()
        dapf8.paged_decode_attn(st.q, kp, vp, st.page_table, st.seq_lens, st.k_scale, st.v_scale, abort, out=out,
                                sm_scale=s.scale(), workspace=ws)
        ev[i][1].record()
    torch.cuda.synchronize()
    attn_ms = sum(a.elapsed_time(b) for a, b in ev) / 61
    by = algorithmic_bytes(w, "fp8")
    gbs = by["total"] / (attn_ms * 1e-3) / 1e9
    worst_pages = -(-(s.len_range[1] + 1) // s.page_size)
    return {"metric": "decode-attn tokens/s + effective KV GB/s (% HBM peak), FP8 vs BF16 KV",
            "value": round(s.B / (step_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8-e4m3 KV, bf16 q/out", "data": "synthetic",
            "config": {"workload": "capacity_b64_61layers_80GB_budget", "batch": s.B, "layers": s.layers,
                       "pages_per_layer": w.num_pages, "attended_tokens_per_layer": by["tokens"],
                       "parallelism": "single-gpu"},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "algorithmic_bytes_per_launch": by["total"], "avg_launch_ms": round(attn_ms, 5)},
            "tag_check": {"verify_ms": round(verify_ms, 5), "attention_ms_per_layer": round(attn_ms, 5),
                          "verify_over_61_layers_attention": round(verify_ms / (61 * attn_ms), 5),
                          "aborted_requests": n_abort, "expected_aborted": int(w.expected_abort.sum())},
            "capacity": {"budget_bytes": s.budget_bytes, "worst_case_pages_per_sequence": worst_pages,
                         "fp8_pages_per_layer": synth.pages_per_layer(s, "fp8"),
                         "bf16_pages_per_layer": synth.pages_per_layer(s, "bf16"),
                         "fp8_admits_sequences": synth.pages_per_layer(s, "fp8") // worst_pages,
                         "bf16_admits_sequences": synth.pages_per_layer(s, "bf16") // worst_pages}}


def copy_calibration(mib: int, reps: int = 5) -> dict:
    """A plain elementwise kernel of known size (out = -x over `mib` MiB of fp32): its rocprofv3
    FETCH_SIZE / WRITE_SIZE per dispatch against the bytes it must read and write give the factor
    that turns those counters into HBM bytes; its event time gives a reachable streaming rate."""
    import torch

    n = mib * (1 << 20) // 4
    x = torch.empty(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    ev = _events(reps)
    for i in range(reps):
        ev[i][0].record()
        torch.neg(x if i % 2 == 0 else y, out=y if i % 2 == 0 else x)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev) / reps
    nbytes = n * 4
    del y
    # the read probe over the same bytes: 16-byte non-temporal loads, the load type of the attention
    # kernels -- the FETCH_SIZE calibration for them
    import decode_attention_paged_fp8_amd as dapf8

    buf = x.view(torch.uint8)
    sink = torch.empty(2048 * 256, dtype=torch.int32, device="cuda")
    for _ in range(reps):
        dapf8.hbm_read_probe(buf, 2048, sink=sink)
    torch.cuda.synchronize()
    del x, buf, sink
    torch.cuda.empty_cache()
    return {"kernel": "torch.neg fp32 (elementwise, reads and writes each byte once); hbm_read_probe over the "
                      "same bytes (non-temporal 16-byte loads)", "read_bytes": nbytes,
            "write_bytes": nbytes, "launches": reps + 1, "probe_launches": reps, "avg_ms": round(ms, 5),
            "gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


# ------------------------------------------------------------------------------------------------
# Offline summaries of rocprofv3 CSV output (no GPU): kernel statistics, and HBM traffic from a
# FETCH_SIZE pass and a WRITE_SIZE pass scaled by the copy calibration measured in the same pass.

def _csv_rows(d: str, suffix: str):
    import csv
    import glob

    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _short(name: str) -> str:
    """Kernel name without return type, namespace and argument list (template arguments kept)."""
    n = name[5:] if name.startswith("void ") else name
    depth = 0
    for i, c in enumerate(n):
        if c == "<":
            depth += 1
        elif c == ">":
            depth -= 1
        elif c == "(" and depth == 0:
            n = n[:i]
            break
    return n.replace("dapf8::", "")[:80]


def summarize_stats(d: str, cmd: str, out: str, bench_json: str | None, count_prefixes=None, title: str = ""):
    rows = _csv_rows(d, "kernel_stats.csv")
    head = "# rocprofv3 kernel statistics" + (f": {title}" if title else "")
    lines = [head, "", "Command (run from the repository root on one MI355X):", "",
             "```", cmd, "```", "", "| kernel | calls | avg us | min us | max us | total % |",
             "|---|---:|---:|---:|---:|---:|"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows[:14]:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    if bench_json and os.path.exists(bench_json):
        with open(bench_json) as fh:
            js = [ln for ln in fh if ln.startswith("{")]
        if js:
            b = json.loads(js[-1])
            rl = b.get("roofline", {})
            lines += ["", "bench line of the same run (under the profiler; avg_launch_ms is the bench's own "
                      "timing of the workload's unit on the library's stream):", "",
                      f"- avg_launch_ms: {rl.get('avg_launch_ms')}", f"- achieved GB/s: {rl.get('achieved')}",
                      f"- frac: {rl.get('frac')}", f"- ms_per_step: {b.get('ms_per_step')}"]
    if count_prefixes:
        # every dispatch of the run is in the kernel trace: count those whose name starts with each prefix
        trace = _csv_rows(d, "kernel_trace.csv")
        lines += ["", "Dispatches in the kernel trace of the whole run:", ""]
        for pre in count_prefixes:
            n = sum(1 for r in trace if _short(r["Kernel_Name"]).startswith(pre))
            lines.append(f"- `{pre}*`: {n}")
    lines += ["", f"library_source_sha256: `{kernel_source_hash(None)}`", ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def summarize_traffic(fetch_dir: str, write_dir: str, cmd_fetch: str, cmd_write: str, out: str, mib: int,
                      title: str = "GQA decode workload"):
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _csv_rows(d, "counter_collection.csv") if r.get("Counter_Name") == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        calib, probe, kv, acc = [], [], None, {}
        for r in rows:
            name, val = r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0  # KiB -> bytes
            if "read_probe_kernel" in name:
                # calibration dispatches read `mib` MiB; the GEMV leg's own probe over its weights is smaller
                if val > 0.25 * mib * (1 << 20):
                    probe.append(val)
            elif "transcode_kernel" in name:
                acc.setdefault(("transcode", "main"), []).append(val)
            elif "w4_gemv_kernel" in name:
                acc.setdefault(("w4gemv", "all"), []).append(val)
            elif "neg" in name and "elementwise" in name:
                calib.append(val)
            elif "attn_sk_kernel<" in name and name.split(">")[0].endswith("true"):
                kv = None  # the in-walk tag-check instantiation (ablation): not the measured call
            elif any(k in name for k in ("attn_sk_kernel<true", "attn_mfma_kernel<true", "attn_latent_kernel<",
                                         "attn_generic_kernel<true")):
                kv = "fp8"
                acc.setdefault(("fp8", "main"), []).append(val)
            elif any(k in name for k in ("attn_sk_kernel<false", "attn_mfma_kernel<false", "attn_generic_kernel<false")):
                kv = "bf16"
                acc.setdefault(("bf16", "main"), []).append(val)
            elif ("merge_sk_kernel" in name or "merge_kernel" in name) and kv is not None:
                acc.setdefault((kv, "merge"), []).append(val)
        if not calib:
            raise SystemExit(f"no calibration dispatch in the {counter} pass")
        # the GEMV leg runs the same number of calls at M = 1, 4, 16, in that order (one kernel for all M)
        gv = acc.pop(("w4gemv", "all"), [])
        if gv:
            if len(gv) % 3:
                raise SystemExit(f"{len(gv)} GEMV dispatches: not three equal batches")
            for i, m in enumerate(("M1", "M4", "M16")):
                acc[("w4gemv", m)] = gv[i * len(gv) // 3:(i + 1) * len(gv) // 3]
        known = mib * (1 << 20)
        # FETCH_SIZE: calibrated on the read probe (non-temporal loads, as the attention kernels use)
        # when it ran; WRITE_SIZE on the elementwise kernel's stores
        src = probe if (counter == "FETCH_SIZE" and probe) else calib
        per[counter] = dict(factor=sum(src) / len(src) / known, n_calib=len(src),
                            neg_factor=sum(calib) / len(calib) / known,
                            probe_factor=(sum(probe) / len(probe) / known) if probe else None,
                            avg={k: sum(v) / len(v) for k, v in acc.items()}, n={k: len(v) for k, v in acc.items()})
    ff, fw = per["FETCH_SIZE"]["factor"], per["WRITE_SIZE"]["factor"]
    lines = [f"# HBM traffic (rocprofv3 --pmc), {title}", "",
             "Two counter passes over the same bench run (one counter each), from the repository root:", "",
             "```", cmd_fetch, cmd_write, "```", "",
             f"Calibration over {mib} MiB of known bytes in the same passes: hbm_read_probe (16-byte "
             f"non-temporal loads, the load type of the attention kernels) reads {mib} MiB per dispatch, and "
             f"FETCH_SIZE reports {ff:.4f} x those bytes"
             + (f" (the elementwise kernel's ordinary loads: {per['FETCH_SIZE']['neg_factor']:.4f} x)"
                if per["FETCH_SIZE"]["probe_factor"] is not None else " (elementwise kernel; no probe ran)")
             + f"; a plain fp32 elementwise kernel (out = -x) writes {mib} MiB per dispatch and WRITE_SIZE "
             f"reports {fw:.4f} x.  The factors divide the measured kernels' counters.", "",
             "| unit | kernel | dispatches | FETCH_SIZE MB | WRITE_SIZE MB | HBM MB (scaled) |",
             "|---|---|---:|---:|---:|---:|"]
    totals = {}
    for kv in ("fp8", "bf16", "transcode", "w4gemv"):
        tot = 0.0
        for part in ("main", "merge", "M1", "M4", "M16"):
            f = per["FETCH_SIZE"]["avg"].get((kv, part))
            w = per["WRITE_SIZE"]["avg"].get((kv, part))
            if f is None or w is None:
                continue
            hb = f / ff + w / fw
            if part not in ("M4", "M16"):  # the GEMV's figure is the M = 1 call's, the one its roofline prices
                tot += hb
            lines.append(f"| {kv} | {part} | {per['FETCH_SIZE']['n'][(kv, part)]} | {f / 1e6:.2f} | {w / 1e6:.2f} | "
                         f"{hb / 1e6:.2f} |")
        if tot:
            totals[kv] = int(round(tot))
    lines += ["", "Machine-readable (bench.py fills roofline.traffic from these while the sources of the measured "
              "call -- kernels, shared headers, launch plan -- hash the same):", ""]
    # the workload is named by the summary file
    base = os.path.basename(out)
    workload = next((k for k, v in TRAFFIC_FILES.items() if v == base),
                    base.removeprefix("traffic_paged_decode_attn_").removesuffix(".md"))
    lines.append(f"kernel_source_sha256: {kernel_source_hash(workload)}")
    lines.append(f"fetch_factor: {ff:.5f}")
    lines.append(f"write_factor: {fw:.5f}")
    for kv, t in totals.items():
        lines.append(f"hbm_bytes_per_call[{kv}]: {t}")
    lines.append("")
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


# Counter passes of one workload: per-kernel averages over the dispatches of each pass, and the
# rocprofv3 derived metrics built from them (the expressions rocprofv3 --list-avail prints for
# MfmaUtil, VALUBusy, LdsUtil and LDSBankConflict).  MI355X: 256 CUs, 1024 SIMDs; the CSV sums
# GRBM_GUI_ACTIVE over its 8 instances (one per XCD), where the expressions take the maximum, so it
# is divided by 8 (it then matches the kernels' durations at 2.4 GHz).  SQ_WAVE_CYCLES and
# SQ_WAIT_INST_ANY count in units of 4 cycles, so their ratio needs no scaling.
CU_NUM, SIMD_NUM, GRBM_INSTANCES = 256, 1024, 8


def summarize_counters(dirs, cmds, out: str, title: str, kernels):
    per = {}  # kernel -> counter -> [values]
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            k = _short(r["Kernel_Name"])
            if not any(k.startswith(x) for x in kernels):
                continue
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 counters: {title}", "", "Counter passes (one rocprofv3 run each, from the repository root "
             "on one MI355X):", "", "```", *cmds, "```", "",
             "Per kernel, averages over its dispatches; GRBM_GUI_ACTIVE below is the per-XCD value (CSV sum / 8), "
             "about the kernel's duration in 2.4 GHz cycles.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x "
             f"{SIMD_NUM} SIMDs); VALU busy = SQ_ACTIVE_INST_VALU / ({CU_NUM} CUs x GRBM_GUI_ACTIVE); LDS busy = "
             "SQ_LDS_IDX_ACTIVE / (CUs x GRBM_GUI_ACTIVE); LDS bank-conflict cycles = SQ_LDS_BANK_CONFLICT / (CUs x "
             "GRBM_GUI_ACTIVE); waiting = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of wave time stalled on a "
             "dependency); instructions per wave = SQ_INSTS_* / SQ_WAVES.", "",
             "| kernel | dispatches | GRBM_GUI_ACTIVE / 8 | MFMA busy % | VALU busy % | LDS busy % | LDS bank-conflict % | waiting % | "
             "VALU / wave | MFMA / wave | LDS / wave | VMEM rd / wave | cvt / wave |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]

    def avg(c, name):
        v = c.get(name)
        return sum(v) / len(v) if v else None

    def pct(num, den):
        return "" if num is None or not den else f"{100.0 * num / den:.1f}"

    def per_wave(c, name):
        v, w = avg(c, name), avg(c, "SQ_WAVES")
        return "" if v is None or not w else f"{v / w:.0f}"

    for k, c in sorted(per.items()):
        g = avg(c, "GRBM_GUI_ACTIVE")
        g = g / GRBM_INSTANCES if g else g
        n = max(len(v) for v in c.values())
        lines.append(
            f"| `{k}` | {n} | {g:.4g} | {pct(avg(c, 'SQ_VALU_MFMA_BUSY_CYCLES'), g and g * SIMD_NUM)} | "
            f"{pct(avg(c, 'SQ_ACTIVE_INST_VALU'), g and g * CU_NUM)} | {pct(avg(c, 'SQ_LDS_IDX_ACTIVE'), g and g * CU_NUM)} | "
            f"{pct(avg(c, 'SQ_LDS_BANK_CONFLICT'), g and g * CU_NUM)} | "
            f"{pct(avg(c, 'SQ_WAIT_INST_ANY'), avg(c, 'SQ_WAVE_CYCLES'))} | {per_wave(c, 'SQ_INSTS_VALU')} | "
            f"{per_wave(c, 'SQ_INSTS_MFMA')} | {per_wave(c, 'SQ_INSTS_LDS')} | {per_wave(c, 'SQ_INSTS_VMEM_RD')} | "
            f"{per_wave(c, 'SQ_INSTS_VALU_CVT')} |")
    lines += ["", "Raw averages per dispatch:", ""]
    for k, c in sorted(per.items()):
        lines.append(f"- `{k}`: " + ", ".join(f"{n}={sum(v) / len(v):.6g}" for n, v in sorted(c.items())))
    lines += ["", f"kernel_source_sha256: `{kernel_source_hash()}`", ""]
    with open(out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--split", type=int, default=0, help="split_tokens (0 = library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="default workload only: skip the read-ceiling, long-context and capacity tag-check legs")
    ap.add_argument("--no-graph", action="store_true", help="time the step with eager launches only")
    ap.add_argument("--no-tag-check", action="store_true",
                    help="GQA step with the no-op tracker (no kv_tag_verify, no abort mask) in place of the checked one")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--workload", default="gqa", choices=["gqa", "long", "capacity", "shared_kv", "transcode", "pages", "w4gemv"],
                    help="gqa (default, the headline line), long, capacity (61 layers), shared_kv, transcode, "
                         "pages, w4gemv")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run a plain elementwise kernel over this many MiB first (counter calibration)")
    ap.add_argument("--summarize", choices=["stats", "traffic", "counters"],
                    help="offline: summarise rocprofv3 CSV output into a profiles/ markdown file")
    ap.add_argument("--prof-dir", nargs="+", help="rocprofv3 output dir(s) (stats: 1; traffic: fetch, write)")
    ap.add_argument("--prof-cmd", nargs="+", help="the command(s) that produced them")
    ap.add_argument("--bench-json", help="stats: the bench output of the profiled run")
    ap.add_argument("--out", help="summary file to write")
    ap.add_argument("--title", default="", help="counters: what the summary covers")
    ap.add_argument("--kernels", nargs="+", default=["attn_", "merge_"],
                    help="counters: kernel name prefixes; stats with --count-dispatches: prefixes to count")
    ap.add_argument("--count-dispatches", action="store_true",
                    help="stats: also count the trace's dispatches of each --kernels prefix")
    args = ap.parse_args()
    if args.summarize == "stats":
        summarize_stats(args.prof_dir[0], args.prof_cmd[0], args.out, args.bench_json,
                        args.kernels if args.count_dispatches else None, args.title)
        return
    if args.summarize == "counters":
        summarize_counters(args.prof_dir, args.prof_cmd, args.out, args.title, args.kernels)
        return
    if args.summarize == "traffic":
        summarize_traffic(args.prof_dir[0], args.prof_dir[1], args.prof_cmd[0], args.prof_cmd[1], args.out,
                          args.copy_calibration_mib, args.title or "GQA decode workload")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    torch.cuda.set_device(0)
    calib = copy_calibration(args.copy_calibration_mib) if args.copy_calibration_mib > 0 else None
    if args.workload == "capacity":
        print(json.dumps(bench_capacity(args.steps, args.warmup)), flush=True)
        return
    if args.workload == "w4gemv":
        print(json.dumps(bench_w4gemv(args.steps, args.warmup)), flush=True)
        return
    if args.workload == "pages":
        print(json.dumps(bench_pages(args.steps, args.warmup)), flush=True)
        return
    if args.workload == "transcode":
        print(json.dumps(bench_transcode(args.steps, args.warmup)), flush=True)
        return
    if args.workload in ("long", "shared_kv"):
        print(json.dumps(bench_attention_only(args.workload, args.steps, args.warmup)), flush=True)
        return
    w = synth.make("gqa", seed=args.seed)
    s = w.spec
    res = {}
    for kv in ("fp8", "bf16"):
        res[kv] = run_kv(w, kv, args.steps, args.warmup, args.split, use_graph=not args.no_graph,
                         no_tag_check=args.no_tag_check)
        res[kv]["bytes"] = algorithmic_bytes(w, kv)
    f = res["fp8"]
    fb = f["bytes"]["total"]
    achieved = fb / (f["attn_ms"] * 1e-3) / 1e9
    line = {
        "metric": "decode-attn tokens/s + effective KV GB/s (% HBM peak), FP8 vs BF16 KV",
        "value": round(s.B / (f["step_ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 KV, bf16 q/out, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) bf16 K/V with 1% x20 outlier channels)",
        "config": {"workload": "gqa_decode_b32_h32kv8_d128_p16_len1024-8192_append1", "batch": s.B,
                   "q_heads": s.Hq, "kv_heads": s.Hkv, "head_dim": s.Dk, "page_size": s.page_size,
                   "attended_tokens": f["bytes"]["tokens"], "split_tokens": f["split"],
                   "variant": f["variant"], "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "paged_decode_attn call (attn_sk_kernel + merge_sk_kernel), back-to-back calls "
                               "replayed from a HIP graph",
                     "algorithmic_bytes_per_launch": fb, "avg_launch_ms": round(f["attn_ms"], 5)},
        "fp8": {"step_ms": round(f["step_ms"], 5), "eager_step_ms": round(f["eager_step_ms"], 5),
                "graph_step_ms": None if f["graph_step_ms"] is None else round(f["graph_step_ms"], 5),
                "attn_ms": round(f["attn_ms"], 5), "attn_eager_event_ms": round(f["attn_eager_event_ms"], 5),
                "verify_ms": None if f["verify_ms"] is None else round(f["verify_ms"], 5),
                "append_ms": round(f["append_ms"], 5),
                "kv_gbs": round(f["bytes"]["kv"] / (f["attn_ms"] * 1e-3) / 1e9, 1),
                "kv_tokens_per_s": round(f["bytes"]["tokens"] / (f["attn_ms"] * 1e-3), 1)},
        "bf16_twin": {},
        "verify_over_attention": None if f["verify_ms"] is None else round(f["verify_ms"] / f["attn_ms"], 4),
    }
    # informational: how far the FP8-KV outputs lie from the BF16-KV ones on the same inputs
    d = (f["out"] - res["bf16"]["out"]).abs()
    line["fp8_vs_bf16_output"] = {"max_abs_diff": round(float(d.max()), 6),
                                  "max_abs_bf16_output": round(float(res["bf16"]["out"].abs().max()), 6),
                                  "mean_abs_diff": round(float(d.mean()), 7)}
    if f["untracked_step_ms"] is not None:
        # the same step with the no-op tracker (no tag check, no abort mask), replayed from a graph
        line["fp8"]["no_op_tracker_step_ms"] = round(f["untracked_step_ms"], 5)
    if f["separate_step_ms"] is not None:
        # the same step as three calls (kv_tag_verify, kv_append, paged_decode_attn), graph-replayed
        line["fp8"]["separate_step_ms"] = round(f["separate_step_ms"], 5)
        line["fp8"]["verify_append_ms"] = round(f["verify_append_ms"], 5)
    line["fp8"]["step"] = ("no-op tracker: kv_append + paged_decode_attn, no tag check, no abort mask"
                           if args.no_tag_check else
                           "kv_tag_verify_append (tag check + guarded append, one launch) + paged_decode_attn")
    b = res["bf16"]
    bb = b["bytes"]["total"]
    line["bf16_twin"] = {"tokens_per_s": round(s.B / (b["step_ms"] * 1e-3), 1), "step_ms": round(b["step_ms"], 5),
                         "attn_ms": round(b["attn_ms"], 5), "achieved_gbs": round(bb / (b["attn_ms"] * 1e-3) / 1e9, 1),
                         "frac": round(bb / (b["attn_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "variant": b["variant"], "split_tokens": b["split"]}
    if f.get("checked"):
        c = f["checked"]
        line["fused_check_ablation"] = {
            "separate_check": {"verify_ms": round(f["verify_ms"], 5), "attn_ms": round(f["attn_ms"], 5),
                               "step_ms": None if f["separate_step_ms"] is None else round(f["separate_step_ms"], 5),
                               "step_ms_check_and_append_one_launch": round(f["step_ms"], 5)},
            "check_in_page_walk": {"attn_ms": round(c["attn_ms"], 5),
                                   "step_ms": None if c["graph_step_ms"] is None else round(c["graph_step_ms"], 5)},
            "note": "in-walk step = unguarded append + checked attention; separate = verify + guarded append + "
                    "attention"}
    if not args.no_legs:
        line["stream_ceiling"] = stream_ceiling(fb)
        line["long_context"] = long_context_leg()
        line["tiny_mha_latency"] = tiny_mha_leg()
        line["capacity_tag_check"] = capacity_tag_check_leg()
    line["roofline"]["traffic"] = measured_traffic("gqa", "fp8")
    line["bf16_twin"]["traffic"] = measured_traffic("gqa", "bf16")
    if calib is not None:
        line["copy_calibration"] = calib
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
