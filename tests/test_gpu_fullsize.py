"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark uses.

The oracle cannot redo a whole full-size step in seconds, so it checks sampled requests: for each
sampled request it rebuilds that request alone in a compact pool (oracle_subproblem) with scales the
oracle computed over the entire fill, and the GPU's pool pages and output rows for that request
must match (codes bit-exact, outputs within the bar).  The abort mask is checked for the whole
batch, and properties that hold at any size (finite outputs, zero rows for aborted requests) for
every row.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_pipeline import GpuState, check_close, out_to_f64, pool_to_numpy
from oracle_pipeline import oracle_subproblem

pytestmark = pytest.mark.gpu


def _run(name, kv, sample, heads=None, **over):
    w = synth.make(name, seed=1, **over)
    s = w.spec
    ak = np.zeros(s.Hkv, np.float32)
    av = np.zeros(s.Hkv, np.float32)

    def feed(b, k, v):  # the oracle's own scale pass over the whole fill
        if k.shape[0]:
            oracle.kv_absmax_update(k, ak)
            if v is not None:
                oracle.kv_absmax_update(v, av)

    st = GpuState(w, kv, on_rows=feed if kv == "fp8" else None)
    ks = oracle.scale_from_absmax(ak) if kv == "fp8" else None
    vs = (None if s.shared_kv else oracle.scale_from_absmax(av)) if kv == "fp8" else None
    if kv == "fp8":
        assert (st.k_scale.cpu().numpy() == ks).all()
        if vs is not None:
            assert (st.v_scale.cpu().numpy() == vs).all()
    verify = s.stale != "none"
    out, abort = st.step(verify=True, split_tokens=s.split_tokens)
    torch.cuda.synchronize()
    ab = abort.cpu().numpy()
    ref_ab = oracle.kv_tag_verify(w.page_table, w.expected_tags, w.seq_lens, w.live_tags, page_size=s.page_size)
    assert (ab == ref_ab).all() and (ab == w.expected_abort).all()
    o = out_to_f64(out)
    assert np.isfinite(o).all()
    assert (o[ab.astype(bool)] == 0).all()
    kpool = st.k_pool
    vpool = st.v_pool
    worst = 0.0
    for b in sample(w):
        print(f"  [row] {name} {kv} b={b} L={int(w.seq_lens[b])} abort={int(ab[b])}", flush=True)
        kp, vp, compact, ref = oracle_subproblem(w, b, kv, ks, vs, abort_b=int(ab[b]), heads=heads)
        pages = torch.from_numpy(w.page_table[b, :w.n_pages(b)].astype(np.int64)).cuda()
        gk = pool_to_numpy(kpool.index_select(0, pages))
        assert (gk == kp[compact]).all(), "K pool pages differ"
        if vp is not None:
            gv = pool_to_numpy(vpool.index_select(0, pages))
            assert (gv == vp[compact]).all(), "V pool pages differ"
        hs = list(range(s.Hq)) if heads is None else list(heads)
        e, tol = check_close(o[b, hs], ref, s.out_dt)
        worst = max(worst, e)
    print(f"  {name} {kv}: worst |err| {worst:.3e} (abort {int(ab.sum())}/{len(ab)})", flush=True)
    return w, st


def _short_long(w, k=2):
    order = np.argsort(w.seq_lens)
    return sorted(set([int(order[0]), int(order[-1])] + [int(x) for x in order[len(order) // 2:len(order) // 2 + k]]))


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_gqa_full(kv):
    print("\n[case] gqa full", kv, flush=True)
    _run("gqa", kv, lambda w: _short_long(w))


def _short_mid_long(w):
    """The shortest, the middle and the longest request (the longest is split over the most
    workers, so its merge combines the most partial results)."""
    order = np.argsort(w.seq_lens)
    return sorted(set([int(order[0]), int(order[len(order) // 2]), int(order[-1])]))


def test_long_context_full():
    print("\n[case] long full fp8", flush=True)
    _run("long", "fp8", _short_mid_long, heads=[0, 7, 9, 37, 56, 63])


def test_capacity_one_layer_full():
    print("\n[case] capacity layer 0 fp8", flush=True)

    def pick(w):
        ab = [b for b, _ in w.stale_refs]
        return sorted(set([ab[0], int(np.argmax(w.seq_lens)), (ab[0] + 1) % w.B]))

    _run("capacity", "fp8", pick, heads=[0, 5, 31])


def test_shared_kv_full():
    print("\n[case] shared_kv full fp8", flush=True)
    _run("shared_kv", "fp8", _short_mid_long, heads=[0, 1, 17, 64, 100, 127])
