"""GPU parity of kv_tag_verify_append, the page-tag check and the append of the unaborted requests'
tokens in one launch: its abort mask and both pools must equal, bit for bit, the oracle's
kv_tag_verify followed by kv_append with that mask -- and the library's two separate calls.

Cases: planted stale tags, bad lengths and page ids outside the pool; tokens with out-of-range
sequence ids, positions and page entries; zero to several tokens per request; FP8 and BF16
pools; fp32 and bf16 inputs; shared-KV pools; wide page tables (the 1024-thread check); and the
slow path (more than 64 tokens of one request, or more tokens than the fast scan covers)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_pipeline import pool_to_numpy, t_act, t_int

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu


def _make(rng, B, Hkv, P, Dk, Dv, stride, tok_counts, kv, in_dt, shared=False, stale=2):
    """A self-consistent case: every (request, page slot) owns a distinct pool page, so no two
    tokens name one slot; then planted faults."""
    npg = B * stride + 7
    perm = rng.permutation(npg).astype(np.int32)
    pt = perm[:B * stride].reshape(B, stride).copy()
    live = rng.integers(0, 2**32, size=npg, dtype=np.uint64).astype(np.uint32)
    exp = live[pt].astype(np.uint32)
    lens = rng.integers(0, stride * P + 1, size=B).astype(np.int32)
    for b in rng.choice(B, size=min(stale, B), replace=False):  # stale tag inside the request's pages
        n = -(-int(lens[b]) // P)
        if n:
            exp[b, int(rng.integers(0, n))] ^= np.uint32(1 << int(rng.integers(0, 32)))
    if B > 3:
        lens[3] = stride * P + 1   # bad length: aborts
        pt[2, stride - 1] = npg + 5  # out of the pool, past request 2's pages unless it is full
    ids, pos = [], []
    for b in range(B):
        slots = rng.permutation(stride * P)[:tok_counts[b]]
        ids += [b] * len(slots)
        pos += [int(x) for x in slots]
    order = rng.permutation(len(ids))
    ids = np.array(ids, np.int32)[order] if ids else np.zeros(0, np.int32)
    pos = np.array(pos, np.int32)[order] if pos else np.zeros(0, np.int32)
    if len(ids) > 3:  # tokens the append must skip
        ids[0] = B + 2
        pos[1] = stride * P + 3
        ids[2] = -1
    T = len(ids)
    k_new = rng.standard_normal((T, Hkv, Dk)).astype(np.float32) * 3
    v_new = None if shared else rng.standard_normal((T, Hkv, Dv)).astype(np.float32) * 3
    if in_dt == "bf16":
        k_new = synth.to_bf16_bits(k_new)
        v_new = None if shared else synth.to_bf16_bits(v_new)
    ks = (rng.random(Hkv) * 0.02 + 0.003).astype(np.float32)
    vs = (rng.random(Hkv) * 0.02 + 0.003).astype(np.float32)
    if kv == "fp8":
        kpool = rng.integers(0, 256, size=(npg, Hkv, Dk // 64, P, 64), dtype=np.uint8)
        vpool = None if shared else rng.integers(0, 256, size=(npg, Hkv, Dv, P), dtype=np.uint8)
    else:
        kpool = rng.integers(0, 2**16, size=(npg, Hkv, Dk // 32, P, 32), dtype=np.uint16)
        vpool = None if shared else rng.integers(0, 2**16, size=(npg, Hkv, Dv, P), dtype=np.uint16)
    return dict(pt=pt, exp=exp, lens=lens, live=live, ids=ids, pos=pos, k_new=k_new, v_new=v_new, ks=ks, vs=vs,
                kpool=kpool, vpool=vpool, P=P, npg=npg, kv=kv, B=B)


def _t_pool(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(a.copy()).cuda()


def _run(c):
    kv_dt = oracle.KV_FP8 if c["kv"] == "fp8" else oracle.KV_BF16
    ref_abort = oracle.kv_tag_verify(c["pt"], c["exp"], c["lens"], c["live"], page_size=c["P"])
    rk, rv = c["kpool"].copy(), None if c["vpool"] is None else c["vpool"].copy()
    if len(c["ids"]):
        oracle.kv_append(c["k_new"], c["v_new"], rk, rv, kv_dt, c["pt"], c["ids"], c["pos"], c["ks"], c["vs"],
                         ref_abort, page_size=c["P"], num_pages=c["npg"])
    args = dict(page_table=t_int(c["pt"]), expected_tags=t_int(c["exp"], torch.uint32), seq_lens=t_int(c["lens"]),
                live_tags=t_int(c["live"], torch.uint32))
    kn, vn = t_act(c["k_new"]), None if c["v_new"] is None else t_act(c["v_new"])
    ids, pos = t_int(c["ids"]), t_int(c["pos"])
    ks, vs = torch.from_numpy(c["ks"]).cuda(), torch.from_numpy(c["vs"]).cuda()
    vs_arg = None if c["vpool"] is None else vs
    # fused
    gk, gv = _t_pool(c["kpool"]), _t_pool(c["vpool"])
    abort = torch.full((c["B"],), 7, dtype=torch.uint8, device="cuda")
    dapf8.kv_tag_verify_append(args["page_table"], args["expected_tags"], args["seq_lens"], args["live_tags"], abort,
                               kn, vn, gk, gv, ids, pos, ks, vs_arg)
    # the two separate calls
    sk, sv = _t_pool(c["kpool"]), _t_pool(c["vpool"])
    abort2 = torch.full((c["B"],), 7, dtype=torch.uint8, device="cuda")
    dapf8.kv_tag_verify(args["page_table"], args["expected_tags"], args["seq_lens"], args["live_tags"], abort2, c["P"])
    if len(c["ids"]):
        dapf8.kv_append(kn, vn, sk, sv, args["page_table"], ids, pos, ks, vs_arg, abort2)
    torch.cuda.synchronize()
    got_abort = abort.cpu().numpy()
    assert (got_abort == ref_abort).all()
    assert (abort2.cpu().numpy() == ref_abort).all()
    for name, got, ref, orig in (("separate K", sk, rk, c["kpool"]), ("fused K", gk, rk, c["kpool"]),
                                 ("separate V", sv, rv, c["vpool"]), ("fused V", gv, rv, c["vpool"])):
        if ref is None:
            continue
        g = pool_to_numpy(got)
        bad = np.argwhere(g != ref)
        assert bad.size == 0, (f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}: got "
                               f"{[int(g[tuple(x)]) for x in bad[:3]]} want {[int(ref[tuple(x)]) for x in bad[:3]]} "
                               f"(before {[int(orig[tuple(x)]) for x in bad[:3]]}); pages touched by the oracle "
                               f"{sorted(set(np.argwhere(ref != orig)[:, 0].tolist()))[:12]}")
    return ref_abort


@pytest.mark.parametrize("kv,in_dt,shared", [("fp8", "bf16", False), ("fp8", "f32", False), ("bf16", "bf16", False),
                                             ("bf16", "f32", False), ("fp8", "bf16", True)])
def test_verify_append_matches_oracle(kv, in_dt, shared):
    print(f"\n[case] verify+append kv={kv} in={in_dt} shared={shared}", flush=True)
    rng = np.random.default_rng(hash((kv, in_dt, shared)) % 2**32)
    outcomes = set()
    for trial in range(4):
        B = int(rng.integers(4, 40))
        counts = rng.integers(0, 4, size=B)
        c = _make(rng, B, Hkv=int(rng.choice([1, 2, 8])), P=int(rng.choice([1, 16, 64])), Dk=int(rng.choice([64, 128])),
                  Dv=int(rng.choice([16, 128])), stride=int(rng.integers(2, 12)), tok_counts=counts, kv=kv,
                  in_dt=in_dt, shared=shared)
        outcomes |= set(int(x) for x in _run(c))
    assert outcomes == {0, 1}


def test_verify_append_decode_step_shape():
    """The GQA decode step's shape: 32 requests, one new token each, 8 KV heads, D 128, P 16."""
    print("\n[case] verify+append decode step B=32", flush=True)
    rng = np.random.default_rng(5)
    c = _make(rng, 32, Hkv=8, P=16, Dk=128, Dv=128, stride=140, tok_counts=np.ones(32, int), kv="fp8", in_dt="bf16")
    _run(c)


def test_verify_append_wide_tables():
    """pt_stride above 1024: the 1024-thread check with its first pass loaded up front."""
    print("\n[case] verify+append wide tables", flush=True)
    rng = np.random.default_rng(6)
    c = _make(rng, 3, Hkv=2, P=1, Dk=64, Dv=16, stride=2600, tok_counts=np.array([3, 1, 2]), kv="fp8", in_dt="f32",
              stale=1)
    _run(c)


@pytest.mark.parametrize("counts", ["many_per_request", "long_token_list"])
def test_verify_append_slow_path(counts):
    """More than 64 new tokens of one request, and more tokens than the fast scan covers (1024):
    the workgroup rescans the token list."""
    print(f"\n[case] verify+append slow path {counts}", flush=True)
    rng = np.random.default_rng(7 if counts == "many_per_request" else 8)
    B = 6
    tok = np.array([90, 2, 0, 5, 1, 70]) if counts == "many_per_request" else np.full(B, 200)
    c = _make(rng, B, Hkv=2, P=16, Dk=64, Dv=32, stride=16, tok_counts=tok, kv="fp8", in_dt="bf16")
    assert len(c["ids"]) == tok.sum()
    _run(c)


def test_verify_append_no_tokens_is_the_check():
    print("\n[case] verify+append T=0", flush=True)
    rng = np.random.default_rng(9)
    c = _make(rng, 9, Hkv=2, P=16, Dk=64, Dv=32, stride=6, tok_counts=np.zeros(9, int), kv="fp8", in_dt="bf16")
    _run(c)


def test_verify_append_graph_replays_match_eager():
    """The one-launch check and append captured in a HIP graph: every replay, with eager work and
    synchronisations between replays, leaves the same mask and pools as the eager call."""
    print("\n[case] verify+append graph replays", flush=True)
    rng = np.random.default_rng(10)
    c = _make(rng, 12, Hkv=2, P=16, Dk=64, Dv=32, stride=8, tok_counts=rng.integers(0, 3, size=12), kv="fp8",
              in_dt="bf16")
    pt, et = t_int(c["pt"]), t_int(c["exp"], torch.uint32)
    lens, live = t_int(c["lens"]), t_int(c["live"], torch.uint32)
    kn, vn = t_act(c["k_new"]), t_act(c["v_new"])
    ids, pos = t_int(c["ids"]), t_int(c["pos"])
    ks, vs = torch.from_numpy(c["ks"]).cuda(), torch.from_numpy(c["vs"]).cuda()
    ek, ev = _t_pool(c["kpool"]), _t_pool(c["vpool"])
    eab = torch.full((c["B"],), 7, dtype=torch.uint8, device="cuda")
    dapf8.kv_tag_verify_append(pt, et, lens, live, eab, kn, vn, ek, ev, ids, pos, ks, vs)
    gk, gv = _t_pool(c["kpool"]), _t_pool(c["vpool"])
    gab = torch.full((c["B"],), 7, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dapf8.kv_tag_verify_append(pt, et, lens, live, gab, kn, vn, gk, gv, ids, pos, ks, vs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dapf8.kv_tag_verify_append(pt, et, lens, live, gab, kn, vn, gk, gv, ids, pos, ks, vs)
    for rep in range(4):
        gk.copy_(_t_pool(c["kpool"]))
        gv.copy_(_t_pool(c["vpool"]))
        gab.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(gab, eab), rep
        assert torch.equal(gk.view(torch.uint8), ek.view(torch.uint8)), rep
        assert torch.equal(gv.view(torch.uint8), ev.view(torch.uint8)), rep
