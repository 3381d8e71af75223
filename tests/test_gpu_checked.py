"""GPU parity of paged_decode_attn_checked (page-tag check inside the attention page walk) against
the oracle's separate check followed by its attention: the abort mask bit-exact, aborted rows exact
zeros, every other row within the attention bar; and against the library's own unfused path."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_pipeline import GpuState, check_close, out_to_f64, t_int
from oracle_pipeline import kv_code, oracle_fill

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu


def _run(w, kv, out_dtype, mutate=None):
    s = w.spec
    # GPU: fill, unguarded append, then (optionally) corrupt tables, then the checked attention
    st = GpuState(w, kv)
    if s.append:
        k_new, v_new, ids, pos = st.step_inputs()
        dapf8.kv_append(k_new, v_new, st.k_pool, st.v_pool, st.page_table, ids, pos, st.k_scale, st.v_scale)
    pt, lens, exp, live = w.page_table.copy(), w.seq_lens.copy(), w.expected_tags.copy(), w.live_tags.copy()
    if mutate is not None:
        mutate(pt, lens, exp, live)
    g_pt, g_lens = t_int(pt), t_int(lens)
    g_exp, g_live = t_int(exp, torch.uint32), t_int(live, torch.uint32)
    mask = torch.full((w.B,), 7, dtype=torch.uint8, device="cuda")
    out = dapf8.paged_decode_attn_checked(st.q, st.k_pool, st.v_pool, g_pt, g_lens, g_exp, g_live, mask, st.k_scale,
                                          st.v_scale, out_dtype=out_dtype, sm_scale=s.scale())
    # unfused library path on the same (corrupted) tables
    ref_mask = torch.zeros_like(mask)
    dapf8.kv_tag_verify(g_pt, g_exp, g_lens, g_live, ref_mask, s.page_size)
    out2 = dapf8.paged_decode_attn(st.q, st.k_pool, st.v_pool, g_pt, g_lens, st.k_scale, st.v_scale, ref_mask,
                                   out_dtype=out_dtype, sm_scale=s.scale())
    torch.cuda.synchronize()
    # oracle: fill, unguarded append, verify on the corrupted tables, attention with that mask
    kd = kv_code(kv)
    kp, vp, ks, vs = oracle_fill(w, kv)
    if s.append:
        k_new, v_new, ids, pos = w.step_tokens(0)
        oracle.kv_append(k_new, v_new, kp, vp, kd, w.page_table, ids, pos, ks, vs, None, page_size=s.page_size,
                         num_pages=w.num_pages)
    abort = oracle.kv_tag_verify(pt, exp, lens, live, page_size=s.page_size)
    ref = oracle.paged_decode_attn(w.q, kp, vp, kd, pt, lens, ks, vs, abort, sm_scale=s.scale(), Hkv=s.Hkv, Dk=s.Dk,
                                   Dv=s.Dv, page_size=s.page_size)
    return mask.cpu().numpy(), out_to_f64(out), ref_mask.cpu().numpy(), out_to_f64(out2), abort, ref


def _check(w, kv, out_dtype, mutate=None):
    got_mask, got, lib_mask, lib_out, abort, ref = _run(w, kv, out_dtype, mutate)
    assert (got_mask == abort).all(), (got_mask, abort)
    assert (lib_mask == abort).all()
    bad = abort.astype(bool)
    assert (got[bad] == 0.0).all()
    tol = "f32" if out_dtype == torch.float32 else "bf16"
    check_close(got, ref, tol)
    check_close(got, lib_out, tol)
    return int(bad.sum())


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_checked_matches_separate_check_stale_tags(kv, out_dtype):
    print(f"\n[case] checked stale-tags {kv} {out_dtype}", flush=True)
    w = synth.make("capacity", seed=3, B=12, len_range=(200, 1500), stale_rate=2e-2, layers=1, budget_bytes=None)
    n_bad = _check(w, kv, out_dtype)
    print(f"  aborted {n_bad} of {w.B}")
    assert 0 < n_bad < w.B


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_checked_bad_ids_and_lengths(kv):
    print(f"\n[case] checked bad ids / lengths {kv}", flush=True)
    w = synth.make("gqa", seed=5, B=10, len_range=(1, 900))
    max_len = w.page_table.shape[1] * w.spec.page_size

    def mutate(pt, lens, exp, live):
        lens[1] = -1                    # negative length
        lens[2] = max_len + 1           # more tokens than the page table holds
        n3 = (int(lens[3]) + 15) // 16
        pt[3, n3 - 1] = -5              # negative page id on the last page
        n4 = (int(lens[4]) + 15) // 16
        pt[4, n4 // 2] = w.num_pages + 3  # id past the pool
        live[pt[5, 0]] ^= 1             # a live tag moved on (the page was reallocated)
        lens[6] = 0                     # empty request: not aborted, zeros
        n7 = (int(lens[7]) + 15) // 16
        if n7 < pt.shape[1]:
            pt[7, n7] = -9              # past the request's pages: ignored

    _check(w, kv, torch.bfloat16, mutate)


def test_checked_clean_batch_gqa_shape():
    print("\n[case] checked clean gqa", flush=True)
    w = synth.make("gqa", seed=2, B=8, len_range=(30, 2000))
    assert _check(w, "fp8", torch.bfloat16) == 0


def test_checked_rejects_other_shapes():
    w = synth.make("shared_kv", seed=1, B=2, len_range=(10, 100))
    st = GpuState(w, "fp8")
    m = torch.zeros(w.B, dtype=torch.uint8, device="cuda")
    with pytest.raises(dapf8.DapfError):
        dapf8.paged_decode_attn_checked(st.q, st.k_pool, st.k_pool, st.page_table, st.seq_lens, st.expected_tags,
                                        st.live_tags, m, st.k_scale, st.k_scale)
