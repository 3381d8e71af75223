"""Slots the attention must not use hold NaN codes.

Every slot of the pools outside the attended tokens -- the tail of each sequence's last page, the
pages a 32-token window or a 64-token page reaches past the end, every page no request owns -- is
set to NaN (e4m3 0x7F or bf16 0x7FC0) before the real rows are appended, so a kernel that multiplies
a stale value by a zero weight (NaN x 0 = NaN) or lets it into a maximum shows up as a non-finite or
wrong output.  Covers the stream-K kernel (FP8 and BF16), the latent kernel (which zeroes a last
page's stale rows in LDS) and the generic kernel, each against the oracle at the parity bar.
"""
import pytest
import torch

import synth
from gpu_pipeline import GpuState, check_close, out_to_f64
from oracle_pipeline import oracle_step

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu

CASES = [
    ("gqa", "fp8", dict(B=6, len_range=(1, 700))),
    ("gqa", "bf16", dict(B=6, len_range=(1, 700))),
    ("shared_kv", "fp8", dict(B=3, len_range=(1, 300))),
    ("tiny_mha", "fp8", {}),
]


def _poison(t: torch.Tensor):
    if t is None:
        return
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(0x7FC0)
    else:
        t.view(torch.uint8).fill_(0x7F)


@pytest.mark.parametrize("name,kv,kw", CASES)
def test_nan_in_unused_slots_never_reaches_the_output(name, kv, kw):
    print(f"\n[case] stale NaN slots {name} {kv} {kw}", flush=True)
    w = synth.make(name, seed=4, **kw)
    ref = oracle_step(w, kv)
    st = GpuState(w, kv)
    _poison(st.k_pool)
    _poison(st.v_pool)
    st.fill()  # the attended rows again; every other slot keeps its NaN
    out, abort = st.step()
    torch.cuda.synchronize()
    assert (abort.cpu().numpy() == ref["abort"]).all()
    worst, tol = check_close(out_to_f64(out), ref["out"], w.spec.out_dt)
    print(f"  max|err| {worst:.3e} (tol {tol:.3e})")
