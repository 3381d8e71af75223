"""GPU parity of the generic (vector-ALU) attention kernel on shapes outside the matrix-core kernels:
grouped query heads (G = 2, 3, 8, 12: one or two head groups per workgroup), head dims from 64 to
1024, odd page sizes (1, 7, 24) where tokens of one load would straddle pages, shared-KV rows with a
V width that is not a multiple of 64, FP8 and BF16 storage, one partition or several (library choice
and explicit splits), each against the oracle at the parity bar."""
import pytest
import torch

import synth
from gpu_pipeline import GpuState, check_close, out_to_f64
from oracle_pipeline import oracle_step

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu

BASE = dict(lens=None, num_pages=None, stale="none")
SHAPES = [
    # (overrides of the tiny MHA workload, split_tokens values)
    (dict(B=5, Hq=12, Hkv=4, Dk=64, Dv=64, page_size=16, len_range=(1, 900)), (0, 96)),
    (dict(B=3, Hq=8, Hkv=1, Dk=192, Dv=80, page_size=7, len_range=(1, 500)), (0, 64)),
    (dict(B=2, Hq=24, Hkv=2, Dk=128, Dv=96, page_size=24, shared_kv=True, len_range=(30, 700)), (0, 256)),
    (dict(B=3, Hq=4, Hkv=2, Dk=64, Dv=32, page_size=1, len_range=(1, 200)), (0, 32)),
    (dict(B=2, Hq=2, Hkv=2, Dk=1024, Dv=1024, page_size=16, len_range=(100, 400)), (0, 128)),
]


@pytest.mark.parametrize("kw,splits", SHAPES)
@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_generic_kernel_parity(kw, splits, kv):
    print(f"\n[case] generic {kw} {kv}", flush=True)
    kw2 = dict(BASE)
    kw2.update(kw)
    w = synth.make("tiny_mha", seed=7, **kw2)
    s = w.spec
    for sp in splits:
        name, _ = dapf8.paged_decode_attn_variant(s.B, s.Hq, s.Hkv, s.Dk, s.Dv, s.page_size, w.pt_stride, sp,
                                                  0 if kv == "fp8" else 1, s.shared_kv)
        assert name == "valu_generic", name
    ref = oracle_step(w, kv)
    st = GpuState(w, kv)
    for sp in splits:
        for od, tol in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            out, abort = st.step(split_tokens=sp, out_dtype=od)
            torch.cuda.synchronize()
            assert (abort.cpu().numpy() == ref["abort"]).all()
            worst, t = check_close(out_to_f64(out), ref["out"], tol)
            print(f"  split {sp} {tol}: max|err| {worst:.3e} (tol {t:.3e})")
