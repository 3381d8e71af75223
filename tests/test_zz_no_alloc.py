"""paged_decode_attn_noalloc -- the entry point for callers that cannot allocate -- against
paged_decode_attn: the same kernels run on the library's own scratch instead of a caller-owned
workspace, so every output must be bit-identical, on two calls in a row (the second with a smaller
input, so stale scratch contents from the first call are around), for the stream-K shape and for
the fixed-partition generic shape (both keep partial results in the scratch).  The first call is
also held to the oracle at the parity bar.  Shapes whose workspace exceeds the scratch are refused
before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_pipeline import GpuState, check_close, out_to_f64
from oracle_pipeline import oracle_step

import decode_attention_paged_fp8_amd as dapf8


def _noalloc(st, w, out, split_tokens=0):
    """Calls the C entry point directly (ctypes), not through the Python wrapper."""
    s = w.spec
    L = dapf8.lib()
    num_pages, Hkv, P = st.k_pool.shape[0], st.k_pool.shape[1], st.k_pool.shape[3]
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    rc = L.paged_decode_attn_noalloc(
        vp(st.q), dapf8.ACT_BF16 if st.q.dtype == torch.bfloat16 else dapf8.ACT_F32, vp(st.k_pool), vp(st.v_pool),
        dapf8.KV_FP8 if st.kv == "fp8" else dapf8.KV_BF16, vp(st.page_table), st.page_table.shape[1],
        vp(st.seq_lens), vp(st.k_scale), vp(st.v_scale), vp(st.abort),
        vp(out), dapf8.ACT_BF16 if out.dtype == torch.bfloat16 else dapf8.ACT_F32, float(s.scale()), s.B, s.Hq, Hkv,
        s.Dk, s.Dv, P, num_pages, int(split_tokens), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, L.dapf8_last_error().decode()


CASES = [
    # (workload, generator overrides, split_tokens): stream-K on the matrix cores, then the generic
    # kernel with fixed 256-token partitions
    ("gqa", dict(B=8, len_range=(600, 3000)), 0, "mfma_streamk"),
    ("tiny_mha", dict(B=4, lens=None, len_range=(700, 1500), num_pages=None), 256, "valu_generic"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,kw,split,variant", CASES)
def test_noalloc_matches_workspace_entry_point(name, kw, split, variant):
    print(f"\n[case] noalloc {name} {kw} split={split}", flush=True)
    for call, shrink in enumerate((1, 2)):
        kw2 = dict(kw)
        kw2["B"] = kw["B"] // shrink
        lo, hi = kw["len_range"]
        kw2["len_range"] = (lo // shrink, hi // shrink)
        w = synth.make(name, seed=7 + call, **kw2)
        s = w.spec
        assert dapf8.paged_decode_attn_variant(s.B, s.Hq, s.Hkv, s.Dk, s.Dv, s.page_size, w.pt_stride, split,
                                               0)[0].startswith(variant)
        st = GpuState(w, "fp8")
        od = torch.float32 if s.out_dt == "f32" else torch.bfloat16
        ref, abort = st.step(split_tokens=split, out_dtype=od)  # tag check + append + paged_decode_attn
        out = torch.full_like(ref, float("nan"))
        _noalloc(st, w, out, split)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if od == torch.bfloat16 else out.view(torch.int32),
                           ref.view(torch.int16) if od == torch.bfloat16 else ref.view(torch.int32)), f"call {call}"
        if call == 0:
            orc = oracle_step(w, "fp8")
            check_close(out_to_f64(out), orc["out"], s.out_dt)
            assert (abort.cpu().numpy() == orc["abort"]).all()


def test_noalloc_refuses_shapes_beyond_its_scratch():
    # the latent-style shape (B64, 128 heads on one 576/512 KV head, page 64, 512-page rows) needs a
    # ~152 MB workspace: refused with DAPF8_EWORKSPACE before any argument is dereferenced or any
    # kernel is launched (the pointers below are never used)
    need = dapf8.paged_decode_attn_workspace_size(64, 128, 1, 576, 512, 64, 512, 0, dapf8.KV_FP8, True)
    assert need > dapf8.NOALLOC_SCRATCH_BYTES
    L = dapf8.lib()
    fake = ctypes.c_void_p(1 << 20)
    rc = L.paged_decode_attn_noalloc(fake, dapf8.ACT_BF16, fake, None, dapf8.KV_FP8, fake, 512, fake, fake, None, None,
                                     fake, dapf8.ACT_BF16, 1.0 / 24, 64, 128, 1, 576, 512, 64, 1000, 0, None)
    assert rc == -3, rc
    assert b"scratch" in L.dapf8_last_error()
