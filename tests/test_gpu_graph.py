"""The decode step (tag check -> append -> attention) captured in a HIP graph must give, on every
replay, exactly the result of the same step run eagerly.  No memset nodes are involved: the
library launches kernels only."""
import pytest
import torch

import synth
from gpu_pipeline import GpuState

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_graph_replays_match_eager(kv):
    w = synth.make("gqa", seed=3, B=8, len_range=(100, 2000))
    s = w.spec
    st = GpuState(w, kv)
    k_new, v_new, ids, pos = st.step_inputs()
    ws = dapf8.make_workspace(st.q, st.k_pool, st.v_pool, st.page_table, s.Dv)
    out = torch.empty((s.B, s.Hq, s.Dv), dtype=torch.bfloat16, device="cuda")

    def step():
        dapf8.kv_tag_verify(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, st.abort, s.page_size)
        dapf8.kv_append(k_new, v_new, st.k_pool, st.v_pool, st.page_table, ids, pos, st.k_scale, st.v_scale,
                        st.abort)
        dapf8.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, st.k_scale, st.v_scale,
                                st.abort, out=out, sm_scale=s.scale(), workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(5):
        out.zero_()
        st.abort.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep} differs"
        assert (st.abort.cpu() == 0).all()
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
