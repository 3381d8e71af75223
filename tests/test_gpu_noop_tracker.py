"""The pages' default no-op tracker: with tag checking disabled, the decode step must launch no tag
check at all.  The step (kv_append + paged_decode_attn, no abort mask) is captured in a HIP graph
and its kernel nodes are listed through the HIP graph API: there is no verify kernel among them, and
the checked step (kv_tag_verify first, its mask passed on) has exactly one more kernel node, the tag
check.  With no stale tag both steps give the same output, bit for bit."""
import ctypes

import pytest
import torch

import synth
from gpu_pipeline import GpuState

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu


class _Dim3(ctypes.Structure):
    _fields_ = [("x", ctypes.c_uint), ("y", ctypes.c_uint), ("z", ctypes.c_uint)]


class _KernelNodeParams(ctypes.Structure):  # hipKernelNodeParams
    _fields_ = [("blockDim", _Dim3), ("extra", ctypes.c_void_p), ("func", ctypes.c_void_p), ("gridDim", _Dim3),
                ("kernelParams", ctypes.c_void_p), ("sharedMemBytes", ctypes.c_uint),
                ("_slack", ctypes.c_char * 64)]  # room to spare past the documented fields


def _hip_runtime():
    """The HIP runtime this process already uses (torch's and the library's): the graph handle is an
    object of that runtime, so it must be queried through the same library."""
    with open("/proc/self/maps") as fh:
        paths = sorted({ln.split()[-1] for ln in fh if "libamdhip64" in ln and "/" in ln})
    assert len(paths) == 1, paths
    return ctypes.CDLL(paths[0])


def _kernel_nodes(graph_handle):
    """Names of the kernel nodes of a captured graph (None where the runtime gives no name)."""
    hip = _hip_runtime()
    g = ctypes.c_void_p(graph_handle)
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(g, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(g, nodes, ctypes.byref(n)) == 0
    name_of = getattr(hip, "hipKernelNameRefByPtr", None)
    if name_of is not None:
        name_of.restype = ctypes.c_char_p
        name_of.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    names = []
    for nd in nodes:
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nd), ctypes.byref(t)) == 0
        assert t.value == 0, f"non-kernel node of type {t.value}"  # the library launches kernels only
        p = _KernelNodeParams()
        assert hip.hipGraphKernelNodeGetParams(ctypes.c_void_p(nd), ctypes.byref(p)) == 0
        nm = name_of(p.func, None) if name_of is not None else None
        names.append(nm.decode() if nm else None)
    return names


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_no_op_tracker_launches_no_tag_check(kv):
    print(f"\n[case] no-op tracker {kv}", flush=True)
    w = synth.make("gqa", seed=3, B=8, len_range=(100, 2000))
    s = w.spec
    st = GpuState(w, kv)
    k_new, v_new, ids, pos = st.step_inputs()
    ws = dapf8.make_workspace(st.q, st.k_pool, st.v_pool, st.page_table, s.Dv)
    outs = {m: torch.empty((s.B, s.Hq, s.Dv), dtype=torch.bfloat16, device="cuda") for m in ("checked", "untracked")}

    def checked():
        dapf8.kv_tag_verify(st.page_table, st.expected_tags, st.seq_lens, st.live_tags, st.abort, s.page_size)
        dapf8.kv_append(k_new, v_new, st.k_pool, st.v_pool, st.page_table, ids, pos, st.k_scale, st.v_scale,
                        st.abort)
        dapf8.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, st.k_scale, st.v_scale,
                                st.abort, out=outs["checked"], sm_scale=s.scale(), workspace=ws)

    def untracked():
        dapf8.kv_append(k_new, v_new, st.k_pool, st.v_pool, st.page_table, ids, pos, st.k_scale, st.v_scale)
        dapf8.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, st.k_scale, st.v_scale,
                                out=outs["untracked"], sm_scale=s.scale(), workspace=ws)

    graphs = {"checked": _capture(checked), "untracked": _capture(untracked)}
    nodes = {m: _kernel_nodes(g.raw_cuda_graph()) for m, g in graphs.items()}
    print("  kernel nodes:", nodes, flush=True)
    assert len(nodes["checked"]) == len(nodes["untracked"]) + 1
    if all(n is not None for v in nodes.values() for n in v):
        assert not any("verify" in n for n in nodes["untracked"])
        assert sum("verify" in n for n in nodes["checked"]) == 1
    for m, g in graphs.items():
        g.instantiate()
        outs[m].zero_()
        g.replay()
    torch.cuda.synchronize()
    assert (st.abort.cpu() == 0).all()
    assert torch.equal(outs["checked"].view(torch.int16), outs["untracked"].view(torch.int16))
