"""Runs a synthetic workload through the HIP library (test and benchmark infrastructure).

Uploads the drawn inputs, sets up scales with the library's own kernels, fills the pools with
kv_append, and runs one decode step: kv_tag_verify -> kv_append -> paged_decode_attn, all on the
current stream.  Nothing here computes any part of the method itself.
"""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_paged_fp8_amd as dapf8


def t_act(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy fp32 array or bf16 bit patterns (uint16) -> torch tensor on the device."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def t_int(a: np.ndarray, dtype=torch.int32, device="cuda") -> torch.Tensor:
    if dtype == torch.int32:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    if dtype == torch.uint32:  # torch has limited uint32 support: carry tags as int32 bit patterns
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(device)
    raise TypeError(dtype)


def pool_to_numpy(p: torch.Tensor) -> np.ndarray:
    if p.dtype == torch.bfloat16:
        return p.view(torch.int16).cpu().numpy().view(np.uint16)
    return p.cpu().numpy()


class GpuState:
    def __init__(self, w, kv="fp8", layer=0, device="cuda", num_pages=None, on_rows=None):
        s = w.spec
        self.w, self.kv, self.layer = w, kv, layer
        self.num_pages = w.num_pages if num_pages is None else num_pages
        self.page_table = t_int(w.page_table)
        self.seq_lens = t_int(w.seq_lens)
        self.live_tags = t_int(w.live_tags, torch.uint32)
        self.expected_tags = t_int(w.expected_tags, torch.uint32)
        self.q = t_act(w.q)
        self.k_pool, self.v_pool = dapf8.alloc_pools(self.num_pages, s.Hkv, s.page_size, s.Dk, s.Dv, kv,
                                                     s.shared_kv, device)
        self.abort = torch.zeros(w.B, dtype=torch.uint8, device=device)
        self.k_scale = self.v_scale = None
        self.fill(on_rows)

    def fill(self, on_rows=None):
        """Initial fill: scales from the fill tokens (FP8), then kv_append of every fill token.
        on_rows(b, k, v) sees each sequence's drawn rows (numpy) before upload."""
        w, s = self.w, self.w.spec
        rows = []
        for b in range(w.B):
            k, v = w.fill_tokens(b, self.layer)
            if on_rows is not None:
                on_rows(b, k, v)
            rows.append((b, t_act(k), None if v is None else t_act(v)))
            del k, v
        if self.kv == "fp8":
            ak = torch.zeros(s.Hkv, dtype=torch.float32, device="cuda")
            av = torch.zeros(s.Hkv, dtype=torch.float32, device="cuda")
            for _, k, v in rows:
                if k.shape[0]:
                    dapf8.kv_absmax_update(k, ak)
                    if v is not None:
                        dapf8.kv_absmax_update(v, av)
            self.k_scale = dapf8.kv_scale_from_absmax(ak)
            self.v_scale = None if s.shared_kv else dapf8.kv_scale_from_absmax(av)
        for b, k, v in rows:
            n = k.shape[0]
            if n == 0:
                continue
            ids = torch.full((n,), b, dtype=torch.int32, device="cuda")
            pos = torch.arange(n, dtype=torch.int32, device="cuda")
            dapf8.kv_append(k, v, self.k_pool, self.v_pool, self.page_table, ids, pos, self.k_scale, self.v_scale)
        del rows

    def step_inputs(self):
        k_new, v_new, ids, pos = self.w.step_tokens(self.layer)
        return (t_act(k_new), None if v_new is None else t_act(v_new), t_int(ids), t_int(pos))

    def step(self, verify=True, split_tokens=0, out_dtype=None, step_inputs=None, workspace=None):
        """One decode step.  Returns (out, abort mask or None)."""
        s = self.w.spec
        abort = None
        if verify:
            dapf8.kv_tag_verify(self.page_table, self.expected_tags, self.seq_lens, self.live_tags, self.abort,
                                s.page_size)
            abort = self.abort
        if s.append:
            k_new, v_new, ids, pos = step_inputs if step_inputs is not None else self.step_inputs()
            dapf8.kv_append(k_new, v_new, self.k_pool, self.v_pool, self.page_table, ids, pos, self.k_scale,
                            self.v_scale, abort)
        od = out_dtype or (torch.float32 if s.out_dt == "f32" else torch.bfloat16)
        out = dapf8.paged_decode_attn(self.q, self.k_pool, self.v_pool, self.page_table, self.seq_lens,
                                      self.k_scale, self.v_scale, abort, out_dtype=od, sm_scale=s.scale(), Dv=s.Dv,
                                      split_tokens=split_tokens, workspace=workspace)
        return out, abort


def out_to_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def check_close(gpu: np.ndarray, ref: np.ndarray, out_dt: str):
    """The parity bar: fp32 output max |err| <= 1e-4 absolute; bf16 output <= 1e-2 * max |ref|."""
    err = np.abs(gpu - ref)
    if out_dt == "f32":
        tol = 1e-4
    else:
        tol = 1e-2 * max(float(np.abs(ref).max()), 1e-30)
    worst = float(err.max()) if err.size else 0.0
    assert np.isfinite(gpu).all(), "non-finite GPU output"
    assert worst <= tol, f"max |err| {worst:.3e} > tol {tol:.3e}"
    return worst, tol
