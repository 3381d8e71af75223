"""Paged FP8 decode attention for AMD MI355X (gfx950) -- Python binding of libdapf8.so.

The binding only marshals arguments: it reads shapes, dtypes and device pointers from torch
tensors and calls the C ABI (include/dapf8.h) on the current HIP stream.  Every step of the
path runs in the library's HIP kernels; if the library is missing the import of any entry
point fails loudly -- there is no fallback.

Entry points (same names as the C ABI):
  kv_absmax_update, kv_scale_from_absmax   per-head scale setup, s = fp32(amax / 448)
  kv_append                                quantize-on-append of new K/V rows into page slots
  kv_tag_verify                            batched page-tag check -> abort mask
  kv_tag_verify_append                     the check and the append of its unaborted tokens, one launch
  kv_transcode_pages                       BF16 pool pages -> FP8 pool pages (prefill -> decode handoff)
  paged_decode_attn                        decode attention, FP8 (dequantised on read) or BF16
  paged_decode_attn_checked                the same with the page-tag check inside the page walk
  kv_pages_init, kv_pages_alloc, kv_pages_free   device page allocator and tag tracker
  w4_pack, w4a16_gemv                      INT4 weight-only decode GEMV (synthetic weights)
  paged_decode_attn_noalloc                paged_decode_attn on the library's own scratch (no allocation)
  hbm_read_probe                           plain read-only streaming kernel (the attainable read rate)
  hbm_copy_probe                           plain read-write streaming kernel (2 bytes read per byte written)

Pools are torch tensors: FP8 pools are uint8 (or float8_e4m3fn) tensors, BF16 pools are bfloat16;
K pool shape [num_pages, Hkv, Dk/C, page_size, C] with C = 64 (FP8) or 32 (BF16) -- each token's
row cut into 64-byte dimension chunks stored chunk by chunk -- and V pool [num_pages, Hkv, Dv,
page_size].  alloc_pools() allocates both.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["KV_FP8", "KV_BF16", "ACT_F32", "ACT_BF16", "DapfError", "lib", "lib_path", "alloc_pools",
           "k_chunk", "kv_absmax_update",
           "kv_scale_from_absmax", "kv_scales", "kv_append", "kv_tag_verify", "kv_tag_verify_append",
           "kv_transcode_pages",
           "paged_decode_attn", "paged_decode_attn_noalloc", "paged_decode_attn_checked", "kv_pages_init", "kv_pages_alloc", "kv_pages_free",
           "alloc_page_allocator", "w4_pack", "w4a16_gemv", "hbm_read_probe", "hbm_copy_probe",
           "paged_decode_attn_workspace_size", "paged_decode_attn_variant", "make_workspace"]

KV_FP8, KV_BF16 = 0, 1
ACT_F32, ACT_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdapf8.so")
_lock = threading.Lock()
_lib = None


class DapfError(RuntimeError):
    pass


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libdapf8.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise DapfError(f"{_LIB_PATH} is missing: build it with "
                                f"`python -c 'import __graft_entry__ as g; g.build()'`")
            L = ctypes.CDLL(_LIB_PATH)
            vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
            ci, f32 = ctypes.c_int, ctypes.c_float
            L.dapf8_last_error.restype = ctypes.c_char_p
            L.dapf8_version.restype = ci
            L.kv_absmax_update.argtypes = [vp, ci, i64, i32, i32, vp, vp]
            L.kv_scale_from_absmax.argtypes = [vp, i32, vp, vp]
            L.kv_append.argtypes = [vp, vp, ci, vp, vp, ci, vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                    i32, i32, vp]
            L.kv_tag_verify.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, i32, vp]
            L.kv_tag_verify_append.argtypes = [vp, i32, vp, vp, vp, i32, vp, vp, vp, ci, vp, vp, ci, vp, vp, i32, vp,
                                               vp, i32, i32, i32, i32, i32, vp]
            L.kv_transcode_pages.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, vp]
            L.paged_decode_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, ci, ci]
            L.paged_decode_attn_workspace_size.restype = sz
            L.paged_decode_attn_variant.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, ci, ci,
                                                    ctypes.POINTER(i32)]
            L.paged_decode_attn_variant.restype = ctypes.c_char_p
            L.paged_decode_attn.argtypes = [vp, ci, vp, vp, ci, vp, i32, vp, vp, vp, vp, vp, ci, f32, i32, i32, i32,
                                            i32, i32, i32, i32, i32, vp, sz, vp]
            L.paged_decode_attn_noalloc.argtypes = [vp, ci, vp, vp, ci, vp, i32, vp, vp, vp, vp, vp, ci, f32, i32,
                                                    i32, i32, i32, i32, i32, i32, i32, vp]
            L.paged_decode_attn_checked.argtypes = [vp, ci, vp, vp, ci, vp, i32, vp, vp, vp, vp, vp, vp, vp, ci, f32,
                                                    i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
            L.kv_pages_init.argtypes = [vp, vp, vp, i32, vp]
            L.kv_pages_alloc.argtypes = [vp, vp, vp, i32, vp, vp, i32, vp, vp, i32, vp, vp]
            L.kv_pages_free.argtypes = [vp, vp, vp, i32, i32, vp, vp]
            L.w4_pack.argtypes = [vp, vp, i32, i32, vp, vp, vp]
            L.hbm_read_probe.argtypes = [vp, vp, i64, i32, vp, i32, vp]
            L.hbm_copy_probe.argtypes = [vp, vp, i64, i32, vp]
            L.w4a16_gemv.argtypes = [vp, vp, vp, vp, ci, i32, i32, i32, vp]
            for f in (L.kv_absmax_update, L.kv_scale_from_absmax, L.kv_append, L.kv_tag_verify, L.kv_tag_verify_append,
                      L.kv_transcode_pages, L.paged_decode_attn, L.paged_decode_attn_noalloc,
                      L.paged_decode_attn_checked, L.kv_pages_init,
                      L.kv_pages_alloc, L.kv_pages_free, L.w4_pack, L.w4a16_gemv, L.hbm_read_probe,
                      L.hbm_copy_probe):
                f.restype = ci
            _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = lib().dapf8_last_error().decode(errors="replace")
        raise DapfError(f"{what} failed ({rc}): {msg}")


def _p(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise DapfError("tensors passed to the library must live on the GPU")
    if not t.is_contiguous():
        raise DapfError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _act_dt(t) -> int:
    if t.dtype == torch.float32:
        return ACT_F32
    if t.dtype == torch.bfloat16:
        return ACT_BF16
    raise DapfError(f"activation tensors must be float32 or bfloat16, got {t.dtype}")


def _kv_dt(pool) -> int:
    if pool.dtype in (torch.uint8, torch.float8_e4m3fn):
        return KV_FP8
    if pool.dtype == torch.bfloat16:
        return KV_BF16
    raise DapfError(f"KV pools must be uint8/float8_e4m3fn (FP8) or bfloat16 (BF16), got {pool.dtype}")


def k_chunk(kv_dt: int) -> int:
    """Dimensions per 64-byte chunk of a K pool row."""
    return 64 if kv_dt == KV_FP8 else 32


def alloc_pools(num_pages, Hkv, page_size, Dk, Dv, kv="fp8", shared_kv=False, device="cuda"):
    """Zeroed K and V pools in the library's layout (V is None in shared-KV mode)."""
    kd = KV_FP8 if kv == "fp8" else KV_BF16
    C = k_chunk(kd)
    if Dk % 64:
        raise DapfError(f"Dk must be a multiple of 64, got {Dk}")
    el = torch.uint8 if kd == KV_FP8 else torch.bfloat16
    k = torch.zeros((num_pages, Hkv, Dk // C, page_size, C), dtype=el, device=device)
    v = None if shared_kv else torch.zeros((num_pages, Hkv, Dv, page_size), dtype=el, device=device)
    return k, v


def _k_dims(k_pool):
    """(num_pages, Hkv, page_size, Dk) of a K pool tensor [num_pages, Hkv, Dk/C, P, C]."""
    if k_pool.dim() != 5:
        raise DapfError("K pool must have shape [num_pages, Hkv, Dk/C, page_size, C]")
    n, H, nc, P, C = k_pool.shape
    if C != k_chunk(_kv_dt(k_pool)):
        raise DapfError(f"K pool chunk width {C} does not match its dtype")
    return n, H, P, nc * C


def kv_absmax_update(x, amax, stream=None):
    """amax[h] = max(amax[h], max |x[:, h, :]|) for x : [T, H, D]."""
    T, H, D = x.shape
    _check(lib().kv_absmax_update(_p(x), _act_dt(x), T, H, D, _p(amax), _stream(stream)), "kv_absmax_update")


def kv_scale_from_absmax(amax, scale=None, stream=None):
    scale = torch.empty_like(amax) if scale is None else scale
    _check(lib().kv_scale_from_absmax(_p(amax), amax.numel(), _p(scale), _stream(stream)), "kv_scale_from_absmax")
    return scale


def kv_scales(x, stream=None):
    """Per-head scales of a whole fill x : [T, H, D] in one call."""
    amax = torch.zeros(x.shape[1], dtype=torch.float32, device=x.device)
    kv_absmax_update(x, amax, stream)
    return kv_scale_from_absmax(amax, stream=stream)


def kv_append(k_new, v_new, k_pool, v_pool, page_table, seq_ids, positions, k_scale=None, v_scale=None,
              abort_mask=None, stream=None):
    """Quantise-on-append.  k_new : [T, Hkv, Dk], v_new : [T, Hkv, Dv] (or None with v_pool None)."""
    T, Hkv, Dk = k_new.shape
    Dv = v_new.shape[2] if v_new is not None else 0
    num_pages, _, P, _ = _k_dims(k_pool)
    B, stride = page_table.shape
    _check(lib().kv_append(_p(k_new), _p(v_new), _act_dt(k_new), _p(k_pool), _p(v_pool), _kv_dt(k_pool),
                           _p(page_table), stride, _p(seq_ids), _p(positions), T, _p(k_scale), _p(v_scale),
                           _p(abort_mask), B, Hkv, Dk, Dv, P, num_pages, _stream(stream)), "kv_append")


def kv_tag_verify(page_table, expected_tags, seq_lens, live_tags, abort_mask, page_size, stream=None):
    B, stride = page_table.shape
    _check(lib().kv_tag_verify(_p(page_table), stride, _p(expected_tags), _p(seq_lens), _p(live_tags),
                               live_tags.numel(), _p(abort_mask), B, page_size, _stream(stream)), "kv_tag_verify")
    return abort_mask


def kv_tag_verify_append(page_table, expected_tags, seq_lens, live_tags, abort_mask, k_new, v_new, k_pool, v_pool,
                         seq_ids, positions, k_scale=None, v_scale=None, stream=None):
    """kv_tag_verify, then kv_append of the unaborted requests' tokens with that mask, in one launch.
    k_new : [T, Hkv, Dk], v_new : [T, Hkv, Dv] (or None with v_pool None).  Returns abort_mask."""
    T, Hkv, Dk = k_new.shape
    Dv = v_new.shape[2] if v_new is not None else 0
    num_pages, _, P, _ = _k_dims(k_pool)
    if live_tags.numel() != num_pages:
        raise DapfError("kv_tag_verify_append: live_tags must hold one tag per pool page")
    B, stride = page_table.shape
    _check(lib().kv_tag_verify_append(_p(page_table), stride, _p(expected_tags), _p(seq_lens), _p(live_tags),
                                      live_tags.numel(), _p(abort_mask), _p(k_new), _p(v_new), _act_dt(k_new),
                                      _p(k_pool), _p(v_pool), _kv_dt(k_pool), _p(seq_ids), _p(positions), T,
                                      _p(k_scale), _p(v_scale), B, Hkv, Dk, Dv, P, _stream(stream)),
           "kv_tag_verify_append")
    return abort_mask


def kv_transcode_pages(k_src, v_src, k_dst, v_dst, src_pages, dst_pages, k_scale, v_scale=None, stream=None):
    """Page src_pages[i] of the BF16 pools -> page dst_pages[i] of the FP8 pools, quantised as on append.
    v_src = v_dst = None for shared-KV pools."""
    if _kv_dt(k_src) != KV_BF16 or _kv_dt(k_dst) != KV_FP8:
        raise DapfError("kv_transcode_pages: source pools must be bfloat16 and destination pools FP8")
    ns, Hkv, P, Dk = _k_dims(k_src)
    nd, Hkv2, P2, Dk2 = _k_dims(k_dst)
    if (Hkv2, P2, Dk2) != (Hkv, P, Dk):
        raise DapfError("kv_transcode_pages: source and destination K pools differ in shape")
    if (v_src is None) != (v_dst is None):
        raise DapfError("kv_transcode_pages: give both V pools or neither")
    Dv = v_src.shape[2] if v_src is not None else 0
    if v_src is not None and (v_dst.shape[1:] != v_src.shape[1:] or _kv_dt(v_dst) != KV_FP8):
        raise DapfError("kv_transcode_pages: source and destination V pools differ in shape or type")
    n = src_pages.numel()
    if dst_pages.numel() != n:
        raise DapfError("kv_transcode_pages: src_pages and dst_pages differ in length")
    _check(lib().kv_transcode_pages(_p(k_src), _p(v_src), _p(k_dst), _p(v_dst), _p(src_pages), _p(dst_pages), n,
                                    _p(k_scale), _p(v_scale), Hkv, Dk, Dv, P, ns, nd, _stream(stream)),
           "kv_transcode_pages")


def paged_decode_attn_workspace_size(B, Hq, Hkv, Dk, Dv, page_size, pt_stride, split_tokens=0, kv_dt=KV_FP8,
                                     shared_kv=False) -> int:
    return int(lib().paged_decode_attn_workspace_size(B, Hq, Hkv, Dk, Dv, page_size, pt_stride, split_tokens,
                                                      kv_dt, int(bool(shared_kv))))


def paged_decode_attn_variant(B, Hq, Hkv, Dk, Dv, page_size, pt_stride, split_tokens=0, kv_dt=KV_FP8,
                              shared_kv=False):
    s = ctypes.c_int32(0)
    name = lib().paged_decode_attn_variant(B, Hq, Hkv, Dk, Dv, page_size, pt_stride, split_tokens, kv_dt,
                                           int(bool(shared_kv)), ctypes.byref(s))
    return name.decode(), int(s.value)


def make_workspace(q, k_pool, v_pool, page_table, Dv, split_tokens=0):
    B, Hq, Dk = q.shape
    _, Hkv, P, _ = _k_dims(k_pool)
    n = paged_decode_attn_workspace_size(B, Hq, Hkv, Dk, Dv, P, page_table.shape[1], split_tokens, _kv_dt(k_pool),
                                         v_pool is None)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def paged_decode_attn(q, k_pool, v_pool, page_table, seq_lens, k_scale=None, v_scale=None, abort_mask=None, *,
                      out=None, out_dtype=None, sm_scale=None, Dv=None, split_tokens=0, workspace=None,
                      stream=None):
    """q : [B, Hq, Dk].  Returns out : [B, Hq, Dv] (float32 or bfloat16)."""
    B, Hq, Dk = q.shape
    num_pages, Hkv, P, Dk2 = _k_dims(k_pool)
    if Dk2 != Dk:
        raise DapfError(f"q head dim {Dk} != K pool head dim {Dk2}")
    if v_pool is not None:
        Dv = v_pool.shape[2]
    elif Dv is None:
        raise DapfError("Dv is required in shared-KV mode (v_pool None)")
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=out_dtype or q.dtype, device=q.device)
    if sm_scale is None:
        sm_scale = Dk ** -0.5
    if workspace is None:
        workspace = make_workspace(q, k_pool, v_pool, page_table, Dv, split_tokens)
    _check(lib().paged_decode_attn(_p(q), _act_dt(q), _p(k_pool), _p(v_pool), _kv_dt(k_pool), _p(page_table),
                                   page_table.shape[1], _p(seq_lens), _p(k_scale), _p(v_scale), _p(abort_mask),
                                   _p(out), _act_dt(out), float(sm_scale), B, Hq, Hkv, Dk, Dv, P, num_pages,
                                   int(split_tokens), _p(workspace), workspace.numel(), _stream(stream)),
           "paged_decode_attn")
    return out


def paged_decode_attn_noalloc(q, k_pool, v_pool, page_table, seq_lens, k_scale=None, v_scale=None, abort_mask=None,
                              *, out, sm_scale=None, Dv=None, split_tokens=0, stream=None):
    """paged_decode_attn with the library's own scratch instead of a workspace: allocates nothing
    (out must be given).  Calls that overlap in time on one GPU race on that scratch."""
    B, Hq, Dk = q.shape
    num_pages, Hkv, P, Dk2 = _k_dims(k_pool)
    if Dk2 != Dk:
        raise DapfError(f"q head dim {Dk} != K pool head dim {Dk2}")
    if v_pool is not None:
        Dv = v_pool.shape[2]
    elif Dv is None:
        raise DapfError("Dv is required in shared-KV mode (v_pool None)")
    if sm_scale is None:
        sm_scale = Dk ** -0.5
    _check(lib().paged_decode_attn_noalloc(_p(q), _act_dt(q), _p(k_pool), _p(v_pool), _kv_dt(k_pool),
                                           _p(page_table), page_table.shape[1], _p(seq_lens), _p(k_scale),
                                           _p(v_scale), _p(abort_mask), _p(out), _act_dt(out), float(sm_scale), B, Hq,
                                           Hkv, Dk, Dv, P, num_pages, int(split_tokens), _stream(stream)),
           "paged_decode_attn_noalloc")
    return out


# DAPF8_NOALLOC_SCRATCH_BYTES of include/dapf8.h: the scratch the no-allocation entry point holds per GPU
NOALLOC_SCRATCH_BYTES = 64 << 20


def paged_decode_attn_checked(q, k_pool, v_pool, page_table, seq_lens, expected_tags, live_tags, abort_mask,
                              k_scale=None, v_scale=None, *, out=None, out_dtype=None, sm_scale=None,
                              workspace=None, stream=None):
    """Attention with the page-tag check inside the page walk; abort_mask [B] uint8 is written.
    Tags are int32 tensors holding the uint32 bit patterns."""
    B, Hq, Dk = q.shape
    num_pages, Hkv, P, Dk2 = _k_dims(k_pool)
    if Dk2 != Dk or v_pool is None:
        raise DapfError("paged_decode_attn_checked: needs a separate V pool and matching head dims")
    Dv = v_pool.shape[2]
    if out is None:
        out = torch.empty((B, Hq, Dv), dtype=out_dtype or q.dtype, device=q.device)
    if sm_scale is None:
        sm_scale = Dk ** -0.5
    if workspace is None:
        workspace = make_workspace(q, k_pool, v_pool, page_table, Dv, 0)
    _check(lib().paged_decode_attn_checked(_p(q), _act_dt(q), _p(k_pool), _p(v_pool), _kv_dt(k_pool), _p(page_table),
                                           page_table.shape[1], _p(seq_lens), _p(expected_tags), _p(live_tags),
                                           _p(k_scale), _p(v_scale), _p(abort_mask), _p(out), _act_dt(out),
                                           float(sm_scale), B, Hq, Hkv, Dk, Dv, P, num_pages, _p(workspace),
                                           workspace.numel(), _stream(stream)),
           "paged_decode_attn_checked")
    return out


def alloc_page_allocator(num_pages, tags=True, device="cuda"):
    """(free_list, free_count, live_tags or None) tensors, initialised by kv_pages_init."""
    free_list = torch.empty(num_pages, dtype=torch.int32, device=device)
    free_count = torch.empty(4, dtype=torch.int32, device=device)  # element 0 is the count
    live_tags = torch.empty(num_pages, dtype=torch.int32, device=device) if tags else None
    kv_pages_init(free_list, free_count, live_tags)
    return free_list, free_count, live_tags


def kv_pages_init(free_list, free_count, live_tags=None, stream=None):
    _check(lib().kv_pages_init(_p(free_list), _p(free_count), _p(live_tags), free_list.numel(), _stream(stream)),
           "kv_pages_init")


def kv_pages_alloc(free_list, free_count, live_tags, counts, first_slot, page_table, expected_tags=None,
                   granted=None, stream=None):
    """Requests b ask for counts[b] pages in slots first_slot[b].. of page_table row b.  Returns granted [B] uint8."""
    B = counts.numel()
    if first_slot.numel() != B:
        raise DapfError("kv_pages_alloc: counts and first_slot differ in length")
    if page_table.dim() != 2 or page_table.shape[0] < B:
        raise DapfError("kv_pages_alloc: page_table must be [>= B][pt_stride]")
    if expected_tags is not None and expected_tags.shape != page_table.shape:
        raise DapfError("kv_pages_alloc: expected_tags must have the page table's shape")
    if granted is None:
        granted = torch.empty(max(B, 1), dtype=torch.uint8, device=counts.device)
    _check(lib().kv_pages_alloc(_p(free_list), _p(free_count), _p(live_tags), free_list.numel(), _p(counts),
                                _p(first_slot), B, _p(page_table), _p(expected_tags), page_table.shape[1],
                                _p(granted), _stream(stream)), "kv_pages_alloc")
    return granted[:B]


def kv_pages_free(free_list, free_count, pages, status=None, stream=None):
    """Push pages onto the free stack.  Returns status [2] int32: (pushed, rejected)."""
    if status is None:
        status = torch.empty(4, dtype=torch.int32, device=free_list.device)
    _check(lib().kv_pages_free(_p(free_list), _p(free_count), _p(pages) if pages.numel() else None, pages.numel(),
                               free_list.numel(), _p(status), _stream(stream)), "kv_pages_free")
    return status[:2]


def w4_pack(q, scales, stream=None):
    """q : [N][K] int8 in [-8, 7], scales : [N][K/128] fp32 -> (packed uint8 [N*K/2], packed_scales [K/128][N])."""
    N, K = q.shape
    if q.dtype != torch.int8 or scales.dtype != torch.float32 or tuple(scales.shape) != (N, K // 128):
        raise DapfError("w4_pack: q must be int8 [N][K] and scales fp32 [N][K/128]")
    packed = torch.empty(N * K // 2, dtype=torch.uint8, device=q.device)
    ps = torch.empty((K // 128, N), dtype=torch.float32, device=q.device)
    _check(lib().w4_pack(_p(q), _p(scales), N, K, _p(packed), _p(ps), _stream(stream)), "w4_pack")
    return packed, ps


def w4a16_gemv(x, packed, packed_scales, N, *, out=None, out_dtype=None, stream=None):
    """y [M][N] = x [M][K] (bf16) times the packed INT4 weights' transpose."""
    M, K = x.shape
    if x.dtype != torch.bfloat16:
        raise DapfError("w4a16_gemv: x must be bfloat16")
    if packed.numel() != N * K // 2 or tuple(packed_scales.shape) != (K // 128, N):
        raise DapfError("w4a16_gemv: packed weights do not match N and K")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=x.device)
    _check(lib().w4a16_gemv(_p(x), _p(packed), _p(packed_scales), _p(out), _act_dt(out), M, N, K, _stream(stream)),
           "w4a16_gemv")
    return out


def hbm_read_probe(buf, block_bytes, block_ids=None, sink=None, workgroups=2048, stream=None):
    """Read-only streaming probe: reads the blocks of `buf` (uint8 tensor) once.  Returns the sink."""
    if buf.dtype != torch.uint8 or buf.numel() % block_bytes:
        raise DapfError("hbm_read_probe: buf must be a uint8 tensor of whole blocks")
    n = buf.numel() // block_bytes if block_ids is None else block_ids.numel()
    if sink is None:
        sink = torch.empty(workgroups * 256, dtype=torch.int32, device=buf.device)
    _check(lib().hbm_read_probe(_p(buf), _p(block_ids), n, block_bytes, _p(sink), workgroups, _stream(stream)),
           "hbm_read_probe")
    return sink


def hbm_copy_probe(src, dst, workgroups=2048, stream=None):
    """Read-write streaming probe: reads 2 * dst.numel() bytes of `src`, writes all of `dst` (uint8)."""
    if src.dtype != torch.uint8 or dst.dtype != torch.uint8 or src.numel() < 2 * dst.numel() or dst.numel() % 16:
        raise DapfError("hbm_copy_probe: uint8 tensors with src.numel() >= 2 * dst.numel(), dst a multiple of 16 bytes")
    _check(lib().hbm_copy_probe(_p(src), _p(dst), dst.numel(), workgroups, _stream(stream)), "hbm_copy_probe")
