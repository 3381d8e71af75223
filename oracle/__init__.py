"""CPU oracle for paged FP8 decode attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product library never calls it; it shares no code with the HIP path.

This module is a thin ctypes wrapper over ``oracle.c`` (plain C99, single-threaded, fp64).
Every function documents the definition it computes in ``oracle.c``; the wrappers only marshal
numpy arrays.  Sources: Cloudflare's "Smaller, faster, safer: running Kimi and GLM at scale"
(Chinese translation on feinterview.poetries.top), sections "量化 KV cache" (FP8 e4m3 KV cache,
converted on read) and "保护共享 KV cache" (per-page tags, batched check, abort on mismatch).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

KV_FP8 = 0
KV_BF16 = 1
ACT_F32 = 0
ACT_BF16 = 1

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain -O2, no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-fno-builtin", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _P(t):
    return ctypes.POINTER(t)


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            L = ctypes.CDLL(_LIB_PATH)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
            L.oracle_e4m3_encode.restype = ctypes.c_uint8
            L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.oracle_e4m3_decode.restype = ctypes.c_double
            L.oracle_quantize_fp8.argtypes = [ctypes.c_float, ctypes.c_float]
            L.oracle_quantize_fp8.restype = ctypes.c_uint8
            L.oracle_bf16_from_f32.argtypes = [ctypes.c_float]
            L.oracle_bf16_from_f32.restype = ctypes.c_uint16
            L.oracle_e4m3_encode_array.argtypes = [vp, i64, vp]
            L.oracle_e4m3_decode_array.argtypes = [vp, i64, vp]
            L.oracle_quantize_fp8_array.argtypes = [vp, ctypes.c_float, i64, vp]
            L.oracle_bf16_from_f32_array.argtypes = [vp, i64, vp]
            L.oracle_kv_scales.argtypes = [vp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, vp]
            L.oracle_kv_absmax_update.argtypes = [vp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, vp]
            L.oracle_scale_from_absmax.argtypes = [ctypes.c_float]
            L.oracle_scale_from_absmax.restype = ctypes.c_float
            L.oracle_kv_append.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i32, vp, vp, i32,
                                           vp, vp, vp, i32, i32, i32, i32, i32, i32]
            L.oracle_kv_tag_verify.argtypes = [vp, i32, vp, vp, vp, i32, vp, i32, i32]
            L.oracle_pages_init.argtypes = [vp, vp, vp, i32]
            L.oracle_w4a16_gemv.argtypes = [vp, vp, vp, i32, i32, i32, vp]
            L.oracle_pages_alloc.argtypes = [vp, vp, vp, i32, vp, vp, i32, vp, vp, i32, vp]
            L.oracle_pages_free.argtypes = [vp, vp, vp, i32, i32, vp]
            L.oracle_kv_transcode_pages.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                                    i32]
            L.oracle_paged_decode_attn.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i32, vp, vp, vp,
                                                   vp, ctypes.c_double, i32, i32, i32, i32, i32, i32, vp]
            L.oracle_paged_decode_attn_rows.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i32, vp, vp,
                                                        vp, vp, ctypes.c_double, i32, i32, i32, i32, i32, vp, vp,
                                                        i32, vp]
            L.oracle_paged_decode_attn_split_rows.argtypes = [vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, i32, vp,
                                                              vp, vp, ctypes.c_double, i32, i32, i32, i32, i32,
                                                              i32, vp, vp, i32, vp]
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _act(a):
    """(array, dt) for an activation array: float32 -> fp32, uint16 -> bf16 bit patterns."""
    if a.dtype == np.float32:
        return _c(a, np.float32), ACT_F32
    if a.dtype == np.uint16:
        return _c(a, np.uint16), ACT_BF16
    raise TypeError(f"activation arrays are float32 or uint16 (bf16 bits), got {a.dtype}")


# ---------------------------------------------------------------- scalar codec definitions

def e4m3_encode(t) -> np.ndarray:
    t = _c(np.atleast_1d(t), np.float32)
    out = np.empty(t.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(t), t.size, _ptr(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = _c(np.atleast_1d(c), np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def quantize_fp8(x, s: float) -> np.ndarray:
    x = _c(np.atleast_1d(x), np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().oracle_quantize_fp8_array(_ptr(x), float(s), x.size, _ptr(out))
    return out


def bf16_from_f32(x) -> np.ndarray:
    x = _c(np.atleast_1d(x), np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_bf16_from_f32_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = _c(np.atleast_1d(h), np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- method steps

def kv_scales(x: np.ndarray) -> np.ndarray:
    """Per-head scale fp32(amax/448) over x : [T][H][D] (fp32 or bf16 bits)."""
    x, dt = _act(x)
    T, H, D = x.shape
    out = np.empty(H, np.float32)
    lib().oracle_kv_scales(_ptr(x), dt, T, H, D, _ptr(out))
    return out


def kv_absmax_update(x: np.ndarray, amax: np.ndarray) -> None:
    """amax[h] = max(amax[h], max |x[:, h, :]|), in place (chunked scale setup)."""
    x, dt = _act(x)
    T, H, D = x.shape
    assert amax.dtype == np.float32 and amax.shape == (H,) and amax.flags.c_contiguous
    lib().oracle_kv_absmax_update(_ptr(x), dt, T, H, D, _ptr(amax))


def scale_from_absmax(amax: np.ndarray) -> np.ndarray:
    return np.array([lib().oracle_scale_from_absmax(float(a)) for a in np.atleast_1d(amax)], np.float32)


def kv_append(k_new, v_new, k_pool, v_pool, kv_dt, page_table, seq_ids, positions, k_scale, v_scale,
              abort_mask=None, *, page_size, num_pages):
    """Quantise-on-append into host pools (modified in place).  Pools are uint8 (FP8 codes) or
    uint16 (bf16 bits) arrays laid out as described in oracle.c."""
    k_new, in_dt = _act(k_new)
    T, Hkv, Dk = k_new.shape
    if v_new is not None:
        v_new, in_dt2 = _act(v_new)
        assert in_dt2 == in_dt
        Dv = v_new.shape[2]
    else:
        Dv = 0
    assert k_pool.flags.c_contiguous and (v_pool is None or v_pool.flags.c_contiguous)
    pt = _c(page_table, np.int32)
    ks = _c(k_scale, np.float32) if k_scale is not None else np.ones(Hkv, np.float32)
    vs = _c(v_scale, np.float32) if v_scale is not None else np.ones(Hkv, np.float32)
    am = _c(abort_mask, np.uint8) if abort_mask is not None else None
    lib().oracle_kv_append(_ptr(k_new), _ptr(v_new), in_dt, _ptr(k_pool), _ptr(v_pool), kv_dt, _ptr(pt),
                           pt.shape[1], _ptr(_c(seq_ids, np.int32)), _ptr(_c(positions, np.int32)), T, _ptr(ks),
                           _ptr(vs), _ptr(am), pt.shape[0], Hkv, Dk, Dv, page_size, num_pages)


def kv_transcode_pages(k_src, v_src, k_dst, v_dst, src_pages, dst_pages, k_scale, v_scale=None, *, page_size):
    """BF16 pool pages -> FP8 pool pages (dst pools modified in place).  k_src/v_src are uint16 (bf16
    bits) pools, k_dst/v_dst uint8 pools, in the layouts described in oracle.c; v_src = v_dst = None
    for shared-KV pools."""
    assert k_src.dtype == np.uint16 and k_dst.dtype == np.uint8
    assert k_src.flags.c_contiguous and k_dst.flags.c_contiguous
    assert (v_src is None) == (v_dst is None)
    ns, Hkv = k_src.shape[0], k_src.shape[1]
    Dk = k_src.size // (ns * Hkv * page_size)
    Dv = 0
    if v_src is not None:
        assert v_src.dtype == np.uint16 and v_dst.dtype == np.uint8
        assert v_src.flags.c_contiguous and v_dst.flags.c_contiguous
        Dv = v_src.size // (ns * Hkv * page_size)
    sp = _c(src_pages, np.int32)
    dp = _c(dst_pages, np.int32)
    assert sp.shape == dp.shape
    ks = _c(k_scale, np.float32)
    vs = _c(v_scale, np.float32) if v_scale is not None else None
    lib().oracle_kv_transcode_pages(_ptr(k_src), _ptr(v_src), _ptr(k_dst), _ptr(v_dst), _ptr(sp), _ptr(dp), sp.size,
                                    _ptr(ks), _ptr(vs), Hkv, Dk, Dv, page_size, ns, k_dst.shape[0])


def w4a16_gemv(x, q, s) -> np.ndarray:
    """y = x . (q * s)^T in fp64.  x : [M][K] bf16 bits (uint16); q : [N][K] int8; s : [N][K/128] fp32."""
    x = _c(x, np.uint16)
    q = _c(q, np.int8)
    s = _c(s, np.float32)
    M, K = x.shape
    N = q.shape[0]
    assert q.shape == (N, K) and s.shape == (N, K // 128) and K % 128 == 0
    y = np.empty((M, N), np.float64)
    lib().oracle_w4a16_gemv(_ptr(x), _ptr(q), _ptr(s), M, N, K, _ptr(y))
    return y


class PageAllocator:
    """The allocator state in host arrays (free_list, free_count, live_tags or None), updated in place
    by the oracle's init / alloc / free."""

    def __init__(self, num_pages: int, tags: bool = True):
        self.num_pages = num_pages
        self.free_list = np.zeros(num_pages, np.int32)
        self.free_count = np.zeros(1, np.int32)
        self.live_tags = np.zeros(num_pages, np.uint32) if tags else None
        lib().oracle_pages_init(_ptr(self.free_list), _ptr(self.free_count), _ptr(self.live_tags), num_pages)

    def alloc(self, counts, first_slot, page_table, expected_tags=None) -> np.ndarray:
        c = _c(counts, np.int32)
        f = _c(first_slot, np.int32)
        assert page_table.dtype == np.int32 and page_table.flags.c_contiguous
        assert expected_tags is None or (expected_tags.dtype == np.uint32 and expected_tags.flags.c_contiguous)
        granted = np.zeros(c.size, np.uint8)
        lib().oracle_pages_alloc(_ptr(self.free_list), _ptr(self.free_count), _ptr(self.live_tags), self.num_pages,
                                 _ptr(c), _ptr(f), c.size, _ptr(page_table), _ptr(expected_tags),
                                 page_table.shape[1], _ptr(granted))
        return granted

    def free(self, pages) -> np.ndarray:
        p = _c(pages, np.int32)
        status = np.zeros(2, np.int32)
        lib().oracle_pages_free(_ptr(self.free_list), _ptr(self.free_count), _ptr(p), p.size, self.num_pages,
                                _ptr(status))
        return status


def kv_tag_verify(page_table, expected_tags, seq_lens, live_tags, *, page_size) -> np.ndarray:
    pt = _c(page_table, np.int32)
    et = _c(expected_tags, np.uint32)
    sl = _c(seq_lens, np.int32)
    lt = _c(live_tags, np.uint32)
    B = pt.shape[0]
    out = np.empty(B, np.uint8)
    lib().oracle_kv_tag_verify(_ptr(pt), pt.shape[1], _ptr(et), _ptr(sl), _ptr(lt), lt.size, _ptr(out), B,
                               page_size)
    return out


def paged_decode_attn(q, k_pool, v_pool, kv_dt, page_table, seq_lens, k_scale, v_scale, abort_mask=None, *,
                      sm_scale, Hkv, Dk, Dv, page_size, rows=None, split=None) -> np.ndarray:
    """fp64 attention.  q : [B][Hq][Dk] (fp32 or bf16 bits).  Returns [B][Hq][Dv] float64, or
    [len(rows)][Dv] when rows = list of (b, h).  split=N uses the N-token partition form."""
    q, q_dt = _act(q)
    B, Hq, _ = q.shape
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    ks = _c(k_scale, np.float32) if k_scale is not None else np.ones(Hkv, np.float32)
    vs = _c(v_scale, np.float32) if v_scale is not None else np.ones(Hkv, np.float32)
    am = _c(abort_mask, np.uint8) if abort_mask is not None else None
    kp = np.ascontiguousarray(k_pool)
    vp = None if v_pool is None else np.ascontiguousarray(v_pool)
    L = lib()
    if rows is None and split is None:
        out = np.empty((B, Hq, Dv), np.float64)
        L.oracle_paged_decode_attn(_ptr(q), q_dt, _ptr(kp), _ptr(vp), kv_dt, _ptr(pt), pt.shape[1], _ptr(sl),
                                   _ptr(ks), _ptr(vs), _ptr(am), float(sm_scale), B, Hq, Hkv, Dk, Dv, page_size,
                                   _ptr(out))
        return out
    if rows is None:
        rows = [(b, h) for b in range(B) for h in range(Hq)]
    rb = np.array([r[0] for r in rows], np.int32)
    rh = np.array([r[1] for r in rows], np.int32)
    out = np.empty((len(rows), Dv), np.float64)
    if split is None:
        L.oracle_paged_decode_attn_rows(_ptr(q), q_dt, _ptr(kp), _ptr(vp), kv_dt, _ptr(pt), pt.shape[1], _ptr(sl),
                                        _ptr(ks), _ptr(vs), _ptr(am), float(sm_scale), Hq, Hkv, Dk, Dv, page_size,
                                        _ptr(rb), _ptr(rh), len(rows), _ptr(out))
    else:
        assert am is None, "split form is used for invariance checks without aborts"
        L.oracle_paged_decode_attn_split_rows(_ptr(q), q_dt, _ptr(kp), _ptr(vp), kv_dt, _ptr(pt), pt.shape[1],
                                              _ptr(sl), _ptr(ks), _ptr(vs), float(sm_scale), Hq, Hkv, Dk, Dv,
                                              page_size, int(split), _ptr(rb), _ptr(rh), len(rows), _ptr(out))
    return out
