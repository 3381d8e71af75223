"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on seeded inputs.

Bar: FP8 codes, bf16 stores, scales and abort masks bit-exact; attention max |err| <= 1e-4 for
fp32 output and <= 1e-2 * max|ref| for bf16 output.  Sizes here span several 32-token windows,
several partitions and ragged tails while keeping the oracle at a few seconds; the full-size
workloads are covered by test_gpu_fullsize.py on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_pipeline import GpuState, check_close, out_to_f64, pool_to_numpy, t_act, t_int
from oracle_pipeline import oracle_step

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu

REDUCED = {
    "tiny_mha": {},
    "gqa": dict(B=6, len_range=(30, 700)),
    "long": dict(B=2, len_range=(4100, 9000)),
    "capacity": dict(B=8, len_range=(200, 1200), stale_rate=5e-3, layers=1, budget_bytes=None),
    "shared_kv": dict(B=3, len_range=(100, 700)),
}


def _case(name, seed=1, **extra):
    kw = dict(REDUCED[name])
    kw.update(extra)
    return synth.make(name, seed=seed, **kw)


@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_pools_scales_and_mask_bit_exact(name, kv):
    print(f"\n[case] pools {name} {kv}", flush=True)
    w = _case(name)
    ref = oracle_step(w, kv)
    st = GpuState(w, kv)
    out, abort = st.step()
    torch.cuda.synchronize()
    if kv == "fp8":
        assert (st.k_scale.cpu().numpy() == ref["k_scale"]).all()
        if ref["v_scale"] is not None:
            assert (st.v_scale.cpu().numpy() == ref["v_scale"]).all()
    assert (pool_to_numpy(st.k_pool) == ref["k_pool"]).all()
    if ref["v_pool"] is not None:
        assert (pool_to_numpy(st.v_pool) == ref["v_pool"]).all()
    assert (abort.cpu().numpy() == ref["abort"]).all()
    assert (ref["abort"] == w.expected_abort).all()


@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("split", [0, 64])
def test_attention_parity(name, kv, split):
    print(f"\n[case] attn {name} {kv} split={split}", flush=True)
    w = _case(name)
    ref = oracle_step(w, kv)
    st = GpuState(w, kv)
    out, _ = st.step(split_tokens=split)
    worst, tol = check_close(out_to_f64(out), ref["out"], w.spec.out_dt)
    print(f"  max|err| {worst:.3e} (tol {tol:.3e})")


@pytest.mark.parametrize("name", ["gqa", "long", "capacity"])
@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_attention_fp32_output_tight(name, kv):
    """fp32 output of the matrix-core path against the 1e-4 absolute bar."""
    print(f"\n[case] attn-f32out {name} {kv}", flush=True)
    w = _case(name, out_dt="f32")
    ref = oracle_step(w, kv)
    st = GpuState(w, kv)
    out, _ = st.step(out_dtype=torch.float32, split_tokens=96)
    check_close(out_to_f64(out), ref["out"], "f32")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_fp32_queries_on_matrix_cores(kv):
    print(f"\n[case] q-f32 gqa {kv}", flush=True)
    w = _case("gqa", q_dt="f32", out_dt="f32")
    ref = oracle_step(w, kv)
    st = GpuState(w, kv)
    assert dapf8.paged_decode_attn_variant(w.B, 32, 8, 128, 128, 16, w.pt_stride)[0].startswith("mfma")
    out, _ = st.step(out_dtype=torch.float32)
    check_close(out_to_f64(out), ref["out"], "f32")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_large_batch_fixed_partition_kernel(kv):
    """Batches above the stream-K limit run the fixed-partition matrix-core kernel."""
    print(f"\n[case] large-batch fixed-partition {kv}", flush=True)
    w = _case("gqa", B=1030, len_range=(1, 40))
    name, split = dapf8.paged_decode_attn_variant(w.B, 32, 8, 128, 128, 16, w.pt_stride)
    assert name == "mfma_g16_d128_p16", name
    ref = oracle_step(w, kv)
    st = GpuState(w, kv)
    for od, tol in ((torch.bfloat16, "bf16"), (torch.float32, "f32")):
        for sp in (0, 32):
            out, _ = st.step(out_dtype=od, split_tokens=sp)
            check_close(out_to_f64(out), ref["out"], tol)


@pytest.mark.parametrize("G,Hkv", [(16, 1), (32, 1), (64, 1), (128, 2)])
def test_latent_kernel_group_sizes(G, Hkv):
    """Shared-KV latent shape on the matrix cores: every supported group size, two KV heads."""
    print(f"\n[case] latent G={G} Hkv={Hkv}", flush=True)
    w = _case("shared_kv", Hq=G * Hkv, Hkv=Hkv, B=3, len_range=(1, 300))
    assert dapf8.paged_decode_attn_variant(w.B, G * Hkv, Hkv, 576, 512, 64, w.pt_stride,
                                           shared_kv=True)[0] == "mfma_latent_d576_p64"
    ref = oracle_step(w, "fp8")
    st = GpuState(w, "fp8")
    for sp in (0, 64, 128):
        out, _ = st.step(split_tokens=sp)
        check_close(out_to_f64(out), ref["out"], "bf16")


def test_latent_kernel_fp32_output_and_fp32_queries():
    """fp32 output (three-term P) on the latent kernel; fp32 queries take the generic kernel."""
    print("\n[case] latent f32 out / f32 q", flush=True)
    w = _case("shared_kv", out_dt="f32")
    ref = oracle_step(w, "fp8")
    st = GpuState(w, "fp8")
    out, _ = st.step(out_dtype=torch.float32)
    check_close(out_to_f64(out), ref["out"], "f32")
    w = _case("shared_kv", q_dt="f32", out_dt="f32")
    ref = oracle_step(w, "fp8")
    st = GpuState(w, "fp8")
    for sp in (0, 64):
        out, _ = st.step(out_dtype=torch.float32, split_tokens=sp)
        check_close(out_to_f64(out), ref["out"], "f32")


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_group_sizes(G):
    print(f"\n[case] G={G}", flush=True)
    w = _case("gqa", Hq=4 * G, Hkv=4, B=3, len_range=(1, 300))
    ref = oracle_step(w, "fp8")
    st = GpuState(w, "fp8")
    out, _ = st.step(split_tokens=128)
    check_close(out_to_f64(out), ref["out"], "bf16")


def test_deterministic_and_split_invariant():
    w = _case("long")
    st = GpuState(w, "fp8")
    a, _ = st.step(split_tokens=4096)
    b, _ = st.step(split_tokens=4096)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    ref = oracle_step(w, "fp8")["out"]
    for sp in (32, 512, 0, 1 << 14):
        o, _ = st.step(split_tokens=sp)
        check_close(out_to_f64(o), ref, "bf16")


def test_physical_page_permutation_gives_identical_bits():
    w = _case("gqa")
    st = GpuState(w, "fp8")
    out1, _ = st.step(verify=False)
    # move every physical page to a new slot and rewrite the page table accordingly
    perm = torch.randperm(st.num_pages, generator=torch.Generator().manual_seed(0)).cuda()
    k2 = torch.empty_like(st.k_pool)
    v2 = torch.empty_like(st.v_pool)
    k2[perm] = st.k_pool
    v2[perm] = st.v_pool
    pt = st.page_table.long()
    pt2 = torch.where(pt >= 0, perm[pt.clamp(min=0)], pt).to(torch.int32).contiguous()
    out2 = dapf8.paged_decode_attn(st.q, k2, v2, pt2, st.seq_lens, st.k_scale, st.v_scale, out_dtype=out1.dtype,
                                   sm_scale=w.spec.scale())
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("variant_dims", [(128, 16), (64, 16), (128, 32)])
def test_dequant_of_every_code_via_single_token_attention(variant_dims):
    """L = 1 makes attention return V_0 exactly; with s_V = 2^-8 every product is exact."""
    D, P = variant_dims
    codes = np.arange(256, dtype=np.uint8)
    nb = 256 // D
    B, Hkv, G = nb, 1, 4
    kp, vp = dapf8.alloc_pools(nb, 1, P, D, D, "fp8")
    for b in range(nb):
        vp[b, 0, :, 0] = torch.from_numpy(codes[b * D:(b + 1) * D]).cuda()
    pt = torch.arange(nb, dtype=torch.int32, device="cuda").view(nb, 1).contiguous()
    lens = torch.ones(nb, dtype=torch.int32, device="cuda")
    q = torch.randn((B, G, D), device="cuda")
    ks = torch.ones(1, device="cuda")
    vs = torch.full((1,), 2.0**-8, device="cuda")
    out = dapf8.paged_decode_attn(q, kp, vp, pt, lens, ks, vs, out_dtype=torch.float32).cpu().numpy()
    expect = oracle.e4m3_decode(codes).reshape(nb, D) * 2.0**-8
    for g in range(G):
        got = out[:, g, :].astype(np.float64)
        nan = np.isnan(expect)
        assert (np.isnan(got) == nan).all()
        assert (got[~nan] == expect[~nan]).all()


def test_verify_random_tables_bit_exact():
    rng = np.random.default_rng(0)
    for trial in range(20):
        B, P, npg, stride = int(rng.integers(1, 300)), int(rng.choice([1, 16, 64])), int(rng.integers(1, 5000)), \
            int(rng.integers(1, 200))
        pt = rng.integers(-3, npg + 3, size=(B, stride)).astype(np.int32)
        live = rng.integers(0, 2**32, size=npg, dtype=np.uint64).astype(np.uint32)
        exp = np.where(pt >= 0, live[np.clip(pt, 0, npg - 1)], 0).astype(np.uint32)
        exp[rng.random((B, stride)) < 1e-3] ^= np.uint32(1)
        lens = rng.integers(-2, stride * P + 5, size=B).astype(np.int32)
        ref = oracle.kv_tag_verify(pt, exp, lens, live, page_size=P)
        got = torch.full((B,), 7, dtype=torch.uint8, device="cuda")
        dapf8.kv_tag_verify(t_int(pt), t_int(exp, torch.uint32), t_int(lens), t_int(live, torch.uint32), got, P)
        assert (got.cpu().numpy() == ref).all(), trial


def test_verify_wide_tables_bit_exact():
    """Page tables wider than one 256 x 4 pass (pt_stride > 1024) take the 1024-thread check:
    long requests over several passes, mismatches placed in the last pass and past the length."""
    rng = np.random.default_rng(1)
    outcomes = set()
    for trial in range(8):
        B, P, npg, stride = int(rng.integers(1, 9)), int(rng.choice([1, 16])), int(rng.integers(100, 70000)), \
            int(rng.integers(1025, 20000))
        pt = rng.integers(0, npg, size=(B, stride)).astype(np.int32)
        live = rng.integers(0, 2**32, size=npg, dtype=np.uint64).astype(np.uint32)
        exp = live[pt].astype(np.uint32)
        lens = rng.integers(0, stride * P + 1, size=B).astype(np.int32)
        for b in range(B):  # a mismatch in some requests: at their last page, or past their length
            n = -(-int(lens[b]) // P)
            if n and rng.random() < 0.5:
                exp[b, n - 1] ^= np.uint32(1 << int(rng.integers(0, 32)))
            elif n < stride:
                exp[b, n] ^= np.uint32(1)
        ref = oracle.kv_tag_verify(pt, exp, lens, live, page_size=P)
        got = torch.full((B,), 7, dtype=torch.uint8, device="cuda")
        dapf8.kv_tag_verify(t_int(pt), t_int(exp, torch.uint32), t_int(lens), t_int(live, torch.uint32), got, P)
        assert (got.cpu().numpy() == ref).all(), trial
        outcomes |= set(int(x) for x in ref)
    assert outcomes == {0, 1}  # aborted and clean requests both occur


def test_empty_and_aborted_rows_are_zero():
    w = _case("gqa", B=4)
    st = GpuState(w, "fp8")
    st.seq_lens[1] = 0
    abort = torch.tensor([0, 0, 1, 0], dtype=torch.uint8, device="cuda")
    for sp in (0, 64):
        out = dapf8.paged_decode_attn(st.q, st.k_pool, st.v_pool, st.page_table, st.seq_lens, st.k_scale,
                                      st.v_scale, abort, out_dtype=torch.float32, split_tokens=sp)
        o = out.cpu()
        assert (o[1] == 0).all() and (o[2] == 0).all() and (o[0] != 0).any() and (o[3] != 0).any()


def test_batch_zero_is_noop_and_bad_args_raise():
    q = torch.zeros((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    kp, vp = dapf8.alloc_pools(1, 2, 16, 128, 128, "fp8")
    pt = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    sl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    s = torch.ones(2, device="cuda")
    dapf8.paged_decode_attn(q, kp, vp, pt, sl, s, s)
    q2 = torch.zeros((1, 6, 128), dtype=torch.bfloat16, device="cuda")     # 6 % 4 heads -> error
    kp2, vp2 = dapf8.alloc_pools(1, 4, 16, 128, 128, "fp8")
    with pytest.raises(dapf8.DapfError):
        dapf8.paged_decode_attn(q2, kp2, vp2, torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
                                torch.ones(1, dtype=torch.int32, device="cuda"), torch.ones(4, device="cuda"),
                                torch.ones(4, device="cuda"))


def test_encode_exhaustive_all_fp32_patterns():
    """Every one of the 2^32 fp32 bit patterns through kv_append (scale 1) against the oracle."""
    import concurrent.futures as cf

    chunk = 1 << 26
    D = 1024
    T = chunk // D
    pt = torch.arange(T, dtype=torch.int32, device="cuda").view(1, T).contiguous()
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    one = torch.ones(1, device="cuda")
    pool = torch.empty((T, 1, D // 64, 1, 64), dtype=torch.uint8, device="cuda")  # page size 1: row order
    with cf.ThreadPoolExecutor(max_workers=16) as ex:
        for start in range(0, 1 << 32, chunk):
            bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
            x = bits.view(np.float32)
            xt = torch.from_numpy(x).cuda().view(T, 1, D)
            dapf8.kv_append(xt, None, pool, None, pt, ids, pos, one, None)
            parts = np.array_split(x, 16)
            refs = list(ex.map(oracle.e4m3_encode, parts))
            got = pool.view(-1).cpu().numpy()
            assert (got == np.concatenate(refs)).all(), hex(start)


def test_append_random_values_and_scales():
    """Quantise-on-append of random (x, s) pairs, bit-exact against the oracle's fp32(x / s) -> e4m3:
    2^25 values over 128 KV heads whose scales are spread log-uniformly over 2^-24 .. 2^24.  Half the
    values are random fp32 bit patterns (every class: zeros, subnormals, NaN, infinities, huge); the
    other half sit at s times a rounding midpoint between neighbouring e4m3 values, so the fp32
    division lands within a few ulps of a tie."""
    import concurrent.futures as cf

    Hkv, D, T = 128, 1024, 256                      # 2^25 values per call
    rng = np.random.default_rng(20261202)
    # e4m3 magnitudes (finite), built here from the format's definition: subnormals m * 2^-9, normals
    # (8 + m) * 2^(e - 10) for e = 1..15 without the NaN code
    mags = [m * 2.0 ** -9 for m in range(8)] + [(8 + m) * 2.0 ** (e - 10) for e in range(1, 16) for m in range(8)]
    mags = np.array(sorted(set(mags))[:-1])          # drop 480 (the NaN code's slot)
    mids = (mags[1:] + mags[:-1]) / 2
    pt = torch.arange(T, dtype=torch.int32, device="cuda").view(1, T).contiguous()
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    pool = torch.empty((T, Hkv, D // 64, 1, 64), dtype=torch.uint8, device="cuda")  # page size 1
    for rep in range(2):
        print(f"\n[case] random (x, s) append rep={rep}", flush=True)
        scales = np.exp2(rng.uniform(-24, 24, size=Hkv)).astype(np.float32)
        bits = rng.integers(0, 2**32, size=(T, Hkv, D // 2), dtype=np.uint64).astype(np.uint32)
        rnd = bits.view(np.float32)
        t = rng.choice(mids, size=(T, Hkv, D // 2)) * rng.choice([-1.0, 1.0], size=(T, Hkv, D // 2))
        near = (t * scales[None, :, None]).astype(np.float32)
        x = np.ascontiguousarray(np.concatenate([rnd, near], axis=2))
        dapf8.kv_append(torch.from_numpy(x).cuda(), None, pool, None, pt, ids, pos, torch.from_numpy(scales).cuda(),
                        None)
        got = pool.cpu().numpy().reshape(T, Hkv, D)   # page size 1: codes in row order
        with cf.ThreadPoolExecutor(max_workers=16) as ex:
            refs = list(ex.map(lambda h: oracle.quantize_fp8(np.ascontiguousarray(x[:, h, :]), float(scales[h])),
                               range(Hkv)))
        for h in range(Hkv):
            assert (got[:, h, :] == refs[h].reshape(T, D)).all(), (rep, h, float(scales[h]))
