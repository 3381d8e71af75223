"""GPU parity of the device page allocator (kv_pages_init / kv_pages_alloc / kv_pages_free) against
the oracle: after every operation of seeded random sequences the whole state -- free stack, count,
live tags, page table, expected tags, grant flags and free status -- is bit-exact.  Batches span
several 1024-request scan chunks and allocations of thousands of pages."""
import numpy as np
import pytest
import torch

import oracle

import decode_attention_paged_fp8_amd as dapf8

pytestmark = pytest.mark.gpu


def _u32(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("tags", [True, False])
@pytest.mark.parametrize("seed", [1, 2])
def test_random_sequences_bit_exact(tags, seed):
    print(f"\n[case] pages seed={seed} tags={tags}", flush=True)
    rng = np.random.default_rng(seed)
    N, stride, Bmax = 6000, 16, 3000
    fl, fc, lt = dapf8.alloc_page_allocator(N, tags)
    ref = oracle.PageAllocator(N, tags)
    pt = torch.full((Bmax, stride), -1, dtype=torch.int32, device="cuda")
    et = torch.zeros((Bmax, stride), dtype=torch.int32, device="cuda")
    pt_ref = np.full((Bmax, stride), -1, np.int32)
    et_ref = np.zeros((Bmax, stride), np.uint32)
    held = []
    for step in range(14):
        if step % 3 != 2:
            B = int(rng.choice([1, 7, 1024, 1500, Bmax]))
            counts = rng.integers(-1, 6, size=B).astype(np.int32)
            if step == 0:
                counts[0] = 1500  # one request needing more than a scan chunk of pages (and a long row)
            first = rng.integers(-1, stride, size=B).astype(np.int32)
            first[0] = 0
            row = np.zeros((B, stride), np.int32)
            if step == 0:
                row = np.zeros((B, 2048), np.int32)
            pt_b = torch.full(row.shape, -1, dtype=torch.int32, device="cuda")
            et_b = torch.zeros(row.shape, dtype=torch.int32, device="cuda")
            pr, er = np.full(row.shape, -1, np.int32), np.zeros(row.shape, np.uint32)
            g = dapf8.kv_pages_alloc(fl, fc, lt, torch.from_numpy(counts).cuda(), torch.from_numpy(first).cuda(),
                                     pt_b, et_b if tags else None)
            gr = ref.alloc(counts, first, pr, er if tags else None)
            torch.cuda.synchronize()
            assert (g.cpu().numpy() == gr).all(), step
            assert (pt_b.cpu().numpy() == pr).all(), step
            if tags:
                assert (_u32(et_b) == er).all(), step
            for b in np.nonzero(gr)[0]:
                n, f = int(counts[b]), int(first[b])
                held.extend(pr[b, f:f + n].tolist())
        else:
            k = int(rng.integers(0, len(held) + 1)) if held else 0
            idx = rng.permutation(len(held))[:k]
            pages = [held[i] for i in idx]
            gone = set(idx.tolist())
            held = [h for i, h in enumerate(held) if i not in gone]
            pages += [-3, N + 10]  # rejected ids
            pages = np.array(rng.permutation(pages), np.int32)
            st = dapf8.kv_pages_free(fl, fc, torch.from_numpy(pages).cuda())
            sr = ref.free(pages)
            torch.cuda.synchronize()
            assert (st.cpu().numpy() == sr).all(), step
        assert int(fc[0].item()) == int(ref.free_count[0]), step
        assert (fl.cpu().numpy() == ref.free_list).all(), step
        if tags:
            assert (_u32(lt) == ref.live_tags).all(), step


def test_max_batch_and_empty_calls():
    print("\n[case] pages max batch", flush=True)
    N = 9000
    fl, fc, lt = dapf8.alloc_page_allocator(N)
    ref = oracle.PageAllocator(N)
    B = 8192
    counts = np.ones(B, np.int32)
    first = np.zeros(B, np.int32)
    pt = torch.full((B, 1), -1, dtype=torch.int32, device="cuda")
    et = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    pr, er = np.full((B, 1), -1, np.int32), np.zeros((B, 1), np.uint32)
    g = dapf8.kv_pages_alloc(fl, fc, lt, torch.from_numpy(counts).cuda(), torch.from_numpy(first).cuda(), pt, et)
    gr = ref.alloc(counts, first, pr, er)
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    st = dapf8.kv_pages_free(fl, fc, e)
    g0 = dapf8.kv_pages_alloc(fl, fc, lt, e, e, pt, et)
    torch.cuda.synchronize()
    assert (g.cpu().numpy() == gr).all() and (pt.cpu().numpy() == pr).all() and (_u32(et) == er).all()
    assert list(st.cpu().numpy()) == [0, 0] and g0.numel() == 0
    assert int(fc[0].item()) == N - B


def test_page_counts_summing_past_32_bits():
    # valid page counts adding up to more than 2^31 (8192 requests of 262208 pages): only the first
    # request (3 pages) fits; the 64-bit prefix refuses every later one
    print("\n[case] pages counts past 2^31", flush=True)
    B, stride, N = 8192, 262208, 100
    fl, fc, lt = dapf8.alloc_page_allocator(N)
    ref = oracle.PageAllocator(N)
    counts = np.full(B, stride, np.int32)
    counts[0] = 3
    first = np.zeros(B, np.int32)
    pt = torch.full((B, stride), -1, dtype=torch.int32, device="cuda")  # 8.6 GB
    pr = np.empty((B, stride), np.int32)
    pr[0] = -1
    g = dapf8.kv_pages_alloc(fl, fc, lt, torch.from_numpy(counts).cuda(), torch.from_numpy(first).cuda(), pt)
    gr = ref.alloc(counts, first, pr)
    torch.cuda.synchronize()
    assert (g.cpu().numpy() == gr).all() and gr[0] == 1 and not gr[1:].any()
    assert (pt[0].cpu().numpy() == pr[0]).all()
    for r in (1, 2, B // 2, B - 1):
        assert bool((pt[r] == -1).all()), r
    assert int(fc[0].item()) == int(ref.free_count[0]) == N - 3
    assert (fl.cpu().numpy() == ref.free_list).all() and (_u32(lt) == ref.live_tags).all()
    del pt
    torch.cuda.empty_cache()
