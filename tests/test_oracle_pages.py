"""Pins of the oracle's page allocator and tag tracker (Cloudflare, "Smaller, faster, safer",
section 保护共享 KV cache: every physical page carries a tag that changes when the page is
reallocated; requests record the (page, tag) pairs they expect; a mismatch aborts the request).

Pinned by worked cases whose pages and tags follow from the stack discipline by hand, by
invariants over long random operation sequences checked against a brute-force Python model of the
pool (every page is either free exactly once or owned by exactly one live request slot; a page's
tag counts how often it was handed out), and end to end through the oracle's tag check: a request
that still holds a page that was freed and handed to another request is aborted, and only then.
"""
import numpy as np

import oracle


def _pt(B, stride):
    return np.full((B, stride), -1, np.int32), np.zeros((B, stride), np.uint32)


def test_worked_example():
    a = oracle.PageAllocator(10)
    assert list(a.free_list) == list(range(9, -1, -1)) and a.free_count[0] == 10
    pt, et = _pt(2, 4)
    g = a.alloc([2, 3], [0, 1], pt, et)
    assert list(g) == [1, 1]
    assert list(pt[0, :2]) == [0, 1] and list(pt[1, 1:4]) == [2, 3, 4]
    assert (et[0, :2] == 1).all() and (et[1, 1:4] == 1).all() and pt[1, 0] == -1
    assert a.free_count[0] == 5
    st = a.free([1, 3])
    assert list(st) == [2, 0] and a.free_count[0] == 7
    pt2, et2 = _pt(1, 4)
    g = a.alloc([3], [0], pt2, et2)
    # last pushed comes out first: 3, then 1, then the old top 5
    assert list(g) == [1] and list(pt2[0, :3]) == [3, 1, 5]
    assert list(et2[0, :3]) == [2, 2, 1]
    assert list(a.live_tags[:6]) == [1, 2, 1, 2, 1, 1]


def test_prefix_grant_and_invalid_requests():
    a = oracle.PageAllocator(8)
    pt, et = _pt(5, 4)
    # request 1 is invalid (range past the row) and asks for nothing; request 3 does not fit,
    # so request 4 is refused even though one page would fit
    g = a.alloc([2, 3, 4, 3, 1], [0, 2, 0, 0, 0], pt, et)
    assert list(g) == [1, 0, 1, 0, 0]
    assert a.free_count[0] == 2
    assert (pt[1] == -1).all() and (pt[3] == -1).all() and (pt[4] == -1).all()
    # negative count / slot: refused, later valid requests still served
    g = a.alloc([-1, 1, 1], [0, -2, 3], *_pt(3, 4))
    assert list(g) == [0, 0, 1] and a.free_count[0] == 1


def test_free_rejects_bad_ids_and_overflow():
    a = oracle.PageAllocator(4)
    pt, et = _pt(1, 4)
    a.alloc([3], [0], pt, et)
    st = a.free([7, -1, 2, 1, 0])  # 2 out of range; room for 3
    assert list(st) == [3, 2] and a.free_count[0] == 4
    st = a.free([3])
    assert list(st) == [0, 1]


def test_no_op_tracker():
    a = oracle.PageAllocator(6, tags=False)
    pt, et = _pt(2, 3)
    g = a.alloc([2, 2], [0, 1], pt, et)
    assert list(g) == [1, 1] and a.live_tags is None
    assert (et == 0).all() and list(pt[0, :2]) == [0, 1] and list(pt[1, 1:3]) == [2, 3]


def test_random_sequences_against_brute_force_model():
    rng = np.random.default_rng(4)
    for trial in range(30):
        N = int(rng.integers(1, 60))
        stride = int(rng.integers(1, 9))
        a = oracle.PageAllocator(N)
        free = list(range(N - 1, -1, -1))  # model stack, top last
        tags = [0] * N
        owned = {}  # (request id, slot) -> (page, tag)
        rid = 0
        for step in range(40):
            if rng.random() < 0.6:
                B = int(rng.integers(0, 5))
                counts = rng.integers(-1, 5, size=B).astype(np.int32)
                first = rng.integers(-1, stride + 1, size=B).astype(np.int32)
                pt, et = _pt(B, stride)
                g = a.alloc(counts, first, pt, et)
                stop = False
                for b in range(B):
                    n, f = int(counts[b]), int(first[b])
                    valid = n >= 0 and f >= 0 and f + n <= stride
                    want = 0
                    if valid and not stop and n <= len(free):
                        want = 1
                        for j in range(n):
                            p = free.pop()
                            tags[p] += 1
                            assert pt[b, f + j] == p and et[b, f + j] == tags[p]
                            owned[(rid + b, f + j)] = (p, tags[p])
                    elif valid:
                        stop = True
                    assert g[b] == want, (trial, step, b)
                rid += B
            elif owned:
                keys = list(owned)
                pick = rng.choice(len(keys), size=int(rng.integers(1, min(6, len(keys)) + 1)), replace=False)
                pages = [owned.pop(keys[i])[0] for i in pick]
                st = a.free(np.array(pages, np.int32))
                assert list(st) == [len(pages), 0]
                free.extend(pages)
            # invariants: the stack is the model's; free + owned pages partition the pool
            assert a.free_count[0] == len(free) and list(a.free_list[:len(free)]) == free
            live = [v[0] for v in owned.values()]
            assert sorted(free + live) == list(range(N))
            assert list(a.live_tags) == tags


def test_reallocated_page_fails_the_tag_check():
    a = oracle.PageAllocator(6)
    P = 4
    pt, et = _pt(2, 3)
    a.alloc([2, 2], [0, 0], pt, et)      # request 0: pages 0, 1; request 1: pages 2, 3
    lens = np.array([8, 8], np.int32)
    assert list(oracle.kv_tag_verify(pt, et, lens, a.live_tags, page_size=P)) == [0, 0]
    a.free(pt[0, :2].copy())             # request 0 ends (but a stale copy of its row survives)
    assert list(oracle.kv_tag_verify(pt, et, lens, a.live_tags, page_size=P)) == [0, 0]  # freeing changes no tag
    pt2, et2 = _pt(1, 3)
    a.alloc([1], [0], pt2, et2)          # page 1 handed to a new request
    assert pt2[0, 0] == 1
    got = oracle.kv_tag_verify(pt, et, lens, a.live_tags, page_size=P)
    assert list(got) == [1, 0]           # the stale holder of page 1 aborts; request 1 is untouched
    assert list(oracle.kv_tag_verify(pt2, et2, np.array([3], np.int32), a.live_tags, page_size=P)) == [0]


def test_page_counts_summing_past_32_bits():
    # 8192 valid requests whose page counts add up to more than 2^31: the first fits, the second
    # does not, so every later request is refused -- whatever a 32-bit running sum would wrap to
    B, stride = 8192, 262208
    assert (B - 1) * stride > 2 ** 31
    a = oracle.PageAllocator(100)
    counts = np.full(B, stride, np.int32)
    counts[0] = 3
    first = np.zeros(B, np.int32)
    pt = np.empty((B, stride), np.int32)  # only row 0 is ever written (untouched pages stay virtual)
    pt[0, :4] = -1
    g = a.alloc(counts, first, pt)
    assert g[0] == 1 and not g[1:].any()
    assert list(pt[0, :4]) == [0, 1, 2, -1] and a.free_count[0] == 97
    assert list(a.live_tags[:4]) == [1, 1, 1, 0]
