"""The frozen oracle fixture and the seeded input generator.

tests/golden/tiny_mha_seed1.txt was written by tests/golden/make_golden.py, which calls only the
oracle and the input generator; re-rendering it must reproduce the file byte for byte.  The pages
print no worked example of the kernel's arithmetic, so no fixture holds values quoted from them.
"""
import os
import sys

import numpy as np
import pytest

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_reproduces_frozen_fixture():
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_golden

    with open(os.path.join(HERE, "golden", "tiny_mha_seed1.txt")) as f:
        assert make_golden.render() == f.read()


@pytest.mark.parametrize("name", ["tiny_mha", "gqa", "long", "capacity", "shared_kv"])
def test_workload_structure(name):
    w = synth.make(name, seed=3)
    s = w.spec
    P = s.page_size
    assert w.q.shape == (s.B, s.Hq, s.Dk)
    assert w.q.dtype == (np.float32 if s.q_dt == "f32" else np.uint16)
    assert (w.seq_lens >= 1).all()
    if s.lens is None:
        lo, hi = s.len_range
        assert (w.ctx_lens >= lo).all() and (w.ctx_lens <= hi).all()
    assert (w.seq_lens - w.ctx_lens == (1 if s.append else 0)).all()
    used = []
    for b in range(s.B):
        n = w.n_pages(b)
        row = w.page_table[b]
        assert (row[:n] >= 0).all() and (row[:n] < w.num_pages).all() and (row[n:] == -1).all()
        used.extend(row[:n].tolist())
    assert len(used) == len(set(used))                  # no physical page shared by two requests
    if s.stale == "none":
        assert w.expected_abort.sum() == 0
        for b in range(s.B):
            n = w.n_pages(b)
            assert (w.expected_tags[b, :n] == w.live_tags[w.page_table[b, :n]]).all()


def test_workload_determinism_and_sequence_streams():
    a = synth.make("gqa", seed=5, B=4, len_range=(40, 90))
    b = synth.make("gqa", seed=5, B=4, len_range=(40, 90))
    assert (a.q == b.q).all() and (a.page_table == b.page_table).all()
    k1, v1 = a.kv_tokens(2)
    k2, v2 = b.kv_tokens(2, t0=10, t1=20)
    assert (k1[10:20] == k2).all() and (v1[10:20] == v2).all()
    c = synth.make("gqa", seed=6, B=4, len_range=(40, 90))
    assert not (a.q == c.q).all()


def test_capacity_budget_fits_fp8_not_bf16():
    s = synth.SPECS["capacity"]
    fp8_pages = synth.pages_per_layer(s, "fp8")
    bf16_pages = synth.pages_per_layer(s, "bf16")
    worst = s.B * -(-(s.len_range[1] + 1) // s.page_size)
    assert fp8_pages >= worst > bf16_pages
    assert 61 * fp8_pages * 16 * 8 * 256 <= 80 * 10**9


def test_outlier_channels():
    w = synth.make("gqa", seed=1, B=2, len_range=(30, 40))
    assert len(w.k_outliers[0]) == 10 and len(w.v_outliers[0]) == 10
