"""Pins of the oracle's INT4 weight-only GEMV (Cloudflare, "Smaller, faster, safer": GLM weights
compressed from 8-bit floats to 4-bit integers to speed memory-bound decode; here synthetic).

Pinned by closed forms -- all-ones weights with unit scales give row sums of x; one-hot weights
pick single activations times their group's scale -- and by brute force in plain Python on small
random cases (a dropped scale, a transposed operand or a wrong group index fails these)."""
import numpy as np

import oracle
import synth


def _x(rng, M, K):
    return synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))


def test_all_ones_gives_row_sums():
    rng = np.random.default_rng(1)
    M, N, K = 3, 5, 256
    xb = _x(rng, M, K)
    x = synth.bf16_bits_to_f32(xb).astype(np.float64)
    y = oracle.w4a16_gemv(xb, np.ones((N, K), np.int8), np.ones((N, K // 128), np.float32))
    assert np.allclose(y, np.repeat(x.sum(axis=1, keepdims=True), N, axis=1), rtol=0, atol=1e-12)


def test_one_hot_picks_scaled_activation():
    rng = np.random.default_rng(2)
    M, N, K = 2, 4, 384
    xb = _x(rng, M, K)
    x = synth.bf16_bits_to_f32(xb).astype(np.float64)
    q = np.zeros((N, K), np.int8)
    picks = [5, 200, 383, 128]
    vals = [-8, 7, 3, -1]
    for n, (k, v) in enumerate(zip(picks, vals)):
        q[n, k] = v
    s = (rng.random((N, K // 128)) + 0.5).astype(np.float32)
    y = oracle.w4a16_gemv(xb, q, s)
    for n, (k, v) in enumerate(zip(picks, vals)):
        assert np.array_equal(y[:, n], x[:, k] * v * float(s[n, k // 128]))


def test_brute_force_small():
    rng = np.random.default_rng(3)
    for trial in range(5):
        M, N, K = int(rng.integers(1, 4)), int(rng.integers(1, 5)), 128 * int(rng.integers(1, 4))
        xb = _x(rng, M, K)
        x = synth.bf16_bits_to_f32(xb).astype(np.float64)
        q = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        s = (rng.random((N, K // 128)) * 0.1).astype(np.float32)
        y = oracle.w4a16_gemv(xb, q, s)
        for m in range(M):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += float(x[m, k]) * int(q[n, k]) * float(s[n, k // 128])
                assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
