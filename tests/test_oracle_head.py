"""Pins for the oracle's vocabulary projection (CPU only).

Full head z = W_full h and SlimSpec's factorised head z = W_up W_down h
("SlimSpec: Low-Rank Draft LM-Head ...", gist.science, '방법론 / 아키텍처').
Pins: explicit loops on tiny sizes (brute force), associativity of the low-rank
product against the dense (W_up W_down) h, scipy's logsumexp for the row
normaliser, and softmax rows summing to one.
"""
import math

import numpy as np
import scipy.special

import oracle
from verification_step_amd import workloads as wl


def test_full_head_brute_force_loops():
    rng = np.random.default_rng(0)
    M, d, V = 3, 6, 11
    H = rng.standard_normal((M, d))
    Wf = rng.standard_normal((V, d)).astype(np.float32)
    z, lse = oracle.lm_head_full(H, Wf, 1.0, "f32", block=4)
    for r in range(M):
        for v in range(V):
            ref = math.fsum(float(Wf[v, k]) * float(H[r, k]) for k in range(d))
            assert z[r, v] == np.float32(ref)
    assert np.abs(lse - scipy.special.logsumexp(z.astype(np.float64), axis=1)).max() < 1e-13


def test_full_head_bf16_weights_decode_and_temperature():
    rng = np.random.default_rng(1)
    M, d, V = 2, 32, 50
    H = rng.standard_normal((M, d))
    w32 = rng.standard_normal((V, d)).astype(np.float32)
    bits = wl.f32_to_bf16_bits(w32)
    z, lse = oracle.lm_head_full(H, bits, 0.7, "bf16")
    Wexact = np.array([[float(np.float32(np.uint32(int(b) << 16).view(np.float32))) for b in row]
                       for row in bits])
    assert np.abs(z - (H @ Wexact.T).astype(np.float32)).max() == 0.0
    assert np.abs(lse - scipy.special.logsumexp(z.astype(np.float64) / 0.7, axis=1)).max() < 1e-13
    p = oracle.head_softmax(z, lse, 0.7)
    assert np.abs(p.sum(axis=1) - 1.0).max() < 1e-13


def test_lowrank_equals_dense_product():
    rng = np.random.default_rng(2)
    M, d, r, V = 7, 64, 8, 300
    H = rng.standard_normal((M, d))
    Wd = wl.f32_to_bf16_bits(rng.standard_normal((r, d)).astype(np.float32) / 8)
    Wu = wl.f32_to_bf16_bits(rng.standard_normal((V, r)).astype(np.float32) / 3)
    z, lse, t = oracle.lm_head_lowrank(H, Wd, Wu, 1.0, "bf16", block=128)
    Wd64 = oracle.bf16_bits_to_f64(Wd)
    Wu64 = oracle.bf16_bits_to_f64(Wu)
    dense = H @ (Wu64 @ Wd64).T                       # (W_up W_down) h, other association
    assert np.abs(z.astype(np.float64) - dense).max() <= 1e-6 * np.abs(dense).max()
    assert np.abs(t - H @ Wd64.T).max() < 1e-12


def test_lowrank_rank_full_identity_reduces_to_full_head():
    """With r = d and W_down = I, the factorised head is the full head W_up."""
    rng = np.random.default_rng(3)
    M, d, V = 2, 16, 40
    H = rng.standard_normal((M, d))
    Wu = rng.standard_normal((V, d)).astype(np.float32)
    z1, l1, _ = oracle.lm_head_lowrank(H, np.eye(d, dtype=np.float32), Wu, 1.0, "f32")
    z2, l2 = oracle.lm_head_full(H, Wu, 1.0, "f32")
    assert np.array_equal(z1, z2) and np.allclose(l1, l2, rtol=0, atol=1e-14)
