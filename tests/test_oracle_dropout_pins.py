"""Pins for the dropout form of the oracle (oracle/dropout.py), on the CPU.

  * generator: Philox4x32-10 reproduces the published known-answer vectors
    (tests/golden/philox4x32_10_kat.json);
  * keep mask: the fraction kept matches T / 256 within binomial noise, neighbouring pairs are
    kept independently, and keep_prob = 1 keeps everything (the result is then the oracle
    without dropout, bit for bit);
  * forward: pure-Python loops (math.exp) with the same mask agree; averaged over many seeds the
    output approaches the output without dropout (the scale 256 / T makes each kept weight
    unbiased);
  * backward: central finite differences of sum(dO * O) with the mask held fixed agree with the
    chain-rule gradients.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle.attention import band_visible, head_attention_band_fp64
from oracle.dropout import (head_attention_bwd_dropout_fp64, head_attention_dropout_fp64, keep_mask, keep_threshold,
                            philox4x32_10)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_philox_known_answers():
    for vec in json.load(open(GOLDEN))["vectors"]:
        c = [np.array([int(x, 16)]) for x in vec["counter"]]
        k = [int(x, 16) for x in vec["key"]]
        out = philox4x32_10(*c, *k)
        assert [int(o[0]) for o in out] == [int(x, 16) for x in vec["output"]]


def test_threshold():
    assert keep_threshold(1.0) == 256 and keep_threshold(0.5) == 128 and keep_threshold(0.0) == 1
    assert keep_threshold(0.9) == 230 and keep_threshold(0.3) == 77


@pytest.mark.parametrize("keep", [0.9, 0.5, 0.3])
def test_keep_fraction_and_independence(keep):
    Z = keep_mask(12345, 7, 3, np.arange(512), np.arange(512), keep)
    p = keep_threshold(keep) / 256.0
    n = Z.size
    assert abs(Z.mean() - p) <= 5 * math.sqrt(p * (1 - p) / n)
    both = (Z[:, :-1] & Z[:, 1:]).mean()
    assert abs(both - p * p) <= 5 * math.sqrt(p * p * (1 - p * p) / Z[:, 1:].size)
    rows = (Z[:-1] & Z[1:]).mean()
    assert abs(rows - p * p) <= 5 * math.sqrt(p * p * (1 - p * p) / Z[1:].size)


def test_keep_one_is_no_dropout():
    g = np.random.Generator(np.random.PCG64(1))
    q, k, v = (g.standard_normal((70, 16)) for _ in range(3))
    Z = keep_mask(5, 0, 0, np.arange(70), np.arange(70), 1.0)
    assert Z.all()
    O, L = head_attention_dropout_fp64(q, k, v, 0.25, None, 0, 0, Z, 1.0)
    O0, L0 = head_attention_band_fp64(q, k, v, 0.25, None, 0, 0)
    np.testing.assert_array_equal(L, L0)
    np.testing.assert_allclose(O, O0, rtol=1e-13, atol=1e-15)


def test_forward_brute_force():
    g = np.random.Generator(np.random.PCG64(2))
    n, N, d = 6, 9, 3
    q, k, v = (g.standard_normal((r, d)) for r in (n, N, N))
    Z = keep_mask(99, 1, 4, np.arange(n), np.arange(N), 0.6)
    O, L = head_attention_dropout_fp64(q, k, v, 0.7, 4, 1, 3, Z, 0.6)
    vis = band_visible(np.arange(n), np.arange(N), 4, 1, 3)
    inv = 256.0 / keep_threshold(0.6)
    for i in range(n):
        js = [j for j in range(N) if vis[i, j]]
        s = {j: 0.7 * sum(q[i, c] * k[j, c] for c in range(d)) for j in js}
        m = max(s.values())
        den = math.fsum(math.exp(s[j] - m) for j in js)
        assert abs(L[i] - (m + math.log(den))) <= 1e-13 * max(1.0, abs(L[i]))
        for c in range(d):
            want = math.fsum(math.exp(s[j] - m) / den * Z[i, j] * inv * v[j, c] for j in js)
            assert abs(O[i, c] - want) <= 1e-13


def test_expectation_over_seeds_is_undropped():
    g = np.random.Generator(np.random.PCG64(3))
    q, k, v = (g.standard_normal((8, 4)) for _ in range(3))
    O0, _ = head_attention_band_fp64(q, k, v, 0.5, None, None, 0)
    acc = np.zeros_like(O0)
    S = 4000
    for seed in range(S):
        Z = keep_mask(seed, 0, 0, np.arange(8), np.arange(8), 0.5)
        acc += head_attention_dropout_fp64(q, k, v, 0.5, None, None, 0, Z, 0.5)[0]
    # per element the sample mean's standard error is below 0.02 here
    assert np.abs(acc / S - O0).max() <= 0.05


def test_backward_finite_differences():
    g = np.random.Generator(np.random.PCG64(4))
    n, N, d = 5, 7, 3
    q, k, v = (g.standard_normal((r, d)) for r in (n, N, N))
    do = g.standard_normal((n, d))
    Z = keep_mask(17, 2, 1, np.arange(n), np.arange(N), 0.7)
    args = (0.6, None, 0, 2, Z, 0.7)
    got = head_attention_bwd_dropout_fp64(q, k, v, do, *args)
    h = 1e-6
    for which, gr in zip(range(3), got):
        x = [q.copy(), k.copy(), v.copy()]
        fd = np.zeros_like(x[which])
        for idx in np.ndindex(fd.shape):
            x0 = x[which][idx]
            x[which][idx] = x0 + h
            lp = np.sum(do * head_attention_dropout_fp64(*x, *args)[0])
            x[which][idx] = x0 - h
            lm = np.sum(do * head_attention_dropout_fp64(*x, *args)[0])
            x[which][idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        assert np.abs(gr - fd).max() <= 1e-7 * max(1.0, np.abs(fd).max())
