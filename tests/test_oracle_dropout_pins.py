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
    chain-rule gradients;
  * backward bar (oracle/backward.py magnitudes with ``drop``): pure-Python enumeration of every
    chain-rule term with its Z / keep factor gives the same magnitude sums; they bound the
    gradients; a numpy emulation of the stated precision (16-bit P and dS in the products, fp32
    sums) stays inside the bar, and planted slips (dP not masked, dV not rescaled, the mask read
    transposed, D from the undropped output) exceed it.
"""
import json
import math
import os

import numpy as np
import pytest

from exact_attention_114_amd import inputs as I
from oracle.attention import band_visible, head_attention_band_fp64
from oracle.backward import bwd_parity_bar, head_attention_bwd_magnitude_fp64
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


# ------------------------------------------------------------------ backward bar with dropout

def enumerate_drop_magnitudes(q, k, v, do, scale, band, Z, keep):
    """Every term of every gradient element with dropout, magnitudes summed in pure Python."""
    n, d = q.shape
    N = k.shape[0]
    O, L = head_attention_dropout_fp64(q, k, v, scale, *band, Z, keep)
    vis = band_visible(np.arange(n), np.arange(N), *band)
    inv = 256.0 / keep_threshold(keep)
    P = [[math.exp(scale * sum(q[i, c] * k[j, c] for c in range(d)) - L[i]) if vis[i, j] else 0.0
          for j in range(N)] for i in range(n)]
    mq = np.zeros((n, d))
    mk = np.zeros((N, d))
    mv = np.zeros((N, d))
    for i in range(n):
        for j in range(N):
            z = Z[i, j] * inv
            for c in range(d):
                mv[j, c] += abs(z * P[i][j] * do[i, c])
                for c2 in range(d):
                    # dP_ij holds (Z_ij / keep) dO_ic2 V_jc2; D_i holds dO_ic2 O_ic2
                    mq[i, c] += abs(scale * P[i][j] * z * do[i, c2] * v[j, c2] * k[j, c])
                    mq[i, c] += abs(scale * P[i][j] * do[i, c2] * O[i, c2] * k[j, c])
                    mk[j, c] += abs(scale * P[i][j] * z * do[i, c2] * v[j, c2] * q[i, c])
                    mk[j, c] += abs(scale * P[i][j] * do[i, c2] * O[i, c2] * q[i, c])
    return mq, mk, mv


def test_drop_magnitudes_equal_term_enumeration():
    g = np.random.Generator(np.random.PCG64(40))
    n, N, d = 5, 8, 3
    q, k, v = (g.standard_normal((r, d)) for r in (n, N, N))
    do = g.standard_normal((n, d))
    Z = keep_mask(8, 3, 2, np.arange(n), np.arange(N), 0.6)
    assert 0 < Z.sum() < Z.size
    band = (5, 1, 3)
    got = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.8, False, band=band, drop=(Z, 0.6))
    want = enumerate_drop_magnitudes(q, k, v, do, 0.8, band, Z, 0.6)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)


def test_drop_magnitudes_dominate_gradients():
    g = np.random.Generator(np.random.PCG64(41))
    q, k, v, do = (g.standard_normal((40, 8)) for _ in range(4))
    for keep, band in ((0.5, (None, 0, 0)), (0.9, (None, None, 0)), (0.2, (7, 3, 0))):
        Z = keep_mask(3, 1, 0, np.arange(40), np.arange(40), keep)
        grads = head_attention_bwd_dropout_fp64(q, k, v, do, 0.4, *band, Z, keep)
        mags = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.4, False, band=band, drop=(Z, keep))
        for a, b in zip(grads, mags):
            assert (np.abs(a) <= b * (1 + 1e-12)).all()


def round16(x, dt):
    x = np.asarray(x, dtype=np.float32)
    return I.bits_to_f64(I.to_bits(x, dt), dt).astype(np.float32)


def emulate_drop_head(q, k, v, do, o_used, lse, scale, band, Z, keep, dt, slip=None):
    """One head's gradients with dropout in the stated precision: S, dP, D and every sum in fp32,
    P (masked) and dS rounded to the input type before the products that consume them."""
    f = np.float32
    q, k, v, do, o_used = (np.asarray(x, dtype=f) for x in (q, k, v, do, o_used))
    n, N = q.shape[0], k.shape[0]
    inv = f(256.0 / keep_threshold(keep))
    Zf = np.asarray(Z.T if slip == "mask_transposed" else Z, dtype=f)
    S = (q @ k.T) * f(scale)
    vis = band_visible(np.arange(n), np.arange(N), *band)
    P = np.where(vis, np.exp(S - np.asarray(lse, dtype=f)[:, None]), f(0)).astype(f)
    dv = round16(P * Zf, dt).T @ do
    if slip != "dv_unscaled":
        dv = dv * inv
    dP = do @ v.T
    if slip != "dp_unmasked":
        dP = dP * Zf * inv
    D = np.sum(do * o_used, axis=1, dtype=f)
    dS = round16(P * (dP - D[:, None]), dt)
    return (dS @ k) * f(scale), (dS.T @ q) * f(scale), dv


def drop_case(n, d, keep, dt, seed, band):
    g = np.random.Generator(np.random.PCG64(seed))
    q, k, v, do = (I.bits_to_f64(I.to_bits(g.standard_normal((n, d), dtype=np.float32), dt), dt)
                   for _ in range(4))
    Z = keep_mask(seed, 0, 0, np.arange(n), np.arange(n), keep)
    O, L = head_attention_dropout_fp64(q, k, v, 0.25, *band, Z, keep)
    return q, k, v, do, O, L, Z


def bar_ratio(q, k, v, do, O, L, Z, keep, dt, band, slip=None, o_used=None):
    n, d = q.shape
    got = emulate_drop_head(q, k, v, do, O if o_used is None else o_used, L, 0.25, band, Z, keep, dt, slip)
    ref = head_attention_bwd_dropout_fp64(q, k, v, do, 0.25, *band, Z, keep)
    mags = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.25, False, band=band, drop=(Z, keep))
    worst = 0.0
    for gg, r, m in zip(got, ref, mags):
        bar = bwd_parity_bar(m, {I.F16: 2.0 ** -11, I.BF16: 2.0 ** -8}[dt], d, n)
        worst = max(worst, float((np.abs(gg - r) / np.maximum(bar, 1e-300)).max()))
    return worst


@pytest.mark.parametrize("dt", [I.F16, I.BF16])
@pytest.mark.parametrize("keep,band", [(0.9, (None, 0, 0)), (0.5, (None, None, 0)), (0.2, (20, 5, 0))])
def test_drop_bar_holds_for_stated_precision(dt, keep, band):
    case = drop_case(96, 32, keep, dt, 50, band)
    r = bar_ratio(*case, keep, dt, band)
    print(f"dropout bwd emulation {dt} keep={keep}: worst error/bar {r:.3f}")
    assert r <= 1.0


@pytest.mark.parametrize("slip", ["dp_unmasked", "dv_unscaled", "mask_transposed", "d_undropped"])
def test_drop_bar_catches_slips(slip):
    dt, keep, band = I.F16, 0.5, (None, 0, 0)
    q, k, v, do, O, L, Z = drop_case(96, 32, keep, dt, 51, band)
    o_used = None
    if slip == "d_undropped":
        o_used, _ = head_attention_band_fp64(q, k, v, 0.25, *band)
    r = bar_ratio(q, k, v, do, O, L, Z, keep, dt, band, None if slip == "d_undropped" else slip, o_used)
    assert r > 1.0, f"{slip}: ratio {r:.3f}"
