"""Pins for the additive-mask oracle (oracle/additive.py) and its backward magnitudes, on the CPU.

  * forward: torch's fp64 scaled_dot_product_attention with a float attn_mask (which it adds to
    the scaled scores) gives O, and torch.logsumexp of the masked scores the LSE; pure-Python loops
    agree on a tiny case; a mask of 0 and -inf equals the boolean-hidden oracle bit for bit; a
    per-row constant leaves O unchanged and shifts the LSE by it; a row whose visible keys all
    carry -inf gives O = 0, LSE = -inf;
  * backward: torch autograd through the same SDPA call, and central finite differences;
  * magnitudes (oracle/backward.py with ``add``): a {0, -inf} mask gives the boolean-hidden
    magnitudes, a pure-Python enumeration of the terms agrees on a generic mask, and they bound
    the gradients.
"""
import math

import numpy as np
import pytest
import torch

from oracle.additive import head_attention_additive_fp64, head_attention_bwd_additive_fp64
from oracle.attention import band_visible, head_attention_band_fp64
from oracle.backward import head_attention_bwd_band_fp64, head_attention_bwd_magnitude_fp64


def draw(n, N, d, seed, mask_scale=2.0, ninf=0.1):
    g = np.random.Generator(np.random.PCG64(seed))
    q, k, v, do = (g.standard_normal((r, d)) for r in (n, N, N, n))
    M = g.standard_normal((n, N)) * mask_scale
    M[g.random((n, N)) < ninf] = -np.inf
    return q, k, v, do, M


def torch_sdpa(q, k, v, M, scale, band):
    n, N = M.shape
    vis = band_visible(np.arange(n), np.arange(N), *band)
    Mt = torch.from_numpy(np.where(vis, M, -np.inf))
    qt, kt, vt = (torch.from_numpy(x)[None, None].requires_grad_(True) for x in (q, k, v))
    O = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=Mt[None, None], scale=scale)
    L = torch.logsumexp(scale * (qt[0, 0] @ kt[0, 0].T) + Mt, dim=1)
    return O, L, (qt, kt, vt)


@pytest.mark.parametrize("band", [(None, None, 0), (None, 0, 3), (6, 2, -2)])
def test_forward_matches_torch_sdpa(band):
    q, k, v, _, M = draw(12, 15, 8, seed=60 + (band[2] or 0))
    O, L = head_attention_additive_fp64(q, k, v, 0.3, *band, M)
    Ot, Lt, _ = torch_sdpa(q, k, v, M, 0.3, band)
    seen = np.isfinite(L)
    assert seen.all(), "the draw should leave every row a key"
    np.testing.assert_allclose(O, Ot[0, 0].detach().numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, Lt.detach().numpy(), rtol=1e-12, atol=1e-13)


def test_forward_brute_force():
    q, k, v, _, M = draw(4, 6, 3, seed=61)
    band = (3, 1, 2)
    O, L = head_attention_additive_fp64(q, k, v, 0.8, *band, M)
    vis = band_visible(np.arange(4), np.arange(6), *band)
    for i in range(4):
        js = [j for j in range(6) if vis[i, j] and M[i, j] != -math.inf]
        if not js:
            assert L[i] == -math.inf and (O[i] == 0).all()
            continue
        s = {j: 0.8 * sum(q[i, c] * k[j, c] for c in range(3)) + M[i, j] for j in js}
        m = max(s.values())
        den = math.fsum(math.exp(s[j] - m) for j in js)
        assert abs(L[i] - (m + math.log(den))) <= 1e-13 * max(1.0, abs(L[i]))
        for c in range(3):
            assert abs(O[i, c] - math.fsum(math.exp(s[j] - m) / den * v[j, c] for j in js)) <= 1e-13


def test_zero_and_neg_inf_is_the_boolean_mask():
    q, k, v, _, M = draw(20, 25, 6, seed=62, ninf=0.3)
    hidden = np.isneginf(M)
    Mz = np.where(hidden, -np.inf, 0.0)
    for band in ((None, None, 5), (None, 0, 5), (4, 4, 5)):
        O, L = head_attention_additive_fp64(q, k, v, 0.5, *band, Mz)
        O0, L0 = head_attention_band_fp64(q, k, v, 0.5, band[0], band[1], band[2], hidden=hidden)
        np.testing.assert_array_equal(O, O0)
        np.testing.assert_array_equal(L, L0)


def test_row_constant_shifts_only_the_lse():
    q, k, v, _, M = draw(10, 10, 4, seed=63, ninf=0.0)
    c = np.linspace(-30.0, 30.0, 10)
    O, L = head_attention_additive_fp64(q, k, v, 0.5, None, 0, 0, M)
    O2, L2 = head_attention_additive_fp64(q, k, v, 0.5, None, 0, 0, M + c[:, None])
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2, L + c, rtol=1e-12, atol=1e-12)


def test_fully_masked_row():
    q, k, v, do, M = draw(5, 7, 3, seed=64, ninf=0.0)
    M[2] = -np.inf
    O, L = head_attention_additive_fp64(q, k, v, 0.5, None, None, 0, M)
    assert L[2] == -np.inf and (O[2] == 0).all() and np.isfinite(L[[0, 1, 3, 4]]).all()
    dq, dk, dv = head_attention_bwd_additive_fp64(q, k, v, do, 0.5, None, None, 0, M)
    assert (dq[2] == 0).all()


@pytest.mark.parametrize("band", [(None, None, 0), (5, 1, 0)])
def test_backward_matches_torch_autograd(band):
    q, k, v, do, M = draw(9, 9, 5, seed=65)
    got = head_attention_bwd_additive_fp64(q, k, v, do, 0.6, *band, M)
    O, _, leaves = torch_sdpa(q, k, v, M, 0.6, band)
    O.backward(torch.from_numpy(do)[None, None])
    for g, t in zip(got, leaves):
        np.testing.assert_allclose(g, t.grad[0, 0].numpy(), rtol=1e-10, atol=1e-12)


def test_backward_finite_differences():
    q, k, v, do, M = draw(5, 6, 3, seed=66)
    args = (0.7, None, None, 0, M)
    got = head_attention_bwd_additive_fp64(q, k, v, do, *args)
    h = 1e-6
    for which, gr in enumerate(got):
        x = [q.copy(), k.copy(), v.copy()]
        fd = np.zeros_like(x[which])
        for idx in np.ndindex(fd.shape):
            x0 = x[which][idx]
            x[which][idx] = x0 + h
            lp = np.sum(do * head_attention_additive_fp64(*x, *args)[0])
            x[which][idx] = x0 - h
            lm = np.sum(do * head_attention_additive_fp64(*x, *args)[0])
            x[which][idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        assert np.abs(gr - fd).max() <= 1e-7 * max(1.0, np.abs(fd).max())


def test_zero_and_neg_inf_backward_is_the_boolean_mask():
    q, k, v, do, M = draw(16, 16, 4, seed=67, ninf=0.25)
    hidden = np.isneginf(M)
    Mz = np.where(hidden, -np.inf, 0.0)
    got = head_attention_bwd_additive_fp64(q, k, v, do, 0.5, None, 0, 0, Mz)
    want = head_attention_bwd_band_fp64(q, k, v, do, 0.5, None, 0, 0, hidden=hidden)
    for a, b in zip(got, want):
        np.testing.assert_array_equal(a, b)


# ------------------------------------------------------------------ magnitudes with an additive mask

def test_magnitudes_zero_and_neg_inf_is_the_boolean_mask():
    q, k, v, do, M = draw(12, 14, 4, seed=68, ninf=0.3)
    hidden = np.isneginf(M)
    band = (None, 1, 2)
    got = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.5, False, band=band, add=np.where(hidden, -np.inf, 0.0))
    want = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.5, False, band=band, hidden=hidden)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-14, atol=0)


def test_magnitudes_equal_term_enumeration():
    q, k, v, do, M = draw(4, 6, 3, seed=69)
    band = (4, 1, 2)
    mq, mk, mv = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.9, False, band=band, add=M)
    O, L = head_attention_additive_fp64(q, k, v, 0.9, *band, M)
    vis = band_visible(np.arange(4), np.arange(6), *band)
    wq, wk, wv = np.zeros((4, 3)), np.zeros((6, 3)), np.zeros((6, 3))
    for i in range(4):
        for j in range(6):
            if not vis[i, j] or M[i, j] == -math.inf or L[i] == -math.inf:
                continue
            P = math.exp(0.9 * sum(q[i, c] * k[j, c] for c in range(3)) + M[i, j] - L[i])
            for c in range(3):
                wv[j, c] += abs(P * do[i, c])
                for c2 in range(3):
                    wq[i, c] += abs(0.9 * P * do[i, c2] * v[j, c2] * k[j, c]) + abs(0.9 * P * do[i, c2] * O[i, c2] * k[j, c])
                    wk[j, c] += abs(0.9 * P * do[i, c2] * v[j, c2] * q[i, c]) + abs(0.9 * P * do[i, c2] * O[i, c2] * q[i, c])
    for a, b in ((mq, wq), (mk, wk), (mv, wv)):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)


def test_magnitudes_dominate_gradients():
    q, k, v, do, M = draw(30, 30, 6, seed=70, mask_scale=4.0)
    for band in ((None, None, 0), (None, 0, 0), (6, 3, 0)):
        g = head_attention_bwd_additive_fp64(q, k, v, do, 0.5, *band, M)
        m = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.5, False, band=band, add=M)
        for a, b in zip(g, m):
            assert (np.abs(a) <= b * (1 + 1e-12)).all()
