"""Pins for the masked oracle forms (a boolean mask whose nonzero entries hide keys, on top of
the band, broadcast over batch and heads).

  * special cases: an all-zero mask is the banded oracle exactly; a mask holding the causal
    pattern (built here by index comparison) is the causal oracle; a mask holding a window
    pattern is the banded oracle with those edges;
  * slicing: every row equals the plain definition on the keys the mask leaves, gathered
    by index in the test;
  * library routine: torch's float64 scaled_dot_product_attention with the inverted mask
    (True = attend) and its autograd;
  * finite differences of the masked forward for the masked gradients;
  * rows the mask hides completely: O = 0, LSE = -inf, zero dQ;
  * broadcast: a [1, 1, Nq, Nk] mask equals the same mask repeated to [B, Hq, Nq, Nk].
"""
import numpy as np
import pytest
import torch

from oracle import attention_fp64
from oracle.attention import attention_band_fp64, head_attention_fp64
from oracle.backward import attention_bwd_band_fp64, head_attention_bwd_magnitude_fp64


def draw(B, Hq, Hkv, Nq, Nk, d, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal((B, Hq, Nq, d)), g.standard_normal((B, Hkv, Nk, d)),
            g.standard_normal((B, Hkv, Nk, d)), g.standard_normal((B, Hq, Nq, d)))


def random_mask(shape, p_hide, seed):
    return (np.random.Generator(np.random.PCG64(seed)).random(shape) < p_hide).astype(np.uint8)


def test_zero_mask_is_the_band_oracle():
    q, k, v, _ = draw(2, 4, 2, 40, 56, 8, 1)
    zero = np.zeros((1, 1, 40, 56), np.uint8)
    for band in ((None, None), (None, 0), (9, 3)):
        O, L = attention_band_fp64(q, k, v, 0.4, *band)
        Om, Lm = attention_band_fp64(q, k, v, 0.4, *band, mask=zero)
        assert np.array_equal(O, Om) and np.array_equal(L, Lm)


def test_causal_and_window_patterns():
    q, k, v, _ = draw(2, 2, 2, 37, 37, 8, 2)
    i = np.arange(37)[:, None]
    j = np.arange(37)[None, :]
    causal = (j > i).astype(np.uint8)[None, None]
    O, L = attention_fp64(q, k, v, 0.3, True)
    Om, Lm = attention_band_fp64(q, k, v, 0.3, None, None, mask=causal)
    np.testing.assert_allclose(Om, O, rtol=0, atol=1e-14)
    np.testing.assert_allclose(Lm, L, rtol=0, atol=1e-13)
    window = ((j > i) | (j < i - 5)).astype(np.uint8)[None, None]
    Ob, Lb = attention_band_fp64(q, k, v, 0.3, 5, 0)
    Ow, Lw = attention_band_fp64(q, k, v, 0.3, None, None, mask=window)
    np.testing.assert_allclose(Ow, Ob, rtol=0, atol=1e-14)
    np.testing.assert_allclose(Lw, Lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("band", [(None, None), (None, 0), (7, 2)])
def test_rows_equal_the_definition_on_their_unmasked_keys(band):
    Nq, Nk = 30, 45
    q, k, v, _ = draw(1, 1, 1, Nq, Nk, 8, 3)
    mask = random_mask((1, 1, Nq, Nk), 0.4, 4)
    mask[0, 0, 5] = 1  # one row hidden completely
    O, L = attention_band_fp64(q, k, v, 0.5, *band, mask=mask)
    off = Nk - Nq
    for i in range(Nq):
        keys = [j for j in range(Nk) if not mask[0, 0, i, j]
                and (band[0] is None or j >= i + off - band[0]) and (band[1] is None or j <= i + off + band[1])]
        if not keys:
            assert (O[0, 0, i] == 0).all() and L[0, 0, i] == -np.inf
            continue
        keys = np.array(keys)
        Oi, Li = head_attention_fp64(q[0, 0, i:i + 1], k[0, 0, keys], v[0, 0, keys], 0.5, False)
        np.testing.assert_allclose(O[0, 0, i], Oi[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[0, 0, i], Li[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("mshape", [(1, 1), (2, 1), (2, 4)])
def test_torch_masked_sdpa_and_autograd(mshape):
    B, Hq, Hkv, Nq, Nk, d = 2, 4, 2, 24, 40, 16
    q, k, v, do = draw(B, Hq, Hkv, Nq, Nk, d, 11)
    mask = random_mask(mshape + (Nq, Nk), 0.5, 12)
    mask[..., :, -1] = 0  # every row keeps a key: torch's empty-row result differs from the reading
    scale = 0.25
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1),
        attn_mask=torch.tensor(mask == 0), scale=scale)
    O, _ = attention_band_fp64(q, k, v, scale, None, None, mask=mask)
    np.testing.assert_allclose(O, out.detach().numpy(), rtol=0, atol=1e-13)
    out.backward(torch.tensor(do))
    got = attention_bwd_band_fp64(q, k, v, do, scale, None, None, mask=mask)
    for a, t in zip(got, (tq, tk, tv)):
        b = t.grad.numpy()
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))


def test_masked_gradients_finite_differences():
    q, k, v, do = draw(1, 2, 1, 5, 8, 3, 21)
    mask = random_mask((1, 2, 5, 8), 0.4, 22)
    got = attention_bwd_band_fp64(q, k, v, do, 0.7, 3, 1, mask=mask)
    h = 1e-5
    for which, g in enumerate(got):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = x[idx]
            x[idx] = x0 + h
            lp = np.sum(do * attention_band_fp64(*args, 0.7, 3, 1, mask=mask)[0])
            x[idx] = x0 - h
            lm = np.sum(do * attention_band_fp64(*args, 0.7, 3, 1, mask=mask)[0])
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        assert np.abs(g - fd).max() <= 1e-7 * max(1.0, np.abs(fd).max())


def test_fully_hidden_rows():
    q, k, v, do = draw(1, 2, 2, 12, 12, 4, 31)
    mask = np.zeros((1, 2, 12, 12), np.uint8)
    mask[0, 1, 3] = 1
    O, L = attention_band_fp64(q, k, v, 0.5, None, None, mask=mask)
    assert (O[0, 1, 3] == 0).all() and L[0, 1, 3] == -np.inf and np.isfinite(L[0, 0]).all()
    dq, dk, dv = attention_bwd_band_fp64(q, k, v, do, 0.5, None, None, mask=mask)
    assert (dq[0, 1, 3] == 0).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    bq, bk, bv = head_attention_bwd_magnitude_fp64(q[0, 1], k[0, 1], v[0, 1], do[0, 1], 0.5, False,
                                                   band=(None, None, 0), hidden=mask[0, 1])
    assert (bq[3] == 0).all() and np.isfinite(bk).all() and np.isfinite(bv).all()


def test_broadcast_equals_repeat():
    q, k, v, do = draw(2, 4, 2, 16, 20, 8, 41)
    m1 = random_mask((1, 1, 16, 20), 0.3, 42)
    mr = np.broadcast_to(m1, (2, 4, 16, 20)).copy()
    a = attention_band_fp64(q, k, v, 0.5, None, 0, mask=m1)
    b = attention_band_fp64(q, k, v, 0.5, None, 0, mask=mr)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ga = attention_bwd_band_fp64(q, k, v, do, 0.5, None, 0, mask=m1)
    gb = attention_bwd_band_fp64(q, k, v, do, 0.5, None, 0, mask=mr)
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)


def test_planted_mistake_is_caught():
    """A mask read with its axes swapped (a plausible indexing slip) fails the slicing pin."""
    q, k, v, _ = draw(1, 1, 1, 10, 10, 4, 51)
    mask = random_mask((1, 1, 10, 10), 0.4, 52)
    O, _ = attention_band_fp64(q, k, v, 0.5, None, None, mask=mask)
    Ot, _ = attention_band_fp64(q, k, v, 0.5, None, None, mask=mask.transpose(0, 1, 3, 2).copy())
    assert np.abs(O - Ot).max() > 1e-3
