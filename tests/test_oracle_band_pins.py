"""Pins for the banded oracle forms (sliding window, separate query and key lengths).

  * special cases: the unlimited band is the plain definition, the band (None, 0) with
    Nq = Nk is the causal definition, and a single query row with (None, 0) sees every key
    (the diagonal sits at the end of the key sequence);
  * slicing: each row of a windowed result equals the plain definition on that row's own
    slice of keys, cut out by index arithmetic in the test;
  * library routine: torch's float64 scaled_dot_product_attention with an explicit boolean
    mask built here element by element from the band's definition, and its autograd;
  * finite differences of the banded forward for the banded gradients;
  * rows that see no key: O = 0 and LSE = -inf, gradients zero for those rows.
"""
import numpy as np
import pytest
import torch

from oracle import attention_fp64, head_attention_fp64
from oracle.attention import attention_band_fp64, head_attention_band_fp64
from oracle.backward import attention_bwd_band_fp64, attention_bwd_fp64, head_attention_bwd_magnitude_fp64


def draw(B, Hq, Hkv, Nq, Nk, d, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return (g.standard_normal((B, Hq, Nq, d)), g.standard_normal((B, Hkv, Nk, d)),
            g.standard_normal((B, Hkv, Nk, d)), g.standard_normal((B, Hq, Nq, d)))


def explicit_mask(Nq, Nk, left, right):
    off = Nk - Nq
    m = np.zeros((Nq, Nk), dtype=bool)
    for i in range(Nq):
        for j in range(Nk):
            ok = True
            if left is not None and j < i + off - left:
                ok = False
            if right is not None and j > i + off + right:
                ok = False
            m[i, j] = ok
    return m


def test_unlimited_and_causal_special_cases():
    q, k, v, _ = draw(2, 4, 2, 37, 37, 8, 1)
    for causal, band in ((False, (None, None)), (True, (None, 0))):
        O, L = attention_fp64(q, k, v, 0.4, causal)
        Ob, Lb = attention_band_fp64(q, k, v, 0.4, *band)
        np.testing.assert_allclose(Ob, O, rtol=0, atol=1e-14)
        np.testing.assert_allclose(Lb, L, rtol=0, atol=1e-13)


def test_single_query_sees_every_key():
    q, k, v, _ = draw(1, 2, 2, 1, 50, 8, 2)
    Ob, Lb = attention_band_fp64(q, k, v, 0.3, None, 0)
    for h in range(2):
        O, L = head_attention_fp64(q[0, h], k[0, h], v[0, h], 0.3, False)
        np.testing.assert_allclose(Ob[0, h], O, rtol=0, atol=1e-14)
        np.testing.assert_allclose(Lb[0, h], L, rtol=0, atol=1e-13)


@pytest.mark.parametrize("Nq,Nk,left,right", [(40, 40, 5, 0), (40, 40, 3, 4), (30, 50, 7, 0), (50, 30, None, 0),
                                              (45, 45, 0, 0), (33, 64, 10, 2)])
def test_rows_equal_the_definition_on_their_key_slice(Nq, Nk, left, right):
    q, k, v, _ = draw(1, 1, 1, Nq, Nk, 8, 3 + Nq + Nk)
    O, L = head_attention_band_fp64(q[0, 0], k[0, 0], v[0, 0], 0.5, left, right, off=Nk - Nq)
    off = Nk - Nq
    for i in range(Nq):
        lo = 0 if left is None else max(0, i + off - left)
        hi = Nk - 1 if right is None else min(Nk - 1, i + off + right)
        if lo > hi:
            assert (O[i] == 0).all() and L[i] == -np.inf
            continue
        Oi, Li = head_attention_fp64(q[0, 0][i:i + 1], k[0, 0][lo:hi + 1], v[0, 0][lo:hi + 1], 0.5, False)
        np.testing.assert_allclose(O[i], Oi[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[i], Li[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("Nq,Nk,left,right", [(40, 40, 6, 0), (24, 56, 9, 3), (56, 24, None, 0), (33, 33, 4, 4)])
def test_torch_masked_sdpa_and_autograd(Nq, Nk, left, right):
    q, k, v, do = draw(2, 4, 2, Nq, Nk, 16, 11 + Nq)
    scale = 0.25
    mask = explicit_mask(Nq, Nk, left, right)
    seen = mask.any(axis=1)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1),
        attn_mask=torch.tensor(mask), scale=scale)
    O, L = attention_band_fp64(q, k, v, scale, left, right)
    np.testing.assert_allclose(O[:, :, seen], out.detach().numpy()[:, :, seen], rtol=0, atol=1e-13)
    assert (O[:, :, ~seen] == 0).all() and (L[:, :, ~seen] == -np.inf).all()
    if seen.all():
        out.backward(torch.tensor(do))
        want = [t.grad.numpy() for t in (tq, tk, tv)]
        got = attention_bwd_band_fp64(q, k, v, do, scale, left, right)
        for a, b in zip(got, want):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * max(1.0, np.abs(b).max()))


def test_band_gradients_finite_differences():
    q, k, v, do = draw(1, 2, 1, 6, 9, 3, 21)
    scale, left, right = 0.7, 2, 1
    got = attention_bwd_band_fp64(q, k, v, do, scale, left, right)
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
            lp = np.sum(do * attention_band_fp64(*args, scale, left, right)[0])
            x[idx] = x0 - h
            lm = np.sum(do * attention_band_fp64(*args, scale, left, right)[0])
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        assert np.abs(g - fd).max() <= 1e-7 * max(1.0, np.abs(fd).max())


def test_band_gradients_match_the_pinned_causal_oracle():
    q, k, v, do = draw(2, 4, 2, 40, 40, 8, 31)
    for causal, band in ((False, (None, None)), (True, (None, 0))):
        a = attention_bwd_fp64(q, k, v, do, 0.4, causal)
        b = attention_bwd_band_fp64(q, k, v, do, 0.4, *band)
        for x, y in zip(a, b):
            np.testing.assert_allclose(y, x, rtol=0, atol=1e-12)


def test_rows_without_keys_have_zero_gradients():
    q, k, v, do = draw(1, 1, 1, 20, 10, 4, 41)  # Nq > Nk, causal: the first 10 rows see nothing
    dq, dk, dv = attention_bwd_band_fp64(q, k, v, do, 0.5, None, 0)
    assert (dq[0, 0, :10] == 0).all()
    O, L = attention_band_fp64(q, k, v, 0.5, None, 0)
    assert (O[0, 0, :10] == 0).all() and (L[0, 0, :10] == -np.inf).all()
    assert np.isfinite(O).all()


def test_magnitudes_band_match_causal_and_cover_empty_rows():
    q, k, v, do = draw(1, 1, 1, 30, 30, 8, 51)
    a = head_attention_bwd_magnitude_fp64(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.5, True)
    b = head_attention_bwd_magnitude_fp64(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.5, False, band=(None, 0, 0))
    for x, y in zip(a, b):
        np.testing.assert_allclose(y, x, rtol=1e-12, atol=0)
    # Nq > Nk with the band (None, 0): rows 0..9 see no key, their dQ magnitudes are 0 and all finite
    q, k, v, do = draw(1, 1, 1, 20, 10, 4, 52)
    mq, mk, mv = head_attention_bwd_magnitude_fp64(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.5, False,
                                                   band=(None, 0, -10))
    assert np.isfinite(mq).all() and np.isfinite(mk).all() and np.isfinite(mv).all()
    assert (mq[:10] == 0).all()
