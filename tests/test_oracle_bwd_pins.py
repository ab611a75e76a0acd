"""Pins for the fp64 gradient oracle (oracle/backward.py): checks that do not retype it.

  * finite differences: central differences of L = sum(dO * O) through the forward
    definition (and, on the smallest shape, through the pure-Python brute force) give every
    element of dQ, dK and dV independently of the chain-rule formula;
  * library routine: torch's float64 autograd through scaled_dot_product_attention on the
    CPU, with K/V heads repeated over their query-head groups (consecutive grouping, the
    reading the forward oracle takes of the intelliparadigm page, section 1.3);
  * invariants: softmax rows sum to one, so sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i for
    every head, causal or not;
  * planted mistakes: copies of the oracle with one plausible slip each (the D term dropped,
    dS transposed, the scale missing, P recomputed without the mask, the GQA sum replaced by
    one head) are rejected by the finite-difference check.
"""
import numpy as np
import pytest
import torch

from oracle import attention_brute, attention_fp64, kv_head_of
from oracle.attention import head_attention_fp64
from oracle.backward import attention_bwd_fp64, head_attention_bwd_fp64


def draw(B, Hq, Hkv, N, d, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, Hq, N, d))
    k = g.standard_normal((B, Hkv, N, d))
    v = g.standard_normal((B, Hkv, N, d))
    do = g.standard_normal((B, Hq, N, d))
    return q, k, v, do


def fd_grads(fwd, q, k, v, do, scale, causal, h=1e-5):
    """Central differences of L = sum(dO * O(q, k, v)) for every input element."""
    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = x[idx]
            x[idx] = x0 + h
            lp = np.sum(do * fwd(*args, scale, causal)[0])
            x[idx] = x0 - h
            lm = np.sum(do * fwd(*args, scale, causal)[0])
            x[idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        out.append(g)
    return out


def assert_grads_close(got, want, rtol, what):
    for name, a, b in zip(("dQ", "dK", "dV"), got, want):
        err = np.abs(a - b).max() / max(1.0, np.abs(b).max())
        assert err <= rtol, f"{what}: {name} differs by {err:.3e}"


SHAPES = [(1, 1, 1, 5, 3), (1, 2, 1, 6, 4), (2, 4, 2, 7, 3)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(shape, causal):
    q, k, v, do = draw(*shape, seed=11 + shape[3])
    scale = 0.37
    got = attention_bwd_fp64(q, k, v, do, scale, causal)
    want = fd_grads(attention_fp64, q, k, v, do, scale, causal)
    assert_grads_close(got, want, 1e-7, f"FD {shape} causal={causal}")


def test_finite_differences_brute_force():
    q, k, v, do = draw(1, 2, 1, 4, 2, seed=5)

    def brute(q, k, v, scale, causal):
        return np.array(attention_brute(q.tolist(), k.tolist(), v.tolist(), scale, causal)[0]), None

    for causal in (False, True):
        got = attention_bwd_fp64(q, k, v, do, 0.8, causal)
        want = fd_grads(brute, q, k, v, do, 0.8, causal)
        assert_grads_close(got, want, 1e-7, f"brute FD causal={causal}")


@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(2, 4, 2, 33, 16), (1, 8, 2, 64, 32), (1, 3, 3, 40, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd_float64(B, Hq, Hkv, N, d, causal):
    q, k, v, do = draw(B, Hq, Hkv, N, d, seed=B * 100 + N)
    scale = 1.0 / np.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), is_causal=causal, scale=scale)
    out.backward(torch.tensor(do))
    want = [t.grad.numpy() for t in (tq, tk, tv)]
    got = attention_bwd_fp64(q, k, v, do, scale, causal)
    assert_grads_close(got, want, 1e-12, f"torch ({B},{Hq},{Hkv},{N},{d}) causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    q, k, v, do = draw(2, 4, 2, 50, 8, seed=77)
    for b in range(2):
        for hq in range(4):
            hk = kv_head_of(hq, 4, 2)
            dq, dk, dv = head_attention_bwd_fp64(q[b, hq], k[b, hk], v[b, hk], do[b, hq], 0.5, causal)
            assert np.abs(dk.sum(axis=0)).max() <= 1e-12 * max(1.0, np.abs(dk).max())
            np.testing.assert_allclose(dv.sum(axis=0), do[b, hq].sum(axis=0), rtol=0, atol=1e-11)


def test_saved_lse_equals_recomputed():
    q, k, v, do = draw(1, 1, 1, 30, 8, seed=3)
    _, lse = head_attention_fp64(q[0, 0], k[0, 0], v[0, 0], 0.6, True)
    a = head_attention_bwd_fp64(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.6, True, lse=lse)
    b = head_attention_bwd_fp64(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 0.6, True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# ---------------------------------------------------------------- planted mistakes

def broken_bwd(mistake):
    """A copy of the oracle's chain rule with one slip, for the checks to reject."""
    def head(q, k, v, do, scale, causal):
        n, N = q.shape[0], k.shape[0]
        _, lse = head_attention_fp64(q, k, v, scale, causal)
        S = scale * (q @ k.T)
        if causal and mistake != "no_mask":
            S = np.where(np.arange(N)[None, :] > np.arange(n)[:, None], -np.inf, S)
        P = np.exp(S - lse[:, None])
        dv = P.T @ do
        dP = do @ v.T
        D = np.sum(P * dP, axis=1)
        dS = P * dP if mistake == "no_D" else P * (dP - D[:, None])
        dq = (dS @ k) * (1.0 if mistake == "no_scale" else scale)
        dk = scale * ((dS @ q) if mistake == "dS_not_transposed" else (dS.T @ q))
        return dq, dk, dv

    def full(q, k, v, do, scale, causal):
        B, Hq = q.shape[:2]
        Hkv = k.shape[1]
        dq = np.empty(q.shape)
        dk = np.zeros(k.shape)
        dv = np.zeros(v.shape)
        for b in range(B):
            for hq in range(Hq):
                hk = kv_head_of(hq, Hq, Hkv)
                a, c, e = head(q[b, hq], k[b, hk], v[b, hk], do[b, hq], scale, causal)
                dq[b, hq] = a
                if mistake == "gqa_last_head_only":
                    dk[b, hk], dv[b, hk] = c, e
                else:
                    dk[b, hk] += c
                    dv[b, hk] += e
        return dq, dk, dv
    return full


@pytest.mark.parametrize("mistake", ["no_D", "no_scale", "dS_not_transposed", "no_mask", "gqa_last_head_only"])
def test_planted_mistakes_are_caught(mistake):
    q, k, v, do = draw(1, 2, 1, 6, 3, seed=21)
    scale = 0.37
    want = fd_grads(attention_fp64, q, k, v, do, scale, True)
    ok = broken_bwd("none")(q, k, v, do, scale, True)
    assert_grads_close(ok, want, 1e-7, "unbroken copy")
    bad = broken_bwd(mistake)(q, k, v, do, scale, True)
    with pytest.raises(AssertionError):
        assert_grads_close(bad, want, 1e-7, mistake)
