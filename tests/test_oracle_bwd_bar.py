"""Pins for the backward parity bar (oracle/backward.py: head_attention_bwd_magnitude_fp64 and
bwd_parity_bar), all on the CPU.

  * term enumeration: pure-Python loops list every term of every gradient element (the chain
    rule written out as products of Q, K, V, dO, P and O) and sum their magnitudes; the
    vectorised magnitude sums must equal that, so a dropped, doubled or misplaced term fails;
  * a single key worked by hand (P = 1, O = V), and the bar's constants on given numbers;
  * validity: a numpy emulation of the stated precision (16-bit operands in the products, fp32
    everything else, O given in fp32 or 16 bits) stays inside the bar on ragged, causal,
    grouped and sharp-row cases, and its worst error-to-bar ratio is printed;
  * planted slips: the same emulation with one plausible implementation mistake each (D from
    the neighbouring row's O, the LSE left in log2 units, the diagonal key hidden, the scale
    missing from dK, the LSE stored in 16 bits, one head's dK dropped from a group) exceeds
    the bar somewhere.
Slips whose effect stays at the input type's rounding level (a score-gradient factor rounded
twice, an LSE off by one fp32 ulp) cannot be told apart from correct rounding by any bar at that
precision; the forward's LSE itself is checked to 1e-4 relative.
"""
import math

import numpy as np
import pytest

from exact_attention_114_amd import inputs as I
from oracle import attention_brute, kv_head_of
from oracle.attention import band_visible, head_attention_band_fp64, head_attention_fp64
from oracle.backward import E32, bwd_parity_bar, head_attention_bwd_fp64, head_attention_bwd_magnitude_fp64

UNIT = {I.F16: 2.0 ** -11, I.BF16: 2.0 ** -8}


def draw(shape_q, shape_kv, seed, k_mult=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal(shape_q)
    k = g.standard_normal(shape_kv) * k_mult
    v = g.standard_normal(shape_kv)
    do = g.standard_normal(shape_q)
    return q, k, v, do


# ------------------------------------------------------------------ term enumeration

def enumerate_magnitudes(q, k, v, do, scale, visible):
    """Every term of every gradient element, its magnitude summed, with P and O from the
    pure-Python brute force (causal or all keys) or from the banded definition."""
    n, d = len(q), len(q[0])
    N = len(k)
    if visible is None:
        O, L = attention_brute([[q.tolist()]], [[k.tolist()]], [[v.tolist()]], scale, False)
        O, L = O[0][0], L[0][0]
        vis = [[True] * N for _ in range(n)]
    else:
        O, L = head_attention_band_fp64(q, k, v, scale, *visible[0], hidden=visible[1])
        vis = (band_visible(np.arange(n), np.arange(N), *visible[0]) & ~visible[1]).tolist()
        O, L = O.tolist(), L.tolist()
    P = [[math.exp(scale * sum(q[i][c] * k[j][c] for c in range(d)) - L[i]) if vis[i][j] else 0.0
          for j in range(N)] for i in range(n)]
    mq = [[0.0] * d for _ in range(n)]
    mk = [[0.0] * d for _ in range(N)]
    mv = [[0.0] * d for _ in range(N)]
    for i in range(n):
        for j in range(N):
            for c in range(d):
                mv[j][c] += abs(P[i][j] * do[i][c])
                for c2 in range(d):
                    # dQ_ic and dK_jc each hold s P_ij dO_ic2 V_jc2 (.) and -s P_ij dO_ic2 O_ic2 (.)
                    mq[i][c] += abs(scale * P[i][j] * do[i][c2] * v[j][c2] * k[j][c])
                    mq[i][c] += abs(scale * P[i][j] * do[i][c2] * O[i][c2] * k[j][c])
                    mk[j][c] += abs(scale * P[i][j] * do[i][c2] * v[j][c2] * q[i][c])
                    mk[j][c] += abs(scale * P[i][j] * do[i][c2] * O[i][c2] * q[i][c])
    return np.array(mq), np.array(mk), np.array(mv)


def test_magnitudes_equal_term_enumeration_all_keys():
    q, k, v, do = draw((5, 3), (5, 3), seed=31)  # the brute force takes as many keys as queries
    got = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.7, False)
    want = enumerate_magnitudes(q, k, v, do, 0.7, None)
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)


def test_magnitudes_equal_term_enumeration_causal():
    q, k, v, do = draw((5, 3), (5, 3), seed=32)
    got = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.45, True)
    # causal is the band (unlimited left edge, right edge 0) with nothing else hidden
    want = enumerate_magnitudes(q, k, v, do, 0.45, ((None, 0, 0), np.zeros((5, 5), dtype=bool)))
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)


def test_magnitudes_equal_term_enumeration_band_and_mask():
    q, k, v, do = draw((4, 2), (7, 2), seed=33)
    hid = np.zeros((4, 7), dtype=bool)
    hid[1, 4] = hid[2, 3] = True
    band = (2, 1, 3)
    got = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.9, False, band=band, hidden=hid)
    want = enumerate_magnitudes(q, k, v, do, 0.9, (band, hid))
    for a, b in zip(got, want):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)


def test_single_key_by_hand():
    """One key: P = 1 and O = V, so Mv = |dO|, Mq_c = 2 s sum_c2 |dO_c2 V_c2| |K_c| and
    Mk_c = 2 s sum_c2 |dO_c2 V_c2| |Q_c|."""
    q = np.array([[0.5, -2.0]])
    k = np.array([[1.5, 0.25]])
    v = np.array([[-3.0, 1.0]])
    do = np.array([[2.0, -0.5]])
    mq, mk, mv = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.25, False)
    a = 2.0 * 3.0 + 0.5 * 1.0  # sum |dO V|
    np.testing.assert_allclose(mv, [[2.0, 0.5]], rtol=1e-15)
    np.testing.assert_allclose(mq, [[2 * 0.25 * a * 1.5, 2 * 0.25 * a * 0.25]], rtol=1e-15)
    np.testing.assert_allclose(mk, [[2 * 0.25 * a * 0.5, 2 * 0.25 * a * 2.0]], rtol=1e-15)


def test_bar_constants():
    """(2u + (d + n) e32) M on given numbers: a changed coefficient or length fails."""
    assert E32 == 2.0 ** -24
    m = np.array([1.0, 3.0])
    np.testing.assert_allclose(bwd_parity_bar(m, 2.0 ** -8, 64, 100), (2.0 ** -7 + 164 * 2.0 ** -24) * m, rtol=1e-15)
    np.testing.assert_allclose(bwd_parity_bar(m, 2.0 ** -11, 128, 8192), (2.0 ** -10 + 8320 * 2.0 ** -24) * m,
                               rtol=1e-15)


def test_magnitude_dominates_gradient():
    """|g| <= M: the magnitude sum of a gradient's terms bounds the gradient."""
    q, k, v, do = draw((30, 8), (30, 8), seed=34)
    for causal in (False, True):
        g = head_attention_bwd_fp64(q, k, v, do, 0.5, causal)
        m = head_attention_bwd_magnitude_fp64(q, k, v, do, 0.5, causal)
        for a, b in zip(g, m):
            assert (np.abs(a) <= b * (1 + 1e-12)).all()


# ------------------------------------------------------------------ emulation of the stated precision

def round16(x, dt):
    x = np.asarray(x, dtype=np.float32)
    return I.bits_to_f64(I.to_bits(x, dt), dt).astype(np.float32)


def emulate_head(q, k, v, do, o_used, lse, scale, causal, dt, slip=None):
    """One head's gradients in the stated precision: S, dP, D and every sum in fp32, P and dS
    rounded to the input type before the products that consume them. ``slip`` plants one
    implementation mistake."""
    f = np.float32
    q, k, v, do, o_used = (np.asarray(x, dtype=f) for x in (q, k, v, do, o_used))
    lse = np.asarray(lse, dtype=f)
    n, N = q.shape[0], k.shape[0]
    s = f(scale)
    S = (q @ k.T) * s
    if slip == "lse_log2":
        P = np.exp2(S * f(1.4426950408889634) - lse[:, None]).astype(f)
    elif slip == "lse_16bit":
        P = np.exp(S - round16(lse, dt)[:, None]).astype(f)
    else:
        P = np.exp(S - lse[:, None]).astype(f)
    if causal:
        hidden = np.arange(N)[None, :] > np.arange(n)[:, None]
        if slip == "diagonal_hidden":
            hidden = np.arange(N)[None, :] >= np.arange(n)[:, None]
        P = np.where(hidden, f(0), P)
    P16 = round16(P, dt)
    dv = P16.T @ do
    dP = do @ v.T
    o_for_d = np.roll(o_used, 1, axis=0) if slip == "d_from_next_row" else o_used
    D = np.sum(do * o_for_d, axis=1, dtype=f)
    dS = round16(P * (dP - D[:, None]), dt)
    dq = (dS @ k) * s
    dk = dS.T @ q
    if slip != "dk_unscaled":
        dk = dk * s
    return dq, dk, dv


def emulate(q, k, v, do, o_used, lse, scale, causal, dt, slip=None):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq = np.empty(q.shape, dtype=np.float32)
    dk = np.zeros(k.shape, dtype=np.float32)
    dv = np.zeros(v.shape, dtype=np.float32)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            a, c, e = emulate_head(q[b, hq], k[b, hk], v[b, hk], do[b, hq], o_used[b, hq], lse[b, hq], scale,
                                   causal, dt, slip)
            dq[b, hq] = a
            if slip == "gqa_one_head" and hq % (Hq // Hkv) == 0:
                continue
            dk[b, hk] += c
            dv[b, hk] += e
    return dq, dk, dv


def case_arrays(B, Hq, Hkv, N, d, dt, causal, seed, k_mult=1.0, o16=False):
    w = I.small_case(B, Hq, Hkv, N, d, dt, causal, seed=seed, k_mult=k_mult)
    qkv = I.workload_qkv(w)
    q, k, v = qkv.f64()
    do = I.bits_to_f64(I.draw_dout(B, Hq, N, d, dt, seed + 1), dt)
    scale = I.scale_f32(w.scale)
    O = np.empty(q.shape)
    L = np.empty((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            O[b, h], L[b, h] = head_attention_fp64(q[b, h], k[b, kv_head_of(h, Hq, Hkv)], v[b, kv_head_of(h, Hq, Hkv)],
                                                   scale, causal)
    o_used = I.bits_to_f64(I.to_bits(O.astype(np.float32), dt), dt) if o16 else O.astype(np.float32).astype(np.float64)
    return q, k, v, do, O, L, o_used, scale


def worst_ratio(q, k, v, do, o_used, L, scale, causal, dt, got):
    """max over elements of |got - ref| / bar, per gradient (dQ, dK, dV)."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    ref_q = np.empty(q.shape)
    ref_k = np.zeros(k.shape)
    ref_v = np.zeros(v.shape)
    mq = np.empty(q.shape)
    mk = np.zeros(k.shape)
    mv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            a, c, e = head_attention_bwd_fp64(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, causal)
            x, y, z = head_attention_bwd_magnitude_fp64(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, causal)
            ref_q[b, h], mq[b, h] = a, x
            ref_k[b, hk] += c
            ref_v[b, hk] += e
            mk[b, hk] += y
            mv[b, hk] += z
    u = UNIT[dt]
    bars = (bwd_parity_bar(mq, u, d, N), bwd_parity_bar(mk, u, d, G * N), bwd_parity_bar(mv, u, d, G * N))
    return [float((np.abs(np.asarray(g, np.float64) - r) / np.maximum(bb, 1e-300)).max())
            for g, r, bb in zip(got, (ref_q, ref_k, ref_v), bars)]


CASES = [
    # (B, Hq, Hkv, N, d, dtype, causal, seed, k_mult, O in 16 bits)
    (1, 2, 1, 1, 64, I.F16, True, 501, 1.0, False),
    (1, 2, 2, 37, 32, I.BF16, False, 502, 1.0, False),
    (1, 2, 1, 200, 128, I.BF16, True, 503, 2.0, False),
    (1, 2, 2, 150, 64, I.F16, True, 504, 1.0, True),
    (1, 4, 1, 100, 64, I.F16, False, 505, 1.0, False),
    (1, 2, 1, 300, 96, I.BF16, True, 506, 2.0, True),
]


@pytest.mark.parametrize("case", CASES)
def test_emulated_precision_within_bar(case):
    B, Hq, Hkv, N, d, dt, causal, seed, km, o16 = case
    q, k, v, do, O, L, o_used, scale = case_arrays(B, Hq, Hkv, N, d, dt, causal, seed, km, o16)
    got = emulate(q, k, v, do, o_used, L, scale, causal, dt)
    r = worst_ratio(q, k, v, do, o_used, L, scale, causal, dt, got)
    print(f"emulated worst error / bar (dQ, dK, dV): {r[0]:.3f} {r[1]:.3f} {r[2]:.3f}")
    assert max(r) <= 1.0


SLIPS = [
    ("d_from_next_row", (1, 2, 1, 64, 32, I.F16, True, 511, 1.0, False)),
    ("lse_log2", (1, 2, 1, 64, 32, I.F16, True, 512, 1.0, False)),
    ("diagonal_hidden", (1, 2, 1, 64, 32, I.BF16, True, 513, 1.0, False)),
    ("dk_unscaled", (1, 2, 1, 64, 32, I.BF16, False, 514, 1.0, False)),
    ("lse_16bit", (1, 4, 1, 64, 32, I.F16, True, 515, 2.0, False)),
    ("gqa_one_head", (1, 4, 2, 64, 32, I.BF16, False, 516, 1.0, False)),
]


@pytest.mark.parametrize("slip,case", SLIPS, ids=[s for s, _ in SLIPS])
def test_planted_slips_exceed_bar(slip, case):
    B, Hq, Hkv, N, d, dt, causal, seed, km, o16 = case
    q, k, v, do, O, L, o_used, scale = case_arrays(B, Hq, Hkv, N, d, dt, causal, seed, km, o16)
    clean = worst_ratio(q, k, v, do, o_used, L, scale, causal, dt, emulate(q, k, v, do, o_used, L, scale, causal, dt))
    assert max(clean) <= 1.0
    bad = worst_ratio(q, k, v, do, o_used, L, scale, causal, dt,
                      emulate(q, k, v, do, o_used, L, scale, causal, dt, slip))
    print(f"{slip}: worst error / bar (dQ, dK, dV) {bad[0]:.2f} {bad[1]:.2f} {bad[2]:.2f}")
    assert max(bad) > 1.0
