"""Comparison of GPU gradients with the fp64 gradient oracle, shared by the GPU backward tests.

Bar (stated up front, independent of how a kernel orders or tiles its sums): every element g of
dQ, dK and dV must satisfy
    |g_gpu - g_ref| <= (2u + (d + n) e32) * M_g
with M_g the sum of the magnitudes of the terms of g (oracle.backward.
head_attention_bwd_magnitude_fp64), u the unit roundoff of the input type (2^-11 fp16,
2^-8 bf16), e32 = 2^-24, d the head dimension and n the terms summed per element (keys for dQ,
rows of the K/V head's whole query group for dK and dV). It is the first-order error of any
evaluation with 16-bit operands in the products and fp32 sums and statistics, the precision of
the method (oracle.backward.bwd_parity_bar).
"""
from __future__ import annotations

import numpy as np

from exact_attention_114_amd import inputs as I
from oracle.attention import kv_head_of
from oracle.backward import bwd_parity_bar, head_attention_bwd_magnitude_fp64  # noqa: F401
from oracle.dropout import keep_mask

UNIT = {I.F16: 2.0 ** -11, I.BF16: 2.0 ** -8}


def mask_plane(mask, b, h):
    if mask is None:
        return None
    return mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0]


def magnitudes(q, k, v, do, scale, causal=False, band=None, mask=None, heads=None, drop=None, add=None):
    """(Mq, Mk, Mv) over [B, Hq, Nq, d] / [B, Hkv, Nk, d] arrays; ``band`` = (left, right) with
    off = Nk - Nq. ``heads``: an optional list of (b, hq) to fill (others stay 0). ``drop`` =
    (keep_prob, seed, offset): dropout with the keep mask of head plane b * Hq + hq. ``add``: an
    additive [B or 1, Hq or 1, Nq, Nk] mask (float64 values)."""
    if (drop is not None or add is not None) and band is None:
        band = (None, 0) if causal else (None, None)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    mq = np.zeros(q.shape)
    mk = np.zeros(k.shape)
    mv = np.zeros(v.shape)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        hk = kv_head_of(h, Hq, Hkv)
        bd = None if band is None else (band[0], band[1], Nk - Nq)
        dr = None
        if drop is not None:
            dr = (keep_mask(drop[1], drop[2], b * Hq + h, np.arange(Nq), np.arange(Nk), drop[0]), drop[0])
        x, y, z = head_attention_bwd_magnitude_fp64(q[b, h], k[b, hk], v[b, hk], do[b, h], scale,
                                                    causal if band is None else False, band=bd,
                                                    hidden=mask_plane(mask, b, h), drop=dr,
                                                    add=mask_plane(add, b, h))
        mq[b, h] = x
        mk[b, hk] += y
        mv[b, hk] += z
    return mq, mk, mv


def check_one(label, name, g, r, m, dt, d, n, extra_rel=0.0):
    """Assert one gradient within the bar (plus ``extra_rel`` times the magnitudes, for an error
    source the caller states); return its worst error-to-bar ratio."""
    assert np.isfinite(g).all(), f"{label}: non-finite {name}"
    bar = bwd_parity_bar(m, UNIT[dt], d, n) + extra_rel * np.asarray(m, dtype=np.float64)
    err = np.abs(np.asarray(g, np.float64) - r)
    ratio = float((err / np.maximum(bar, 1e-300)).max()) if err.size else 0.0
    assert ratio <= 1.0, f"{label}: {name} error reaches {ratio:.3f} of the bar (max err {err.max():.3e})"
    return ratio


def check(label, got, ref, mags, dt, d, n_q, n_kv, select=None, extra_rel=0.0):
    """Assert every compared element within the bar and return the worst error-to-bar ratio per
    gradient (dQ, dK, dV). n_q: terms per dQ element (keys); n_kv: terms per dK/dV element
    (query rows of the group). ``select``: optional (dQ index, dK/dV index) to compare a part."""
    ratios = []
    for i, (name, g, r, m) in enumerate(zip(("dQ", "dK", "dV"), got, ref, mags)):
        if select is not None:
            sel = select[0] if i == 0 else select[1]
            g, r, m = g[sel], r[sel], m[sel]
        ratios.append(check_one(label, name, g, r, m, dt, d, n_q if i == 0 else n_kv, extra_rel))
    print(f"[bar] {label}: worst error/bar dQ {ratios[0]:.4f} dK {ratios[1]:.4f} dV {ratios[2]:.4f}", flush=True)
    return ratios
