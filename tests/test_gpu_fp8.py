"""GPU parity of the fp8-input forward (fa_fwd_fp8: OCP e4m3 Q, K, V with per-tensor descales)
against the fp64 oracle on the represented values (byte value times descale), within the fp8 bar
of oracle/precision.py: the fp32 bar of the arithmetic plus, per element of O,
    sum_j (2^-4 w_ij + min(w_ij, 2^-10 w_max,i)) |V_jc - O_ic| / (1 - 2^-4 - sum_j min(w_ij, 2^-10 w_max,i))
for the probabilities rounded to e4m3 in the P V product (LSE: the fp32 bar). Inputs: seeded
N(0,1) draws stored as e4m3 with descale = max|x| / 448 per tensor. Each case prints its worst
error-to-bar ratio."""
import numpy as np
import pytest
import torch

from exact_attention_114_amd import binding as bnd
from exact_attention_114_amd import inputs as I
from oracle.attention import head_attention_band_fp64, kv_head_of
from oracle.precision import head_attention_fp8_bar_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run(B, Hq, Hkv, Nq, Nk, d, seed, causal=False, window=None, k_mult=1.0, rows=None, heads=None):
    (q8, k8, v8), (dq, dk, dv) = I.draw_qkv_fp8(B, Hq, Hkv, Nq, d, seed, k_mult, Nk)
    scale = d ** -0.5
    print(f"[gpu] fa_fwd_fp8 B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} window={window}",
          flush=True)
    o, lse = bnd.fwd_fp8(*(torch.from_numpy(x).to(DEV) for x in (q8, k8, v8)), dq, dk, dv, scale=scale,
                         causal=causal, window=window)
    torch.cuda.synchronize()
    O = o.cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    left, right = (None, 0) if causal else (window if window is not None else (None, None))
    sc = I.scale_f32(scale)
    q, k, v = (I.e4m3_bits_to_f64(x) * s for x, s in ((q8, dq), (k8, dk), (v8, dv)))
    worst = [0.0, 0.0]
    for b, h in (heads or [(b, h) for b in range(B) for h in range(Hq)]):
        hk = kv_head_of(h, Hq, Hkv)
        kk, vv = k[b, hk], v[b, hk]
        sel = range(Nq) if rows is None else rows
        O_ref = np.empty((len(sel), d)); L_ref = np.empty(len(sel))
        bo = np.empty((len(sel), d)); bl = np.empty(len(sel))
        if rows is None:
            O_ref, L_ref = head_attention_band_fp64(q[b, h], kk, vv, sc, left, right, Nk - Nq)
            bo, bl = head_attention_fp8_bar_fp64(q[b, h], kk, vv, sc, left, right, Nk - Nq)
        else:
            for n, r in enumerate(rows):
                a, c = head_attention_band_fp64(q[b, h][r:r + 1], kk, vv, sc, left, right, r + Nk - Nq)
                x, y = head_attention_fp8_bar_fp64(q[b, h][r:r + 1], kk, vv, sc, left, right, r + Nk - Nq)
                O_ref[n], L_ref[n], bo[n], bl[n] = a[0], c[0], x[0], y[0]
        Og, Lg = O[b, h][list(sel)], L[b, h][list(sel)]
        assert np.isfinite(Og).all()
        seen = np.isfinite(L_ref)
        assert (Og[~seen] == 0).all() and (Lg[~seen] == -np.inf).all()
        ro = (np.abs(Og - O_ref) / np.maximum(bo, 1e-300))[seen].max() if seen.any() else 0.0
        rl = (np.abs(Lg[seen] - L_ref[seen]) / np.maximum(bl[seen], 1e-300)).max() if seen.any() else 0.0
        worst = [max(worst[0], ro), max(worst[1], rl)]
        assert ro <= 1.0, f"b={b} h={h}: O error reaches {ro:.3f} of the fp8 bar"
        assert rl <= 1.0, f"b={b} h={h}: LSE error reaches {rl:.3f} of the fp8 bar"
    print(f"[fp8 bar] worst error/bar O {worst[0]:.4f} LSE {worst[1]:.4f}", flush=True)


@pytest.mark.parametrize("N", [1, 17, 64, 65, 129, 257])
@pytest.mark.parametrize("d", [32, 48, 64, 80, 96, 112, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged(N, d, causal):
    run(1, 2, 1, N, N, d, 4000 + N + d, causal=causal)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 1)])
def test_fp8_gqa_sharp_rows(Hq, Hkv):
    run(2, Hq, Hkv, 333, 333, 128, 4100 + Hq + Hkv, causal=True, k_mult=2.0)


@pytest.mark.parametrize("Nq,Nk,window", [(300, 300, (64, 0)), (200, 450, (None, 0)), (450, 200, (None, 0)),
                                          (160, 96, (20, 70)), (1, 500, (None, 0))])
def test_fp8_bands(Nq, Nk, window):
    run(1, 4, 2, Nq, Nk, 64, 4200 + Nq + Nk, window=window)


def test_fp8_causal_n8192_workload_sampled_rows():
    """The grouped-query causal N = 8192 shape (B=4, Hq=32, Hkv=8, d=128, K x2) in fp8: every
    query head of one K/V group and heads of the other batch elements, on rows the oracle
    computes one by one (both ends, tile edges and the middle)."""
    rows = np.array([0, 1, 63, 64, 127, 128, 4095, 4096, 8190, 8191])
    heads = [(1, 12), (1, 13), (1, 14), (1, 15), (0, 0), (2, 31), (3, 7)]
    run(4, 32, 8, 8192, 8192, 128, 4300, causal=True, k_mult=2.0, rows=rows, heads=heads)


def test_fp8_errors():
    (q8, k8, v8), (dq, dk, dv) = I.draw_qkv_fp8(1, 2, 2, 64, 64, 4400)
    q, k, v = (torch.from_numpy(x).to(DEV) for x in (q8, k8, v8))
    with pytest.raises(bnd.FaError):
        bnd.fwd_fp8(q, k, v, 0.0, dk, dv)  # descales must be positive
    with pytest.raises(bnd.FaError):
        bnd.fwd_fp8(q[..., :40].contiguous(), k[..., :40].contiguous(), v[..., :40].contiguous(), dq, dk, dv)
