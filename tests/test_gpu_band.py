"""GPU parity of the banded entry points (fa_fwd_ex, fa_bwd_ex) against the fp64 oracle.

The band: query row i sits at key position i + Nk - Nq and sees keys i + Nk - Nq - left ..
i + Nk - Nq + right (None: unlimited), the reading the oracle's band_visible documents. A row
that sees no key must give O = 0 and LSE = -inf exactly. The forward bar is the one of
test_gpu_parity (2e-3 fp16, 1e-2 bf16 on O; 1e-4 relative with a floor of 1 on LSE), the
backward bar the one of test_gpu_bwd (bwd_check.py: the input type's rounding and fp32 sums
applied to the magnitude sum of each gradient element's terms).
"""
import math

import numpy as np
import pytest
import torch

import bwd_check
import exact_attention_114_amd as fa
from exact_attention_114_amd import inputs as I
from oracle.attention import attention_band_fp64
from oracle.backward import attention_bwd_band_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {I.F16: 2e-3, I.BF16: 1e-2}
TOL_LSE = 1e-4


def to_dev(bits, dt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dt == I.F16 else torch.bfloat16).to(DEV)


def draw(B, Hq, Hkv, Nq, Nk, d, dt, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    q = I.to_bits(g.standard_normal((B, Hq, Nq, d), dtype=np.float32), dt)
    k = I.to_bits(g.standard_normal((B, Hkv, Nk, d), dtype=np.float32), dt)
    v = I.to_bits(g.standard_normal((B, Hkv, Nk, d), dtype=np.float32), dt)
    do = I.draw_dout(B, Hq, Nq, d, dt, seed + 1)
    return q, k, v, do


def check_fwd(O, L, O_ref, L_ref, dt, what):
    empty = np.isneginf(L_ref)
    assert (np.isneginf(L) == empty).all(), f"{what}: rows without keys differ"
    assert (O[empty] == 0).all(), f"{what}: O of a row without keys is not 0"
    seen = ~empty
    assert np.isfinite(O).all()
    err_o = np.abs(O - O_ref).max()
    err_l = (np.abs(L[seen] - L_ref[seen]) / np.maximum(1.0, np.abs(L_ref[seen]))).max() if seen.any() else 0.0
    assert err_o <= TOL_O[dt], f"{what}: max|dO| = {err_o:.3e}"
    assert err_l <= TOL_LSE, f"{what}: LSE rel err {err_l:.3e}"


BANDS = [  # (Nq, Nk, left, right)
    (300, 300, 64, 0), (300, 300, 100, 17), (300, 300, 0, 0), (257, 257, 5, 5),
    (200, 333, None, 0), (333, 200, None, 0), (200, 333, 40, 0), (1, 500, None, 0),
    (129, 129, None, 31), (96, 160, None, None), (160, 96, 20, 70),
]


@pytest.mark.parametrize("Nq,Nk,left,right", BANDS)
@pytest.mark.parametrize("d,dt", [(64, I.F16), (128, I.BF16), (96, I.F16), (32, I.BF16)])
def test_fwd_band(Nq, Nk, left, right, d, dt):
    seed = 900 + Nq + 3 * Nk + d
    qb, kb, vb, _ = draw(2, 4, 2, Nq, Nk, d, dt, seed)
    scale = 1.0 / math.sqrt(d)
    print(f"[gpu] fa_fwd_ex Nq={Nq} Nk={Nk} band=({left},{right}) d={d} {dt}", flush=True)
    O, L = fa.fwd(to_dev(qb, dt), to_dev(kb, dt), to_dev(vb, dt), scale=scale, window=(left, right))
    torch.cuda.synchronize()
    q, k, v = (I.bits_to_f64(x, dt) for x in (qb, kb, vb))
    O_ref, L_ref = attention_band_fp64(q, k, v, I.scale_f32(scale), left, right)
    check_fwd(O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64), O_ref, L_ref, dt,
              f"band ({left},{right}) Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("left,right", [(96, 0), (None, 0), (33, 33)])
def test_fwd_band_large_grid(left, right):
    # d = 128 grids beyond 512 work-groups take the 32-key step
    Nq, Nk, d, dt = 300, 300, 128, I.BF16
    qb, kb, vb, _ = draw(2, 88, 8, Nq, Nk, d, dt, 950)
    scale = 1.0 / math.sqrt(d)
    O, L = fa.fwd(to_dev(qb, dt), to_dev(kb, dt), to_dev(vb, dt), scale=scale, window=(left, right))
    torch.cuda.synchronize()
    q, k, v = (I.bits_to_f64(x, dt) for x in (qb, kb, vb))
    O_ref, L_ref = attention_band_fp64(q, k, v, I.scale_f32(scale), left, right)
    check_fwd(O.cpu().numpy().astype(np.float64), L.cpu().numpy().astype(np.float64), O_ref, L_ref, dt, "large grid")


def test_causal_flag_equals_band():
    qb, kb, vb, _ = draw(1, 4, 2, 333, 333, 64, I.F16, 960)
    q, k, v = (to_dev(x, I.F16) for x in (qb, kb, vb))
    a = fa.fwd(q, k, v, causal=True)
    b = fa.fwd(q, k, v, window=(None, 0))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("Nq,Nk,left,right", [(300, 300, 64, 0), (200, 333, None, 0), (333, 200, None, 0),
                                              (257, 257, 5, 5), (160, 96, 20, 70), (1, 300, None, 0)])
@pytest.mark.parametrize("d,dt", [(64, I.F16), (128, I.BF16), (96, I.BF16), (32, I.F16)])
def test_bwd_band(Nq, Nk, left, right, d, dt):
    B, Hq, Hkv = 1, 4, 2
    seed = 970 + Nq + Nk + d
    qb, kb, vb, dob = draw(B, Hq, Hkv, Nq, Nk, d, dt, seed)
    scale = 1.0 / math.sqrt(d)
    sc = I.scale_f32(scale)
    q, k, v, do = (I.bits_to_f64(x, dt) for x in (qb, kb, vb, dob))
    O, L = attention_band_fp64(q, k, v, sc, left, right)
    o32 = O.astype(np.float32)
    print(f"[gpu] fa_bwd_ex Nq={Nq} Nk={Nk} band=({left},{right}) d={d} {dt}", flush=True)
    grads = fa.bwd(to_dev(qb, dt), to_dev(kb, dt), to_dev(vb, dt), torch.from_numpy(o32).to(DEV),
                   torch.from_numpy(L.astype(np.float32)).to(DEV), to_dev(dob, dt), scale=scale, window=(left, right))
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in grads]
    ref = attention_bwd_band_fp64(q, k, v, do, sc, left, right)
    mags = bwd_check.magnitudes(q, k, v, do, sc, band=(left, right))
    bwd_check.check(f"band Nq={Nq} Nk={Nk} ({left},{right}) d={d} {dt}", got, ref, mags, dt, d, Nk, (Hq // Hkv) * Nq)


def test_window_workload_sampled_rows():
    """The full-size sliding-window workload as the benchmark times it, on rows the oracle
    computes one by one (rows at the window's edge and spread over the sequence)."""
    from oracle.attention import head_attention_band_fp64

    w = I.WORKLOADS["window_b4_h48_n16384_d64_f16_w2048"]
    qkv = I.workload_qkv(w)
    print(f"[gpu] fa_fwd_ex {w.name}", flush=True)
    O, L = fa.fwd(*(to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v)), scale=w.scale, window=w.band)
    torch.cuda.synchronize()
    O = O.cpu().numpy()
    L = L.cpu().numpy()
    rng = np.random.Generator(np.random.PCG64(7))
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 2049, 8191, w.N - 1], rng.integers(0, w.N, 24)]))
    for b, h in [(0, 0), (1, 17), (3, 47)]:
        q = I.bits_to_f64(qkv.q[b, h][rows], w.dtype)
        k = I.bits_to_f64(qkv.k[b, h], w.dtype)
        v = I.bits_to_f64(qkv.v[b, h], w.dtype)
        O_ref, L_ref = head_attention_band_fp64(q, k, v, I.scale_f32(w.scale), w.window_left, 0, q_pos=rows)
        check_fwd(O[b, h][rows].astype(np.float64), L[b, h][rows].astype(np.float64), O_ref, L_ref, w.dtype,
                  f"{w.name} head ({b},{h})")
