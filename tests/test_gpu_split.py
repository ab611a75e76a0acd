"""GPU parity of split keys (fa_fwd_split): chunks of keys per Q-tile, merged by their LSEs.

The result is the same attention as fa_fwd_ex (the merge is the online-softmax combination of
partial results), so the bars are the forward's: O within 2e-3 (fp16) or 1e-2 (bf16) of the
fp64 oracle, LSE within 1e-4 relative with a floor of 1, rows without keys exactly O = 0 and
LSE = -inf; O stored in 16 bits adds half an ulp of that type.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_114_amd as fa
from exact_attention_114_amd import binding as bnd
from exact_attention_114_amd import inputs as I
from oracle.attention import attention_band_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {I.F16: 2e-3, I.BF16: 1e-2}
TOL_LSE = 1e-4


def to_dev(bits, dt):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dt == I.F16 else torch.bfloat16).to(DEV)


def half_ulp(x, dt):
    bits = I.to_bits(np.abs(x).astype(np.float32), dt)
    return 0.5 * (I.bits_to_f64(bits + np.uint16(1), dt) - I.bits_to_f64(bits, dt))


def run(B, Hq, Hkv, Nq, Nk, d, dt, band, splits, seed, out16=False):
    g = np.random.Generator(np.random.PCG64(seed))
    qb = I.to_bits(g.standard_normal((B, Hq, Nq, d), dtype=np.float32), dt)
    kb = I.to_bits(g.standard_normal((B, Hkv, Nk, d), dtype=np.float32), dt)
    vb = I.to_bits(g.standard_normal((B, Hkv, Nk, d), dtype=np.float32), dt)
    scale = 1.0 / math.sqrt(d)
    print(f"[gpu] fa_fwd_split B={B} Hq={Hq} Nq={Nq} Nk={Nk} d={d} {dt} band={band} splits={splits}", flush=True)
    tq, tk, tv = (to_dev(x, dt) for x in (qb, kb, vb))
    out_dtype = tq.dtype if out16 else torch.float32
    O, L = fa.fwd(tq, tk, tv, scale=scale, window=band, splits=splits, out_dtype=out_dtype)
    O0, L0 = fa.fwd(tq, tk, tv, scale=scale, window=band, out_dtype=out_dtype)
    torch.cuda.synchronize()
    q, k, v = (I.bits_to_f64(x, dt) for x in (qb, kb, vb))
    O_ref, L_ref = attention_band_fp64(q, k, v, I.scale_f32(scale), *band)
    O = O.float().cpu().numpy().astype(np.float64)
    L = L.cpu().numpy().astype(np.float64)
    empty = np.isneginf(L_ref)
    assert (np.isneginf(L) == empty).all() and (O[empty] == 0).all()
    bar = TOL_O[dt] + (half_ulp(O_ref, dt) if out16 else 0.0)
    assert (np.abs(O - O_ref) <= bar).all(), f"max|dO| {np.abs(O - O_ref).max():.3e}"
    seen = ~empty
    if seen.any():
        err_l = (np.abs(L[seen] - L_ref[seen]) / np.maximum(1.0, np.abs(L_ref[seen]))).max()
        assert err_l <= TOL_LSE, f"LSE rel err {err_l:.3e}"
    # the unsplit path on the same inputs
    d_o = np.abs(O - O0.float().cpu().numpy()).max()
    assert d_o <= 2 * TOL_O[dt], d_o
    return bnd.split_workspace_bytes(B, Hq, Nq, Nk, d, splits)


@pytest.mark.parametrize("splits", [0, 2, 3, 16])
@pytest.mark.parametrize("d,dt", [(64, I.F16), (128, I.BF16)])
@pytest.mark.parametrize("band", [(None, None), (None, 0), (300, 0)])
def test_split_small_grid(splits, d, dt, band):
    ws = run(1, 4, 2, 200, 1500, d, dt, band, splits, 1100 + splits + d)
    assert ws > 0  # these shapes do split


@pytest.mark.parametrize("Nq,Nk", [(256, 4096), (1, 3000), (33, 65), (129, 1000)])
@pytest.mark.parametrize("band", [(None, 0), (None, None)])
def test_split_prefill_and_decode_shapes(Nq, Nk, band):
    run(1, 8, 2, Nq, Nk, 128, I.BF16, band, 0, 1200 + Nq + Nk)


@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("band", [(None, None), (None, 0)])
def test_split_head_dims_32_and_96(d, band):
    # 96 / 4 = 24 merge lanes per row do not divide a 256-thread work-group: the tail idles
    ws = run(1, 4, 2, 200, 1500, d, I.BF16, band, 3, 1400 + d)
    assert ws > 0
    run(1, 2, 1, 77, 1000, d, I.F16, band, 0, 1410 + d, out16=True)


@pytest.mark.parametrize("dt", [I.F16, I.BF16])
def test_split_output_in_input_dtype(dt):
    run(1, 4, 4, 300, 2048, 64, dt, (None, 0), 4, 1300, out16=True)


def test_split_long_head_workload():
    w = I.WORKLOADS["long_head_b1_h16_n2048_d128_f16"]
    run(w.B, w.Hq, w.Hkv, w.N, w.N, w.d, w.dtype, (None, None), 0, w.seed)


def test_split_chunk_workload_sampled_rows():
    """The query-block workload (512 causal rows against 32768 keys) at full size, split as the
    benchmark runs it, on rows the oracle computes one by one: each Q-tile's first and last rows,
    the tail, and random rows."""
    from oracle.attention import head_attention_band_fp64

    w = I.WORKLOADS["chunk_causal_b1_hq32_hkv8_nq512_nk32768_d128_bf16"]
    qkv = I.workload_qkv(w)
    ns = bnd.split_workspace_bytes(w.B, w.Hq, w.N, w.nk, w.d, 0) // (w.B * w.Hq * w.N * (w.d + 1) * 4)
    assert ns > 1  # the grid is too small to fill the chip: the library splits the keys
    print(f"[gpu] fa_fwd_split {w.name} splits={ns}", flush=True)
    O, L = fa.fwd(*(to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v)), scale=w.scale, window=w.band, splits=0)
    torch.cuda.synchronize()
    O = O.cpu().numpy().astype(np.float64)
    L = L.cpu().numpy().astype(np.float64)
    rng = np.random.Generator(np.random.PCG64(9))
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 255, 256, 383, 384, 510, 511], rng.integers(0, w.N, 16)]))
    for b, h in [(0, 0), (0, 13), (0, 31)]:
        q = I.bits_to_f64(qkv.q[b, h][rows], w.dtype)
        k = I.bits_to_f64(qkv.k[b, h // (w.Hq // w.Hkv)], w.dtype)
        v = I.bits_to_f64(qkv.v[b, h // (w.Hq // w.Hkv)], w.dtype)
        O_ref, L_ref = head_attention_band_fp64(q, k, v, I.scale_f32(w.scale), None, 0, off=w.nk - w.N, q_pos=rows)
        err_o = np.abs(O[b, h][rows] - O_ref).max()
        assert err_o <= TOL_O[w.dtype], f"head ({b},{h}) max|dO| {err_o:.3e}"
        err_l = (np.abs(L[b, h][rows] - L_ref) / np.maximum(1.0, np.abs(L_ref))).max()
        assert err_l <= TOL_LSE, f"head ({b},{h}) LSE rel err {err_l:.3e}"
