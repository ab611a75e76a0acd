"""GPU parity of the backward pass (fa_bwd through the C ABI) against the fp64 gradient oracle.

The backward consumes O and LSE. In most tests they come from the oracle (O stored as float32,
or in the input type where a test says so; LSE as float32), so that these tests measure the
backward kernels alone; the end-to-end tests at the benchmark's causal N = 8192 shapes take them
from fa.fwd instead. dO is a seeded standard normal in the input type.

Bar (bwd_check.py, stated before any kernel choice): every element g satisfies
    |g_gpu - g_ref| <= (2u + (d + n) e32) * M_g
with M_g the sum of the magnitudes of the terms of g (the chain rule written out as products of
the inputs, P and O), u the input type's unit roundoff (2^-11 fp16, 2^-8 bf16), e32 = 2^-24 and
n the terms per element. Each case prints its worst error-to-bar ratio per gradient.
"""
import math

import numpy as np
import pytest
import torch

import bwd_check
import exact_attention_114_amd as fa
from exact_attention_114_amd import binding as bnd
from exact_attention_114_amd import inputs as I
from oracle import attention_fp64, kv_head_of
from oracle.backward import attention_bwd_fp64, head_attention_bwd_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def tdtype(dt):
    return torch.float16 if dt == I.F16 else torch.bfloat16


def to_dev(bits, dt):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdtype(dt)).to(DEV)


def run_case(w, o_in_dtype=False, seed_do=None):
    qkv = I.workload_qkv(w)
    q, k, v = qkv.f64()
    do_bits = I.draw_dout(w.B, w.Hq, w.N, w.d, w.dtype, w.seed + 1000 if seed_do is None else seed_do)
    do = I.bits_to_f64(do_bits, w.dtype)
    scale = I.scale_f32(w.scale)
    O, L = attention_fp64(q, k, v, scale, w.causal)
    print(f"[gpu] fa_bwd {w.name} o_in_dtype={o_in_dtype}", flush=True)
    if o_in_dtype:
        o_dev = to_dev(I.to_bits(O.astype(np.float32), w.dtype), w.dtype)
    else:
        o_dev = torch.from_numpy(O.astype(np.float32)).to(DEV)
    lse_dev = torch.from_numpy(L.astype(np.float32)).to(DEV)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    dq, dk, dv = fa.bwd(qd, kd, vd, o_dev, lse_dev, to_dev(do_bits, w.dtype), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    ref = attention_bwd_fp64(q, k, v, do, scale, w.causal)
    mags = bwd_check.magnitudes(q, k, v, do, scale, w.causal)
    G = w.Hq // w.Hkv
    return bwd_check.check(w.name, got, ref, mags, w.dtype, w.d, w.N, G * w.N)


RAGGED_N = [1, 17, 64, 65, 127, 129, 257]


@pytest.mark.parametrize("N", RAGGED_N)
@pytest.mark.parametrize("d,dt", [(64, I.F16), (64, I.BF16), (128, I.F16), (128, I.BF16)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged_shapes(N, d, dt, causal):
    run_case(I.small_case(1, 2, 1, N, d, dt, causal, seed=700 + N + d))


@pytest.mark.parametrize("N", [1, 65, 129, 257])
@pytest.mark.parametrize("d,dt", [(32, I.F16), (32, I.BF16), (48, I.F16), (48, I.BF16), (80, I.F16), (80, I.BF16),
                                  (96, I.F16), (96, I.BF16), (112, I.F16), (112, I.BF16)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_head_dims_not_64_or_128(N, d, dt, causal):
    run_case(I.small_case(1, 2, 1, N, d, dt, causal, seed=770 + N + d))


@pytest.mark.parametrize("d", [32, 48, 80, 96, 112])
def test_bwd_head_dims_gqa(d):
    run_case(I.small_case(2, 8, 2, 400, d, I.BF16, True, seed=780 + d, k_mult=2.0))
    run_case(I.small_case(1, 4, 4, 300, d, I.F16, False, seed=790 + d), o_in_dtype=True)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (8, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_gqa_groups(Hq, Hkv, causal):
    run_case(I.small_case(2, Hq, Hkv, 200, 128, I.BF16, causal, seed=720 + Hq + Hkv))


@pytest.mark.parametrize("dt", [I.F16, I.BF16])
def test_bwd_o_in_input_dtype(dt):
    run_case(I.small_case(1, 4, 2, 300, 64, dt, True, seed=730), o_in_dtype=True)


@pytest.mark.parametrize("name,shape", [
    ("c4 shape at N=1024", (1, 4, 4, 1024, 64, I.F16, True, 0.125, 1.0)),
    ("GQA shape at N=1024, K x2", (1, 8, 2, 1024, 128, I.BF16, True, 1.0 / math.sqrt(128), 2.0)),
    ("gpt2 shape", (1, 4, 4, 1024, 64, I.BF16, False, 0.125, 1.0)),
])
def test_bwd_workload_shapes(name, shape):
    B, Hq, Hkv, N, d, dt, causal, scale, km = shape
    w = I.small_case(B, Hq, Hkv, N, d, dt, causal, seed=740 + N + d, scale=scale, k_mult=km)
    print(name, run_case(w), flush=True)


def test_bwd_deterministic():
    w = I.small_case(1, 4, 2, 333, 128, I.BF16, True, seed=750)
    qkv = I.workload_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    o, lse = fa.fwd(qd, kd, vd, scale=w.scale, causal=True)
    do = to_dev(I.draw_dout(1, 4, 333, 128, w.dtype, 751), w.dtype)
    a = fa.bwd(qd, kd, vd, o, lse, do, scale=w.scale, causal=True)
    b = fa.bwd(qd, kd, vd, o, lse, do, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_errors_raise():
    w = I.small_case(1, 2, 2, 64, 64, I.F16, False, seed=760)
    qkv = I.workload_qkv(w)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    o, lse = fa.fwd(qd, kd, vd)
    with pytest.raises(bnd.FaError):
        fa.bwd(qd, kd, vd, o, lse, qd.float())  # dout in the wrong dtype
    with pytest.raises(bnd.FaError):
        fa.bwd(qd, kd, vd, o, lse, qd, workspace=torch.empty(8, dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("name,heads", [
    ("gqa_causal_b4_hq32_hkv8_n8192_d128_bf16", [(1, 12), (1, 13), (1, 14), (1, 15)]),
    ("causal_b4_h48_n8192_d64_f16", [(0, 0), (2, 17), (3, 47)]),
])
def test_bwd_end_to_end_timed_shapes(name, heads):
    """The backward as the benchmark times it: the full-size causal N = 8192 workload, O and
    LSE from fa.fwd (fp32 O), dO drawn as the benchmark draws it, then fa_bwd. Every row of the
    listed query heads (dQ) and of their K/V heads (dK, dV: each listed group is complete, so the
    oracle's sum over the group's query heads is the whole gradient) is compared with the oracle.
    O carries the forward's own rounding of P into D here; the bar's second rounding covers it."""
    w = I.WORKLOADS[name]
    print(f"[gpu] fa_fwd + fa_bwd end to end {name}", flush=True)
    qkv = I.workload_qkv(w)
    dob = I.draw_dout(w.B, w.Hq, w.N, w.d, w.dtype, w.seed + 1000)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    dod = to_dev(dob, w.dtype)
    o, lse = fa.fwd(qd, kd, vd, scale=w.scale, causal=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    del o, lse
    G = w.Hq // w.Hkv
    groups = sorted({(b, kv_head_of(h, w.Hq, w.Hkv)) for b, h in heads})
    assert all(sum(1 for bb, hh in heads if bb == b and kv_head_of(hh, w.Hq, w.Hkv) == hk) == G
               for b, hk in groups), "each listed K/V group must be complete"
    scale = I.scale_f32(w.scale)
    worst = [0.0, 0.0, 0.0]
    for b, hk in groups:
        k = I.bits_to_f64(qkv.k[b, hk], w.dtype)
        v = I.bits_to_f64(qkv.v[b, hk], w.dtype)
        gk = np.zeros(k.shape)
        gv = np.zeros(k.shape)
        mk = np.zeros(k.shape)
        mv = np.zeros(k.shape)
        for h in range(hk * G, (hk + 1) * G):
            q = I.bits_to_f64(qkv.q[b, h], w.dtype)
            do = I.bits_to_f64(dob[b, h], w.dtype)
            a, c, e = head_attention_bwd_fp64(q, k, v, do, scale, True)
            x, y, z = bwd_check.head_attention_bwd_magnitude_fp64(q, k, v, do, scale, True)
            gk += c
            gv += e
            mk += y
            mv += z
            got_q = dq[b, h].cpu().numpy().astype(np.float64)
            worst[0] = max(worst[0], bwd_check.check_one(f"{name} b={b} hq={h}", "dQ", got_q, a, x, w.dtype, w.d, w.N))
        got_k = dk[b, hk].cpu().numpy().astype(np.float64)
        got_v = dv[b, hk].cpu().numpy().astype(np.float64)
        worst[1] = max(worst[1], bwd_check.check_one(f"{name} b={b} hkv={hk}", "dK", got_k, gk, mk, w.dtype, w.d,
                                                     G * w.N))
        worst[2] = max(worst[2], bwd_check.check_one(f"{name} b={b} hkv={hk}", "dV", got_v, gv, mv, w.dtype, w.d,
                                                     G * w.N))
    print(f"[bar] {name} end to end: worst error/bar dQ {worst[0]:.4f} dK {worst[1]:.4f} dV {worst[2]:.4f}",
          flush=True)
