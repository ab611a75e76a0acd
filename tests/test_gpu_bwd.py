"""GPU parity of the backward pass (fa_bwd through the C ABI) against the fp64 gradient oracle.

The backward consumes O and LSE. Here they come from the oracle (O stored as float32, or in
the input type where a test says so; LSE as float32), so that these tests measure the backward
kernels alone; dO is a seeded standard normal in the input type.

Bar (derived from the arithmetic, written here): the kernels form S, dP and D in fp32, take
P = exp2(S*c - LSE*log2(e)) in fp32, round P and dS to the input type (unit roundoff
u = 2^-11 for fp16, 2^-8 for bf16) before dV = P^T dO, dK = s dS^T Q and dQ = s dS K, and
accumulate those in fp32. The oracle's first-order error analysis of exactly that arithmetic
(head_attention_bwd_bound_fp64: the rounding of P and dS, the fp32 error of S, of dP - D
including its cancellation, of D from the O the kernels are given, and of the fp32
accumulations) gives an elementwise bound B_g, and every element must satisfy
    |g_gpu - g_ref| <= 2 * B_g
where the factor 2 covers the second-order terms the analysis drops.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_114_amd as fa
from exact_attention_114_amd import binding as bnd
from exact_attention_114_amd import inputs as I
from oracle import attention_fp64, kv_head_of
from oracle.backward import attention_bwd_fp64, head_attention_bwd_bound_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
UNIT = {I.F16: 2.0 ** -11, I.BF16: 2.0 ** -8}


def tdtype(dt):
    return torch.float16 if dt == I.F16 else torch.bfloat16


def to_dev(bits, dt):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdtype(dt)).to(DEV)


def bounds(q, k, v, do, o_used, scale, causal, u):
    """Elementwise bounds for all heads; o_used is the O the kernels read."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    bq = np.empty(q.shape)
    bk = np.zeros(k.shape)
    bv = np.zeros(v.shape)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            x, y, z = head_attention_bwd_bound_fp64(q[b, hq], k[b, hk], v[b, hk], do[b, hq], o_used[b, hq],
                                                    scale, causal, u)
            bq[b, hq] = x
            bk[b, hk] += y
            bv[b, hk] += z
    return bq, bk, bv


def run_case(w, o_in_dtype=False, seed_do=None):
    qkv = I.workload_qkv(w)
    q, k, v = qkv.f64()
    do_bits = I.draw_dout(w.B, w.Hq, w.N, w.d, w.dtype, w.seed + 1000 if seed_do is None else seed_do)
    do = I.bits_to_f64(do_bits, w.dtype)
    scale = I.scale_f32(w.scale)
    O, L = attention_fp64(q, k, v, scale, w.causal)
    print(f"[gpu] fa_bwd {w.name} o_in_dtype={o_in_dtype}", flush=True)
    if o_in_dtype:
        o_bits = I.to_bits(O.astype(np.float32), w.dtype)
        o_dev = to_dev(o_bits, w.dtype)
        o_used = I.bits_to_f64(o_bits, w.dtype)
    else:
        o32 = O.astype(np.float32)
        o_dev = torch.from_numpy(o32).to(DEV)
        o_used = o32.astype(np.float64)
    lse_dev = torch.from_numpy(L.astype(np.float32)).to(DEV)
    qd, kd, vd = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    dq, dk, dv = fa.bwd(qd, kd, vd, o_dev, lse_dev, to_dev(do_bits, w.dtype), scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    got = [t.cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    ref = attention_bwd_fp64(q, k, v, do, scale, w.causal)
    bnds = bounds(q, k, v, do, o_used, scale, w.causal, UNIT[w.dtype])
    worst = []
    for name, g, r, b in zip(("dQ", "dK", "dV"), got, ref, bnds):
        assert np.isfinite(g).all(), f"{w.name}: non-finite {name}"
        err = np.abs(g - r)
        bar = 2.0 * b
        ratio = (err / np.maximum(bar, 1e-300)).max()
        worst.append(ratio)
        assert ratio <= 1.0, f"{w.name}: {name} error reaches {ratio:.3f} of the bar (max err {err.max():.3e})"
    return worst


RAGGED_N = [1, 17, 64, 65, 127, 129, 257]


@pytest.mark.parametrize("N", RAGGED_N)
@pytest.mark.parametrize("d,dt", [(64, I.F16), (64, I.BF16), (128, I.F16), (128, I.BF16)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged_shapes(N, d, dt, causal):
    run_case(I.small_case(1, 2, 1, N, d, dt, causal, seed=700 + N + d))


@pytest.mark.parametrize("N", [1, 65, 129, 257])
@pytest.mark.parametrize("d,dt", [(32, I.F16), (32, I.BF16), (96, I.F16), (96, I.BF16)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_head_dims_32_and_96(N, d, dt, causal):
    run_case(I.small_case(1, 2, 1, N, d, dt, causal, seed=770 + N + d))


@pytest.mark.parametrize("d", [32, 96])
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
