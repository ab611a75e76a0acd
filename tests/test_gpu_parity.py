"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars (written here, applied everywhere below):
  * O: max |O_gpu - O_ref| <= 2e-3 for fp16 inputs, <= 1e-2 for bf16 inputs (N(0,1) data);
    when O is stored in the input type, plus half an ulp of that type at |O_ref| (the storage
    rounding, which the fp64 definition does not have);
  * LSE: |LSE_gpu - LSE_ref| <= 1e-4 * max(1, |LSE_ref|) (relative, with a floor of 1 so that
    rows whose LSE is near 0 -- causal row 0 is a single score -- are not held to an
    ill-posed relative bound).
Inputs are the seeded generator's bit patterns; oracle and kernel see identical bits.
Small and ragged shapes are compared element by element; the full-size workloads (the
shapes and launch configuration the benchmark times) on sampled rows the oracle computes
one by one.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_114_amd as fa
from exact_attention_114_amd import binding as bnd
from exact_attention_114_amd import inputs as I
from oracle import attention_fp64, head_attention_fp64, kv_head_of
from oracle.pool import attention_rows_pool, available_cores

pytestmark = pytest.mark.gpu

TOL_O = {I.F16: 2e-3, I.BF16: 1e-2}
TOL_LSE = 1e-4
DEV = "cuda:0"


def tdtype(dt):
    return torch.float16 if dt == I.F16 else torch.bfloat16


def to_dev(bits, dt):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdtype(dt)).to(DEV)


def run_gpu(w, qkv, out_dtype=torch.float32):
    print(f"[gpu] fa_fwd {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} d={w.d} {w.dtype} "
          f"causal={w.causal} seed={w.seed} out={out_dtype}", flush=True)
    q, k, v = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    o, lse = fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def half_ulp(x, dt):
    """Half the spacing of the fp16/bf16 grid at |x|: the error of storing x in that type."""
    bits = I.to_bits(np.abs(x).astype(np.float32), dt)
    lo = I.bits_to_f64(bits, dt)
    hi = I.bits_to_f64(bits + np.uint16(1), dt)
    return 0.5 * (hi - lo)


def assert_close(O, L, O_ref, L_ref, dt, what="", stored_dt=None):
    """O within the bar of the input type; when O is stored in a 16-bit type (stored_dt), that
    storage rounding, half an ulp at |O_ref|, is added to the bar element by element."""
    assert np.isfinite(O).all() and np.isfinite(L).all(), f"{what}: non-finite output"
    bar = TOL_O[dt] if stored_dt is None else TOL_O[dt] + half_ulp(O_ref, stored_dt)
    excess = np.abs(O - O_ref) - bar
    err_o = np.abs(O - O_ref).max()
    err_l = (np.abs(L - L_ref) / np.maximum(1.0, np.abs(L_ref))).max()
    assert excess.max() <= 0, f"{what}: max|dO| = {err_o:.3e}, exceeds the bar by {excess.max():.3e}"
    assert err_l <= TOL_LSE, f"{what}: max LSE rel err = {err_l:.3e} > {TOL_LSE}"
    return err_o, err_l


def check_full(w, out_dtype=torch.float32):
    qkv = I.workload_qkv(w)
    O, L = run_gpu(w, qkv, out_dtype)
    O_ref, L_ref = attention_fp64(*qkv.f64(), I.scale_f32(w.scale), w.causal)
    stored = None if out_dtype == torch.float32 else w.dtype
    return assert_close(O, L, O_ref, L_ref, w.dtype, w.name, stored_dt=stored)


# ---------------------------------------------------------------- the boundary's entry point

@pytest.mark.parametrize("case", ["single_head_n256_d64_f16", "gqa_causal_small"])
def test_fa_fwd_through_ctypes(case):
    """fa_fwd itself, called through ctypes with raw device addresses and torch's stream: the
    single-head workload (fp32 O) and a causal grouped-query case with O in the input type."""
    if case == "single_head_n256_d64_f16":
        w, out_code = I.WORKLOADS[case], bnd.FA_F32
    else:
        w, out_code = I.small_case(2, 8, 2, 777, 128, I.BF16, True, seed=660, k_mult=2.0), bnd.FA_BF16
    qkv = I.workload_qkv(w)
    q, k, v = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    in_code = bnd.FA_F16 if w.dtype == I.F16 else bnd.FA_BF16
    o = torch.empty((w.B, w.Hq, w.N, w.d), dtype=torch.float32 if out_code == bnd.FA_F32 else tdtype(w.dtype),
                    device=DEV)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=DEV)
    print(f"[gpu] fa_fwd via ctypes {w.name}", flush=True)
    st = bnd.fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.Hq, w.Hkv, w.N,
                     w.d, I.scale_f32(w.scale), w.causal, in_code, out_code,
                     torch.cuda.current_stream().cuda_stream)
    assert st == bnd.FA_OK, bnd.status_str(st)
    torch.cuda.synchronize()
    O_ref, L_ref = attention_fp64(*qkv.f64(), I.scale_f32(w.scale), w.causal)
    assert_close(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), O_ref, L_ref,
                 w.dtype, f"fa_fwd {w.name}", stored_dt=None if out_code == bnd.FA_F32 else w.dtype)


# ---------------------------------------------------------------- small and ragged shapes

RAGGED_N = [1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 257]


@pytest.mark.parametrize("N", RAGGED_N)
@pytest.mark.parametrize("d,dt", [(64, I.F16), (64, I.BF16), (128, I.F16), (128, I.BF16)])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_shapes(N, d, dt, causal):
    check_full(I.small_case(1, 2, 1, N, d, dt, causal, seed=100 + N))


@pytest.mark.parametrize("N", [1, 17, 64, 65, 129, 257])
@pytest.mark.parametrize("d,dt", [(32, I.F16), (32, I.BF16), (48, I.F16), (48, I.BF16), (80, I.F16), (80, I.BF16),
                                  (96, I.F16), (96, I.BF16), (112, I.F16), (112, I.BF16)])
@pytest.mark.parametrize("causal", [False, True])
def test_head_dims_not_64_or_128(N, d, dt, causal):
    """Head dimensions that are not 64 or 128: rows sit at a padded LDS pitch, and for 48, 80 and
    112 the last 32-column block of P V is half filled."""
    check_full(I.small_case(1, 2, 1, N, d, dt, causal, seed=700 + N + d))


@pytest.mark.parametrize("d", [32, 48, 80, 96, 112])
def test_head_dims_gqa_many_tiles(d):
    check_full(I.small_case(2, 8, 2, 700, d, I.BF16, True, seed=750 + d, k_mult=2.0))
    check_full(I.small_case(1, 4, 4, 1000, d, I.F16, False, seed=760 + d), out_dtype=torch.float16)


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (8, 2), (8, 1), (16, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_groups(Hq, Hkv, causal):
    check_full(I.small_case(2, Hq, Hkv, 300, 64, I.F16, causal, seed=200 + Hq))
    check_full(I.small_case(1, Hq, Hkv, 200, 128, I.BF16, causal, seed=300 + Hq, k_mult=2.0))


@pytest.mark.parametrize("N", [1, 33, 65, 300])
@pytest.mark.parametrize("dt", [I.F16, I.BF16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [128, 112, 96, 80])
def test_d128_large_grid_shapes(N, dt, causal, d):
    """Grids above two work-groups per CU with d > 64 run the kernel with 32-key steps."""
    T = (N + 127) // 128
    Hq = 4 * (-(-520 // (2 * T * 4)))  # B = 2: at least 520 work-groups, heads a multiple of 4
    w = I.small_case(2, Hq, Hq // 4, N, d, dt, causal, seed=600 + N + d, k_mult=2.0)
    assert bnd.tile(w.B, w.Hq, w.Hkv, w.N, w.d, w.causal, bnd.FA_F16)[1] == 32
    check_full(w)


@pytest.mark.parametrize("dt", [I.F16, I.BF16])
@pytest.mark.parametrize("causal", [False, True])
def test_output_in_input_dtype(dt, causal):
    check_full(I.small_case(2, 4, 2, 333, 64, dt, causal, seed=400), out_dtype=tdtype(dt))
    check_full(I.small_case(1, 2, 2, 190, 128, dt, causal, seed=401), out_dtype=tdtype(dt))


def test_scale_values():
    for s in (1.0, 0.05, 0.3):
        check_full(I.small_case(1, 2, 2, 150, 64, I.F16, True, seed=402, scale=s))


# ---------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["single_head_n256_d64_f16", "gpt2_b8_h12_n1024_d64_bf16",
                                  "long_head_b1_h16_n2048_d128_f16", "causal_b4_h48_n1024_d64_f16"])
def test_workload_full(name):
    check_full(I.WORKLOADS[name])


def sampled_rows(N, rng, n_random=24):
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, N // 2, N - 129, N - 128, N - 65, N - 64, N - 2, N - 1]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(int(x) for x in rng.integers(0, N, n_random))
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["causal_b4_h48_n2048_d64_f16", "causal_b4_h48_n4096_d64_f16",
                                  "causal_b4_h48_n8192_d64_f16", "causal_b4_h48_n16384_d64_f16",
                                  "gqa_causal_b4_hq32_hkv8_n8192_d128_bf16", "causal_b4_h48_n8192_d96_bf16",
                                  "causal_b4_h48_n8192_d32_f16"])
def test_workload_sampled(name):
    w = I.WORKLOADS[name]
    qkv = I.workload_qkv(w)
    O, L = run_gpu(w, qkv)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    rng = np.random.default_rng(w.seed)
    heads = {(0, 0), (w.B - 1, w.Hq - 1), (w.B // 2, w.Hq // 2), (1, min(w.Hq - 1, 5))}
    scale = I.scale_f32(w.scale)
    for (b, hq) in sorted(heads):
        hk = kv_head_of(hq, w.Hq, w.Hkv)
        rows = sampled_rows(w.N, rng)
        q = I.bits_to_f64(qkv.q[b, hq][rows], w.dtype)
        k = I.bits_to_f64(qkv.k[b, hk], w.dtype)
        v = I.bits_to_f64(qkv.v[b, hk], w.dtype)
        O_ref, L_ref = head_attention_fp64(q, k, v, scale, w.causal, q_pos=rows)
        assert_close(O[b, hq][rows], L[b, hq][rows], O_ref, L_ref, w.dtype, f"{name} b={b} h={hq}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["gqa_causal_b4_hq32_hkv8_n8192_d128_bf16", "causal_b4_h48_n4096_d64_f16",
                                  "causal_b4_h48_n8192_d64_f16", "causal_b4_h48_n16384_d64_f16"])
def test_workload_every_output(name):
    """Every O and LSE element of a full-size workload (the launch the benchmark times) against
    the fp64 oracle, computed per batch element on a process pool of the host's cores (at most
    16 processes, the CPU share of one GPU)."""
    w = I.WORKLOADS[name]
    qkv = I.workload_qkv(w)
    O, L = run_gpu(w, qkv)
    workers = max(1, min(16, available_cores()))
    scale = I.scale_f32(w.scale)
    worst_o = worst_l = 0.0
    for b in range(w.B):
        q = I.bits_to_f64(qkv.q[b:b + 1], w.dtype)
        k = I.bits_to_f64(qkv.k[b:b + 1], w.dtype)
        v = I.bits_to_f64(qkv.v[b:b + 1], w.dtype)
        units = [(0, h, range(r0, min(w.N, r0 + 1024))) for h in range(w.Hq) for r0 in range(0, w.N, 1024)]
        for (_, h, rows, o_ref, l_ref) in attention_rows_pool(q, k, v, scale, w.causal, units, workers):
            rows = np.asarray(rows)
            eo, el = assert_close(O[b, h][rows], L[b, h][rows], o_ref, l_ref, w.dtype, f"{name} b={b} h={h}")
            worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
        print(f"{name}: batch element {b} done, max|dO| so far {worst_o:.3e}", flush=True)
    print(f"{name}: every output, max|dO| {worst_o:.3e}, max LSE rel {worst_l:.3e}", flush=True)


# ---------------------------------------------------------------- rescale paths
# The kernel exponentiates each tile against its running reference and accepts the tile while
# every lane's sum of exponentials stays at or below 2^8; otherwise it moves the reference to
# the exact running max and forms the tile again. Seeded N(0,1) data rarely takes that path
# after the first tile, so these inputs force it: scores that keep rising along the sequence
# (a new reference every few tiles), and one late key whose exponential against the stale
# reference is huge (near 2^100 at d = 64) or overflows fp32 (d = 128).

def structured_qkv(w, kind):
    g = np.random.Generator(np.random.PCG64(w.seed))
    q = g.standard_normal(w.q_shape(), dtype=np.float32) + np.float32(1.0)
    k = g.standard_normal(w.kv_shape(), dtype=np.float32)
    v = g.standard_normal(w.kv_shape(), dtype=np.float32)
    if kind == "rising":
        # key j gains 3*j/N along the all-ones direction: its score grows by about 3*sqrt(d)*j/N
        k += (np.float32(3.0) * np.arange(w.N, dtype=np.float32) / np.float32(w.N))[:, None]
    else:
        # a key near the end aligned with the queries' positive mean: score about s*(sqrt(d) + z),
        # z ~ N(0, 1) per row, which puts its exponential near 2^100 (d = 64) or past fp32's
        # range (d >= 96) against the reference the earlier keys set. At d = 32 the spike is
        # s = 64 so that every row's score stays above 60 out to z = -4.5.
        k[:, :, w.N - 5, :] = np.float32(16.0 if w.d >= 64 else 64.0)
    return I.QKV(I.to_bits(q, w.dtype), I.to_bits(k, w.dtype), I.to_bits(v, w.dtype), w.dtype)


@pytest.mark.parametrize("kind", ["rising", "late_spike"])
@pytest.mark.parametrize("d,dt,Hq,Hkv", [(64, I.F16, 4, 2), (64, I.BF16, 4, 2), (128, I.F16, 4, 2),
                                         (128, I.BF16, 4, 2), (128, I.BF16, 88, 8), (32, I.F16, 4, 2),
                                         (96, I.BF16, 4, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_rescale_paths(kind, d, dt, Hq, Hkv, causal):
    w = I.small_case(2, Hq, Hkv, 333, d, dt, causal, seed=600 + d + Hq)
    qkv = structured_qkv(w, kind)
    O, L = run_gpu(w, qkv)
    O_ref, L_ref = attention_fp64(*qkv.f64(), I.scale_f32(w.scale), w.causal)
    if kind == "late_spike":
        seen = slice(w.N - 5, None) if causal else slice(None)
        assert (L_ref[:, :, seen] > 60).all()  # the spike dominates: exp overflows fp32 by far
    assert_close(O, L, O_ref, L_ref, dt, f"{w.name} {kind}")


C_LOG2E = 1.4426950408889634


@pytest.mark.parametrize("dt", [I.F16, I.BF16])
def test_dominant_key_stale_reference(dt):
    """A key that dominates its row arrives in a later tile than the key that set the row's
    reference, 7 to 7.95 (log2 units) above it: the lane-sum check accepts the tile, so the
    dominant weight is an exponential 2^x with an arbitrary mantissa, rounded to the input type
    before it multiplies V = +-5. Normalised by the unrounded sum that rounding would reach O as
    about u |V| (2.4e-3 in fp16, above the bar; tests/test_normaliser_model.py); with the sum of
    the rounded weights it cancels. The rows sweep the alignment: the precondition below checks
    on the CPU that some row would break the bar with the unrounded sum."""
    N, d = 256, 64
    w = I.small_case(1, 1, 1, N, d, dt, False, seed=650)
    g = np.random.Generator(np.random.PCG64(651))
    q = np.zeros((1, 1, N, d), np.float32)
    k = np.zeros((1, 1, N, d), np.float32)
    v = (0.1 * g.standard_normal((1, 1, N, d))).astype(np.float32)
    q[0, 0, :, 0] = np.linspace(38.9, 44.0, N)
    q[0, 0, :, 1] = g.uniform(-1.0, 1.0, N)
    k[0, 0, :, 0] = -8.0                      # every other key: weight below 2^-60
    k[0, 0, 0, 0] = 1.0                       # the reference key, in the first tile
    k[0, 0, 100, :2] = (2.0, 1.0 / 64.0)      # the dominant key, in a later tile
    v[0, 0, 100] = np.where(np.arange(d) % 2 == 0, 5.0, -5.0)
    v[0, 0, 0] = -v[0, 0, 100]
    qkv = I.QKV(I.to_bits(q, dt), I.to_bits(k, dt), I.to_bits(v, dt), dt)
    qf, kf, vf = qkv.f64()
    # precondition (CPU model of the kernel's arithmetic): the unrounded sum would break the bar
    c = np.float32(np.float32(w.scale) * np.float32(C_LOG2E))
    s_ref = (qf[0, 0] @ kf[0, 0, 0]).astype(np.float32)
    s_dom = (qf[0, 0] @ kf[0, 0, 100]).astype(np.float32)
    x = (s_dom.astype(np.float64) * np.float64(c) - (s_ref * c).astype(np.float64)).astype(np.float32)
    p = np.exp2(x.astype(np.float64)).astype(np.float32).astype(np.float64)
    assert (p < 256).all() and (p > 128).all()
    p16 = I.bits_to_f64(I.to_bits(p.astype(np.float32), dt), dt)
    model_err = np.abs((p16 - p) / (p + 1.0))[:, None] * np.abs(vf[0, 0, 100] - vf[0, 0, 0])[None, :]
    assert model_err.max() > TOL_O[dt]
    O, L = run_gpu(w, qkv)
    O_ref, L_ref = attention_fp64(qf, kf, vf, I.scale_f32(w.scale), False)
    err_o, _ = assert_close(O, L, O_ref, L_ref, dt, f"dominant key {dt}")
    print(f"dominant key {dt}: max|dO| {err_o:.3e} (the unrounded-sum model reaches {model_err.max():.3e})")


# ---------------------------------------------------------------- invariants

def test_v_ones_gives_ones():
    w = I.small_case(2, 4, 2, 513, 128, I.BF16, True, seed=500)
    qkv = I.workload_qkv(w)
    qkv.v[...] = I.to_bits(np.ones(qkv.v.shape, np.float32), w.dtype)
    O, _ = run_gpu(w, qkv)
    # O is divided by the sum of the very (rounded) weights that multiply V, so V = 1 gives 1 up
    # to fp32 rounding of the two sums.
    assert np.abs(O - 1.0).max() <= 1e-5


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean(causal):
    w = I.small_case(1, 2, 2, 400, 64, I.F16, causal, seed=501)
    qkv = I.workload_qkv(w)
    qkv.q[...] = 0
    O, L = run_gpu(w, qkv)
    v = I.bits_to_f64(qkv.v, w.dtype)
    n = np.arange(1, w.N + 1)
    for h in range(2):
        if causal:
            exp_O, exp_L = np.cumsum(v[0, h], axis=0) / n[:, None], np.log(n)
        else:
            exp_O, exp_L = np.broadcast_to(v[0, h].mean(axis=0), v[0, h].shape), np.full(w.N, math.log(w.N))
        assert np.abs(O[0, h] - exp_O).max() <= TOL_O[w.dtype]
        assert (np.abs(L[0, h] - exp_L) / np.maximum(1, exp_L)).max() <= TOL_LSE


def test_gqa_equals_repeated_heads_bitwise():
    w = I.small_case(2, 8, 2, 260, 64, I.F16, True, seed=502)
    qkv = I.workload_qkv(w)
    O1, L1 = run_gpu(w, qkv)
    rep = I.QKV(qkv.q, np.repeat(qkv.k, 4, axis=1), np.repeat(qkv.v, 4, axis=1), qkv.dtype)
    w2 = I.small_case(2, 8, 8, 260, 64, I.F16, True, seed=502)
    O2, L2 = run_gpu(w2, rep)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def test_deterministic_and_stream_respected():
    w = I.WORKLOADS["gpt2_b8_h12_n1024_d64_bf16"]
    qkv = I.workload_qkv(w)
    q, k, v = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    o1, l1 = fa.fwd(q, k, v, scale=w.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = fa.fwd(q, k, v, scale=w.scale, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_outputs_written_in_place_and_errors_raise():
    w = I.small_case(1, 2, 2, 100, 64, I.F16, False, seed=503)
    qkv = I.workload_qkv(w)
    q, k, v = (to_dev(x, w.dtype) for x in (qkv.q, qkv.k, qkv.v))
    out = torch.full((1, 2, 100, 64), float("nan"), device=DEV)
    lse = torch.full((1, 2, 100), float("nan"), device=DEV)
    o, l = fa.fwd(q, k, v, scale=w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr() and torch.isfinite(out).all() and torch.isfinite(lse).all()
    with pytest.raises(bnd.FaError):
        fa.fwd(q[..., :40].contiguous(), k[..., :40].contiguous(), v[..., :40].contiguous())  # d = 40
    with pytest.raises(bnd.FaError):
        fa.fwd(q[:, :1].expand(1, 3, 100, 64).contiguous(), k, v)  # 3 query heads over 2 K/V heads
