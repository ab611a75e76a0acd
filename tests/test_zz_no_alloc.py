"""GPU check of fa_fwd_split_noalloc, the allocation-free split forward (split partials in the
library's static scratch array), through the C ABI: its output must equal fa_fwd_split's (the
same kernels and plan, with the partials in a caller workspace) bit for bit and lie within the
forward bar of the fp64 oracle, on two calls in a row, the second with a smaller problem (the
scratch then still holds the first call's partials)."""
import numpy as np
import pytest
import torch

from exact_attention_114_amd import binding as bnd
from exact_attention_114_amd import inputs as I
from oracle import attention_band_fp64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O = {I.F16: 2e-3, I.BF16: 1e-2}


def to_dev(bits, dt):
    tdt = torch.float16 if dt == I.F16 else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).to(DEV)


def one_call(B, Hq, Hkv, Nq, Nk, d, dt, left, right, n_splits, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    qb, kb, vb = (I.to_bits(g.standard_normal(s, dtype=np.float32), dt)
                  for s in ((B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)))
    q, k, v = to_dev(qb, dt), to_dev(kb, dt), to_dev(vb, dt)
    in_code = bnd.FA_F16 if dt == I.F16 else bnd.FA_BF16
    scale = I.scale_f32(d ** -0.5)
    need = bnd.split_workspace_bytes(B, Hq, Nq, Nk, d, n_splits)
    assert 0 < need <= bnd.NOALLOC_SCRATCH_BYTES, "the case must split and fit the scratch"
    stream = torch.cuda.current_stream().cuda_stream
    o_a = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=DEV)
    l_a = torch.empty((B, Hq, Nq), dtype=torch.float32, device=DEV)
    o_b, l_b = torch.empty_like(o_a), torch.empty_like(l_a)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    print(f"[gpu] fa_fwd_split_noalloc B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dt} band=({left},{right}) "
          f"splits={n_splits}", flush=True)
    st = bnd.fwd_split_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_a.data_ptr(), l_a.data_ptr(), B, Hq,
                                   Hkv, Nq, Nk, d, scale, left, right, n_splits, in_code, bnd.FA_F32, stream)
    assert st == bnd.FA_OK, bnd.status_str(st)
    st = bnd.fwd_split_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_b.data_ptr(), l_b.data_ptr(), ws.data_ptr(),
                           B, Hq, Hkv, Nq, Nk, d, scale, left, right, n_splits, in_code, bnd.FA_F32, stream)
    assert st == bnd.FA_OK, bnd.status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(l_a, l_b), "differs from fa_fwd_split"
    qf, kf, vf = (I.bits_to_f64(x, dt) for x in (qb, kb, vb))
    O, L = attention_band_fp64(qf, kf, vf, scale, None if left < 0 else left, None if right < 0 else right)
    Og = o_a.cpu().numpy().astype(np.float64)
    Lg = l_a.cpu().numpy().astype(np.float64)
    assert np.abs(Og - O).max() <= TOL_O[dt]
    seen = np.isfinite(L)
    assert (np.abs(Lg[seen] - L[seen]) / np.maximum(1.0, np.abs(L[seen]))).max() <= 1e-4
    assert (Lg[~seen] == -np.inf).all()


def test_noalloc_two_calls_second_smaller():
    one_call(1, 8, 2, 200, 4096, 128, I.BF16, -1, 0, 4, 1901)
    one_call(1, 4, 1, 77, 1500, 64, I.F16, -1, -1, 3, 1902)
