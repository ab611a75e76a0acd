"""Seeded synthetic attention inputs and the workload table.

This module only draws and rounds numbers; it computes nothing of attention.
Both the fp64 oracle (through the tests and the benchmark's CPU leg) and the
HIP path consume what it produces, so the two sides see bit-identical inputs.

Recipe (the same for every workload):
  * ``numpy.random.Generator(PCG64(seed))``;
  * draw Q, then K, then V with ``standard_normal(shape, dtype=float32)``;
  * optionally multiply K by a power of two (exact in fp32);
  * round each fp32 value to the storage type with round-to-nearest-even:
    fp16 through numpy's ``astype(float16)``, bf16 by rounding the fp32 bit
    pattern to its upper 16 bits.

Storage is returned as ``uint16`` bit patterns (numpy has no bf16 type) plus
an exact float64 upcast for the oracle.

Shapes follow the pages' workloads: the [B, H, L, D] layout of the memory
table in the CUDA-fusion lecture page (section 1, "traditional attention
memory bottleneck"), the GPT-2 N=1024, d=64 check in the Triton FA2
walkthrough, and that walkthrough's benchmark shape B=4, H=48, d=64 with a
causal mask; grouped-query attention is named in the FA-principles page,
section 1.3.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

F16 = "f16"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention forward problem, fully determined by its fields."""

    name: str
    B: int
    Hq: int
    Hkv: int
    N: int  # query rows per head (and key rows, unless n_keys is given)
    d: int
    dtype: str  # F16 or BF16: storage type of Q, K, V
    causal: bool
    scale: float  # passed to the kernel as a float32
    seed: int
    k_mult: float = 1.0  # exact power-of-two multiplier applied to K before rounding
    window_left: Optional[int] = None  # causal sliding window: row i sees keys i - window_left .. i
    n_keys: Optional[int] = None  # key rows per head when they differ from the query rows

    @property
    def nk(self) -> int:
        return self.N if self.n_keys is None else self.n_keys

    @property
    def band(self):
        """(left, right) edges for the binding: causal, a causal window, or unmasked."""
        if self.window_left is not None:
            return (self.window_left, 0)
        return (None, 0) if self.causal else (None, None)

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs: 4 d per visible (query, key) pair: two N x N x d contractions,
        halved when causal, over the band when windowed. With separate key rows, query row i
        sits at key position i + nk - N and sees the keys up to it when causal."""
        if self.nk != self.N:
            assert self.window_left is None
            n, off = self.N, self.nk - self.N
            pairs = float(n) * self.nk if not self.causal else \
                sum(max(0, min(self.nk, i + off + 1)) for i in range(n))
            return 4.0 * self.B * self.Hq * self.d * pairs
        if self.window_left is not None:
            w, n = self.window_left, self.N
            m = min(w, n)
            pairs = m * (m + 1) / 2.0 + (n - m) * (w + 1.0)
            return 4.0 * self.B * self.Hq * self.d * pairs
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def q_shape(self):
        return (self.B, self.Hq, self.N, self.d)

    def kv_shape(self):
        return (self.B, self.Hkv, self.nk, self.d)


def _c4(n: int) -> Workload:
    return Workload(f"causal_b4_h48_n{n}_d64_f16", 4, 48, 48, n, 64, F16, True, 0.125,
                    40 + int(round(math.log2(n // 1024))))


# The five workloads: single-head, GPT-2 shaped, long head dim, the causal
# sweep, and GQA causal long sequence with K scaled by 2; then four for the
# widened path: a causal sliding window, head dimensions 96 and 32, and a query
# block against long keys.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("single_head_n256_d64_f16", 1, 1, 1, 256, 64, F16, False, 0.125, 1),
        Workload("gpt2_b8_h12_n1024_d64_bf16", 8, 12, 12, 1024, 64, BF16, False, 0.125, 2),
        Workload("long_head_b1_h16_n2048_d128_f16", 1, 16, 16, 2048, 128, F16, False,
                 1.0 / math.sqrt(128.0), 3),
        _c4(1024), _c4(2048), _c4(4096), _c4(8192), _c4(16384),
        Workload("gqa_causal_b4_hq32_hkv8_n8192_d128_bf16", 4, 32, 8, 8192, 128, BF16, True,
                 1.0 / math.sqrt(128.0), 5, k_mult=2.0),
        # the walkthrough's benchmark shape under the operator's sliding window
        # (pre_tokens = 2048, next_tokens = 0; intelliparadigm page, section 2.2)
        Workload("window_b4_h48_n16384_d64_f16_w2048", 4, 48, 48, 16384, 64, F16, True, 0.125, 46,
                 window_left=2048),
        # the walkthrough's causal benchmark shape at N = 8192 with head dimensions that are
        # not 64 or 128 (the intelliparadigm page, section 1.3)
        Workload("causal_b4_h48_n8192_d96_bf16", 4, 48, 48, 8192, 96, BF16, True,
                 1.0 / math.sqrt(96.0), 48),
        Workload("causal_b4_h48_n8192_d32_f16", 4, 48, 48, 8192, 32, F16, True,
                 1.0 / math.sqrt(32.0), 49),
        # a short block of new queries against a long key sequence (the last 512 rows of a
        # causal 32768-token sequence), GQA heads as above: a grid too small to fill the chip
        # unless the keys are split
        Workload("chunk_causal_b1_hq32_hkv8_nq512_nk32768_d128_bf16", 1, 32, 8, 512, 128, BF16, True,
                 1.0 / math.sqrt(128.0), 47, n_keys=32768),
    ]
}

CAUSAL_SWEEP: List[str] = [_c4(n).name for n in (1024, 2048, 4096, 8192, 16384)]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # 32-bit arithmetic cannot overflow for finite values: the largest finite pattern,
    # 0xFF7FFFFF, plus 0x8000 stays below 2^32
    if not np.isfinite(x).all():
        raise ValueError("bf16 rounding expects finite values")
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    return r.astype(np.uint16)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (round to nearest even); uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of fp16/bf16 bit patterns to float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return f32_to_f16_bits(x)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclasses.dataclass
class QKV:
    """Storage bit patterns (uint16) for Q, K, V."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str

    def f64(self):
        return (bits_to_f64(self.q, self.dtype), bits_to_f64(self.k, self.dtype),
                bits_to_f64(self.v, self.dtype))


def draw_qkv(B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str, seed: int,
             k_mult: float = 1.0, Nk: Optional[int] = None) -> QKV:
    """Draw Q [B,Hq,N,d], K and V [B,Hkv,Nk,d] (Nk defaults to N) per the recipe in the module doc."""
    Nk = N if Nk is None else Nk
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = g.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = g.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    if k_mult != 1.0:
        k = k * np.float32(k_mult)
    return QKV(to_bits(q, dtype), to_bits(k, dtype), to_bits(v, dtype), dtype)


def draw_qkv_f32(B: int, Hq: int, Hkv: int, N: int, d: int, seed: int, k_mult: float = 1.0,
                 Nk: Optional[int] = None):
    """The same draws as draw_qkv kept in float32 (the fp32-input path): (q, k, v) arrays."""
    Nk = N if Nk is None else Nk
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, Hq, N, d), dtype=np.float32)
    k = g.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = g.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    if k_mult != 1.0:
        k = k * np.float32(k_mult)
    return q, k, v


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP fp8 e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
    no infinities, largest finite 448), nearest even; values beyond 448 saturate to +-448; uint8
    bits. Normal numbers have exponents -6..8; below 2^-6 the grid is the subnormal one, 2^-9."""
    x = np.asarray(x, dtype=np.float64)
    if not np.isfinite(x).all():
        raise ValueError("e4m3 rounding expects finite values")
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), 448.0)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)                         # below 2^-6: the subnormal spacing 2^-9
    q = np.ldexp(1.0, (e - 3).astype(np.int64))   # grid spacing in this binade
    r = np.round(a / q) * q                       # numpy rounds halves to even
    r = np.minimum(r, 448.0)
    e2 = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    normal = r >= 2.0 ** -6
    exp_f = np.where(normal, e2 + 7, 0).astype(np.int64)
    man = np.where(normal, np.round((r / np.ldexp(1.0, e2.astype(np.int64)) - 1.0) * 8), np.round(r / 2.0 ** -9))
    return (sign | (exp_f.astype(np.uint8) << 3) | man.astype(np.uint8)).astype(np.uint8)


def e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of OCP e4m3 bit patterns (the NaN patterns 0x7F and 0xFF are not produced)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    e = (b >> 3) & 15
    m = b & 7
    v = np.where(e == 0, np.ldexp(m.astype(np.float64), -9), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where(b >> 7 != 0, -v, v)


def draw_qkv_fp8(B: int, Hq: int, Hkv: int, N: int, d: int, seed: int, k_mult: float = 1.0,
                 Nk: Optional[int] = None):
    """fp8 inputs: the draws of draw_qkv_f32, each tensor stored as e4m3 bytes of x / descale with
    descale = max|x| / 448 (float32), the per-tensor scaling that uses e4m3's whole range. Returns
    (q, k, v) uint8 arrays and (descale_q, descale_k, descale_v) floats; the represented values are
    e4m3(bytes) * descale."""
    xs = draw_qkv_f32(B, Hq, Hkv, N, d, seed, k_mult, Nk)
    out, ds = [], []
    for x in xs:
        dsc = float(np.float32(np.abs(x).max() / 448.0))
        out.append(f32_to_e4m3_bits(x.astype(np.float64) / dsc))
        ds.append(dsc)
    return tuple(out), tuple(ds)


def draw_dout(B: int, Hq: int, N: int, d: int, dtype: str, seed: int) -> np.ndarray:
    """The gradient arriving at O for the backward pass: [B,Hq,N,d] standard normal from its
    own PCG64 stream (seed), rounded to the storage type; returns the bit pattern."""
    g = np.random.Generator(np.random.PCG64(seed))
    return to_bits(g.standard_normal((B, Hq, N, d), dtype=np.float32), dtype)


def workload_qkv(w: Workload) -> QKV:
    return draw_qkv(w.B, w.Hq, w.Hkv, w.N, w.d, w.dtype, w.seed, w.k_mult, w.nk)


def scale_f32(scale: float) -> float:
    """The scale as the kernel receives it: rounded to float32, returned as a Python float."""
    return float(np.float32(scale))


def small_case(B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str, causal: bool,
               seed: int, scale: Optional[float] = None, k_mult: float = 1.0) -> Workload:
    """An ad-hoc workload (parity sweeps over odd shapes)."""
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return Workload(f"case_b{B}_hq{Hq}_hkv{Hkv}_n{N}_d{d}_{dtype}_{'c' if causal else 'nc'}_s{seed}",
                    B, Hq, Hkv, N, d, dtype, causal, scale, seed, k_mult)


def document_lengths(B: int, N: int, seed: int, min_len: int, max_len: int) -> List[List[int]]:
    """Lengths of the documents packed into each of B sequences of N tokens: each drawn
    uniformly from [min_len, max_len] with PCG64(seed), the last one cut at N."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(B):
        lens, total = [], 0
        while total < N:
            n = int(min(N - total, g.integers(min_len, max_len + 1)))
            lens.append(n)
            total += n
        out.append(lens)
    return out


def document_mask(lengths: List[List[int]], N: int) -> np.ndarray:
    """[B, 1, N, N] uint8 mask of packed documents: 1 (hidden) where query i and key j lie in
    different documents of their sequence, 0 where they share one."""
    B = len(lengths)
    m = np.ones((B, 1, N, N), np.uint8)
    for b, lens in enumerate(lengths):
        s = 0
        for n in lens:
            m[b, 0, s:s + n, s:s + n] = 0
            s += n
    return m
