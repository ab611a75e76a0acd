// fa_fwd_fp8_kernel.hpp — exact-attention forward for fp8 (OCP e4m3) inputs on gfx950.
//
// The zyxy lecture (section 5) names fp8 among the input types of the FA2 generation of kernels.
// Here Q, K and V arrive as e4m3 bytes with one float descale per tensor (the real value is
// byte * descale), and both products run on gfx950's fp8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales: 64 products per lane pair and
// instruction, twice the bf16 rate), accumulating in fp32:
//   * S^T = K Q^T, so a lane holds one query and 16 keys of each 32-key block; a step takes 64
//     keys (two blocks), the K-length of one instruction of the P V product;
//   * scale * descale_q * descale_k * log2(e) is folded into one fma before v_exp_f32, and the
//     running max moves every step (exact online softmax);
//   * P is rounded to e4m3 (v_cvt_pk_fp8_f32, nearest even) as the B operand of O^T += V^T P^T:
//     lane (query, half h) holds the keys 32kb + 8g + 4h + i (kb, g < 2, 4; i < 4), in that
//     order, so V^T's 64 keys are stored in the same order: key 32kb + 8g + 4h + i at position
//     32h + 16kb + 4g + i. V reaches LDS transposed by 4x4 byte transposes in registers
//     (v_perm_b32) as the tile is staged;
//   * O is divided by the sum of the rounded P values, formed by one more MFMA of the P operand
//     against an all-ones operand, so that the weights applied to V sum to one; the LSE uses the
//     fp32 sum of the unrounded exponentials; O is finally multiplied by descale_v.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_fwd_kernel.hpp"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned lds_u32;

// The fp8 product of one 32x32 output block and one 64-long K range: unit block scales (E8M0 127).
__device__ inline f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// LDS row pitch (bytes) of the K tile: the head dimension rounded up to the 64-byte K-range of an
// instruction (the rounding is zero padding), plus 16 bytes, an odd number of 16-byte units, so
// that 16 rows read at one column land in 16 different bank groups.
constexpr int fp8_k_pitch(int d) { return ((d + 63) / 64) * 64 + 16; }
constexpr int kFp8VtPitch = 80;  // V^T rows: 64 keys + 16 bytes, 5 units of 16 bytes

template <int D, bool BAND>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_fp8_kernel(const Params p) {
  static_assert(D % 16 == 0 && D >= 32 && D <= 128, "head dimension: a multiple of 16 from 32 to 128");
  constexpr int BM = 128, BN = 64;
  constexpr int NKT = (D + 63) / 64;   // 64-long K ranges of Q K^T
  constexpr int NDB = (D + 31) / 32;   // 32-column blocks of O
  constexpr int KP = fp8_k_pitch(D);
  constexpr int VP = kFp8VtPitch;
  constexpr int KCH = BN * D / 16;     // 16-byte chunks of a K tile
  constexpr int KPER = (KCH + 255) / 256;
  constexpr int VU = 2 * D;            // V units of 4 keys x 8 columns per tile
  constexpr int VPER = (VU + 255) / 256;
  __shared__ __attribute__((aligned(16))) unsigned char sK[BN * KP];
  __shared__ __attribute__((aligned(16))) unsigned char sVt[NDB * 32 * VP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // ---- work: as the fp32 kernel (XCD-aware remap, GQA siblings side by side, banded tiles
  // longest first)
  const int wg = blockIdx.x;
  const int xcd = wg & 7, local = wg >> 3;
  const int per = p.total_wg >> 3, rem = p.total_wg & 7;
  const int L = xcd * per + min(xcd, rem) + local;
  const int G = p.group;
  const int per_kv = p.n_qtiles * G;
  const int bk = L / per_kv;
  const int r0 = L - bk * per_kv;
  const int t_ord = r0 / G;
  const int g = r0 - t_ord * G;
  const int t = BAND ? (p.n_qtiles - 1 - t_ord) : t_ord;
  const int b = bk / p.Hkv, hkv = bk - b * p.Hkv, hq = hkv * G + g;
  const int Nq = p.Nq, Nk = p.Nk;

  const unsigned char* __restrict__ Qp = (const unsigned char*)p.q + (int64_t)(b * p.Hq + hq) * Nq * D;
  const unsigned char* __restrict__ Kp = (const unsigned char*)p.k + (int64_t)bk * Nk * D;
  const unsigned char* __restrict__ Vp = (const unsigned char*)p.v + (int64_t)bk * Nk * D;
  const int q0 = t * BM, q0w = q0 + 32 * wave, qrow = q0w + l32;
  const int qr = min(qrow, Nq - 1);
  const int lo_t = BAND ? max(0, q0 + p.off - p.left) : 0;
  const int hi_t = BAND ? min(Nk - 1, min(q0 + BM, Nq) - 1 + p.off + p.right) : Nk - 1;
  const int j_lo = lo_t / BN;
  const int nt = hi_t >= lo_t ? hi_t / BN - j_lo + 1 : 0;
  const int khi = BAND ? min(Nk - 1, qr + p.off + p.right) : Nk - 1;
  const int klo = BAND ? qr + p.off - p.left : 0;
  const int64_t orow = (int64_t)(b * p.Hq + hq) * Nq + qrow;
  float* const Of = (float*)p.o;

  if (nt == 0) {
    if (qrow < Nq) {
#pragma unroll
      for (int c4 = 0; c4 < D / 8; ++c4) *(f32x4*)(Of + orow * D + 8 * c4 + 4 * h) = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (h == 0) p.lse[orow] = -__builtin_inff();
    }
    return;
  }

  // the padding of the K rows (columns D .. 64 NKT) and the V^T rows past D stay zero
  if constexpr (NKT * 64 != D || NDB * 32 != D) {
    for (int i = tid; i < BN * KP / 4; i += 256) ((unsigned*)sK)[i] = 0u;
    for (int i = tid; i < NDB * 32 * VP / 4; i += 256) ((unsigned*)sVt)[i] = 0u;
  }

  // Q as the B operand of S^T = K Q^T: range tt holds columns 64 tt + 32 h .. + 31 (zeros past D)
  i32x8 qreg[NKT];
#pragma unroll
  for (int tt = 0; tt < NKT; ++tt) {
#pragma unroll
    for (int w4 = 0; w4 < 2; ++w4) {
      const int col = 64 * tt + 32 * h + 16 * w4;
      const u32x4 x = col < D ? *(const u32x4*)(Qp + (int64_t)qr * D + col) : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) qreg[tt][4 * w4 + e] = (int)x[e];
    }
  }

  // ---- tile staging through registers. K: 16-byte chunks (row idx / (D/16)); V: units of 4 keys
  // x 8 columns (4 row segments of 8 bytes), transposed to 8 words of 4 keys
  u32x4 pk[KPER];
  unsigned pv[VPER][8];
  auto fetch = [&](int j) {
#pragma unroll
    for (int n = 0; n < KPER; ++n) {
      const int idx = tid + 256 * n;
      const int row = idx / (D / 16), c16 = idx - row * (D / 16);
      const int key = j * BN + row;
      const bool ok = idx < KCH && key < Nk;
      pk[n] = ok ? *(const u32x4*)(Kp + (int64_t)key * D + 16 * c16) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int n = 0; n < VPER; ++n) {
      const int idx = tid + 256 * n;
      const int kq = idx / (D / 8), c8 = idx - kq * (D / 8);  // keys 4 kq .. + 3, columns 8 c8 .. + 7
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j * BN + 4 * kq + r;
        const bool ok = idx < VU && key < Nk;
        const u32x2 x = ok ? *(const u32x2*)(Vp + (int64_t)key * D + 8 * c8) : (u32x2){0u, 0u};
        pv[n][r] = x[0];
        pv[n][4 + r] = x[1];
      }
    }
  };
  // 4x4 byte transpose: in[r] holds bytes (r, 0..3); out[e] gets bytes (0..3, e)
  auto transpose4 = [](const unsigned (&in)[8], int base, unsigned (&out)[4]) {
    const unsigned t0 = __builtin_amdgcn_perm(in[base + 1], in[base + 0], 0x05010400u);
    const unsigned t1 = __builtin_amdgcn_perm(in[base + 1], in[base + 0], 0x07030602u);
    const unsigned t2 = __builtin_amdgcn_perm(in[base + 3], in[base + 2], 0x05010400u);
    const unsigned t3 = __builtin_amdgcn_perm(in[base + 3], in[base + 2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
  };
  auto store = [&]() {
#pragma unroll
    for (int n = 0; n < KPER; ++n) {
      const int idx = tid + 256 * n;
      if (idx < KCH) {
        const int row = idx / (D / 16), c16 = idx - row * (D / 16);
        *(u32x4*)(sK + row * KP + 16 * c16) = pk[n];
      }
    }
#pragma unroll
    for (int n = 0; n < VPER; ++n) {
      const int idx = tid + 256 * n;
      if (idx < VU) {
        const int kq = idx / (D / 8), c8 = idx - kq * (D / 8);
        // keys 4 kq .. + 3 = 32 kb + 8 g + 4 hh + (0..3) go to positions 32 hh + 16 kb + 4 g + (0..3)
        const int pos = 32 * (kq & 1) + 16 * (kq >> 3) + 4 * ((kq >> 1) & 3);
        unsigned lo[4], hi[4];
        transpose4(pv[n], 0, lo);
        transpose4(pv[n], 4, hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          *(unsigned*)(sVt + (8 * c8 + e) * VP + pos) = lo[e];
          *(unsigned*)(sVt + (8 * c8 + 4 + e) * VP + pos) = hi[e];
        }
      }
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};
  f32x16 acc_l = {};                 // sums of the rounded P, every row of a column alike
  float m_run = -__builtin_inff();
  float l_run = 0.f;                 // this lane's part of the unrounded row sum
  const float c = p.c;
  i32x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = 0x38383838;  // e4m3 1.0

  fetch(j_lo);
  for (int r = 0; r < nt; ++r) {
    const int j = j_lo + r;
    __syncthreads();
    store();
    __syncthreads();
    if (r + 1 < nt) fetch(j + 1);

    // S^T for the step's two 32-key blocks: lane (key l32 of block kb, half h) supplies K columns
    // 64 tt + 32 h .. + 31
    f32x16 st[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      st[kb] = (f32x16){};
#pragma unroll
      for (int tt = 0; tt < NKT; ++tt) {
        const unsigned char* src = sK + (32 * kb + l32) * KP + 64 * tt + 32 * h;
        const u32x4 x0 = *(const u32x4*)src, x1 = *(const u32x4*)(src + 16);
        const i32x8 a = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        st[kb] = mfma_fp8(a, qreg[tt], st[kb]);
      }
    }
    const int kbase = j * BN;
    const bool need_mask = (BAND && (kbase + BN - 1 > min(q0w, Nq - 1) + p.off + p.right ||
                                     kbase < min(q0w + 31, Nq - 1) + p.off - p.left)) ||
                           (kbase + BN > Nk);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
          const bool hide = BAND ? (key > khi || key < klo) : key > khi;
          st[kb][i] = hide ? -__builtin_inff() : st[kb][i];
        }
    }
    float mx = st[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kb][i]);
    const float m_new = fmaxf(fmaxf(m_run, wave_half_max(mx) * c), kRefFloor);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    acc_l *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    // P = 2^(S c - m), summed unrounded and packed to e4m3: byte 16 kb + i of the operand
    i32x8 pw;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][4 * q + 0], c, -m_run));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][4 * q + 1], c, -m_run));
        const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][4 * q + 2], c, -m_run));
        const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][4 * q + 3], c, -m_run));
        l_run += (e0 + e1) + (e2 + e3);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, w, true);
        pw[4 * kb + q] = w;
      }
    // O^T += V^T P^T: lane (column 32 db + l32, half h) supplies V^T row positions 32 h .. + 31
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const unsigned char* src = sVt + (32 * db + l32) * VP + 32 * h;
      const u32x4 x0 = *(const u32x4*)src, x1 = *(const u32x4*)(src + 16);
      const i32x8 a = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      acc[db] = mfma_fp8(a, pw, acc[db]);
    }
    acc_l = mfma_fp8(ones, pw, acc_l);
  }

  // ---- epilogue: O = descale_v * acc / l~ (l~: the rounded sum, element 0 of this lane's column),
  // LSE = ln2 (m + log2 l) from the unrounded sum
  const float l_tot = wave_half_sum(l_run);
  const float lr = acc_l[0];
  if (qrow < Nq) {
    const float inv = lr > 0.f ? p.vscale / lr : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        if (32 * db + 8 * g4 >= D) continue;
        const int dcol = 32 * db + 8 * g4 + 4 * h;
        *(f32x4*)(Of + orow * D + dcol) = (f32x4){acc[db][4 * g4] * inv, acc[db][4 * g4 + 1] * inv,
                                                  acc[db][4 * g4 + 2] * inv, acc[db][4 * g4 + 3] * inv};
      }
    if (h == 0) p.lse[orow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : -__builtin_inff();
  }
}

}  // namespace fa
