// fa_fwd_f32_kernel.hpp — exact-attention forward for fp32 inputs on gfx950.
//
// The Ascend operator on the intelliparadigm page (section 2.2) takes query, key and value in
// fp16, bf16 or fp32. fp32 inputs keep fp32 arithmetic throughout: both products run on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32, K = 2 per instruction; gfx950 has no reduced-precision
// xf32 form), so no input or probability is rounded below fp32. The structure is the 16-bit
// kernel's without its 16-bit tricks:
//   * one work-group of 4 waves per (batch, query head, 128-row Q-tile), 32 rows per wave;
//   * K/V tiles of 32 keys staged through LDS (rows padded by 8 floats so that the two halves of
//     a wave read disjoint banks), the next tile fetched into registers while the current one is
//     used;
//   * S^T = K Q^T, so a lane holds one query and 16 of the tile's keys: the row statistics are
//     in-lane plus one swap between the wave's halves;
//   * the online softmax with the running max moved every tile (exact: no 16-bit overflow to
//     avoid here), exponentials in base 2 with scale * log2(e) folded into one fma;
//   * O^T += V^T P^T with P taken straight from the S^T accumulator (fp32, unrounded): for
//     accumulator element i the lane's key is 8(i/4) + 4h + i%4, so each of the 16 MFMAs of a
//     32-column block pairs the two halves' keys of element i;
//   * O = acc / l and LSE = ln2 (m + log2 l) at the end; bands as the 16-bit kernel (causal is
//     the band (unlimited, 0)).
#pragma once

#include <hip/hip_runtime.h>

#include "fa_fwd_kernel.hpp"

namespace fa {

template <int D, bool BAND>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) __attribute__((amdgpu_waves_per_eu(2)))
void fa_fwd_f32_kernel(const Params p) {
  static_assert(D % 16 == 0 && D >= 32 && D <= 128, "head dimension: a multiple of 16 from 32 to 128");
  constexpr int BM = 128, BN = 32;
  constexpr int NDB = (D + 31) / 32;      // 32-column blocks of O (the last one half filled for D % 32 == 16)
  constexpr int NS = D / 8;               // 8-column slices of Q K^T (4 columns per wave half)
  constexpr int PITCH = D + 8;            // LDS row pitch in floats: row r + 4 starts 32 banks further
  constexpr int V4 = BN * D / 4;          // float4 per tile
  constexpr int PER = (V4 + 255) / 256;   // float4 per thread per tile
  __shared__ __attribute__((aligned(16))) float sK[BN * PITCH];
  __shared__ __attribute__((aligned(16))) float sV[BN * PITCH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // ---- work: XCD-aware remap (work-group i runs on XCD i % 8), then (b, hkv) groups with their
  // GQA siblings side by side, Q-tiles longest first when banded
  const int wg = blockIdx.x;
  const int xcd = wg & 7, local = wg >> 3;
  const int per = p.total_wg >> 3, rem = p.total_wg & 7;
  const int L = xcd * per + min(xcd, rem) + local;
  const int G = p.group;
  const int per_kv = p.n_qtiles * G;
  const int bk = L / per_kv;  // b * Hkv + hkv
  const int r0 = L - bk * per_kv;
  const int t_ord = r0 / G;
  const int g = r0 - t_ord * G;
  const int t = BAND ? (p.n_qtiles - 1 - t_ord) : t_ord;
  const int b = bk / p.Hkv, hkv = bk - b * p.Hkv, hq = hkv * G + g;
  const int Nq = p.Nq, Nk = p.Nk;

  const float* __restrict__ Qp = (const float*)p.q + (int64_t)(b * p.Hq + hq) * Nq * D;
  const float* __restrict__ Kp = (const float*)p.k + (int64_t)bk * Nk * D;
  const float* __restrict__ Vp = (const float*)p.v + (int64_t)bk * Nk * D;
  const int q0 = t * BM, q0w = q0 + 32 * wave, qrow = q0w + l32;
  const int qr = min(qrow, Nq - 1);  // rows past Nq behave as the last row (never stored)
  const int lo_t = BAND ? max(0, q0 + p.off - p.left) : 0;
  const int hi_t = BAND ? min(Nk - 1, min(q0 + BM, Nq) - 1 + p.off + p.right) : Nk - 1;
  const int j_lo = lo_t / BN;
  const int nt = hi_t >= lo_t ? hi_t / BN - j_lo + 1 : 0;
  const int khi = BAND ? min(Nk - 1, qr + p.off + p.right) : Nk - 1;
  const int klo = BAND ? qr + p.off - p.left : 0;
  const int64_t orow = (int64_t)(b * p.Hq + hq) * Nq + qrow;
  float* const Of = (float*)p.o;

  if (nt == 0) {  // no row of this Q-tile sees a key: O = 0, LSE = -inf (the whole work-group returns)
    if (qrow < Nq) {
#pragma unroll
      for (int c4 = 0; c4 < D / 8; ++c4) *(f32x4*)(Of + orow * D + 8 * c4 + 4 * h) = (f32x4){0.f, 0.f, 0.f, 0.f};
      if (h == 0) p.lse[orow] = -__builtin_inff();
    }
    return;
  }

  // Q as the B operand of S^T = K Q^T: slice s, element e is column 8s + 4h + e
  f32x4 qv[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) qv[s] = *(const f32x4*)(Qp + (int64_t)qr * D + 8 * s + 4 * h);

  // tile loads: float4 n of this thread is float4 idx = tid + 256 n of the tile (row idx / (D/4));
  // rows past Nk and threads past the tile's end read zeros
  f32x4 pk[PER], pv[PER];
  auto fetch = [&](int j) {
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int idx = tid + 256 * n;
      const int row = idx / (D / 4), c4 = idx - row * (D / 4);
      const int key = j * BN + row;
      const bool ok = idx < V4 && key < Nk;
      const int64_t off = (int64_t)(ok ? key : 0) * D + 4 * c4;
      pk[n] = ok ? *(const f32x4*)(Kp + off) : (f32x4){0.f, 0.f, 0.f, 0.f};
      pv[n] = ok ? *(const f32x4*)(Vp + off) : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int idx = tid + 256 * n;
      if (idx < V4) {
        const int row = idx / (D / 4), c4 = idx - row * (D / 4);
        *(f32x4*)(sK + row * PITCH + 4 * c4) = pk[n];
        *(f32x4*)(sV + row * PITCH + 4 * c4) = pv[n];
      }
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};
  float m_run = -__builtin_inff();  // running max of the scaled scores, log2 units
  float l_run = 0.f;                // this lane's part of the row sum
  const float c = p.c;

  fetch(j_lo);
  for (int r = 0; r < nt; ++r) {
    const int j = j_lo + r;
    __syncthreads();  // every wave is done reading the previous tile
    store();
    __syncthreads();
    if (r + 1 < nt) fetch(j + 1);  // in flight while this tile is used

    // S^T = K Q^T: lane (key l32, half h) supplies K[l32][8s + 4h + e] for MFMA (s, e)
    f32x16 st = {};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const f32x4 a = *(const f32x4*)(sK + l32 * PITCH + 8 * s + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) st = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qv[s][e], st, 0, 0, 0);
    }
    // keys outside the lane's band [klo, khi] (khi also stops at the end of the keys)
    const int kbase = j * BN;
    const bool need_mask = (BAND && (kbase + BN - 1 > min(q0w, Nq - 1) + p.off + p.right ||
                                     kbase < min(q0w + 31, Nq - 1) + p.off - p.left)) ||
                           (kbase + BN > Nk);
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + 8 * (i >> 2) + 4 * h + (i & 3);
        const bool hide = BAND ? (key > khi || key < klo) : key > khi;
        st[i] = hide ? -__builtin_inff() : st[i];
      }
    }
    // online softmax: the running max moves to this tile's row max, O and l are rescaled
    float mx = st[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, st[i]);
    const float m_new = fmaxf(fmaxf(m_run, wave_half_max(mx) * c), kRefFloor);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[i], c, -m_run));
      l_run += st[i];
    }
    // O^T += V^T P^T: MFMA i of block db pairs key 8(i/4) + i%4 (half 0) with the key 4 further
    // (half 1); lane (column l32, half h) supplies V[8(i/4) + 4h + i%4][32 db + l32]
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int dcol = 32 * db + l32;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * h + (i & 3);
        const float a = (D % 32 == 0 || dcol < D) ? sV[key * PITCH + dcol] : 0.f;
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, st[i], acc[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln2 (m + log2 l); a row that saw no key gets O = 0, LSE = -inf
  const float l_tot = wave_half_sum(l_run);
  if (qrow < Nq) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
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
