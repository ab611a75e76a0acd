// fa_fwd_kernel.hpp — exact-attention forward kernel for gfx950 (CDNA4, MI355X).
//
// One work-group computes BM = 32*NW query rows of one (batch, query head):
// the FA2 decomposition over (batch, head, Q-tile) with the Q-outer / K,V-inner
// loop order (Triton FA2 walkthrough, xrbh.cn: the loop swap and the
// sequence-dimension grid). Each wave owns 32 query rows for the whole K/V
// sweep (the walkthrough's split of Q across warps, no inter-wave exchange).
//
// Per K/V tile of BN = 64 keys (intelliparadigm page, sections 1.2.1-1.2.2 and
// 2.4: load a block, Q K^T, scale, online-softmax update, P V, accumulate):
//   1. K and V tiles stream from HBM straight into LDS with gfx950's
//      global_load_lds_dwordx4 (no VGPR staging), double-buffered so tile j+1
//      loads while tile j computes (intelliparadigm page, section 3.1, double
//      buffering). Rows are XOR-swizzled in 16-byte chunks so every LDS read
//      below is bank-conflict free (section 3.1's goal; the printed padding
//      formula is not used: a swizzle wastes no LDS).
//   2. S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16}: A = K from LDS
//      (ds_read_b128), B = Q^T held in VGPRs for the whole sweep (Q is read
//      once, the FA2 point). Computing S^T rather than S puts one query per
//      lane: lane l holds 16 keys of query l%32 per 32-key block, so row
//      statistics are in-lane except one swap between the wave's halves.
//   3. Online softmax in fp32 registers (cnblogs page, 时间复杂度: the running
//      max and the denominator taken relative to it). Scores are scaled by
//      c = scale*log2(e) and exponentiated with v_exp_f32 (2^x). The
//      denominator and output are rescaled by 2^(m_old - m_new) only when the
//      row max grows by more than 8 (log2 units): between rescales the
//      exponentials stay <= 2^8, exact-math identical and well inside
//      fp16/bf16 range, and the final division uses the same reference max.
//      The 1/l normalisation is deferred to the epilogue (FA2's fewer
//      non-matmul operations).
//   4. O^T += V^T P^T on the same MFMA: B = P^T comes straight from the S^T
//      accumulator registers (packed to fp16/bf16 with round-to-nearest-even),
//      A = V^T is read from the row-major V tile with ds_read_b64_tr_b16
//      (gfx950's transposing LDS read), so V is never transposed in memory.
//      The row sum l is accumulated in fp32 from the unrounded exponentials.
//   5. Causal (intelliparadigm page, section 1.3: skip the masked half): tiles
//      past a work-group's last row are never loaded or computed, and only tiles
//      straddling the diagonal (or the ragged end of the sequence) are masked.
// Epilogue: O = acc / l, LSE = ln2 * (m + log2 l), stored with one lane per row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBN = 64;             // keys per inner tile
constexpr float kRescaleSlack = 8.0f;  // log2 units the row max may grow before rescaling

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N;
  int group;     // Hq / Hkv
  int n_qtiles;  // ceil(N / BM)
  int total_wg;  // B * Hq * n_qtiles
  float c;       // scale * log2(e)
};

// ---- element-type traits ------------------------------------------------------------------
template <bool BF16>
struct Elt;
template <>
struct Elt<false> {
  using x8 = f16x8;
  static __device__ inline unsigned pack2(float a, float b) {
    return __builtin_bit_cast(unsigned, (f16x2){(_Float16)a, (_Float16)b});  // v_cvt_pk_f16_f32 (RNE)
  }
  static __device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Elt<true> {
  using x8 = bf16x8;
  static __device__ inline unsigned pack2(float a, float b) {
    return __builtin_bit_cast(unsigned, (bf16x2){(__bf16)a, (__bf16)b});  // v_cvt_pk_bf16_f32 (RNE)
  }
  static __device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// ---- LDS swizzles (16-byte chunk index XOR, per row) ----------------------------------------
// LDS has 64 banks x 4 B. K is read with ds_read_b128 by 16 lanes at a time, one row each,
// same logical chunk: 16 consecutive rows must land in 16 different 16-byte bank slots.
// V is read with ds_read_b64_tr_b16: 32 lanes read 4 consecutive rows x 64 contiguous bytes;
// the 4 row segments must land in 4 different 64-byte bank quarters.
template <int D>
__device__ inline int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ inline int swz_v(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// v_permlane32_swap a, b exchanges the upper 32 lanes of a with the lower 32 lanes of b. With
// a = b = x on entry, a ends as the low half of x in both halves and b as the high half. The
// instruction is issued through inline asm on two distinct registers: the compiler builtin,
// given one value for both operands, folds its two results into one, which loses a half.
__device__ inline void halves_of(float x, float& lo, float& hi) {
  unsigned a = __builtin_bit_cast(unsigned, x), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
__device__ inline float wave_half_max(float x) {
  float lo, hi;
  halves_of(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ inline float wave_half_sum(float x) {
  float lo, hi;
  halves_of(x, lo, hi);
  return lo + hi;
}

template <int N>
struct IC {
  static constexpr int value = N;
};

template <bool BF16, int D, bool CAUSAL, bool OUT_F32, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(2))) void fa_fwd_kernel(const Params p) {
  using E = Elt<BF16>;
  constexpr int BM = 32 * NW;
  constexpr int BN = kBN;
  constexpr int KCH = D / 8;             // 16-byte chunks per row
  constexpr int ROWB = D * 2;            // bytes per row
  constexpr int TILE_BYTES = BN * ROWB;  // one K or one V tile
  constexpr int NKS = D / 16;            // MFMA k-steps of Q K^T
  constexpr int NDB = D / 32;            // MFMA d-blocks of P V
  constexpr int NLD = KCH / NW;          // 1 KiB tile-load instructions per wave per matrix
  static_assert(KCH % NW == 0, "each wave issues the same number of tile loads");

  // Two K/V buffers as four separate arrays: the compiler can then prove that the prefetch
  // into one buffer never aliases the reads of the other, and does not stall on it.
  __shared__ __attribute__((aligned(1024))) char sK0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[TILE_BYTES];
  lds_char* const K0 = (lds_char*)sK0;
  lds_char* const V0 = (lds_char*)sV0;
  lds_char* const K1 = (lds_char*)sK1;
  lds_char* const V1 = (lds_char*)sV1;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;  // which half of the wave
  const int l32 = lane & 31;
  const int i16 = lane & 15;
  const int dh = (lane >> 4) & 1;

  // ---- work decomposition: XCD-aware remap, then (b, hkv) groups, longest Q-tiles first ----
  // Work-group i is dispatched to XCD i % 8. Logical work L is laid out so each XCD gets a
  // contiguous range: consecutive L share a K/V head (and GQA siblings run side by side),
  // keeping that head's K/V in the XCD's own L2.
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
  const int t = CAUSAL ? (p.n_qtiles - 1 - t_ord) : t_ord;
  const int b = bk / p.Hkv;
  const int hkv = bk - b * p.Hkv;
  const int hq = hkv * G + g;
  const int N = p.N;

  using T = unsigned short;
  const T* __restrict__ Qp = (const T*)p.q + ((int64_t)(b * p.Hq + hq)) * N * D;
  const char* __restrict__ Kp = (const char*)((const T*)p.k + ((int64_t)bk) * N * D);
  const char* __restrict__ Vp = (const char*)((const T*)p.v + ((int64_t)bk) * N * D);

  const int q0 = t * BM;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + l32;  // this lane's query row
  const int kv_end = CAUSAL ? min(N, q0 + BM) : N;
  const int nt = (kv_end + BN - 1) / BN;

  // ---- per-lane tile-load offsets: instruction ii of this wave fills LDS bytes
  // [ii*1024, ii*1024 + 1024) of a tile; lane l writes physical chunk ii*64 + l, which holds
  // logical chunk (pch ^ swizzle(row)) of tile row `row`.
  int ld_row[NLD], ld_koff[NLD], ld_voff[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int ii = n * NW + wave;
    const int c_lin = ii * 64 + lane;
    const int row = c_lin / KCH, pch = c_lin % KCH;
    ld_row[n] = row;
    ld_koff[n] = (pch ^ swz_k<D>(row)) << 4;
    ld_voff[n] = (pch ^ swz_v<D>(row)) << 4;
  }
  auto load_tile = [&](int j, lds_char* kdst, lds_char* vdst) {
    const int jrow = j * BN;
    const bool full = jrow + BN <= N;  // uniform: only the ragged last tile clamps rows
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int ii = n * NW + wave;
      const int grow = full ? jrow + ld_row[n] : min(jrow + ld_row[n], N - 1);
      const int gbase = grow * ROWB;
      // (the sources go through named locals: passed as expressions, the host compilation
      // silently drops the kernel stub)
      const char* ksrc = Kp + gbase + ld_koff[n];
      const char* vsrc = Vp + gbase + ld_voff[n];
      __builtin_amdgcn_global_load_lds(ksrc, (__attribute__((address_space(3))) void*)(kdst + ii * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vsrc, (__attribute__((address_space(3))) void*)(vdst + ii * 1024), 16, 0, 0);
    }
  };

  // ---- per-lane LDS read offsets, loop invariant
  // K (A operand of S^T = K Q^T): row 32kb + l32 (kb adds an immediate), logical chunk 2ks + h.
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = l32 * ROWB + (((2 * ks + h) ^ swz_k<D>(l32)) << 4);
  // V^T via transposing reads: lane reads row 16t + 8u + 4h + i16/4 (t, u add immediates),
  // columns 32db + 16dh + 4(i16%4) .. +3.
  int voff[NDB];
  {
    const int vrow = 4 * h + (i16 >> 2);
    const int sv = swz_v<D>(vrow);  // equals the swizzle of every row 16t + 8u + vrow
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      voff[db] = vrow * ROWB + (((4 * db + 2 * dh + ((i16 & 3) >> 1)) ^ sv) << 4) + ((i16 & 1) << 3);
  }

  load_tile(0, K0, V0);

  // ---- Q tile -> registers as the MFMA B operand (Q^T): lane l: query l%32, d = 16ks + 8h + 0..7
  u32x4 qreg[NKS];
  {
    const int qr = min(qrow, N - 1);
    const u32x4* src = (const u32x4*)(Qp + (int64_t)qr * D + 8 * h);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[ks] = src[2 * ks];
  }

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = (f32x16){};
  float m_run = -__builtin_inff();  // reference max (scaled, log2 units) shared by both halves
  float l_run = 0.f;                // this lane's partial row sum (its 16 keys of each block)
  const float c = p.c;

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  auto iter = [&](const int j, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const lds_char* kd = BUF ? K1 : K0;
    const lds_char* vd = BUF ? V1 : V0;
    if (j + 1 < nt) load_tile(j + 1, BUF ? K0 : K1, BUF ? V0 : V1);

    const int kbase = j * BN;
    // ---- S^T = K Q^T for two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x16){};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const u32x4 a = *(const lds_u32x4*)(kd + 32 * kb * ROWB + koff[ks]);
        s[kb] = E::mfma(a, qreg[ks], s[kb]);
      }
    }

    // ---- mask: keys after the query (causal) or past the sequence end
    const bool need_mask = (CAUSAL && kbase + BN - 1 > q0w) || (kbase + BN > N);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
          const bool hide = (CAUSAL && key > qrow) || key >= N;
          s[kb][i] = hide ? -__builtin_inff() : s[kb][i];
        }
    }

    // ---- online softmax: row max over the tile (in-lane, then across the two halves)
    float mx = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
    mx = wave_half_max(mx);
    const float mt = mx * c;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      m_run = m_new;
    }

    // ---- P = 2^(S*c - m): fp32 for the row sum (the LSE needs it unrounded), packed to the
    // input type (round to nearest even) as the B operand of P V, one u32x4 per 16-key step
    u32x4 pk[4];
    float rs[16];  // pairwise partial row sums
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int i = 8 * hf + 2 * w;
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, -m_run));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i + 1], c, -m_run));
          pk[2 * kb + hf][w] = E::pack2(e0, e1);
          rs[8 * kb + 4 * hf + w] = e0 + e1;
        }
#pragma unroll
    for (int n = 8; n >= 1; n >>= 1)
#pragma unroll
      for (int i = 0; i < n; ++i) rs[i] += rs[i + n];
    l_run += rs[0];

    // ---- O^T += V^T P^T: A = V^T through transposing LDS reads (two per operand)
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x4 a;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const lds_char* ap = vd + (16 * t2 + 8 * u) * ROWB + voff[db];
          const u32x2 v2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ap));
          a[2 * u] = v2[0];
          a[2 * u + 1] = v2[1];
        }
        acc_o[db] = E::mfma(a, pk[t2], acc_o[db]);
      }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  for (int j = 0; j < nt; j += 2) {
    iter(j, IC<0>{});
    if (j + 1 < nt) iter(j + 1, IC<1>{});
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l)
  const float l_tot = wave_half_sum(l_run);
  if (qrow < N) {
    const float inv = 1.0f / l_tot;
    const int64_t obase = ((int64_t)(b * p.Hq + hq) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int dcol = 32 * db + 8 * g4 + 4 * h;
        const float o0 = acc_o[db][4 * g4 + 0] * inv, o1 = acc_o[db][4 * g4 + 1] * inv;
        const float o2 = acc_o[db][4 * g4 + 2] * inv, o3 = acc_o[db][4 * g4 + 3] * inv;
        if (OUT_F32) {
          *(f32x4*)((float*)p.o + obase + dcol) = (f32x4){o0, o1, o2, o3};
        } else {
          *(u32x2*)((unsigned short*)p.o + obase + dcol) = (u32x2){E::pack2(o0, o1), E::pack2(o2, o3)};
        }
      }
    if (h == 0) p.lse[(int64_t)(b * p.Hq + hq) * N + qrow] = (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
  }
}

}  // namespace fa
