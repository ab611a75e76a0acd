// fa_bwd_kernel.hpp — exact-attention backward kernels for gfx950 (CDNA4, MI355X).
//
// The backward pass recomputes the attention matrix from Q, K, V and the forward's saved
// statistics instead of storing it (intelliparadigm page, section 1.2.3, recomputation; the
// cnblogs page's summary; the Triton FA2 walkthrough keeps logsumexp L for it). Per head, with
// s the scale and dO the gradient arriving at O:
//   P = exp(s Q K^T - LSE)      (masked entries 0)
//   dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,  dS = P o (dP - D)
//   dQ = s dS K,  dK = s dS^T Q  (K/V-head gradients summed over the head's query group)
// Three kernels:
//   1. prep: per query row, D = rowsum(dO o O) and the LSE in log2 units, into a workspace laid
//      out per 32-row block as [32 LSE*log2(e) | 32 -D] (rows past Nq hold zeros; a row that
//      sees no key holds +inf, which makes its P zero).
// Masks are the forward's band (causal is left unlimited, right 0; query row i sits at key
// position i + Nk - Nq); each kernel visits only the tiles a band touches.
//   2. dK/dV: a work-group owns 32*NW keys of one (batch, K/V head); each wave keeps its 32 keys'
//      K and V rows as MFMA operands and its dK, dV accumulators in registers, and sweeps every
//      32-row query block of every query head of the group. Q and dO blocks stream through LDS
//      (LDS-DMA, double-buffered). S = Q K^T and dP = dO V^T come out with one key per lane, so
//      P and dS pack straight into the A operand of dV += P^T dO and dK += dS^T Q, whose
//      B operands are Q and dO read transposed from LDS (ds_read_b64_tr_b16). No atomics.
//   3. dQ: a work-group owns 32*NW query rows of one (batch, query head), like the forward;
//      K and V tiles stream through LDS. S^T = K Q^T and dP^T = V dO^T put one query per lane, so
//      dS packs into the A operand of dQ += dS K, whose B operand is K read transposed.
// dQ is kept out of the dK/dV kernel: forming it there would need dS transposed and a
// cross-work-group sum over key tiles (atomics). Re-forming S and dP in a second kernel costs
// two more products per tile instead, with no atomics.
#pragma once

#include "fa_fwd_kernel.hpp"

namespace fa {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  float* ws;     // per (b, hq) and 32-row block: 32 floats LSE*log2(e), then 32 floats -D
  int B, Hq, Hkv;
  int Nq, Nk;    // query and key rows per head
  int off;       // Nk - Nq: key position of query row 0
  int left, right;  // band edges (1 << 30: unlimited), as in the forward
  int group;     // Hq / Hkv
  int n_blk32;   // ceil(Nq / 32): query blocks the dK/dV kernel sweeps
  int ws_blk;    // 32-row blocks per head in the workspace: 4 * ceil(Nq / 128), so that every
                 // wave of a dQ work-group finds its block (rows past Nq hold zeros)
  int n_tiles;   // work-group tiles along the sequence: ceil(Nk / 128) for dK/dV, ceil(Nq / 128) for dQ
  int total_wg;
  int ilv;       // (b, hkv) groups whose tiles are interleaved longest first (1, 2 or 4)
  float c;       // scale * log2(e)
  float scale;
  // optional byte mask (kernels built with AM), as in the forward's Params: nonzero hides key j
  // from query i of head (b, hq) at am + b*am_sb + hq*am_sh + i*am_ld + j
  const unsigned char* am;
  long long am_sb, am_sh;
  int am_ld;
  // the mask as fa_mask_prep_kernel leaves it (kernels built with AM; strides 0 along an axis
  // the mask shares): bits as in the forward's Params (dQ), the key hull of each 128-row Q-tile
  // (dQ), and a flag per 128-key tile and Q-tile where the block has a visible pair (dK/dV)
  const unsigned* am_bits;
  long long bits_sb, bits_sh;
  int am_nw;
  const int2* am_hull;
  long long hull_sb, hull_sh;
  int hull_nch;
  const unsigned char* am_flags;  // plane (b, hq) at am_flags + b*flags_sb + hq*flags_sh: [kt][t]
  long long flags_sb, flags_sh;
  int flags_nq;                   // Q-tiles per row of flags
  // the mask as column words (dK/dV): plane (b, hq) at am_cbits + b*cbits_sb + hq*cbits_sh,
  // word [j][qb] with bit r set where key j is hidden from query 32 qb + r
  const unsigned* am_cbits;
  long long cbits_sb, cbits_sh;
  int cbits_nqb;                  // 32-row query blocks per key
  // dropout (kernels built with DROP), as in the forward's Params: pair (i, j) of head plane
  // b * Hq + hq is kept iff its Philox byte is below keep_t; kept terms are scaled by drop_scale
  unsigned seed_lo, seed_hi, drop_offset;
  int keep_t;
  float drop_scale;
  // additive mask (kernels built with FM = its element bytes), as in the forward's Params
  const void* fm;
  long long fm_sb, fm_sh;
  int fm_ld;
  float inv_scale;
};

// One additive-mask value (FM = 2: fp16, 4: fp32) at byte offset vo of a plane's descriptor.
template <int FM>
__device__ inline float fm_load1(__amdgpu_buffer_rsrc_t r, int vo) {
  if constexpr (FM == 4)
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, vo, 0, 0));
  else
    return (float)__builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(r, vo, 0, 0));
}

// 4x4 byte transpose: out[t] byte r = byte t of w[r].
__device__ inline void byte_transpose4(const unsigned (&w)[4], unsigned (&out)[4]) {
  // (w0.b0, w1.b0, w0.b1, w1.b1) and (w0.b2, w1.b2, w0.b3, w1.b3); the same for w2, w3
  const unsigned a_lo = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
  const unsigned a_hi = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
  const unsigned b_lo = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const unsigned b_hi = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
}

// Keep test of one pair: byte `sel` of word (bits 8 sel ..) below t.
__device__ inline bool kept(unsigned word, int sel, int t) { return (int)((word >> (8 * sel)) & 0xFFu) < t; }

// One LDS swizzle for tiles that are read both as rows (ds_read_b128: 16 consecutive rows at one
// logical 16-byte chunk must hit 16 different bank slots) and transposed (ds_read_b64_tr_b16: an
// aligned group of 4 rows at one 64-byte segment must hit 4 different 64-byte bank quarters).
// The chunk index is XORed with a bijection of the row's low bits whose two high result bits come
// from the row's two lowest bits.
// DP is the LDS row pitch in elements (lds_pitch: 64 or 128).
template <int DP>
__device__ inline int swz_u(int row) {
  return DP == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

__device__ inline float half_lo(unsigned w, bool bf16) {
  return bf16 ? __builtin_bit_cast(float, w << 16) : (float)__builtin_bit_cast(f16x2, w)[0];
}
__device__ inline float half_hi(unsigned w, bool bf16) {
  return bf16 ? __builtin_bit_cast(float, w & 0xffff0000u) : (float)__builtin_bit_cast(f16x2, w)[1];
}

// Lanes per row of the prep kernel: D/8 rounded up to a power of two (the row sum is a
// butterfly over them); lanes past D/8 hold zeros.
constexpr int prep_lanes(int d) { return d <= 32 ? 4 : d <= 64 ? 8 : 16; }

// ---- 1. prep: D = rowsum(dO o O) and LSE*log2(e), one row per prep_lanes(D) lanes -----------
template <bool BF16, int D, bool O_F32>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(const BwdParams p) {
  constexpr int TPR = prep_lanes(D);  // lanes per row, 8 elements each
  constexpr int RPB = 256 / TPR;      // rows per work-group
  const int64_t rows_per_head = (int64_t)p.ws_blk * 32;
  const int64_t rows = (int64_t)p.B * p.Hq * rows_per_head;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int ch = threadIdx.x % TPR;
  const int64_t head = row / rows_per_head;
  const int i = (int)(row - head * rows_per_head);
  float acc = 0.f, lse2 = 0.f;
  if (row < rows && i < p.Nq && ch * 8 < D) {
    const int64_t e = (head * p.Nq + i) * D + ch * 8;
    const u32x4 g = *(const u32x4*)((const unsigned short*)p.dout + e);
    float o[8];
    if (O_F32) {
      const f32x4 a = *(const f32x4*)((const float*)p.o + e);
      const f32x4 b = *(const f32x4*)((const float*)p.o + e + 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        o[t] = a[t];
        o[t + 4] = b[t];
      }
    } else {
      const u32x4 w = *(const u32x4*)((const unsigned short*)p.o + e);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        o[2 * t] = half_lo(w[t], BF16);
        o[2 * t + 1] = half_hi(w[t], BF16);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) acc += half_lo(g[t], BF16) * o[2 * t] + half_hi(g[t], BF16) * o[2 * t + 1];
  }
  // a row that sees no key (LSE = -inf) gets +inf, so that every P of the row is 0
  if (row < rows && i < p.Nq && ch == 0) {
    const float l = p.lse[head * p.Nq + i];
    lse2 = l == -__builtin_inff() ? __builtin_inff() : l * 1.44269504088896340736f;
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && ch == 0) {
    float* w = p.ws + (head * p.ws_blk + i / 32) * 64;
    w[i % 32] = lse2;
    w[32 + i % 32] = -acc;  // -D: the dK/dV kernel's dP accumulator starts from it
  }
}

// Work-group id -> logical work, each XCD taking a contiguous range (work-group i runs on
// XCD i % 8), so neighbouring logical work shares that XCD's L2.
__device__ inline int xcd_remap(int wg, int total) {
  const int xcd = wg & 7, local = wg >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + min(xcd, rem) + local;
}

// LDS-DMA of rows [r0, r0 + 32) of a [N][D] plane into a 32-row tile at LDS pitch DP.
// Instruction n of wave w fills tile bytes [(n*NW + w)*1024, +1024), RPI rows further on per
// instruction; lane offsets are loop invariant (the swizzle repeats every 16 rows), the
// instruction's first byte goes into the descriptor base, rows past N read as zero and so do
// the row-padding chunks (their lanes' offset lies past every descriptor's end).
template <int D, int NW>
__device__ inline void dma_rows(const char* plane, int N, int r0, lds_char* dst, int wave, int voff) {
  constexpr int ROWB = D * 2, ROWBL = lds_pitch(D) * 2, TB = 32 * ROWBL, NLD = TB / (NW * 1024);
  constexpr int RPI = NW * 1024 / ROWBL;
  static_assert(NLD >= 1 && TB % (NW * 1024) == 0, "whole 1 KiB DMA instructions per wave");
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int first = r0 * ROWB + n * RPI * ROWB;
    const int left = N * ROWB - first;
    const int bytes = left > 0 ? left : 0;
    void* bp = (void*)(plane + first);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(bp, (short)0, bytes, kBufferWord3);
    lds_void* ldst = (lds_void*)(dst + (n * NW + wave) * 1024);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ldst, 16, voff, 0, 0, 0);
  }
}

// The DMA lane offset of a tile: lane l of wave w writes physical chunk (w*64 + l) of the
// tile's first 1 KiB blocks, which holds logical chunk (pch ^ swizzle) of its row.
template <int D>
__device__ inline int dma_lane_off(int wave, int lane) {
  constexpr int DP = lds_pitch(D), KCH = D / 8, KCHP = DP / 8;
  const int row = (wave * 64 + lane) / KCHP, pch = lane % KCHP;
  const int c = pch ^ swz_u<DP>(row);
  return (KCH == KCHP || c < KCH) ? row * D * 2 + (c << 4) : kPadOffset;
}

// Lane offsets of a tile read as an MFMA operand. Rows: lane holds row l32, chunk 2ks + h.
template <int D>
__device__ inline int row_off(int l32, int h, int ks) {
  constexpr int DP = lds_pitch(D);
  return l32 * DP * 2 + (((2 * ks + h) ^ swz_u<DP>(l32)) << 4);
}
// Transposed: lane reads rows 16t + 8u + 4h + i16/4 (t adds an immediate; u changes the swizzle,
// see tr_half1), columns 32db + 16dh + 4(i16%4) .. +3.
template <int D>
__device__ inline int tr_off(int lane, int u, int db) {
  constexpr int DP = lds_pitch(D);
  const int h = lane >> 5, i16 = lane & 15, dh = (lane >> 4) & 1;
  const int row = 8 * u + 4 * h + (i16 >> 2);
  return row * DP * 2 + (((4 * db + 2 * dh + ((i16 & 3) >> 1)) ^ swz_u<DP>(row)) << 4) + ((i16 & 1) << 3);
}
// The second half (rows + 8) has the swizzle's bit 1 flipped for every lane (rows 8u + 4h + r
// give (row >> 2) & 3 = 2u + h), so its offset is (off0 ^ 32) + 8 rows: one VGPR per d-block,
// with the XOR re-done inside the loop (x1 = off0 ^ 32, pinned there) instead of a second
// loop-invariant register.
__device__ inline int tr_half1(int off0) {
  int x = off0 ^ 32;
  asm volatile("" : "+v"(x));
  return x;
}
__device__ inline u32x4 tr_operand(const lds_char* tile, int rowb, int t2, int off0, int x1) {
  u32x4 a;
  const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + 16 * t2 * rowb + off0)));
  const u32x2 y = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + (16 * t2 + 8) * rowb + x1)));
  a[0] = x[0];
  a[1] = x[1];
  a[2] = y[0];
  a[3] = y[1];
  return a;
}

// At d = 112 and 128 the dK/dV kernel keeps V's rows in LDS rather than registers, which brings
// it under the 256 VGPRs two waves per SIMD allow.
constexpr bool bwd_v_in_lds(int d) { return d > 96; }
// Waves per SIMD the dK/dV kernel is built for: three at d <= 64 without the dropout, mask and
// additive-mask inputs (whose registers need the room of two).
constexpr int bwd_waves_per_simd(int d, bool plain) { return d <= 64 && plain ? 3 : 2; }

// 4 * (lane id), formed from scratch where it is used: as an opaque instruction sequence it
// cannot be hoisted out of a loop, so it holds no register across the loop (the dK/dV kernel
// at d = 128 has none to spare).
__device__ inline int lane_bytes4() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\tv_lshlrev_b32 %0, 2, %0" : "=v"(v));
  return v;
}
// (lane_id_here, the lane id formed the same opaque way, is in fa_fwd_kernel.hpp.)

// ---- 2. dK/dV ---------------------------------------------------------------------------------
template <bool BF16, int D, bool BAND, int NW, bool AM, bool DROP = false, int FM = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd(D, !AM && !DROP && FM == 0)))) void fa_bwd_dkdv_kernel(const BwdParams p) {
  using E = Elt<BF16>;
  static_assert(D % 16 == 0 && D >= 32 && D <= 128, "head dimension: a multiple of 16 from 32 to 128");
  constexpr int ROWBL = lds_pitch(D) * 2, TB = 32 * ROWBL;  // LDS row pitch and tile bytes
  constexpr int NKS = D / 16, NDB = (D + 31) / 32;  // a half-filled last d-block reads LDS padding
  __shared__ __attribute__((aligned(1024))) char sQ0[TB];
  __shared__ __attribute__((aligned(1024))) char sQ1[TB];
  __shared__ __attribute__((aligned(1024))) char sG0[TB];
  __shared__ __attribute__((aligned(1024))) char sG1[TB];
  __shared__ __attribute__((aligned(256))) float sW0[64];
  __shared__ __attribute__((aligned(256))) float sW1[64];
  constexpr bool VL = bwd_v_in_lds(D);
  __shared__ __attribute__((aligned(1024))) char sV[VL ? NW * TB : 16];
  __shared__ __attribute__((aligned(16))) unsigned sDrop[DROP ? NW * 256 : 4];
  static_assert(!AM || BAND, "the masked kernels are built on the banded ones");
  static_assert(!(AM && DROP), "dropout kernels take no mask input");
  static_assert(FM == 0 || (BAND && !AM && !DROP), "the additive mask runs on the banded kernel, alone");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk, G = p.group;

  const int L = xcd_remap(blockIdx.x, p.total_wg);
  // key tiles in order (the first ones see the most queries under a causal band), ilv (b, hkv)
  // groups interleaved
  const int per_blk = p.ilv * p.n_tiles;
  const int blk = L / per_blk;
  const int r0 = L - blk * per_blk;
  const int kt = r0 / p.ilv;
  const int bk = blk * p.ilv + (r0 - kt * p.ilv);  // b * Hkv + hkv
  const int b = bk / p.Hkv, hkv = bk - b * p.Hkv;
  const int k0 = kt * 32 * NW, k0w = k0 + 32 * wave;

  using T = unsigned short;
  const T* Kp = (const T*)p.k + (int64_t)bk * Nk * D;
  const T* Vp = (const T*)p.v + (int64_t)bk * Nk * D;
  const int ld_off = dma_lane_off<D>(wave, lane);
  // this wave's 32 keys as the B operands of S = Q K^T and dP = dO V^T: lane holds key l32,
  // d = 16ks + 8h .. +7 (keys past Nk repeat row Nk-1, or read as zero from LDS; their gradients
  // are never stored). V's rows go to LDS when registers are short: 32 rows per wave, read with
  // the same lane offsets as a Q tile.
  u32x4 kreg[NKS], vreg[VL ? 1 : NKS];
  {
    const int kr = min(k0w + l32, Nk - 1);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      kreg[ks] = *(const u32x4*)(Kp + (int64_t)kr * D + 16 * ks + 8 * h);
      if constexpr (!VL) vreg[ks] = *(const u32x4*)(Vp + (int64_t)kr * D + 16 * ks + 8 * h);
    }
    if constexpr (VL) {
#pragma unroll
      for (int m = 0; m < NW; ++m) dma_rows<D, NW>((const char*)Vp, Nk, k0 + 32 * m, (lds_char*)sV + m * TB, wave, ld_off);
    }
  }
  int aoff[NKS], toff[NDB];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) aoff[ks] = row_off<D>(l32, h, ks);
#pragma unroll
  for (int db = 0; db < NDB; ++db) toff[db] = tr_off<D>(lane, 0, db);

  // query blocks whose band reaches keys [k0, k0 + 32*NW): rows i with
  // i + off - left <= k0 + 32*NW - 1 and i + off + right >= k0
  int q_lo = BAND ? max(0, k0 - p.off - p.right) : 0;
  int q_hi = BAND ? min(Nq - 1, k0 + 32 * NW - 1 - p.off + p.left) : Nq - 1;
  if constexpr (AM) {
    // narrow to the Q-tiles of 128 rows whose block with this key tile has a visible pair, over
    // the G query heads' mask planes (one plane when the mask shares the head axis)
    static_assert(32 * NW == 128, "the flags cover 128-key tiles");
    // (lanes read 64 flags at a time; the ballot keeps the result wave-uniform)
    int tmin = 0x7fffffff, tmax = -1;
    if (q_hi >= q_lo) {
      const int ng = p.flags_sh != 0 ? G : 1;
      const int t0 = q_lo / 128, t1 = q_hi / 128;
      for (int g = 0; g < ng; ++g) {
        const unsigned char* fl = p.am_flags + b * p.flags_sb + (hkv * G + g) * p.flags_sh + (int64_t)kt * p.flags_nq;
        for (int tb = t0; tb <= t1; tb += 64) {
          const int tt = tb + lane;
          const unsigned long long bal = __builtin_amdgcn_ballot_w64(tt <= t1 && fl[tt] != 0);
          if (bal != 0) {
            tmin = min(tmin, tb + (int)__builtin_ctzll(bal));
            tmax = max(tmax, tb + 63 - (int)__builtin_clzll(bal));
          }
        }
      }
    }
    q_lo = max(q_lo, tmin == 0x7fffffff ? Nq : 128 * tmin);
    q_hi = min(q_hi, 128 * tmax + 127);
  }
  const int qb0 = q_lo / 32;
  const int nqb = q_hi >= q_lo ? q_hi / 32 - qb0 + 1 : 0;
  const int n_it = G * nqb;
  // With one mask plane for the G heads, lane l holds the flag of Q-tile q_lo/128 + l: an
  // iteration whose block the mask leaves wholly visible (flag 2) loads no mask tile and
  // applies none (the band is still applied). Q-tiles past the first 64 always apply it.
  int mflag = 1;
  if constexpr (AM) {
    const int tt = q_lo / 128 + lane;
    if (p.flags_sh == 0 && nqb > 0 && tt <= q_hi / 128)
      mflag = p.am_flags[b * p.flags_sb + (int64_t)kt * p.flags_nq + tt];
  }
  // qb: an iteration's query block (wave-uniform)
  auto mask_free = [&](int qb) -> bool {
    if constexpr (!AM) {
      return false;
    } else {
      if (p.flags_sh != 0) return false;
      const int qt = qb / 4 - q_lo / 128;  // wave-uniform, >= 0
      return qt < 64 && __builtin_amdgcn_readlane(mflag, qt) == 2;
    }
  };

  // Iteration it visits query block qb0 + it % nqb of head g = it / nqb. Both the iteration and
  // the loads (one iteration ahead) carry their (g, qb) and head planes along, one block at a
  // time, so the loop does no division and no 64-bit multiply.
  const int64_t head0 = (int64_t)b * p.Hq + hkv * G;
  const int64_t plane_b = (int64_t)Nq * D * 2;
  const int64_t wplane = (int64_t)p.ws_blk * 64;
  const char* ld_q = (const char*)p.q + head0 * plane_b;
  const char* ld_go = (const char*)p.dout + head0 * plane_b;
  const float* ld_w = p.ws + head0 * wplane;
  int ld_g = 0, ld_qb = qb0;

  // The lane's mask column word for the block being loaded (head ld_g, block ld_qb, its key),
  // one iteration ahead; the key's offset is formed from an opaque lane id where it is used (no
  // register holds it across the loop). Keys past Nk read the last key's word: their results
  // are never stored.
  unsigned mw = 0u, mw_next = 0u;
  auto load_mw = [&]() {
    const int key = min(k0w + (lane_id_here() & 31), Nk - 1);
    mw_next = p.am_cbits[b * p.cbits_sb + (hkv * G + ld_g) * p.cbits_sh + (int64_t)key * p.cbits_nqb + ld_qb];
  };
  // the next iteration's Q and dO rows and row statistics, then one block further on
  auto issue_loads = [&](lds_char* dq_, lds_char* dg_, float* dw_) {
    dma_rows<D, NW>(ld_q, Nq, ld_qb * 32, dq_, wave, ld_off);
    dma_rows<D, NW>(ld_go, Nq, ld_qb * 32, dg_, wave, ld_off);
    if constexpr (AM)
      if (!mask_free(ld_qb)) load_mw();
    if (wave == 0) {
      void* wp = (void*)(ld_w + ld_qb * 64);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(wp, (short)0, 256, kBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dw_, 4, lane_bytes4(), 0, 0, 0);
    }
    if (++ld_qb == qb0 + nqb) {
      ld_qb = qb0;
      ++ld_g;
      ld_q += plane_b;
      ld_go += plane_b;
      ld_w += wplane;
    }
  };
  int cur_g = 0, cur_qb = qb0;  // of the iteration running

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = (f32x16){};
    dv[db] = (f32x16){};
  }
  const float c = p.c;

  if (n_it > 0) issue_loads((lds_char*)sQ0, (lds_char*)sG0, sW0);
  // One iteration; even iterations read the 0 buffers and odd ones the 1 buffers. The loop runs
  // them in pairs, so each buffer's address is a compile-time constant of its iteration and the
  // LDS reads take it as an immediate offset.
  auto iter = [&](const int it, auto oddc) {
    constexpr bool odd = decltype(oddc)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const lds_char* tq = (const lds_char*)(odd ? sQ1 : sQ0);
    const lds_char* tg = (const lds_char*)(odd ? sG1 : sG0);
    const float* tw = odd ? sW1 : sW0;
    if constexpr (AM) mw = mw_next;  // loaded during the previous iteration (or before the loop)
    [[maybe_unused]] const int g = cur_g;
    const int qb = cur_qb;
    if (++cur_qb == qb0 + nqb) {
      cur_qb = qb0;
      ++cur_g;
    }
    const int q0 = qb * 32;
    const bool mfree = mask_free(qb);
    // Dropout: the lane's key meets queries q0 + 8 g4 + 4h + r; Philox call (key / 4, query / 4)
    // covers a 4 x 4 block, byte 4 (query & 3) + (key & 3). The quad of lanes with keys 4a .. 4a+3
    // (one half) needs the calls of its 4 query groups g4: lane s computes group s, transposes
    // the block's bytes so that word t holds key t's 4 query bytes, writes word t to slot [t][s]
    // and reads back slot [s][0..3]: zw[g4] byte r is the lane's byte for query 8 g4 + 4h + r.
    // A wave's LDS operations complete in order, so no barrier is needed.
    unsigned zw[DROP ? 4 : 1];
    if constexpr (DROP) {
      const int sq = lane & 3;
      __attribute__((address_space(3))) unsigned* slot =
          (__attribute__((address_space(3))) unsigned*)sDrop + wave * 256 + (lane >> 2) * 16;
      unsigned w[4], tw4[4];
      philox4x32_10((unsigned)(k0w + (l32 & ~3)) >> 2, (unsigned)(q0 >> 2) + 2 * sq + h,
                    (unsigned)(b * p.Hq + hkv * G + g), p.drop_offset, p.seed_lo, p.seed_hi, w);
      byte_transpose4(w, tw4);
#pragma unroll
      for (int r = 0; r < 4; ++r) slot[4 * r + sq] = tw4[r];
      asm volatile("" ::: "memory");
      const u32x4 x = *(__attribute__((address_space(3))) u32x4*)(slot + 4 * sq);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) zw[g4] = x[g4];
    }

    // Additive mask: the lane's key meets queries q0 + 8 g4 + 4h + r; value i = 4 g4 + r, read
    // before the products so that their latency hides the loads. Query rows past Nq lie past the
    // plane's descriptor and read zeros; keys past Nk only reach gradients that are not stored.
    float fmv[FM ? 16 : 1];
    if constexpr (FM != 0) {
      const char* plane = (const char*)p.fm + (b * p.fm_sb + (hkv * G + g) * p.fm_sh) * FM;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)plane, (short)0, Nq * p.fm_ld * FM, kBufferWord3);
      const int v0 = ((q0 + 4 * h) * p.fm_ld + k0w + l32) * FM;
#pragma unroll
      for (int i = 0; i < 16; ++i) fmv[i] = fm_load1<FM>(rs, v0 + (8 * (i >> 2) + (i & 3)) * p.fm_ld * FM);
    }
    // S = Q K^T, dP = dO V^T: lane holds key l32 (column), queries 8(i/4) + 4h + i%4 (rows).
    // Without dropout dP accumulates onto -D of its queries (4 groups of 4 consecutive rows in
    // the statistics), so the products give dP - D directly.
    f32x16 s = (f32x16){}, dp = (f32x16){};
    if constexpr (!DROP) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 nd = *(const __attribute__((address_space(3))) f32x4*)((const lds_char*)tw + 128 + (8 * g4 + 4 * h) * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) dp[4 * g4 + r] = nd[r];
      }
    }
    // band: key k0w + l32 is hidden from query q0 + part + 4h when it lies after the query's
    // right edge (part < t_lo) or before its left edge (part > t_hi)
    const bool diag = BAND && (k0w + 31 > q0 + p.off + p.right || k0w < q0 + 31 + p.off - p.left);
    // visible iff t - right <= part <= t + left (t = key - q0 - 4h - off): one unsigned range
    // check of part - (t - right) against left + right
    const int vlo = k0w + l32 - q0 - 4 * h - p.off - p.right;
    const unsigned width = (unsigned)p.left + (unsigned)p.right;

    // The products run as slots of one MFMA each, in the order S (NKS), dP (NKS), dV (2 NDB),
    // dK (2 NDB). A slot issues the LDS reads of a later slot's MFMA and its share of the
    // VALU work, so that the work of one block overlaps its own products: P is formed from S
    // while the dP products run, dS while the dV products run.
    constexpr int M = 2 * NKS + 4 * NDB;
    constexpr int MDV = 2 * NKS, MDK = 2 * NKS + 2 * NDB;  // first slots of dV and dK
    int x1[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) x1[db] = tr_half1(toff[db]);
    u32x4 opnd[M], vop[VL ? NKS : 1];
    f32x2 a2[8];  // pair q's two rows' statistics
    float ex[16];
    u32x4 pw[2], sw[2];
    auto fetch = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NKS) {
        opnd[m] = *(const lds_u32x4*)(tq + aoff[m]);
      } else if constexpr (m < MDV) {
        opnd[m] = *(const lds_u32x4*)(tg + aoff[m - NKS]);
        if constexpr (VL) vop[m - NKS] = *(const lds_u32x4*)((const lds_char*)sV + wave * TB + aoff[m - NKS]);
      } else if constexpr (m < MDK) {
        constexpr int t2 = (m - MDV) / NDB, db = (m - MDV) % NDB;
        opnd[m] = tr_operand(tg, ROWBL, t2, toff[db], x1[db]);
      } else {
        constexpr int t2 = (m - MDK) / NDB, db = (m - MDK) % NDB;
        opnd[m] = tr_operand(tq, ROWBL, t2, toff[db], x1[db]);
      }
    };
    auto issue = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NKS) {
        s = E::mfma(opnd[m], kreg[m], s);
      } else if constexpr (m < MDV) {
        if constexpr (VL)
          dp = E::mfma(opnd[m], vop[m - NKS], dp);
        else
          dp = E::mfma(opnd[m], vreg[m - NKS], dp);
      } else if constexpr (m < MDK) {
        constexpr int t2 = (m - MDV) / NDB, db = (m - MDV) % NDB;
        dv[db] = E::mfma(pw[t2], opnd[m], dv[db]);
      } else {
        constexpr int t2 = (m - MDK) / NDB, db = (m - MDK) % NDB;
        dk[db] = E::mfma(sw[t2], opnd[m], dk[db]);
      }
    };
    // The hidden scores, once S is complete: the band (one uniform branch over the whole block:
    // only the blocks that cross a band edge pay for the selects) and the byte mask's bits.
    auto mask_s = [&]() {
      if (diag) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[i] = (unsigned)(8 * (i >> 2) + (i & 3) - vlo) > width ? -__builtin_inff() : s[i];
      }
      if constexpr (AM) {
        if (!mfree) {
          // bit 4h + 8(i/4) + i%4 of the lane's column word: query 8(i/4) + 4h + i%4
          const unsigned x = mw >> (4 * h);
#pragma unroll
          for (int i = 0; i < 16; ++i)
            s[i] = ((x >> (8 * (i >> 2) + (i & 3))) & 1u) != 0u ? -__builtin_inff() : s[i];
        }
      }
    };
    // pair q (queries of elements 2q, 2q + 1): P, packed for dV (dropout hides the dropped halves)
    auto p_item = [&](auto qc) {
      constexpr int q = decltype(qc)::value, i = 2 * q, g4 = q >> 1, r2 = q & 1;
      float s0 = s[i], s1 = s[i + 1];
      if constexpr (FM != 0) {
        // the additive mask (a hidden key's -inf stays -inf)
        s0 = __builtin_fmaf(fmv[i], p.inv_scale, s0);
        s1 = __builtin_fmaf(fmv[i + 1], p.inv_scale, s1);
      }
      ex[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, c, -a2[q][0]));
      ex[i + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, -a2[q][1]));
      if constexpr (DROP)
        pw[q >> 2][q & 3] = E::pack2(ex[i], ex[i + 1]) & keep_pair_mask(zw[g4], r2 != 0, p.keep_t);
      else
        pw[q >> 2][q & 3] = E::pack2(ex[i], ex[i + 1]);
    };
    // pair q: dS = P o (dP - D), packed for dK; with dropout dS = P o (Z dP / keep - D)
    auto ds_item = [&](auto qc) {
      constexpr int q = decltype(qc)::value, i = 2 * q, g4 = q >> 1, r2 = q & 1;
      if constexpr (DROP) {
        const f32x2 nd2 = *(const __attribute__((address_space(3))) f32x2*)((const lds_char*)tw + 128 + (8 * g4 + 4 * h + 2 * r2) * 4);
        const float g0 = kept(zw[g4], 2 * r2, p.keep_t) ? dp[i] * p.drop_scale : 0.f;
        const float g1 = kept(zw[g4], 2 * r2 + 1, p.keep_t) ? dp[i + 1] * p.drop_scale : 0.f;
        sw[q >> 2][q & 3] = E::pack2(ex[i] * (g0 + nd2[0]), ex[i + 1] * (g1 + nd2[1]));
      } else {
        sw[q >> 2][q & 3] = E::pack2(ex[i] * dp[i], ex[i + 1] * dp[i + 1]);
      }
    };
    // slot of each pair: P once S is complete, before the first dV product; dS once dP is
    // complete, before the first dK product. A pair's two rows' statistics are read two slots
    // before it.
    auto p_slot = [](int q) { return NKS + 1 + (q * (NKS - 1)) / 8; };
    auto ds_slot = [](int q) { return MDV + 1 + (q * (2 * NDB - 1)) / 8; };

    // operands are read FD slots ahead (one at d >= 112, where registers are shortest)
    constexpr int FD = (D >= 112 || D == 64) ? 1 : 2;
    static_for<0, FD>([&](auto mc) { fetch(mc); });
    static_for<0, M>([&](auto slc) {
      constexpr int sl = decltype(slc)::value;
      if constexpr (sl + FD < M) fetch(IC<sl + FD>{});
      static_for<0, 8>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (p_slot(q) - 2 == sl)
          a2[q] = *(const __attribute__((address_space(3))) f32x2*)((const lds_char*)tw + (8 * (q >> 1) + 4 * h + 2 * (q & 1)) * 4);
      });
      // the next iteration's loads, issued in the shadow of the products (into the buffers the
      // barrier above freed)
      if constexpr (sl == 1)
        if (it + 1 < n_it) issue_loads((lds_char*)(odd ? sQ0 : sQ1), (lds_char*)(odd ? sG0 : sG1), odd ? sW0 : sW1);
      if constexpr (sl == NKS + 1) mask_s();
      static_for<0, 8>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (p_slot(q) == sl) p_item(qc);
      });
      static_for<0, 8>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (ds_slot(q) == sl) ds_item(qc);
      });
      issue(slc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int it = 0; it < n_it; it += 2) {
    iter(it, IC<false>{});
    if (it + 1 < n_it) iter(it + 1, IC<true>{});
  }

  // no LDS-DMA may still be in flight when the work-group ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // element i of block db: key k0w + 8(i/4) + 4h + i%4, column 32db + l32
  float* dkp = p.dk + (int64_t)bk * Nk * D;
  float* dvp = p.dv + (int64_t)bk * Nk * D;
  const float sc = p.scale, vsc = DROP ? p.drop_scale : 1.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = k0w + 8 * (i >> 2) + 4 * h + (i & 3);
    if (key < Nk) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if (D % 32 != 0 && db == NDB - 1 && l32 >= 16) continue;  // padding columns of a half block
        dkp[(int64_t)key * D + 32 * db + l32] = dk[db][i] * sc;
        dvp[(int64_t)key * D + 32 * db + l32] = DROP ? dv[db][i] * vsc : dv[db][i];
      }
    }
  }
}

// ---- 3. dQ ------------------------------------------------------------------------------------
template <bool BF16, int D, bool BAND, int NW, bool AM, bool DROP = false, int FM = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(2))) void fa_bwd_dq_kernel(const BwdParams p) {
  using E = Elt<BF16>;
  static_assert(D % 16 == 0 && D >= 32 && D <= 128, "head dimension: a multiple of 16 from 32 to 128");
  constexpr int ROWBL = lds_pitch(D) * 2, TB = 32 * ROWBL, BM = 32 * NW;  // LDS row pitch, tile bytes
  constexpr int NKS = D / 16, NDB = (D + 31) / 32;  // a half-filled last d-block reads LDS padding
  __shared__ __attribute__((aligned(1024))) char sK0[TB];
  __shared__ __attribute__((aligned(1024))) char sK1[TB];
  __shared__ __attribute__((aligned(1024))) char sV0[TB];
  __shared__ __attribute__((aligned(1024))) char sV1[TB];
  __shared__ __attribute__((aligned(16))) unsigned sDrop[DROP ? NW * 256 : 4];
  static_assert(!(AM && DROP), "dropout kernels take no mask input");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int Nq = p.Nq, Nk = p.Nk, G = p.group;

  // (b, hkv) groups with the G sibling query heads side by side, longest Q-tiles first
  const int L = xcd_remap(blockIdx.x, p.total_wg);
  const int per_kv = p.n_tiles * G;
  const int per_blk = p.ilv * per_kv;  // ilv (b, hkv) groups interleaved, as in the forward
  const int blk = L / per_blk;
  const int r0 = L - blk * per_blk;
  const int t_ord = r0 / (p.ilv * G);
  const int r1 = r0 - t_ord * (p.ilv * G);
  const int sub = r1 / G, g = r1 - sub * G;
  const int bk = blk * p.ilv + sub;
  const int t = BAND ? (p.n_tiles - 1 - t_ord) : t_ord;
  const int b = bk / p.Hkv, hkv = bk - b * p.Hkv, hq = hkv * G + g;
  const int64_t head = (int64_t)b * p.Hq + hq;
  const int q0 = t * BM, q0w = q0 + 32 * wave, qrow = q0w + l32;

  using T = unsigned short;
  const char* Kp = (const char*)((const T*)p.k + (int64_t)bk * Nk * D);
  const char* Vp = (const char*)((const T*)p.v + (int64_t)bk * Nk * D);
  const int qr = min(qrow, Nq - 1);  // rows past Nq behave as the last row (never stored)
  // this wave's queries as B operands of S^T = K Q^T and dP^T = V dO^T
  u32x4 qreg[NKS], greg[NKS];
  {
    const T* qs = (const T*)p.q + (head * Nq + qr) * D + 8 * h;
    const T* gs = (const T*)p.dout + (head * Nq + qr) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qreg[ks] = *(const u32x4*)(qs + 16 * ks);
      greg[ks] = *(const u32x4*)(gs + 16 * ks);
    }
  }
  // the lane's query's statistics (rows past Nq hold zeros)
  const float* w = p.ws + (head * p.ws_blk + q0w / 32) * 64;
  const float lse2 = w[l32], ndlt = w[32 + l32];  // ndlt = -D

  const int ld_off = dma_lane_off<D>(wave, lane);
  int aoff[NKS], toff[NDB];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) aoff[ks] = row_off<D>(l32, h, ks);
#pragma unroll
  for (int db = 0; db < NDB; ++db) toff[db] = tr_off<D>(lane, 0, db);

  // the K/V tiles the Q-tile's band touches: [j_lo, j_lo + nt), and the lane's keys [klo, khi]
  int lo_t = BAND ? max(0, q0 + p.off - p.left) : 0;
  int hi_t = BAND ? min(Nk - 1, min(q0 + BM, Nq) - 1 + p.off + p.right) : Nk - 1;
  if constexpr (AM) {
    // narrow to the mask's key hull for this Q-tile (as the forward)
    static_assert(BM == 128, "the hull covers 128-row Q-tiles");
    if (hi_t >= lo_t) {
      const int2 kr = hull_range(p.am_hull + b * p.hull_sb + hq * p.hull_sh + (int64_t)t * p.hull_nch,
                                 lo_t / kHullKeys, hi_t / kHullKeys);
      lo_t = max(lo_t, kr.x);
      hi_t = min(hi_t, kr.y);
    }
  }
  const int j_lo = lo_t / 32;
  const int nt = hi_t >= lo_t ? hi_t / 32 - j_lo + 1 : 0;
  const int khi = BAND ? min(Nk - 1, qr + p.off + p.right) : Nk - 1;
  const int klo = BAND ? qr + p.off - p.left : 0;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x16){};
  const float c = p.c;

  // the mask word of the lane's query for a 32-key tile (as in the forward: score 4g + i, key
  // 32j + 8g + 4h + i, is bit 8i + 2g + h); loaded one tile ahead, the offset wholly in the
  // vector operand so reads past the plane return zeros
  unsigned am_w = 0u;
  __amdgpu_buffer_rsrc_t am_rs;
  int am_v0 = 0;
  auto load_am = [&](int jt) { am_w = __builtin_amdgcn_raw_buffer_load_b32(am_rs, am_v0 + 4 * jt, 0, 0); };
  if constexpr (AM) {
    const unsigned* plane = p.am_bits + b * p.bits_sb + hq * p.bits_sh;
    am_rs = __builtin_amdgcn_make_buffer_rsrc((void*)plane, (short)0, Nq * p.am_nw * 4, kBufferWord3);
    am_v0 = qr * p.am_nw * 4;
    if (nt > 0) load_am(j_lo);
  }
  // Additive mask: fmw[g] holds the values of keys 32j + 8g + 4h .. +3 of the lane's query, loaded
  // one tile ahead; reads past the plane return zeros and the key-end select replaces the scores
  // of keys past Nk.
  using FV = FmVec<FM == 4 ? 4 : 2>;
  typename FV::T fmw[FM ? 4 : 1];
  __amdgpu_buffer_rsrc_t fm_rs;
  auto load_fm = [&](int jt) {
    if constexpr (FM != 0) {
      const int vo = (qr * p.fm_ld + 32 * jt + 4 * h) * FM;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) fmw[g4] = FV::load(fm_rs, vo + 8 * g4 * FM);
    }
  };
  if constexpr (FM != 0) {
    const char* plane = (const char*)p.fm + (b * p.fm_sb + hq * p.fm_sh) * FM;
    fm_rs = __builtin_amdgcn_make_buffer_rsrc((void*)plane, (short)0, Nq * p.fm_ld * FM, kBufferWord3);
    if (nt > 0) load_fm(j_lo);
  }
  if (nt > 0) {
    dma_rows<D, NW>(Kp, Nk, j_lo * 32, (lds_char*)sK0, wave, ld_off);
    dma_rows<D, NW>(Vp, Nk, j_lo * 32, (lds_char*)sV0, wave, ld_off);
  }
  // dP^T accumulates onto -D of the lane's query (without dropout), so the products give dP - D:
  // one loop-invariant operand tuple
  f32x16 nd16;
#pragma unroll
  for (int i = 0; i < 16; ++i) nd16[i] = DROP ? 0.f : ndlt;
  // One tile; even tiles read the 0 buffers, odd ones the 1 buffers: the loop runs them in
  // pairs, so each buffer's address is a compile-time constant for the LDS reads.
  auto tile = [&](const int r, auto oddc) {
    constexpr bool odd = decltype(oddc)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int j = j_lo + r;
    const lds_char* tk = (const lds_char*)(odd ? sK1 : sK0);
    const lds_char* tv = (const lds_char*)(odd ? sV1 : sV0);
    if (r + 1 < nt) {
      dma_rows<D, NW>(Kp, Nk, (j + 1) * 32, (lds_char*)(odd ? sK0 : sK1), wave, ld_off);
      dma_rows<D, NW>(Vp, Nk, (j + 1) * 32, (lds_char*)(odd ? sV0 : sV1), wave, ld_off);
    }
    // Dropout, as in the forward: the quad of lanes with queries 4a .. 4a+3 (one half) needs the
    // Philox calls of its 4 key groups (keys 32j + 8g + 4h .. +3); lane s computes group s,
    // writes word r (query 4a + r) to slot [r][s] and reads back slot [s][0..3]: zw[g] holds the
    // lane's query's bytes for key group g, byte key & 3.
    const int kbase = 32 * j;
    unsigned zw[DROP ? 4 : 1];
    if constexpr (DROP) {
      const int sq = lane & 3;
      __attribute__((address_space(3))) unsigned* slot =
          (__attribute__((address_space(3))) unsigned*)sDrop + wave * 256 + (lane >> 2) * 16;
      unsigned wd[4];
      philox4x32_10((unsigned)(kbase + 8 * sq + 4 * h) >> 2, (unsigned)(q0w + l32) >> 2, (unsigned)head,
                    p.drop_offset, p.seed_lo, p.seed_hi, wd);
#pragma unroll
      for (int r = 0; r < 4; ++r) slot[4 * r + sq] = wd[r];
      asm volatile("" ::: "memory");
      const u32x4 x = *(__attribute__((address_space(3))) u32x4*)(slot + 4 * sq);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) zw[g4] = x[g4];
    }

    // S^T = K Q^T, dP^T = V dO^T: lane holds query l32, keys 32j + 8(i/4) + 4h + i%4. The products
    // run as slots of one MFMA each, in the order S^T (NKS), dP^T (NKS), dQ (2 NDB), each slot
    // also reading a later slot's operands and doing a share of the VALU work: the exponentials
    // run while the dP^T products do, dS while the dQ products do.
    f32x16 s = (f32x16){}, dp = nd16;
    constexpr int M = 2 * NKS + 2 * NDB, MDQ = 2 * NKS;
    int x1[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) x1[db] = tr_half1(toff[db]);
    u32x4 opnd[M];
    float ex[16];
    u32x4 sw[2];
    auto fetch = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NKS) {
        opnd[m] = *(const lds_u32x4*)(tk + aoff[m]);
      } else if constexpr (m < MDQ) {
        opnd[m] = *(const lds_u32x4*)(tv + aoff[m - NKS]);
      } else {
        constexpr int t2 = (m - MDQ) / NDB, db = (m - MDQ) % NDB;
        opnd[m] = tr_operand(tk, ROWBL, t2, toff[db], x1[db]);
      }
    };
    auto issue = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NKS) {
        s = E::mfma(opnd[m], qreg[m], s);
      } else if constexpr (m < MDQ) {
        dp = E::mfma(opnd[m], greg[m - NKS], dp);
      } else {
        constexpr int t2 = (m - MDQ) / NDB, db = (m - MDQ) % NDB;
        acc[db] = E::mfma(sw[t2], opnd[m], acc[db]);
      }
    };
    // the hidden scores, once S^T is complete: the band and the key end (one uniform branch for
    // the tiles that cross them), the byte mask's bits
    auto mask_s = [&]() {
      if ((BAND && (kbase + 31 > min(q0w, Nq - 1) + p.off + p.right || kbase < min(q0w + 31, Nq - 1) + p.off - p.left)) ||
          kbase + 32 > Nk) {
        const int hi = khi - kbase - 4 * h, lo = klo - kbase - 4 * h;  // hide if part > hi or part < lo
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int part = 8 * (i >> 2) + (i & 3);
          s[i] = (part > hi || (BAND && part < lo)) ? -__builtin_inff() : s[i];
        }
      }
      if constexpr (AM) {
        const unsigned x = am_w >> h;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[i] = ((x >> (8 * (i & 3) + 2 * (i >> 2))) & 1u) != 0u ? -__builtin_inff() : s[i];
      }
    };
    // element pair q: P (the additive mask first; a hidden key's -inf stays -inf)
    auto p_item = [&](auto qc) {
      constexpr int q = decltype(qc)::value, i = 2 * q;
      float s0 = s[i], s1 = s[i + 1];
      if constexpr (FM != 0) {
        s0 = __builtin_fmaf(FV::at(fmw[i >> 2], i & 3), p.inv_scale, s0);
        s1 = __builtin_fmaf(FV::at(fmw[i >> 2], (i & 3) + 1), p.inv_scale, s1);
      }
      ex[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, c, -lse2));
      ex[i + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, c, -lse2));
    };
    // element pair q: dS = P o (dP - D), packed for dQ; with dropout dS = P o (Z dP / keep - D),
    // key 32j + 8(i/4) + 4h + i%4 being byte i%4 of zw[i/4]
    auto ds_item = [&](auto qc) {
      constexpr int q = decltype(qc)::value, i = 2 * q;
      if constexpr (DROP) {
        const float g0 = kept(zw[q >> 1], i & 3, p.keep_t) ? dp[i] * p.drop_scale : 0.f;
        const float g1 = kept(zw[q >> 1], (i & 3) + 1, p.keep_t) ? dp[i + 1] * p.drop_scale : 0.f;
        sw[q >> 2][q & 3] = E::pack2(ex[i] * (g0 + ndlt), ex[i + 1] * (g1 + ndlt));
      } else {
        sw[q >> 2][q & 3] = E::pack2(ex[i] * dp[i], ex[i + 1] * dp[i + 1]);
      }
    };
    // slots: P pairs once S^T is complete, through the dP^T products; dS pairs 0-3 once dP^T is
    // complete, before the first dQ product (they are its operand), pairs 4-7 before the second half
    auto p_slot = [](int q) { return NKS + 1 + (q * (NKS - 1)) / 8; };
    auto ds_slot = [](int q) { return q < 4 ? MDQ : MDQ + ((q - 4) * NDB) / 4; };
    static_for<0, 2>([&](auto mc) { fetch(mc); });
    static_for<0, M>([&](auto slc) {
      constexpr int sl = decltype(slc)::value;
      if constexpr (sl + 2 < M) fetch(IC<sl + 2>{});
      if constexpr (sl == NKS + 1) {
        mask_s();
        // the next tile's mask words and values (the next iteration's opening wait covers them)
        if constexpr (AM)
          if (r + 1 < nt) load_am(j + 1);
      }
      static_for<0, 8>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (p_slot(q) == sl) p_item(qc);
      });
      if constexpr (FM != 0 && sl == 2 * NKS - 1)
        if (r + 1 < nt) load_fm(j + 1);  // after the last use of this tile's values
      static_for<0, 8>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (ds_slot(q) == sl) ds_item(qc);
      });
      issue(slc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int r = 0; r < nt; r += 2) {
    tile(r, IC<false>{});
    if (r + 1 < nt) tile(r + 1, IC<true>{});
  }

  // element i of block db: query q0w + 8(i/4) + 4h + i%4, column 32db + l32
  float* dqp = p.dq + head * Nq * D;
  const float sc = p.scale;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int q = q0w + 8 * (i >> 2) + 4 * h + (i & 3);
    if (q < Nq) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if (D % 32 != 0 && db == NDB - 1 && l32 >= 16) continue;  // padding columns of a half block
        dqp[(int64_t)q * D + 32 * db + l32] = acc[db][i] * sc;
      }
    }
  }
}

}  // namespace fa
