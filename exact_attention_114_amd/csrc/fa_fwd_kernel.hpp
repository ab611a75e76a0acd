// fa_fwd_kernel.hpp — exact-attention forward kernel for gfx950 (CDNA4, MI355X).
//
// One work-group computes BM = 32*NW query rows of one (batch, query head):
// the FA2 decomposition over (batch, head, Q-tile) with the Q-outer / K,V-inner
// loop order (Triton FA2 walkthrough, xrbh.cn: the loop swap and the
// sequence-dimension grid). Each wave owns 32 query rows for the whole K/V
// sweep (the walkthrough's split of Q across warps, no inter-wave exchange).
//
// Per K/V tile of BN = 32*KB keys (intelliparadigm page, sections 1.2.1-1.2.2 and
// 2.4: load a block, Q K^T, scale, online-softmax update, P V, accumulate):
//   1. K and V tiles stream from HBM straight into LDS with buffer loads in LDS-DMA
//      form (no VGPR staging), double-buffered so later tiles load while the
//      current ones compute (intelliparadigm page, section 3.1, double
//      buffering). Each tile gets its own buffer descriptor (base at the tile,
//      size up to the sequence end), so the per-lane offsets never change and
//      rows past the end read as zero. Rows are XOR-swizzled in 16-byte chunks
//      so every LDS read below is bank-conflict free (section 3.1's goal; the
//      printed padding formula is not used: a swizzle wastes no LDS).
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
//      Row sums are kept in fp32: l of the unrounded exponentials, for the LSE, and l~ of
//      the rounded values that enter the MFMA (one v_dot2 per packed pair), which
//      normalises O. The weights that multiply V then sum to one, so the rounding of a
//      dominant weight (up to 2^-9 relative in bf16, 2^-11 in fp16) cancels rather than
//      scaling the row.
//   5. Masks. Causal attention (intelliparadigm page, section 1.3: skip the masked half) is one
//      case of a band: the operator on that page bounds a sliding window by pre_tokens and
//      next_tokens (section 2.2), and its tiling takes separate query and key lengths (2.3).
//      Query row i sits at key position i + off, off = Nk - Nq, and sees keys j with
//      i + off - left <= j <= i + off + right; causal is left = unlimited, right = 0. Only the
//      K/V tiles a Q-tile's band touches are loaded and computed, and only tiles crossing a
//      band edge (or the ragged end of the keys) are masked. A row that sees no key gets
//      O = 0 and LSE = -inf.
//   6. Mask input. The operator's optional boolean attn_mask (intelliparadigm page, section 2.2;
//      the Mask step of FlashAttention-1's Algorithm 2 that the cnblogs page points to) hides a
//      key from a query where its byte is nonzero, on top of the band. A lane reads the mask
//      word of its query row for each 32-key block one step ahead, and a wave skips the
//      per-score selects on tiles its mask leaves whole. A pre-pass
//      (fa_mask_prep_kernel) packs the byte mask into one bit per key, so a lane reads one word
//      per 32-key block, and records, per Q-tile and chunk of keys, the first and last key any
//      row of the tile may see; the attention kernel visits only the tiles between them, so
//      keys a mask hides from a whole Q-tile (other documents, padding) cost nothing.
//   7. Split keys. When batch x heads x Q-tiles leaves the GPU under-filled, the keys of each
//      Q-tile can be cut into chunks handled by separate work-groups (the FA2 walkthrough's
//      point about adding parallelism along the sequence when batch and heads are small); each
//      writes its chunk's normalised O and LSE, and a merge kernel combines them.
//
// Software pipeline. A wave's softmax is VALU work and its two products are MFMA
// work; on gfx950 an MFMA leaves the issue port free for about four VALU
// instructions of the same wave while it runs. So iteration j exponentiates S_j
// while the MFMAs of the neighbouring tiles run: S_{j+1} = K_{j+1} Q^T and
// O += P_{j-1} V_{j-1}. K runs two tiles ahead of V in LDS: iteration j reads
// K_{j+1} and V_{j-1} and loads K_{j+2} and V_j into the buffers it frees.
// Epilogue: O = acc / l~, LSE = ln2 * (m + log2 l), stored with one lane per row.
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_uchar;

// A lane's sum of one tile's exponentials above this (2^8) triggers a rescale; below it every
// exponential of the tile is at most 2^8.
constexpr float kSumLimit = 256.0f;
// Floor of the running reference (log2 units): a row whose first tiles hold no visible key
// keeps a finite reference, so the next visible score overflows the check and moves it.
constexpr float kRefFloor = -1.0e30f;
// Word 3 of a raw buffer descriptor on gfx9-family parts (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;
// A buffer offset past every descriptor's size (sizes stay below 2^31 - 2^17): a load from it
// returns zeros without touching memory. Lanes that fill the padding of an LDS row use it.
constexpr int kPadOffset = 0x7FFF0000;

// LDS row pitch (elements) for a head dimension: rows are stored at a power-of-two pitch so
// the XOR swizzles below stay inside a row; a head dimension below the pitch (32, 48, 80, 96,
// 112) leaves padding chunks at the end of each row that are loaded as zeros; only the P V
// operand of a half-filled last d-block reads them.
constexpr int lds_pitch(int d) { return d <= 64 ? 64 : 128; }

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv;
  int Nq, Nk;    // query and key rows per head
  int off;       // Nk - Nq: key position of query row 0
  int left, right;  // band edges (the host passes 1 << 30 for an unlimited edge)
  int group;     // Hq / Hkv
  int n_qtiles;  // ceil(Nq / BM)
  int nsplit;    // key chunks per Q-tile (1: none); chunk s covers keys [s*kchunk, (s+1)*kchunk)
  int kchunk;    // keys per chunk, a multiple of 64 (every key-tile size)
  int total_wg;  // B * Hq * n_qtiles * nsplit
  int ilv;       // (b, hkv) groups whose Q-tiles are interleaved longest first (1, 2 or 4)
  float c;       // scale * log2(e) (fp8 inputs: times the query and key descales)
  float vscale;  // fp8 inputs: the value descale, applied to O (1 otherwise)
  // dropout (kernels built with DROP): a pair is kept iff its Philox byte is below keep_t, and kept
  // probabilities are scaled by drop_scale = 256 / keep_t
  unsigned seed_lo, seed_hi, drop_offset;
  int keep_t;
  float drop_scale;
  // optional mask (kernels built with AM), as fa_mask_prep_kernel leaves it: one bit per
  // (query, key), set where the key is hidden, in rows of am_nw 32-bit words; the (b, hq)
  // plane starts at am_bits + b*bits_sb + hq*bits_sh (strides 0 along an axis the mask shares)
  const unsigned* am_bits;
  long long bits_sb, bits_sh;
  int am_nw;
  // the mask's key hull: int2 {first, last} visible key per plane, Q-tile and chunk of
  // kHullKeys keys at am_hull + b*hull_sb + hq*hull_sh + t*hull_nch + chunk
  const int2* am_hull;
  long long hull_sb, hull_sh;
  int hull_nch;
  // additive mask (kernels built with FM = its element bytes: 2 fp16, 4 fp32): score (i, j) of
  // head (b, hq) gains fm[b*fm_sb + hq*fm_sh + i*fm_ld + j] (element strides; 0 along an axis the
  // mask shares) before the softmax. It enters the unscaled score as M * inv_scale.
  const void* fm;
  long long fm_sb, fm_sh;
  int fm_ld;
  float inv_scale;  // 1 / scale
};

// The additive mask's values of 4 consecutive keys: 4 fp16 in two words, or 4 fp32.
template <int FM>
struct FmVec {
  typedef u32x2 T;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, int vo) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, vo, 0, 0));
  }
  // (the word is copied out first: a bit cast applied straight to a vector element compiles to a
  // read of element 0)
  __device__ static float at(const T& w, int e) {
    const unsigned x = w[e >> 1];
    return (float)__builtin_bit_cast(f16x2, x)[e & 1];
  }
};
template <>
struct FmVec<4> {
  typedef f32x4 T;
  __device__ static T load(__amdgpu_buffer_rsrc_t r, int vo) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, vo, 0, 0));
  }
  __device__ static float at(const T& w, int e) { return w[e]; }
};

// The lane id, formed where it is used by an opaque instruction sequence: it cannot be hoisted
// out of a loop, so it holds no register across the loop.
__device__ inline int lane_id_here() {
  int v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
  return v;
}

// Keys per chunk of the mask hull.
constexpr int kHullKeys = 1024;

// The key range a mask leaves to a Q-tile: the least first key and the greatest last key over
// its hull entries [c0, c1], {INT_MAX, -1} when none has a visible key. The wave's lanes load
// the entries in parallel and reduce them; the results are made wave-uniform, so the loop
// bounds built from them stay scalar. Every lane of the wave must call it.
__device__ inline int2 hull_range(const int2* hl, int c0, int c1) {
  int kmin = 0x7fffffff, kmax = -1;
  const int lane = (int)(threadIdx.x & 63);
  for (int cb = c0; cb <= c1; cb += 64) {
    const int c = cb + lane;
    if (c <= c1) {
      const int2 e = hl[c];
      kmin = min(kmin, e.x);
      kmax = max(kmax, e.y);
    }
  }
#pragma unroll
  for (int sft = 32; sft >= 1; sft >>= 1) {
    kmin = min(kmin, __shfl_xor(kmin, sft));
    kmax = max(kmax, __shfl_xor(kmax, sft));
  }
  return make_int2(__builtin_amdgcn_readfirstlane(kmin), __builtin_amdgcn_readfirstlane(kmax));
}

// ---- element-type traits ------------------------------------------------------------------
template <bool BF16>
struct Elt;
template <>
struct Elt<false> {
  static __device__ inline unsigned pack2(float a, float b) {
    return __builtin_bit_cast(unsigned, (f16x2){(_Float16)a, (_Float16)b});  // v_cvt_pk_f16_f32 (RNE)
  }
  // acc + the two packed values, summed in fp32 (v_dot2c_f32_f16 with (1, 1))
  static __device__ inline float sum2(unsigned w, float acc) {
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones, acc, false);
  }
  static __device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};
template <>
struct Elt<true> {
  static __device__ inline unsigned pack2(float a, float b) {
    return __builtin_bit_cast(unsigned, (bf16x2){(__bf16)a, (__bf16)b});  // v_cvt_pk_bf16_f32 (RNE)
  }
  // acc + the two packed values, summed in fp32 (v_dot2c_f32_bf16 with (1, 1))
  static __device__ inline float sum2(unsigned w, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
  }
  static __device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// ---- LDS swizzles (16-byte chunk index XOR, per row), by LDS row pitch DP -----------------
// LDS has 64 banks x 4 B. K is read with ds_read_b128 by 16 lanes at a time, one row each,
// same logical chunk: 16 consecutive rows must land in 16 different 16-byte bank slots.
// V is read with ds_read_b64_tr_b16: 32 lanes read 4 consecutive rows x 64 contiguous bytes;
// the 4 row segments must land in 4 different 64-byte bank quarters.
template <int DP>
__device__ inline int swz_k(int row) {
  return DP == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int DP>
__device__ inline int swz_v(int row) {
  return DP == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
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

// An empty asm that claims to read and rewrite x: the value must exist at this point of the
// program, so the compiler cannot sink its computation past it. (Inline asm with VGPR
// operands lives in __device__ helpers: in a kernel body the host pass rejects the
// constraint and silently drops the kernel's host stub.)
__device__ inline void pin(unsigned& x) { asm volatile("" : "+v"(x)); }
__device__ inline void pin(float& x) { asm volatile("" : "+v"(x)); }

// Maximum of v[o .. o+7] as a chain the compiler folds into three v_max3_f32 and one v_max_f32.
__device__ inline float max8(const f32x16& v, int o) {
  float m = fmaxf(fmaxf(v[o], v[o + 1]), v[o + 2]);
  m = fmaxf(fmaxf(m, v[o + 3]), v[o + 4]);
  m = fmaxf(fmaxf(m, v[o + 5]), v[o + 6]);
  return fmaxf(m, v[o + 7]);
}

template <int N>
struct IC {
  static constexpr int value = N;
};

// f(IC<i>) for i = B .. E-1 with i a compile-time constant: a step's slots are expanded by
// template recursion rather than loop unrolling, which gives up on long steps and would then
// index register arrays at run time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IC<B>{});
    static_for<B + 1, E>(f);
  }
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011): ten rounds over the counter (c0..c3) with the key (k0, k1) bumped by the Weyl
// constants between rounds; each round multiplies two counter words by the round constants and
// mixes the 32-bit halves of the products with the other words and the key.
__device__ inline void philox4x32_10(unsigned c0, unsigned c1, unsigned c2, unsigned c3, unsigned k0, unsigned k1,
                                     unsigned (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // each 32 x 32 -> 64-bit product as one 64-bit multiply (one v_mad_u64_u32, both halves)
    const unsigned long long m0 = (unsigned long long)0xD2511F53u * c0;
    const unsigned long long m1 = (unsigned long long)0xCD9E8D57u * c2;
    const unsigned hi0 = (unsigned)(m0 >> 32), lo0 = (unsigned)m0;
    const unsigned hi1 = (unsigned)(m1 >> 32), lo1 = (unsigned)m1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));
// Keep mask of a packed pair of 16-bit probabilities: word holds the random bytes of four
// consecutive keys; the pair is keys (0, 1) or, with `upper`, (2, 3). A half is kept (0xFFFF)
// iff its byte is below t: the two bytes go to 16-bit lanes and byte - t is negative.
__device__ inline unsigned keep_pair_mask(unsigned word, bool upper, int t) {
  const unsigned x = __builtin_amdgcn_perm(0u, word, upper ? 0x0C030C02u : 0x0C010C00u);
  const s16x2 d = __builtin_bit_cast(s16x2, x) - (s16x2){(short)t, (short)t};
  return __builtin_bit_cast(unsigned, d >> (s16x2){15, 15});
}

// Waves that share a SIMD for a tile shape: registers bound it (a d = 128 step with two key
// blocks holds 189 VGPRs, with one 168; d = 64 about 150) and so does LDS (4 tiles of
// 32*KB rows at the LDS pitch per work-group). Dropout's random words need about 20 more
// registers, which at three waves would spill.
constexpr int waves_per_simd(int d, int kb, bool drop) { return d > 64 && kb == 1 && !drop ? 3 : 2; }

// One work-group of NW waves computes BM = 32*NW query rows of one (batch, query head); a
// pipeline step takes KB blocks of 32 keys.
template <bool BF16, int D, bool BAND, bool OUT_F32, int NW, int KB, bool AM, bool DROP = false, int FM = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64)))
__attribute__((amdgpu_waves_per_eu(waves_per_simd(D, KB, DROP || FM != 0)))) void fa_fwd_kernel(const Params p) {
  using E = Elt<BF16>;
  static_assert(D % 16 == 0 && D >= 32 && D <= 128, "head dimension: a multiple of 16 from 32 to 128");
  constexpr int BM = 32 * NW;
  constexpr int BN = 32 * KB;
  constexpr int DP = lds_pitch(D);        // LDS row pitch (elements)
  constexpr int KCH = D / 8;              // 16-byte chunks per row in HBM
  constexpr int KCHP = DP / 8;            // 16-byte chunks per row in LDS
  constexpr int ROWB = D * 2;             // bytes per row in HBM
  constexpr int ROWBL = DP * 2;           // bytes per row in LDS
  constexpr int TILE_BYTES = BN * ROWBL;  // one K or one V tile in LDS
  constexpr int NKS = D / 16;             // MFMA k-steps of Q K^T
  // MFMA d-blocks of P V. A head dimension that is an odd multiple of 16 leaves the last block half
  // filled: its upper 16 columns read the LDS row padding (zeros) and are never stored.
  constexpr int NDB = (D + 31) / 32;
  constexpr int NLD = TILE_BYTES / (NW * 1024);  // 1 KiB tile-load instructions per wave per matrix
  constexpr int RPI = NW * 1024 / ROWBL;  // tile rows between a wave's consecutive load instructions
  static_assert(NLD >= 1 && TILE_BYTES % (NW * 1024) == 0, "each wave issues the same number of tile loads");
  static_assert(!AM || BAND, "the masked kernel is built on the banded one");
  static_assert(FM == 0 || (BAND && !AM && !DROP), "the additive mask runs on the banded kernel, alone");

  // Two K and two V buffers as four separate arrays: the compiler can then prove that a
  // prefetch into one buffer never aliases the reads of another, and does not stall on it.
  __shared__ __attribute__((aligned(1024))) char sK0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[TILE_BYTES];
  // dropout: the four Philox words of each lane's call, exchanged within its quad (16 words a quad)
  __shared__ __attribute__((aligned(16))) unsigned sDrop[DROP ? NW * 256 : 4];
  // additive mask: each wave's 32 rows x BN keys of the step's mask tile, two buffers
  static_assert(FM == 0 || KB == 1, "the additive mask takes 32-key steps");
  constexpr int MROW = BN * (FM ? FM : 2);  // mask bytes per row and step
  __shared__ __attribute__((aligned(1024))) char sM0[FM ? NW * 32 * MROW : 16];
  __shared__ __attribute__((aligned(1024))) char sM1[FM ? NW * 32 * MROW : 16];
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
  const int LS = xcd * per + min(xcd, rem) + local;
  const int split = LS % p.nsplit;  // the key chunk (0 when keys are not split)
  const int L = LS / p.nsplit;
  const int G = p.group;
  // With bands, Q-tiles differ in length: ilv consecutive (b, hkv) groups are taken together,
  // longest Q-tiles of all of them first, so that no group's long tiles start near the end.
  const int per_kv = p.n_qtiles * G;
  const int per_blk = p.ilv * per_kv;
  const int blk = L / per_blk;
  const int r0 = L - blk * per_blk;
  const int t_ord = r0 / (p.ilv * G);
  const int r1 = r0 - t_ord * (p.ilv * G);
  const int sub = r1 / G;
  const int g = r1 - sub * G;
  const int bk = blk * p.ilv + sub;  // b * Hkv + hkv
  const int t = BAND ? (p.n_qtiles - 1 - t_ord) : t_ord;
  const int b = bk / p.Hkv;
  const int hkv = bk - b * p.Hkv;
  const int hq = hkv * G + g;
  const int Nq = p.Nq, Nk = p.Nk;

  // outputs: with split keys, chunk s writes fp32 O and LSE into its own plane (the host
  // passes the workspace and an fp32 output then)
  const int64_t rows_all = (int64_t)p.B * p.Hq * Nq;
  float* const Of = (float*)p.o + (int64_t)split * rows_all * D;
  float* const Ls = p.lse + (int64_t)split * rows_all;

  using T = unsigned short;
  const T* __restrict__ Qp = (const T*)p.q + ((int64_t)(b * p.Hq + hq)) * Nq * D;
  const char* __restrict__ Kp = (const char*)((const T*)p.k + ((int64_t)bk) * Nk * D);
  const char* __restrict__ Vp = (const char*)((const T*)p.v + ((int64_t)bk) * Nk * D);

  // ---- tile loads: instruction n of this wave fills LDS bytes [ii*1024, ii*1024 + 1024) of a
  // tile (ii = n*NW + wave); lane l writes physical chunk ii*64 + l, which holds logical chunk
  // (pch ^ swizzle(row)) of tile row `row`. Moving to the next instruction moves RPI rows
  // (16 or 32), which leaves the swizzle unchanged, so the source offset of instruction n is
  // the lane's offset for n = 0 plus n*RPI rows of HBM: one loop-invariant VGPR per matrix,
  // and the steps go into the (scalar) buffer base. A logical chunk past the head dimension
  // is row padding: its lane reads from past the descriptor's end and writes zeros.
  int ld_koff, ld_voff;
  {
    const int row = (wave * 64 + lane) / KCHP, pch = lane % KCHP;
    const int ck = pch ^ swz_k<DP>(row), cv = pch ^ swz_v<DP>(row);
    ld_koff = (KCH == KCHP || ck < KCH) ? row * ROWB + (ck << 4) : kPadOffset;
    ld_voff = (KCH == KCHP || cv < KCH) ? row * ROWB + (cv << 4) : kPadOffset;
  }
  // One descriptor per tile and instruction: base at the instruction's first byte of the tile,
  // size up to the sequence end, so rows past N (ragged last tile, or a prefetch past the end)
  // read as zero. (The builtin's pointer and offset go through named locals: given as
  // expressions, the host compilation silently drops the kernel's host stub.)
  auto load_tile = [&](const char* base, int j, lds_char* dst, const int voffs) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      // 32-bit: the host keeps Nk*ROWB plus the few tiles a prefetch reaches past it below 2^31
      const int first = j * (BN * ROWB) + n * RPI * ROWB;  // this instruction's part
      const int rest = Nk * ROWB - first;
      const int bytes = rest > 0 ? rest : 0;
      void* bp = (void*)(base + first);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(bp, (short)0, bytes, kBufferWord3);
      lds_void* ldst = (lds_void*)(dst + (n * NW + wave) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ldst, 16, voffs, 0, 0, 0);
    }
  };
  auto load_k = [&](int j, lds_char* dst) { load_tile(Kp, j, dst, ld_koff); };
  auto load_v = [&](int j, lds_char* dst) { load_tile(Vp, j, dst, ld_voff); };

  // ---- per-lane LDS read offsets, loop invariant
  // K (A operand of S^T = K Q^T): row 32kb + l32 (kb adds an immediate), logical chunk 2ks + h.
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = l32 * ROWBL + (((2 * ks + h) ^ swz_k<DP>(l32)) << 4);
  // V^T via transposing reads: lane reads row 16t + 8u + 4h + i16/4 (t, u add immediates),
  // columns 32db + 16dh + 4(i16%4) .. +3.
  int voff[NDB];
  {
    const int vrow = 4 * h + (i16 >> 2);
    const int sv = swz_v<DP>(vrow);  // equals the swizzle of every row 16t + 8u + vrow
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      voff[db] = vrow * ROWBL + (((4 * db + 2 * dh + ((i16 & 3) >> 1)) ^ sv) << 4) + ((i16 & 1) << 3);
  }

  // A ragged sequence end leaves tile rows that no load writes (if out-of-range lanes skip
  // the LDS write) or writes as zero: clear the buffers once so they never hold stale bits
  // that could be non-finite.
  if (Nk % BN != 0) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int n = 0; n < TILE_BYTES / (NW * 64 * 16); ++n) {
      const int off = (n * NW * 64 + (int)threadIdx.x) * 16;
      *(lds_u32x4*)(K0 + off) = z;
      *(lds_u32x4*)(K1 + off) = z;
      *(lds_u32x4*)(V0 + off) = z;
      *(lds_u32x4*)(V1 + off) = z;
    }
    __syncthreads();
  }

  // MFMA operands from LDS. K (A operand of S^T = K Q^T): block kb of 32 keys, k-step ks.
  auto k_operand = [&](const lds_char* kd, int kb, int ks) -> u32x4 {
    return *(const lds_u32x4*)(kd + 32 * kb * ROWBL + koff[ks]);
  };
  // V^T (A operand of O^T += V^T P^T) for 16-key step t2 and d-block db: two transposing reads.
  auto v_operand = [&](const lds_char* vd, int t2, int db) -> u32x4 {
    u32x4 a;
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const lds_char* ap = vd + (16 * t2 + 8 * uu) * ROWBL + voff[db];
      const u32x2 v2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ap));
      a[2 * uu] = v2[0];
      a[2 * uu + 1] = v2[1];
    }
    return a;
  };
  auto sync_tiles = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  const float c = p.c;

  // ---- the Q-tile: rows [t*BM, t*BM + BM) of head (b, hq) against its visible K/V tiles;
  // wave w owns rows t*BM + 32w + (0..31)
  const int q0 = t * BM;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + l32;  // this lane's query row
  const int qr = min(qrow, Nq - 1);  // rows past Nq behave as the last row (never stored)
  // the K/V tiles the Q-tile's band touches: [j_lo, j_lo + nt)
  // keys this work-group may use: its chunk [split*kchunk, kend) (all keys when not split)
  const int kend = min(Nk, (split + 1) * p.kchunk);
  int lo_t = max(split * p.kchunk, BAND ? q0 + p.off - p.left : 0);
  int hi_t = min(kend - 1, BAND ? min(q0 + BM, Nq) - 1 + p.off + p.right : Nk - 1);
  if constexpr (AM) {
    // narrow to the mask's hull for this Q-tile: keys outside it are hidden from every row
    if (hi_t >= lo_t) {
      const int2 kr = hull_range(p.am_hull + b * p.hull_sb + hq * p.hull_sh + (int64_t)t * p.hull_nch,
                                 lo_t / kHullKeys, hi_t / kHullKeys);
      lo_t = max(lo_t, kr.x);
      hi_t = min(hi_t, kr.y);
    }
  }
  const int j_lo = lo_t / BN;
  const int nt = hi_t >= lo_t ? hi_t / BN - j_lo + 1 : 0;
  // the lane's visible keys: [klo, khi]. khi also stops at the chunk's end: the steps run past
  // the last tile (and, with split keys, into the next chunk) must add nothing.
  const int khi = BAND ? min(kend - 1, qr + p.off + p.right) : kend - 1;
  const int klo = BAND ? qr + p.off - p.left : 0;
  if (nt == 0) {
    // no row of this Q-tile sees a key: O = 0, LSE = -inf
    if (qrow < Nq) {
      const int64_t obase = ((int64_t)(b * p.Hq + hq) * Nq + qrow) * D;
#pragma unroll
      for (int c8 = 0; c8 < D / 2; c8 += 4) {
        const int dcol = 2 * c8 + 4 * h;  // lanes h = 0, 1 cover alternate groups of 4
        if (OUT_F32)
          *(f32x4*)(Of + obase + dcol) = (f32x4){0.f, 0.f, 0.f, 0.f};
        else
          *(u32x2*)((unsigned short*)p.o + obase + dcol) = (u32x2){0u, 0u};
      }
      if (h == 0) Ls[(int64_t)(b * p.Hq + hq) * Nq + qrow] = -__builtin_inff();
    }
    return;
  }

  // ---- prologue: K_0, K_1 into LDS; Q tile -> registers as the MFMA B operand (Q^T):
  // lane l: query l%32, d = 16ks + 8h + 0..7
  load_k(j_lo, K0);
  load_k(j_lo + 1, K1);
  // Mask bits: am_w[kb] is the word of keys kbase + 32kb .. + 31 of this lane's query row; the
  // lane's score 4g + i of block kb (key 32kb + 8g + 4h + i) is bit 8i + 2g + h. One
  // descriptor spans the plane; the whole offset goes into the vector operand (the scalar one
  // stays 0), so the range check covers it and a prefetch past the plane reads zeros.
  // The lane's row offset is formed at each load from an opaque lane id (the masked d = 128
  // kernel has no register to keep it in); rows past Nq read the last row.
  unsigned am_w[AM ? KB : 1];
  __amdgpu_buffer_rsrc_t am_rs;
  auto load_am = [&](int jt, unsigned(&w)[AM ? KB : 1]) {
    const int row = min(q0w + (lane_id_here() & 31), Nq - 1);
    const int vo = (row * p.am_nw + jt * KB) * 4;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) w[kb] = __builtin_amdgcn_raw_buffer_load_b32(am_rs, vo + 4 * kb, 0, 0);
  };
  // hide the scores whose bit is set; a wave whose words are all zero skips it
  auto apply_am = [&](f32x16(&st)[KB], const unsigned(&w)[AM ? KB : 1]) {
    unsigned any = 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) any |= w[kb];
    if (__builtin_amdgcn_ballot_w64(any != 0u) != 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const unsigned x = w[kb] >> h;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          st[kb][i] = ((x >> (8 * (i & 3) + 2 * (i >> 2))) & 1u) != 0u ? -__builtin_inff() : st[kb][i];
      }
    }
  };
  // Additive mask, staged through LDS: each wave's 32 rows x 32 keys of a step (64 or 128 bytes a
  // row) arrive by LDS-DMA in 1 KiB instructions of RPM rows (16 rows of 4 chunks of 16 bytes for
  // fp16, 8 rows of 8 chunks for fp32). Chunk c of row r sits at chunk c ^ (r & (CPR - 1)) of its
  // LDS row, so that the lanes' reads (one row each, the same logical chunk) spread over the banks;
  // the swizzle repeats every RPM rows, so the lane's source offset is the same for every
  // instruction, and each instruction's first row goes into its descriptor's base. The
  // descriptor runs to the plane's end: rows past Nq read zeros, keys past a row's end read the
  // next row, and the band and key-end selects below replace those scores.
  constexpr int CPR = MROW / 16, RPM = 64 / CPR, NLM = 32 / RPM;
  int fm_voff = 0, fm_roff = 0;
  const char* fm_plane = nullptr;
  int fm_bytes = 0;
  if constexpr (FM != 0) {
    fm_plane = (const char*)p.fm + (b * p.fm_sb + hq * p.fm_sh) * FM;
    fm_bytes = Nq * p.fm_ld * FM;
    const int r = lane / CPR, c = lane % CPR;
    fm_voff = r * p.fm_ld * FM + ((c ^ (r & (CPR - 1))) << 4);
    // the lane's own row (l32) and its logical chunks, read back after the step's wait
    fm_roff = wave * 32 * MROW + l32 * MROW;
  }
  auto load_fm = [&](int jt, lds_char* dst) {
    if constexpr (FM != 0) {
#pragma unroll
      for (int n = 0; n < NLM; ++n) {
        const int first = (q0w + n * RPM) * p.fm_ld * FM + jt * BN * FM;
        const int rest = fm_bytes - first;
        void* bp = (void*)(fm_plane + first);
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(bp, (short)0, rest > 0 ? rest : 0, kBufferWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + wave * 32 * MROW + n * 1024), 16, fm_voff, 0,
                                                 0, 0);
      }
    }
  };
  // the unscaled score gains M / scale (before the band's selects): group g (keys 8g + 4h .. +3)
  // is half h of logical chunk g (fp16) or chunk 2g + h (fp32)
  auto apply_fm = [&](f32x16(&st)[KB], const lds_char* src) {
    if constexpr (FM != 0) {
      const lds_char* row = src + fm_roff;
      const int sw = l32 & (CPR - 1);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float m4[4];
        if constexpr (FM == 2) {
          const u32x2 w = *(const __attribute__((address_space(3))) u32x2*)(row + ((g4 ^ sw) << 4) + 8 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned x = w[e >> 1];
            m4[e] = (float)__builtin_bit_cast(f16x2, x)[e & 1];
          }
        } else {
          const f32x4 w = *(const __attribute__((address_space(3))) f32x4*)(row + (((2 * g4 + h) ^ sw) << 4));
#pragma unroll
          for (int e = 0; e < 4; ++e) m4[e] = w[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) st[0][4 * g4 + e] = __builtin_fmaf(m4[e], p.inv_scale, st[0][4 * g4 + e]);
      }
    }
  };
  if constexpr (FM != 0) load_fm(j_lo, (lds_char*)sM0);
  // Dropout: Philox call (key tile, row tile, plane, offset) covers 4 rows x 4 keys, byte
  // 4 (row & 3) + (key & 3). The 4 lanes of a quad (rows 4a .. 4a+3, one half) need the calls of
  // their 4 key groups g (keys 32 kb + 8 g + 4 h .. + 3 of a block): lane s of the quad computes
  // group s, writes word r (row 4a + r) to slot [r][s] of the quad's LDS area, and reads back
  // slot [s][0..3], word g of which holds its own row's 4 bytes for group g. LDS operations of a
  // wave complete in order, so no barrier is needed.
  unsigned drop_w[DROP ? KB : 1][4];
  auto drop_words = [&](int jt) {
    if constexpr (DROP) {
      const int s = lane & 3;
      __attribute__((address_space(3))) unsigned* slot =
          (__attribute__((address_space(3))) unsigned*)sDrop + wave * 256 + (lane >> 2) * 16;
      const unsigned rtile = (unsigned)(q0w + l32) >> 2;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        unsigned w[4];
        philox4x32_10((unsigned)(jt * BN + 32 * kb + 8 * s + 4 * h) >> 2, rtile, (unsigned)(b * p.Hq + hq),
                      p.drop_offset, p.seed_lo, p.seed_hi, w);
#pragma unroll
        for (int r = 0; r < 4; ++r) slot[4 * r + s] = w[r];
        asm volatile("" ::: "memory");
        const u32x4 x = *(__attribute__((address_space(3))) u32x4*)(slot + 4 * s);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) drop_w[kb][g4] = x[g4];
      }
    }
  };
  if constexpr (AM) {
    const unsigned* plane = p.am_bits + b * p.bits_sb + hq * p.bits_sh;
    am_rs = __builtin_amdgcn_make_buffer_rsrc((void*)plane, (short)0, Nq * p.am_nw * 4, kBufferWord3);
    load_am(j_lo, am_w);
  }
  u32x4 qreg[NKS];
  {
    const u32x4* src = (const u32x4*)(Qp + (int64_t)qr * D + 8 * h);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qreg[ks] = src[2 * ks];
  }

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = (f32x16){};
  float m_run = -__builtin_inff();  // reference max (scaled, log2 units), one per row
  float l_run = 0.f;   // this lane's partial row sum of the exponentials (its 16 keys of each block)
  float lr_run = 0.f;  // the same sum over the rounded values that enter P V

  sync_tiles();
  f32x16 sA[KB], sB[KB];
  u32x4 pA[2 * KB], pB[2 * KB];
  // S^T of tile 0, block by block
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    sA[kb] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) sA[kb] = E::mfma(k_operand(K0, kb, ks), qreg[ks], sA[kb]);
  }
  // Every wave must be done reading K_0 before the first step refills its buffer.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __syncthreads();

  // One pipeline step for tile j (PAR = j % 2): softmax of S_j (scur) into P_j (pcur), with the
  // MFMAs of O += P_{j-1} V_{j-1} (HAS_PV) and of S_{j+1} (HAS_S) interleaved with it. The step
  // is laid out as slots of one MFMA each; a slot also issues the LDS reads of the MFMA two
  // slots ahead and an even share of the softmax's VALU work, and scheduling barriers keep that
  // order, so the MFMA pipe stays fed while the VALU work issues in its shadow.
  auto step = [&](const int r, auto par, auto has_s, auto has_pv, f32x16 (&scur)[KB], f32x16 (&snext)[KB],
                  const u32x4 (&pprev)[2 * KB], u32x4 (&pcur)[2 * KB]) {
    const int j = j_lo + r;  // the K/V tile (buffers alternate with r)
    constexpr int PAR = decltype(par)::value;
    constexpr bool HAS_S = decltype(has_s)::value;
    constexpr bool HAS_PV = decltype(has_pv)::value;
    constexpr int NPV = HAS_PV ? 2 * KB * NDB : 0;  // MFMAs of P_{j-1} V_{j-1}
    constexpr int NSM = HAS_S ? KB * NKS : 0;       // MFMAs of S_{j+1}
    constexpr int NM = NPV + NSM;
    constexpr int NSLOT = NM > 0 ? NM : 1;
    const lds_char* kread = PAR ? K0 : K1;  // K_{j+1}
    const lds_char* vread = PAR ? V0 : V1;  // V_{j-1}

    // ---- mask S_j: keys outside the lane's band [klo, khi] (khi also stops at the chunk's last key).
    // In the S^T layout element i of block kb holds key kbase + 32kb + 8(i/4) + 4h + i%4: two
    // per-lane thresholds on the constant part. A tile needs masking when it crosses the wave's
    // band edges or the end of the keys.
    const int kbase = j * BN;
    const bool need_mask = (BAND && (kbase + BN - 1 > min(q0w, Nq - 1) + p.off + p.right ||
                                     kbase < min(q0w + 31, Nq - 1) + p.off - p.left)) ||
                           (kbase + BN > kend);
    auto mask = [&](f32x16(&st)[KB]) {
      const int hi = khi - kbase - 4 * h;  // hide if part > hi
      const int lo = klo - kbase - 4 * h;  // hide if part < lo
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int part = 32 * kb + 8 * (i >> 2) + (i & 3);
          const bool hide = BAND ? (part > hi || part < lo) : part > hi;
          st[kb][i] = hide ? -__builtin_inff() : st[kb][i];
        }
    };
    if constexpr (FM != 0) apply_fm(scur, (const lds_char*)(PAR ? sM1 : sM0));
    if (need_mask) mask(scur);
    if constexpr (AM) {
      apply_am(scur, am_w);
      load_am(j + 1, am_w);  // the next step's words; its closing wait covers them
    }
    drop_words(j);  // dropout: this tile's random bytes (no work without DROP)

    // ---- the MFMA stream: P V first (its operands are ready), then S_{j+1}
    u32x4 opnd[NM > 0 ? NM : 1];
    auto fetch = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NPV)
        opnd[m] = v_operand(vread, m / NDB, m % NDB);
      else
        opnd[m] = k_operand(kread, (m - NPV) / NKS, (m - NPV) % NKS);
    };
    auto issue = [&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < NPV) {
        acc_o[m % NDB] = E::mfma(opnd[m], pprev[m / NDB], acc_o[m % NDB]);
      } else {
        constexpr int kb = (m - NPV) / NKS, ks = (m - NPV) % NKS;
        snext[kb] = E::mfma(opnd[m], qreg[ks], ks == 0 ? (f32x16){} : snext[kb]);
      }
    };

    // ---- the VALU work, as small items spread over the slots. The first tile sets the
    // reference from its row max (2*KB partial maxima of 8 scores, then the wave row max). Later
    // tiles are exponentiated against the current reference straight away and checked after
    // the slots. Then one item per score (exponential, and for odd scores the pack and the pair
    // sums); then the lane's totals.
    constexpr bool MAXFIRST = !HAS_PV;
    constexpr int NMAXI = MAXFIRST ? 2 * KB + 1 : 0, NITEM = NMAXI + 16 * KB + 1;
    float pm[2 * KB], ex[16 * KB], part[2], tile_sum = 0.f, tile_rsum = 0.f;
    auto row_max = [&](const float(&pmx)[2 * KB]) -> float {
      float mx;
      if constexpr (KB == 1)
        mx = fmaxf(pmx[0], pmx[1]);
      else
        mx = fmaxf(fmaxf(fmaxf(pmx[0], pmx[1]), pmx[2]), pmx[3]);
      return wave_half_max(mx) * c;
    };
    auto item = [&](auto itc) {
      constexpr int it = decltype(itc)::value;
      if constexpr (it < NMAXI - 1) {
        pm[it] = max8(scur[it >> 1], 8 * (it & 1));
      } else if constexpr (it == NMAXI - 1) {
        // Nothing has been accumulated yet: the reference is simply this tile's row max,
        // floored so that a row with no visible key here keeps a finite reference.
        m_run = fmaxf(row_max(pm), kRefFloor);
      } else if constexpr (it < NITEM - 1) {
        // P = 2^(S*c - m): fp32 for the row sum (the LSE needs it unrounded), packed to the
        // input type (round to nearest even) as the B operand of P V, one u32x4 per 16 keys
        constexpr int e = it - NMAXI, kb = e >> 4, i = e & 15;
        ex[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(scur[kb][i], c, -m_run));
        if constexpr ((e & 1) != 0) {
          constexpr int q = e >> 1;  // pair index: u32x4 (q / 4), word q % 4
          unsigned w = E::pack2(ex[e - 1], ex[e]);
          // Keep the packing in this slot: the value is only used after the step's closing
          // branch, and the compiler would otherwise sink it out of the interleaved block.
          pin(w);
          // dropout hides the pair's dropped halves from P V; the sums keep every probability
          if constexpr (DROP)
            pcur[q >> 2][q & 3] = w & keep_pair_mask(drop_w[kb][i >> 2], (i & 2) != 0, p.keep_t);
          else
            pcur[q >> 2][q & 3] = w;
          const float s2 = ex[e - 1] + ex[e];
          part[q & 1] = q < 2 ? s2 : part[q & 1] + s2;
          tile_rsum = E::sum2(w, q == 0 ? 0.f : tile_rsum);
        }
      } else {
        tile_sum = part[0] + part[1];
        pin(tile_sum);
        pin(tile_rsum);
      }
    };

    // Register reuse decides the split with two key blocks: block 0 of S_j (items below I1) is
    // consumed during the P V MFMAs, before the MFMAs of S_{j+1} overwrite that block, so the
    // two tiles' first blocks can share registers (without P V MFMAs those items run first).
    // With one key block the items simply spread over every slot.
    constexpr bool SPLIT = HAS_S && KB > 1;
    constexpr int I1 = SPLIT ? NMAXI + 16 : NITEM;  // items of phase 1: [0, I1)
    constexpr int S1 = SPLIT ? NPV : NSLOT;         // slots of phase 1: [0, S1)
    if constexpr (S1 == 0) static_for<0, I1>(item);
    if constexpr (NM > 0) fetch(IC<0>{});
    if constexpr (NM > 1) fetch(IC<1>{});
    static_for<0, NSLOT>([&](auto slc) {
      constexpr int sl = decltype(slc)::value;
      if constexpr (sl + 2 < NM) fetch(IC<sl + 2>{});
      // Loads for the next step go into the buffers this step does not read: V_j where V_{j-2}
      // was, K_{j+2} where K_j was. They are issued once the first MFMA runs, so their scalar
      // address and size arithmetic issues in its shadow rather than ahead of it.
      if constexpr (sl == (NM > 1 ? 1 : 0)) {
        load_v(j, PAR ? V1 : V0);
        if (HAS_S) load_k(j + 2, PAR ? K1 : K0);
        if constexpr (FM != 0) load_fm(j + 1, (lds_char*)(PAR ? sM0 : sM1));  // the next step's mask tile
      }
      // items [lo, hi) of this slot: phase 1 spreads [0, I1) over slots [0, S1), phase 2
      // spreads [I1, NITEM) over slots [S1, NSLOT)
      constexpr int D1 = S1 > 0 ? S1 : 1, D2 = NSLOT - S1 > 0 ? NSLOT - S1 : 1;
      constexpr int lo = sl < S1 ? (sl * I1) / D1 : I1 + ((sl - S1) * (NITEM - I1)) / D2;
      constexpr int hi = sl < S1 ? ((sl + 1) * I1) / D1 : I1 + ((sl + 1 - S1) * (NITEM - I1)) / D2;
      static_for<lo, hi>(item);
      if constexpr (sl < NM) issue(IC<sl>{});
      __builtin_amdgcn_sched_barrier(0);
    });

    // The exponentials were taken against the current reference. While the reference is no
    // more than 8 (log2 units) below the true running max, each is at most 2^8 and a lane's sum
    // of them stays under kSumLimit, so the tile is accepted as it is. A larger sum (or an
    // overflow) is rare: the reference moves to the exact running max, the tile's exponentials
    // are taken again (all then at most 1), and the sums and the partial output up to
    // P_{j-1} V_{j-1}, relative to the old reference, are scaled by 2^(m_old - m_new). The
    // scores are gone by then (their registers were reused and the K_j buffer is being
    // refilled), so S_j is formed again with K_j read straight from global memory.
    if constexpr (!MAXFIRST) {
      if (__builtin_amdgcn_ballot_w64(tile_sum > kSumLimit) != 0) {
        f32x16 st[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int krow = min(kbase + 32 * kb + l32, Nk - 1);  // rows past Nk are masked below
          const u32x4* src = (const u32x4*)(Kp + (int64_t)krow * ROWB) + h;
          st[kb] = (f32x16){};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) st[kb] = E::mfma(src[2 * ks], qreg[ks], st[kb]);
        }
        if constexpr (FM != 0) apply_fm(st, (const lds_char*)(PAR ? sM1 : sM0));
        if (need_mask) mask(st);
        if constexpr (AM) {
          unsigned wj[AM ? KB : 1];
          load_am(j, wj);
          apply_am(st, wj);
        }
#pragma unroll
        for (int i = 0; i < 2 * KB; ++i) pm[i] = max8(st[i >> 1], 8 * (i & 1));
        const float m_new = fmaxf(m_run, row_max(pm));
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float prt = 0.f, rs = 0.f;
#pragma unroll
        for (int q = 0; q < 8 * KB; ++q) {
          const int kb = q >> 3, i = 2 * (q & 7);
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][i], c, -m_run));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[kb][i + 1], c, -m_run));
          const unsigned w = E::pack2(e0, e1);
          if constexpr (DROP)
            pcur[q >> 2][q & 3] = w & keep_pair_mask(drop_w[kb][(q & 7) >> 1], (q & 1) != 0, p.keep_t);
          else
            pcur[q >> 2][q & 3] = w;
          prt += e0 + e1;
          rs = E::sum2(w, rs);
        }
        tile_sum = prt;
        tile_rsum = rs;
        l_run *= alpha;
        lr_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      }
    }
    l_run += tile_sum;
    lr_run += tile_rsum;
    sync_tiles();
  };

  // The last product, O += P_{nt-1} V_{nt-1}, alone: V_{nt-1} is in the buffer of parity nt % 2
  // (loaded and waited for by step nt - 1), P_{nt-1} in the registers that step filled.
  auto pv_tail = [&](auto par, const u32x4(&pprev)[2 * KB]) {
    constexpr int PAR = decltype(par)::value;
    const lds_char* vread = PAR ? V0 : V1;
    static_for<0, 2 * KB * NDB>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      acc_o[m % NDB] = E::mfma(v_operand(vread, m / NDB, m % NDB), pprev[m / NDB], acc_o[m % NDB]);
    });
  };

  // Buffers and registers alternate with j: even j uses (sA -> sB, pA), odd j (sB -> sA, pB).
  // Tiles from nt on lie wholly past the last visible key (past the Q-tile's last row when
  // causal, else past the sequence end), so the mask hides all their scores: a step on one adds
  // exactly zero (no rescale, P = 0, zero row sum).
  const IC<0> E0;
  const IC<1> E1;
  const IC<true> Y;
  const IC<false> Nn;
  step(0, E0, Y, Nn, sA, sB, pB, pA);
  if constexpr (KB == 2) {
    // Full steps in pairs while both tiles of the pair exist; the step of the last tile forms
    // no S of a further tile, and the last P V product runs on its own, so no step is spent on a
    // tile past the band.
    int r = 1;
    for (; r + 1 < nt; r += 2) {
      step(r, E1, Y, Y, sB, sA, pA, pB);
      step(r + 1, E0, Y, Y, sA, sB, pB, pA);
    }
    // r is odd and r >= nt - 1
    if (r < nt) {
      // nt even: step nt - 1 (odd) without S_nt, then P_{nt-1} V_{nt-1} from pB
      step(r, E1, Nn, Y, sB, sA, pA, pB);
      pv_tail(E0, pB);
    } else {
      // nt odd: P_{nt-1} V_{nt-1} from the registers of the even step nt - 1
      pv_tail(E1, pA);
    }
  } else {
    // 32-key steps (the instances whose registers are shortest): one code path with a fixed
    // register assignment, full steps in pairs until step nt has added P_{nt-1} V_{nt-1}; this
    // costs at most one and a half extra steps per Q-tile. (A separate last step and product
    // raise the register pressure past what three waves per SIMD allow.)
    for (int r = 1; r <= nt; r += 2) {
      step(r, E1, Y, Y, sB, sA, pA, pB);
      step(r + 1, E0, Y, Y, sA, sB, pB, pA);
    }
  }

  // ---- epilogue: O = acc / lr, LSE = ln2 * (m + log2 l). O is divided by the sum of the very
  // values P V was formed with, so the weights that multiply V sum to one: the rounding of a
  // dominant weight to the input type (up to 2^-9 relative in bf16, 2^-11 in fp16) then cancels
  // instead of scaling the whole row, which with |V| = 5 would cost about 2.4e-3 in fp16. The
  // LSE keeps the unrounded sum. A row that saw no key (a band can leave one empty) has both
  // sums zero: O = 0 and LSE = -inf.
  const float l_tot = wave_half_sum(l_run);
  const float lr_tot = wave_half_sum(lr_run);
  if (qrow < Nq) {
    const float inv = lr_tot > 0.f ? (DROP ? p.drop_scale : 1.0f) / lr_tot : 0.f;
    const int64_t obase = ((int64_t)(b * p.Hq + hq) * Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        if (32 * db + 8 * g4 >= D) continue;  // the padding columns of a half-filled last block
        const int dcol = 32 * db + 8 * g4 + 4 * h;
        const float o0 = acc_o[db][4 * g4 + 0] * inv, o1 = acc_o[db][4 * g4 + 1] * inv;
        const float o2 = acc_o[db][4 * g4 + 2] * inv, o3 = acc_o[db][4 * g4 + 3] * inv;
        if (OUT_F32) {
          *(f32x4*)(Of + obase + dcol) = (f32x4){o0, o1, o2, o3};
        } else {
          *(u32x2*)((unsigned short*)p.o + obase + dcol) = (u32x2){E::pack2(o0, o1), E::pack2(o2, o3)};
        }
      }
    if (h == 0)
      Ls[(int64_t)(b * p.Hq + hq) * Nq + qrow] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : -__builtin_inff();
  }
}

// Merge of split-key partials (the online-softmax combination of partial results: the cnblogs
// page's running maximum and denominator, applied to whole chunks). For a row with chunk
// results (O_s, LSE_s): LSE = ln sum_s e^{LSE_s}, O = sum_s e^{LSE_s - LSE} O_s; chunks whose
// keys the row cannot see carry LSE_s = -inf and weigh nothing, and a row that sees no key
// keeps O = 0 and LSE = -inf. D/4 lanes per row, 4 columns each.
template <bool BF16, int D, bool OUT_F32>
__global__ __launch_bounds__(256) void fa_merge_kernel(const float* __restrict__ ow, const float* __restrict__ lw,
                                                       void* o, float* lse, int64_t rows, int nsplit) {
  using E = Elt<BF16>;
  constexpr int TPR = D / 4;
  constexpr int RPW = 256 / TPR;  // rows per work-group (threads past RPW * TPR idle)
  if ((int)threadIdx.x >= RPW * TPR) return;
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / TPR;
  const int c4 = (threadIdx.x % TPR) * 4;
  if (row >= rows) return;
  float m = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, lw[s * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (m != -__builtin_inff()) {
    for (int s = 0; s < nsplit; ++s) {
      const float wgt = __expf(lw[s * rows + row] - m);
      den += wgt;
      acc += wgt * *(const f32x4*)(ow + (s * rows + row) * D + c4);
    }
    acc *= 1.0f / den;
  }
  if (OUT_F32)
    *(f32x4*)((float*)o + row * D + c4) = acc;
  else
    *(u32x2*)((unsigned short*)o + row * D + c4) = (u32x2){E::pack2(acc[0], acc[1]), E::pack2(acc[2], acc[3])};
  if (c4 == 0) lse[row] = m == -__builtin_inff() ? m : m + __logf(den);
}

}  // namespace fa
