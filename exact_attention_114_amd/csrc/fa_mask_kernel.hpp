// fa_mask_kernel.hpp — the mask pre-pass kernel for gfx950, shared by the forward and backward
// entry points that take a byte attention mask (the host side is fa_mask.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernel.hpp"

namespace fa {

// Mask preparation, run once per call before the attention kernel. For one mask plane, one
// Q-tile of BM rows and one chunk of kHullKeys keys it
//   - packs the byte mask into bits, 32 keys to a word: key 32w + 4s + b of a row (s < 8,
//     b < 4) is bit 8b + s of the row's word w, set where the key is hidden (a nonzero byte, a
//     key past Nk, or a group of four keys outside the row's band, which the band hides
//     anyway), for every row of the tile;
//   - records the chunk's hull: the first and last key some row of the tile may see, or
//     {INT_MAX, -1} when there is none (a group of four keys counts whole when the band reaches
//     it: the hull only has to contain the visible keys, and the attention kernel intersects
//     it with the Q-tile's band);
//   - optionally flags each 128-key tile of the chunk: 0 where no row of the tile may see it, 2
//     where the mask hides none of the block's pairs inside the band, else 1 (the backward's
//     dK/dV kernel takes its query range from these flags and skips the mask on blocks of 2).
// 256 threads: thread x reads dword x of the chunk (keys k0 + 4x .. + 3) of every row of the
// tile whose band reaches it (a wave reads 256 consecutive bytes of a row; every read lies
// inside the plane), and the eight threads of one word gather its bits by DPP moves.
struct PrepParams {
  const unsigned char* am;   // byte [i][j] of plane (pb, ph) at am + pb*am_sb + ph*am_sh + i*am_ld + j
  long long am_sb, am_sh;
  int am_ld;
  int2* hull;                // [planes][n_qtiles][nch]
  unsigned* bits;            // [planes][Nq][nw]
  unsigned char* flags;      // optional (nullptr: not written): [planes][n_ktiles][n_qtiles]: 0
                             // where no row of Q-tile t may see a key of 128-key tile kt, 2 where
                             // the mask hides none of the block's pairs inside the band, else 1
  unsigned* cbits;           // kernels built with COLS: [planes][Nk][nqb] column words, bit r of
                             // word (j, qb) set where key j is hidden from query 32 qb + r
  int planes_h;              // Hq or 1 (planes are numbered pb * planes_h + ph)
  int Nq, Nk, off, left, right;
  int n_qtiles, nch, nw, n_ktiles, nqb;
};

template <int BM, bool COLS>
__global__ __launch_bounds__(256) void fa_mask_prep_kernel(const PrepParams p) {
  static_assert(BM % 32 == 0, "whole 32-row query blocks per tile");
  int wg = blockIdx.x;
  const int ch = wg % p.nch;
  wg /= p.nch;
  const int t = wg % p.n_qtiles;
  const int plane = wg / p.n_qtiles;
  const int pb = plane / p.planes_h, ph = plane - pb * p.planes_h;
  const int q0 = t * BM, q1 = min(q0 + BM, p.Nq) - 1;
  const int x = (int)threadIdx.x;
  const int sl = x & 7;                                    // this thread's slot in its word
  const int key = ch * kHullKeys + 4 * x;                  // its first key
  const int nk = max(0, min(4, p.Nk - key));               // its keys below Nk
  const unsigned mine = 0x01010101u << sl;                 // its bits in the word: 8b + sl
  const unsigned tail = nk >= 4 ? 0u : (0xffffffffu << (8 * nk)) & mine;  // keys past Nk: hidden
  const int wi = ch * (kHullKeys / 32) + (x >> 3);         // the word it contributes to
  const bool store = sl == 0 && wi < p.nw;                 // one thread per existing word stores
  const unsigned char* base = p.am + (long long)pb * p.am_sb + (long long)ph * p.am_sh;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, p.Nq * p.am_ld,
                                                                      kBufferWord3);
  unsigned* const bcol = p.bits + (int64_t)plane * p.Nq * p.nw + wi;
  unsigned vis = 0u;  // bits (8b + sl) of this thread's keys that some row may see
  unsigned hidm = 0u;  // bits of its keys below Nk that the mask hides from some row it read
  // COLS: the column words of this thread's four keys for the current 32-row block, all hidden
  // until a row shows a key visible (rows past q1, or whose band misses the key, stay hidden)
  unsigned cw[4] = {~0u, ~0u, ~0u, ~0u};
  const unsigned vbytes = nk >= 4 ? 0x80808080u : nk <= 0 ? 0u : (0x80808080u >> (8 * (4 - nk)));  // below Nk
  for (int r0 = q0; r0 <= q1; r0 += 16) {
    unsigned w[16];
    bool need[16];
    bool any = false;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int r = r0 + u;  // band edges are at most 2^30: r + off +- edge fits in 32 bits
      need[u] = nk > 0 && r <= q1 && key <= r + p.off + p.right && key + nk - 1 >= r + p.off - p.left;
      any |= need[u];
      w[u] = need[u] ? __builtin_amdgcn_raw_buffer_load_b32(rs, r * p.am_ld + key, 0, 0) : ~0u;
    }
    if (__builtin_amdgcn_ballot_w64(any) == 0) {
      // no row of this batch reaches the wave's keys: every word is all hidden
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (store && r0 + u <= q1) bcol[(int64_t)(r0 + u) * p.nw] = 0xffffffffu;
    } else {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      // bit 7 of each byte: set when the byte is nonzero (its low seven bits plus 0x7f carry
      // into bit 7 unless they are zero, and bit 7 itself comes in through the OR)
      const unsigned y = (((w[u] & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w[u]) & 0x80808080u;
      unsigned word = (y >> (7 - sl)) | tail;  // byte b's flag to bit 8b + sl
      vis |= ~word & mine;
      hidm |= need[u] ? word & ~tail : 0u;
      // OR over the eight lanes of the word by DPP moves: swap neighbours and pairs within each
      // quad (quad_perm [1,0,3,2] and [2,3,0,1]), then mirror within each half-row of eight
      // lanes (row_half_mirror: lane i takes lane 7 - i, from the other quad)
      word |= (unsigned)__builtin_amdgcn_mov_dpp((int)word, 0xB1, 0xF, 0xF, false);
      word |= (unsigned)__builtin_amdgcn_mov_dpp((int)word, 0x4E, 0xF, 0xF, false);
      word |= (unsigned)__builtin_amdgcn_mov_dpp((int)word, 0x141, 0xF, 0xF, false);
      if (store && r0 + u <= q1) bcol[(int64_t)(r0 + u) * p.nw] = word;
      if constexpr (COLS) {
        // bit 8b + 7 of `seen`: key + b is visible to this row
        const unsigned seen = need[u] ? ~y & vbytes : 0u;
        const unsigned rb = 1u << ((r0 + u) & 31);
#pragma unroll
        for (int b = 0; b < 4; ++b) cw[b] = (seen >> (8 * b + 7)) & 1u ? cw[b] & ~rb : cw[b];
      }
    }
    }
    if constexpr (COLS) {
      // a 32-row block ends with this batch: store the four keys' column words
      if ((r0 & 31) == 16 || r0 + 16 > q1) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b < nk) p.cbits[((int64_t)plane * p.Nk + key + b) * p.nqb + (r0 >> 5)] = cw[b];
          cw[b] = ~0u;
        }
      }
    }
  }
  int kmin = 0x7fffffff, kmax = -1;
  if (vis != 0u) {
    kmin = key + (__builtin_ctz(vis) >> 3);
    kmax = key + ((31 - __builtin_clz(vis)) >> 3);
  }
  if (p.flags != nullptr) {
    // a wave covers 256 keys, two 128-key tiles: lanes 0..31 and 32..63
    const unsigned long long bv = __builtin_amdgcn_ballot_w64(vis != 0u);
    const unsigned long long bh = __builtin_amdgcn_ballot_w64(hidm != 0u);
    const int lane = x & 63;
    const int kt = ch * (kHullKeys / 128) + (x >> 5);
    if ((lane & 31) == 0 && kt < p.n_ktiles) {
      const bool v = (lane == 0 ? (unsigned)bv : (unsigned)(bv >> 32)) != 0u;
      const bool hd = (lane == 0 ? (unsigned)bh : (unsigned)(bh >> 32)) != 0u;
      p.flags[((int64_t)plane * p.n_ktiles + kt) * p.n_qtiles + t] = !v ? 0 : hd ? 1 : 2;
    }
  }
  // work-group reduction: within each wave, then across the four waves through LDS
#pragma unroll
  for (int sft = 32; sft >= 1; sft >>= 1) {
    kmin = min(kmin, __shfl_xor(kmin, sft));
    kmax = max(kmax, __shfl_xor(kmax, sft));
  }
  __shared__ int red[2][4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int a = min(min(red[0][0], red[0][1]), min(red[0][2], red[0][3]));
    const int z = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    p.hull[((int64_t)plane * p.n_qtiles + t) * p.nch + ch] = make_int2(a, z);
  }
}

}  // namespace fa
