// fa_mask.hpp — host side of the mask pre-pass shared by fa_fwd_mask and fa_bwd_mask: the
// workspace layout of the packed mask and its summaries, and the launch of fa_mask_prep_kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa_mask_kernel.hpp"

namespace fa {

// Parts of a masked call's workspace after `base` bytes the entry point keeps for itself (the
// forward's split partials, the backward's row statistics), each at a 256-byte boundary: the
// key hull (an int2 per plane, Q-tile and chunk of kHullKeys keys), the mask as bits
// (ceil(Nk / 32) words per row of each plane) and, for the backward, a flag byte per plane,
// 128-key tile and Q-tile, then the mask as column words (ceil(Nq / 32) per key of each plane).
// A plane per batch element and/or head where the mask's stride along that axis is nonzero.
struct MaskLayout {
  int64_t planes_b, planes_h, nq, nch, nw, nkt, nqb;
  int64_t hull_off, bits_off, flags_off, cbits_off, bytes;
};

inline int64_t mask_align256(int64_t x) { return (x + 255) / 256 * 256; }

inline MaskLayout mask_layout(int64_t base, int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t b_stride,
                              int64_t h_stride, bool with_flags) {
  MaskLayout m;
  m.planes_b = b_stride ? B : 1;
  m.planes_h = h_stride ? Hq : 1;
  m.nq = (Nq + 127) / 128;
  m.nch = (Nk + kHullKeys - 1) / kHullKeys;
  m.nw = (Nk + 31) / 32;
  m.nkt = (Nk + 127) / 128;
  m.nqb = (Nq + 31) / 32;
  const int64_t planes = m.planes_b * m.planes_h;
  m.hull_off = mask_align256(base);
  m.bits_off = mask_align256(m.hull_off + planes * m.nq * m.nch * 8);
  m.flags_off = mask_align256(m.bits_off + planes * Nq * m.nw * 4);
  m.cbits_off = mask_align256(m.flags_off + planes * m.nkt * m.nq);
  m.bytes = with_flags ? m.cbits_off + planes * Nk * m.nqb * 4 : m.bits_off + planes * Nq * m.nw * 4;
  return m;
}

// The pre-pass grid must fit one launch dimension.
inline bool mask_prep_fits(const MaskLayout& m) { return m.planes_b * m.planes_h * m.nq * m.nch < ((int64_t)1 << 31); }

// Launch fa_mask_prep_kernel over the mask into the workspace parts of `m` (flags and column
// words only when the layout has them). The band edges are as the kernels take them (1 << 30:
// unlimited).
inline hipError_t launch_mask_prep(const MaskLayout& m, bool with_flags, char* ws, const void* mask,
                                   int64_t b_stride, int64_t h_stride, int64_t row_stride, int Nq, int Nk,
                                   int left, int right, hipStream_t s) {
  PrepParams pp;
  pp.am = static_cast<const unsigned char*>(mask);
  pp.am_sb = b_stride;
  pp.am_sh = h_stride;
  pp.am_ld = (int)row_stride;
  pp.hull = reinterpret_cast<int2*>(ws + m.hull_off);
  pp.bits = reinterpret_cast<unsigned*>(ws + m.bits_off);
  pp.flags = with_flags ? reinterpret_cast<unsigned char*>(ws + m.flags_off) : nullptr;
  pp.cbits = with_flags ? reinterpret_cast<unsigned*>(ws + m.cbits_off) : nullptr;
  pp.planes_h = (int)m.planes_h;
  pp.Nq = Nq;
  pp.Nk = Nk;
  pp.off = Nk - Nq;
  pp.left = left;
  pp.right = right;
  pp.n_qtiles = (int)m.nq;
  pp.nch = (int)m.nch;
  pp.nw = (int)m.nw;
  pp.n_ktiles = (int)m.nkt;
  pp.nqb = (int)m.nqb;
  const dim3 grid((unsigned)(m.planes_b * m.planes_h * m.nq * m.nch));
  if (with_flags)
    hipLaunchKernelGGL((fa_mask_prep_kernel<128, true>), grid, dim3(256), 0, s, pp);
  else
    hipLaunchKernelGGL((fa_mask_prep_kernel<128, false>), grid, dim3(256), 0, s, pp);
  return hipGetLastError();
}

}  // namespace fa
