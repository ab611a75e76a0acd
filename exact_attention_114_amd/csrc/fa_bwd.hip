// fa_bwd.hip — host launcher and C ABI (include/fa.h) of the gfx950 exact-attention backward.
//
// Checks every argument on the host before any HIP call, then enqueues three kernels on the
// caller's stream: the per-row statistics (D = rowsum(dO o O) and LSE in log2 units) into the
// caller's workspace, dK/dV over key tiles, and dQ over query tiles (recomputation of the
// attention matrix from the forward's LSE: intelliparadigm page, section 1.2.3).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/fa.h"
#include "fa_bwd_launch.hpp"
#include "fa_mask.hpp"
#include "fa_status.hpp"

namespace {

constexpr int kTile = 32 * fa::kBwdWaves;                                // keys or queries per work-group
constexpr int64_t kMaxPlaneElems = ((int64_t)1 << 30) - ((int64_t)1 << 16);  // as the forward
constexpr int kUnlimited = 1 << 30;                                       // an unlimited band edge


// The optional mask of fa_bwd_mask (data == nullptr: none).
struct MaskArg {
  const void* data = nullptr;
  int64_t b_stride = 0, h_stride = 0, row_stride = 0;
};

// The additive float mask of fa_bwd_float_mask (data == nullptr: none); strides in elements.
struct FloatMaskArg {
  const void* data = nullptr;
  int bytes = 0;  // 2: fp16, 4: fp32
  int64_t b_stride = 0, h_stride = 0, row_stride = 0;
};

// The dropout of fa_bwd_dropout (keep_t == 0: none).
struct DropArg {
  int keep_t = 0;
  uint64_t seed = 0;
  uint32_t offset = 0;
};

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Shape checks shared by fa_bwd_ex and fa_bwd_workspace_bytes; fills the derived sizes.
fa_status check_bwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int64_t* ws_blk,
                    int64_t* tq, int64_t* tk) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d % 16 != 0 || d < 32 || d > 128) return FA_ERR_UNSUPPORTED;
  if (Nq * d > kMaxPlaneElems || Nk * d > kMaxPlaneElems) return FA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 31;
  const int64_t t = (Nq + kTile - 1) / kTile, u = (Nk + kTile - 1) / kTile;
  if (B >= lim / Hq || B * Hq >= lim / (4 * t) || B * Hq * 4 * t >= lim / 64 || B * Hq >= lim / u) return FA_ERR_SHAPE;
  *ws_blk = 4 * t;
  *tq = t;
  *tk = u;
  return FA_OK;
}

// fa_bwd_ex and fa_bwd_mask: validation and the three launches.
fa_status bwd_run(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  float* dq, float* dk, float* dv, float* workspace, const MaskArg& mask, int64_t B, int64_t Hq,
                  int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int64_t window_left,
                  int64_t window_right, fa_dtype in_dtype, fa_dtype o_dtype, void* stream,
                  const DropArg& drop = DropArg{}, const FloatMaskArg& fmask = FloatMaskArg{}) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_NULLPTR;
  int64_t ws_blk = 0, tq = 0, tk = 0;
  const fa_status st = check_bwd(B, Hq, Hkv, Nq, Nk, d, &ws_blk, &tq, &tk);
  if (st != FA_OK) return st;
  if (!(std::isfinite(scale) && scale > 0.0f)) return FA_ERR_SHAPE;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (o_dtype != FA_F32 && o_dtype != in_dtype) return FA_ERR_UNSUPPORTED;
  const bool am = mask.data != nullptr;
  if (am) {
    // as the forward's mask: dword-aligned rows and planes, 32-bit offsets within a plane
    if (mask.row_stride < Nk || mask.b_stride < 0 || mask.h_stride < 0) return FA_ERR_SHAPE;
    if (Nq * mask.row_stride > ((int64_t)1 << 31) - ((int64_t)1 << 16)) return FA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(mask.data) & 3u) || (mask.row_stride & 3) || (mask.b_stride & 3) ||
        (mask.h_stride & 3))
      return FA_ERR_ALIGN;
  }
  const int fm = fmask.data != nullptr ? fmask.bytes : 0;
  if (fm != 0) {
    // as the forward's float mask; the dK/dV kernel reads up to 32 rows past Nq (as zeros)
    if (fmask.row_stride < Nk || fmask.b_stride < 0 || fmask.h_stride < 0) return FA_ERR_SHAPE;
    if ((Nq + 32) * fmask.row_stride * fm > ((int64_t)1 << 31) - ((int64_t)1 << 16)) return FA_ERR_SHAPE;
    if (!aligned16(fmask.data) || (fmask.row_stride & 3) || (fmask.b_stride & 3) || (fmask.h_stride & 3))
      return FA_ERR_ALIGN;
  }
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv, workspace};
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_ALIGN;
  // with a mask, the pre-pass's parts follow the row statistics in the workspace
  const fa::MaskLayout ml = fa::mask_layout(B * Hq * ws_blk * 64 * 4, B, Hq, Nq, Nk, am ? mask.b_stride : 0,
                                            am ? mask.h_stride : 0, true);
  if (am && !fa::mask_prep_fits(ml)) return FA_ERR_SHAPE;

  fa::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws = workspace;
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.off = (int)(Nk - Nq);
  p.left = window_left < 0 || window_left >= kUnlimited ? kUnlimited : (int)window_left;
  p.right = window_right < 0 || window_right >= kUnlimited ? kUnlimited : (int)window_right;
  p.group = (int)(Hq / Hkv);
  p.n_blk32 = (int)((Nq + 31) / 32);
  p.ws_blk = (int)ws_blk;
  p.n_tiles = 0;
  p.total_wg = 0;
  p.ilv = fa::interleave_groups(p.left, p.right, kUnlimited, am, B * Hkv, Nk, d);
  p.c = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
  p.scale = scale;
  p.am = static_cast<const unsigned char*>(mask.data);
  p.am_sb = mask.b_stride;
  p.am_sh = mask.h_stride;
  p.am_ld = (int)mask.row_stride;
  char* const wsb = reinterpret_cast<char*>(workspace);
  p.am_bits = am ? reinterpret_cast<const unsigned*>(wsb + ml.bits_off) : nullptr;
  p.am_nw = (int)ml.nw;
  p.bits_sh = ml.planes_h > 1 ? Nq * ml.nw : 0;
  p.bits_sb = ml.planes_b > 1 ? ml.planes_h * Nq * ml.nw : 0;
  p.am_hull = am ? reinterpret_cast<const int2*>(wsb + ml.hull_off) : nullptr;
  p.hull_nch = (int)ml.nch;
  p.hull_sh = ml.planes_h > 1 ? ml.nq * ml.nch : 0;
  p.hull_sb = ml.planes_b > 1 ? ml.planes_h * ml.nq * ml.nch : 0;
  p.am_flags = am ? reinterpret_cast<const unsigned char*>(wsb + ml.flags_off) : nullptr;
  p.flags_nq = (int)ml.nq;
  p.flags_sh = ml.planes_h > 1 ? ml.nkt * ml.nq : 0;
  p.flags_sb = ml.planes_b > 1 ? ml.planes_h * ml.nkt * ml.nq : 0;
  p.am_cbits = am ? reinterpret_cast<const unsigned*>(wsb + ml.cbits_off) : nullptr;
  p.cbits_nqb = (int)ml.nqb;
  p.cbits_sh = ml.planes_h > 1 ? Nk * ml.nqb : 0;
  p.cbits_sb = ml.planes_b > 1 ? ml.planes_h * Nk * ml.nqb : 0;
  const bool dropping = drop.keep_t > 0;
  p.seed_lo = (unsigned)(drop.seed & 0xFFFFFFFFu);
  p.seed_hi = (unsigned)(drop.seed >> 32);
  p.drop_offset = drop.offset;
  p.keep_t = dropping ? drop.keep_t : 256;
  p.drop_scale = dropping ? 256.0f / (float)drop.keep_t : 1.0f;
  p.fm = fmask.data;
  p.fm_sb = fmask.b_stride;
  p.fm_sh = fmask.h_stride;
  p.fm_ld = (int)fmask.row_stride;
  p.inv_scale = 1.0f / scale;

  const bool band = p.left != kUnlimited || p.right != kUnlimited;
  const int64_t prep_rows = B * Hq * ws_blk * 32;
  const int64_t grid_kv = B * Hkv * tk;
  const int64_t grid_q = B * Hq * tq;
  const bool bf16 = in_dtype == FA_BF16, o_f32 = o_dtype == FA_F32;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (am) {
    const hipError_t e = fa::launch_mask_prep(ml, true, wsb, mask.data, mask.b_stride, mask.h_stride,
                                              mask.row_stride, p.Nq, p.Nk, p.left, p.right, s);
    if (e != hipSuccess) {
      fa::last_hip_error = (int)e;
      return FA_ERR_HIP;
    }
  }
  switch (d) {
#define FA_BWD_D(DD)                                                                            \
  case DD:                                                                                      \
    return bf16 ? fa::bwd_dispatch_slice<true, DD>(p, band, am, dropping, fm, o_f32, prep_rows, grid_kv, grid_q, s) \
                : fa::bwd_dispatch_slice<false, DD>(p, band, am, dropping, fm, o_f32, prep_rows, grid_kv, grid_q, s);
    FA_BWD_D(32)
    FA_BWD_D(48)
    FA_BWD_D(64)
    FA_BWD_D(80)
    FA_BWD_D(96)
    FA_BWD_D(112)
    FA_BWD_D(128)
#undef FA_BWD_D
  }
  return FA_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

size_t fa_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t N, int64_t d) {
  int64_t wb = 0, t = 0, u = 0;
  if (check_bwd(B, Hq, 1, N, 1, d, &wb, &t, &u) != FA_OK) return 0;
  return (size_t)(B * Hq * wb * 64 * (int64_t)sizeof(float));
}

size_t fa_bwd_mask_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t d,
                                   int64_t mask_b_stride, int64_t mask_h_stride) {
  int64_t wb = 0, t = 0, u = 0;
  if (mask_b_stride < 0 || mask_h_stride < 0) return 0;
  if (check_bwd(B, Hq, 1, Nq, Nk, d, &wb, &t, &u) != FA_OK) return 0;
  return (size_t)fa::mask_layout(B * Hq * wb * 64 * 4, B, Hq, Nq, Nk, mask_b_stride, mask_h_stride, true).bytes;
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, float* dq, float* dk, float* dv, float* workspace, int64_t B, int64_t Hq,
                    int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int64_t window_left,
                    int64_t window_right, fa_dtype in_dtype, fa_dtype o_dtype, void* stream) {
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, workspace, MaskArg{}, B, Hq, Hkv, Nq, Nk, d, scale, window_left,
                 window_right, in_dtype, o_dtype, stream);
}

fa_status fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, float* dq, float* dk, float* dv, float* workspace, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int64_t window_left,
                         int64_t window_right, float keep_prob, uint64_t seed, uint32_t offset, fa_dtype in_dtype,
                         fa_dtype o_dtype, void* stream) {
  if (!(keep_prob > 0.0f && keep_prob <= 1.0f)) return FA_ERR_SHAPE;
  DropArg dr;
  dr.keep_t = std::min(256, std::max(1, (int)std::lround(256.0 * (double)keep_prob)));
  dr.seed = seed;
  dr.offset = offset;
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, workspace, MaskArg{}, B, Hq, Hkv, Nq, Nk, d, scale, window_left,
                 window_right, in_dtype, o_dtype, stream, dr);
}

fa_status fa_bwd_float_mask(const void* q, const void* k, const void* v, const void* o, const float* lse,
                            const void* dout, float* dq, float* dk, float* dv, float* workspace, const void* mask,
                            fa_dtype mask_dtype, int64_t mask_b_stride, int64_t mask_h_stride,
                            int64_t mask_row_stride, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                            int64_t d, float scale, int64_t window_left, int64_t window_right, fa_dtype in_dtype,
                            fa_dtype o_dtype, void* stream) {
  if (!mask) return FA_ERR_NULLPTR;
  if (mask_dtype != FA_F16 && mask_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  FloatMaskArg fmk;
  fmk.data = mask;
  fmk.bytes = mask_dtype == FA_F16 ? 2 : 4;
  fmk.b_stride = mask_b_stride;
  fmk.h_stride = mask_h_stride;
  fmk.row_stride = mask_row_stride;
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, workspace, MaskArg{}, B, Hq, Hkv, Nq, Nk, d, scale, window_left,
                 window_right, in_dtype, o_dtype, stream, DropArg{}, fmk);
}

fa_status fa_bwd_mask(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, float* dq, float* dk, float* dv, float* workspace, const void* mask,
                      int64_t mask_b_stride, int64_t mask_h_stride, int64_t mask_row_stride, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int64_t window_left,
                      int64_t window_right, fa_dtype in_dtype, fa_dtype o_dtype, void* stream) {
  if (!mask) return FA_ERR_NULLPTR;
  MaskArg m;
  m.data = mask;
  m.b_stride = mask_b_stride;
  m.h_stride = mask_h_stride;
  m.row_stride = mask_row_stride;
  return bwd_run(q, k, v, o, lse, dout, dq, dk, dv, workspace, m, B, Hq, Hkv, Nq, Nk, d, scale, window_left,
                 window_right, in_dtype, o_dtype, stream);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 float* dq, float* dk, float* dv, float* workspace, int64_t B, int64_t Hq, int64_t Hkv,
                 int64_t N, int64_t d, float scale, int causal, fa_dtype in_dtype, fa_dtype o_dtype,
                 void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_NULLPTR;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  return fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, N, d, scale, -1, causal ? 0 : -1,
                   in_dtype, o_dtype, stream);
}

}  // extern "C"
