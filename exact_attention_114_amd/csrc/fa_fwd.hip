// fa_fwd.hip — host launcher and C ABI (include/fa.h) of the gfx950 exact-attention forward.
//
// Argument checking happens on the host before any HIP call (the operator-interface
// checks of the intelliparadigm page, section 2.2: 4-D [batch, heads, seq, head_dim]
// inputs, outputs shaped like the query, fp32 statistics [batch, heads, seq]).
// The launch is the FA2 grid over (batch, head, Q-tile) of the Triton FA2 walkthrough,
// flattened to one dimension so the kernel can remap work-groups onto XCDs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/fa.h"
#include "fa_fwd_launch.hpp"
#include "fa_mask.hpp"
#include "fa_status.hpp"

namespace fa {

fa_status fwd_dispatch(const Params& p, bool bf16, int d, bool band, bool am, bool drop, int fm, bool out_f32, int kb,
                       hipStream_t s) {
  switch (d) {
#define FA_SLICE(DD)                                                                          \
  case DD:                                                                                    \
    return bf16 ? fwd_dispatch_slice<true, DD>(p, band, am, drop, fm, out_f32, kb, s)        \
                : fwd_dispatch_slice<false, DD>(p, band, am, drop, fm, out_f32, kb, s);
    FA_SLICE(32)
    FA_SLICE(48)
    FA_SLICE(64)
    FA_SLICE(80)
    FA_SLICE(96)
    FA_SLICE(112)
    FA_SLICE(128)
#undef FA_SLICE
  }
  return FA_ERR_UNSUPPORTED;
}

void merge_dispatch(bool bf16, int d, bool out_f32, dim3 mg, const float* ow, const float* lw, void* o, float* lse,
                    int64_t rows, int nsplit, hipStream_t s) {
  switch (d) {
#define FA_SLICE(DD)                                                                                      \
  case DD:                                                                                                \
    if (bf16)                                                                                             \
      merge_dispatch_slice<true, DD>(out_f32, mg, ow, lw, o, lse, rows, nsplit, s);                      \
    else                                                                                                  \
      merge_dispatch_slice<false, DD>(out_f32, mg, ow, lw, o, lse, rows, nsplit, s);                     \
    break;
    FA_SLICE(32)
    FA_SLICE(48)
    FA_SLICE(64)
    FA_SLICE(80)
    FA_SLICE(96)
    FA_SLICE(112)
    FA_SLICE(128)
#undef FA_SLICE
  }
}

}  // namespace fa

// The scratch array of fa_fwd_split_noalloc (FA_NOALLOC_SCRATCH_BYTES per device). Host code
// never uses this name as an address: it holds the per-device pointer from hipGetSymbolAddress.
static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kBlockM = 32 * fa::kFwdWaves;  // query rows per work-group
// MI355X has 256 CUs. At d > 64 a step of one 32-key block needs fewer registers and
// half the LDS of a two-block step, so three work-groups fit on a CU instead of two; that pays
// when the grid can fill them, while a small grid does better with the longer step (fewer
// barriers). At d = 96 the one-block step measured 4-6% faster on grids above 512.
constexpr int64_t kOneBlockMinGrid = 2 * 256;

// Largest N*d accepted (2^30 - 2^16): a head plane of 2-byte values plus the 64 KiB the last
// prefetches may reach beyond it stays below 2^31 bytes.
constexpr int64_t kMaxPlaneElems = ((int64_t)1 << 30) - ((int64_t)1 << 16);

int key_blocks(int64_t d, int64_t grid) { return d > 64 && grid > kOneBlockMinGrid ? 1 : 2; }

// A band edge of this size or more is unlimited: every in-range index difference is smaller.
constexpr int kUnlimited = 1 << 30;

// Split keys: at most this many chunks per Q-tile, each a whole number of 64-key tiles and at
// least two of them.
constexpr int kMaxSplits = 16;
// The automatic choice aims at two work-groups per CU (256 CUs), but only cuts chunks of at
// least kMinChunkKeys(grid) keys: a chunk's fixed cost (loading its Q-tile, writing an fp32
// partial O, the merge) must stay small against its keys. Measured on MI355X over grids of
// 16..384 work-groups and 1k..32k keys: splitting a grid that already has a work-group on
// every CU pays only for long key ranges; small grids gain from chunks of 512 keys up.
constexpr int64_t kSplitTarget = 2 * 256;
int64_t min_chunk_keys(int64_t grid) { return grid <= 32 ? 512 : grid < 256 ? 1024 : 4096; }

// Chunks for a problem (requested: 0 = automatic) and the keys per chunk.
void split_plan(int64_t grid, int64_t Nk, int requested, int* nsplit, int* kchunk) {
  const int64_t tiles64 = (Nk + 63) / 64;
  int64_t s;
  if (requested > 0)
    s = requested;
  else if (grid >= kSplitTarget)
    s = 1;
  else
    s = std::min<int64_t>((kSplitTarget + grid - 1) / grid, Nk / min_chunk_keys(grid));
  s = std::min<int64_t>(s, kMaxSplits);
  s = std::max<int64_t>(1, std::min<int64_t>(s, tiles64 / 2));
  const int64_t chunk = ((tiles64 + s - 1) / s) * 64;
  *kchunk = (int)chunk;
  *nsplit = (int)((Nk + chunk - 1) / chunk);
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Shared shape/type validation. Returns FA_OK and fills the derived sizes.
fa_status check_problem(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, fa_dtype in_dtype,
                        int64_t* n_qtiles, int64_t* grid) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d % 16 != 0 || d < 32 || d > 128) return FA_ERR_UNSUPPORTED;
  if (in_dtype != FA_F16 && in_dtype != FA_BF16 && in_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  // The kernel sizes its tile loads in 32-bit byte offsets from the start of a K/V head
  // plane, which can reach a few tiles past its end: N*d*2 bytes plus that margin stay below 2^31.
  if (Nq * d > kMaxPlaneElems || Nk * d > kMaxPlaneElems) return FA_ERR_SHAPE;
  if (B >= lim / Hq || B * Hq >= lim / Nq) return FA_ERR_SHAPE;  // LSE index / head planes
  const int64_t nq = (Nq + kBlockM - 1) / kBlockM;
  if (B * Hq >= lim / nq) return FA_ERR_SHAPE;           // grid size
  *n_qtiles = nq;
  *grid = B * Hq * nq;
  return FA_OK;
}

// The optional mask of fa_fwd_mask (data == nullptr: none).
struct MaskArg {
  const void* data = nullptr;
  int64_t b_stride = 0, h_stride = 0, row_stride = 0;
};

// The additive float mask of fa_fwd_float_mask (data == nullptr: none); strides in elements.
struct FloatMaskArg {
  const void* data = nullptr;
  int bytes = 0;  // 2: fp16, 4: fp32
  int64_t b_stride = 0, h_stride = 0, row_stride = 0;
};

// Dropout on the probabilities (fa_fwd_dropout; keep_t == 0: none).
struct DropArg {
  int keep_t = 0;
  uint64_t seed = 0;
  uint32_t offset = 0;
};

// Every forward entry point: validation, the split plan (n_splits = 1: never split; workspace
// is then unused unless there is a mask), the mask hull, the attention kernel and, with split
// keys, the merge.
fa_status fwd_run(const void* q, const void* k, const void* v, void* o, float* lse, float* workspace, int64_t B,
                  int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int64_t window_left,
                  int64_t window_right, int n_splits, const MaskArg& mask, fa_dtype in_dtype, fa_dtype out_dtype,
                  void* stream, const DropArg& drop = DropArg{}, const FloatMaskArg& fmask = FloatMaskArg{}) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
  if (n_splits < 0 || n_splits > kMaxSplits) return FA_ERR_SHAPE;
  int64_t nq = 0, grid = 0;
  fa_status st = check_problem(B, Hq, Hkv, Nq, Nk, d, in_dtype, &nq, &grid);
  if (st != FA_OK) return st;
  const bool am = mask.data != nullptr;
  const bool f32_in = in_dtype == FA_F32;
  // fp32 inputs run their own kernel: no split keys (an automatic plan keeps one chunk), no mask
  // input, fp32 O
  if (f32_in && (n_splits > 1 || am || out_dtype != FA_F32)) return FA_ERR_UNSUPPORTED;
  const bool dropping = drop.keep_t > 0;
  if (dropping && (f32_in || am || n_splits != 1)) return FA_ERR_UNSUPPORTED;
  const int fm = fmask.data != nullptr ? fmask.bytes : 0;
  if (fm != 0 && (f32_in || am || dropping || n_splits != 1)) return FA_ERR_UNSUPPORTED;
  int ns = 1, kc = (int)(((Nk + 63) / 64) * 64);
  if (!f32_in) split_plan(grid, Nk, n_splits, &ns, &kc);
  if (ns == 1) kc = (int)(((Nk + 63) / 64) * 64);
  if ((ns > 1 || am) && !workspace) return FA_ERR_NULLPTR;
  if (!(std::isfinite(scale) && scale > 0.0f)) return FA_ERR_SHAPE;
  if (out_dtype != FA_F32 && out_dtype != in_dtype) return FA_ERR_UNSUPPORTED;
  if (am) {
    // dword reads of the mask: rows, planes and the pointer 4-byte aligned; a head's plane
    // addressed with 32-bit offsets
    if (mask.row_stride < Nk || mask.b_stride < 0 || mask.h_stride < 0) return FA_ERR_SHAPE;
    // (offsets reach a few tiles past a row's end: keep a 64 KiB margin below 2^31)
    if (Nq * mask.row_stride > ((int64_t)1 << 31) - ((int64_t)1 << 16)) return FA_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(mask.data) & 3u) || (mask.row_stride & 3) || (mask.b_stride & 3) ||
        (mask.h_stride & 3))
      return FA_ERR_ALIGN;
  }
  if (fm != 0) {
    // 8- or 16-byte reads of 4 keys: rows and planes whole groups of 4 elements, the pointer
    // 16-byte aligned; a head's plane addressed with 32-bit byte offsets
    if (fmask.row_stride < Nk || fmask.b_stride < 0 || fmask.h_stride < 0) return FA_ERR_SHAPE;
    if ((Nq + 32) * fmask.row_stride * fm > ((int64_t)1 << 31) - ((int64_t)1 << 16)) return FA_ERR_SHAPE;
    if (!aligned16(fmask.data) || (fmask.row_stride & 3) || (fmask.b_stride & 3) || (fmask.h_stride & 3))
      return FA_ERR_ALIGN;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      ((ns > 1 || am) && !aligned16(workspace)))
    return FA_ERR_ALIGN;
  const int64_t rows = B * Hq * Nq;
  if (grid * ns >= ((int64_t)1 << 31) || rows * d * ns >= ((int64_t)1 << 40)) return FA_ERR_SHAPE;
  const fa::MaskLayout ml = fa::mask_layout(ns > 1 ? ns * B * Hq * Nq * (d + 1) * 4 : 0, B, Hq, Nq, Nk,
                                            am ? mask.b_stride : 0, am ? mask.h_stride : 0, false);
  if (am && !fa::mask_prep_fits(ml)) return FA_ERR_SHAPE;

  fa::Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = ns > 1 ? (void*)workspace : o;             // split: ns planes of fp32 O [rows][d]
  p.lse = ns > 1 ? workspace + ns * rows * d : lse;  // then ns planes of fp32 LSE [rows]
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.off = (int)(Nk - Nq);
  p.left = window_left < 0 || window_left >= kUnlimited ? kUnlimited : (int)window_left;
  p.right = window_right < 0 || window_right >= kUnlimited ? kUnlimited : (int)window_right;
  p.group = (int)(Hq / Hkv);
  p.n_qtiles = (int)nq;
  p.nsplit = ns;
  p.kchunk = kc;
  p.total_wg = (int)(grid * ns);
  p.ilv = fa::interleave_groups(p.left, p.right, kUnlimited, am, B * Hkv, Nk, d);
  p.c = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
  p.vscale = 1.0f;
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
  char* const wsb = reinterpret_cast<char*>(workspace);
  int2* const hull = am ? reinterpret_cast<int2*>(wsb + ml.hull_off) : nullptr;
  unsigned* const bits = am ? reinterpret_cast<unsigned*>(wsb + ml.bits_off) : nullptr;
  p.am_bits = bits;
  p.am_nw = (int)ml.nw;
  p.bits_sh = ml.planes_h > 1 ? Nq * ml.nw : 0;
  p.bits_sb = ml.planes_b > 1 ? ml.planes_h * Nq * ml.nw : 0;
  p.am_hull = hull;
  p.hull_nch = (int)ml.nch;
  p.hull_sh = ml.planes_h > 1 ? nq * ml.nch : 0;
  p.hull_sb = ml.planes_b > 1 ? ml.planes_h * nq * ml.nch : 0;

  // With both edges unlimited every key is visible and no band is applied.
  const bool band = p.left != kUnlimited || p.right != kUnlimited;
  const bool bf16 = in_dtype == FA_BF16;
  const bool out_f32 = ns > 1 || out_dtype == FA_F32;
  const int kb = key_blocks(d, grid * ns);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (am) {
    const hipError_t e = fa::launch_mask_prep(ml, false, wsb, mask.data, mask.b_stride, mask.h_stride,
                                              mask.row_stride, p.Nq, p.Nk, p.left, p.right, s);
    if (e != hipSuccess) {
      fa::last_hip_error = (int)e;
      return FA_ERR_HIP;
    }
  }
  if (f32_in) return fa::fwd_dispatch_f32(p, (int)d, band, s);
  st = fa::fwd_dispatch(p, bf16, (int)d, band, am, dropping, fm, out_f32, kb, s);
  if (st != FA_OK || ns == 1) return st;
  const int rows_per_wg = 256 / (int)(d / 4);  // the merge kernel's rows per work-group
  const dim3 mg((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  const float* ow = workspace;
  const float* lw = workspace + ns * rows * d;
  fa::merge_dispatch(bf16, (int)d, out_dtype == FA_F32, mg, ow, lw, o, lse, rows, ns, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    fa::last_hip_error = (int)e;
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// Device addresses of `scratch`, one per device, looked up on the first call on that device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch array; the stream must belong to that device.
fa_status device_scratch(void* stream, float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fa::last_hip_error = (int)e;
    return FA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) {
      fa::last_hip_error = (int)e;
      return FA_ERR_HIP;
    }
    if ((int)sdev != dev) return FA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      fa::last_hip_error = (int)e;
      return FA_ERR_HIP;
    }
    g_scratch_ptr[dev] = reinterpret_cast<float*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                    int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int64_t window_left,
                    int64_t window_right, fa_dtype in_dtype, fa_dtype out_dtype, void* stream) {
  return fwd_run(q, k, v, o, lse, nullptr, B, Hq, Hkv, Nq, Nk, d, scale, window_left, window_right, 1, MaskArg{},
                 in_dtype, out_dtype, stream);
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                 int64_t Hkv, int64_t N, int64_t d, float scale, int causal, fa_dtype in_dtype,
                 fa_dtype out_dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  return fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, N, d, scale, -1, causal ? 0 : -1, in_dtype, out_dtype, stream);
}

size_t fa_fwd_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t d, int n_splits) {
  int64_t nq = 0, grid = 0;
  if (n_splits < 0 || n_splits > kMaxSplits) return 0;
  if (check_problem(B, Hq, 1, Nq, Nk, d, FA_F16, &nq, &grid) != FA_OK) return 0;
  int ns = 1, kc = 0;
  split_plan(grid, Nk, n_splits, &ns, &kc);
  if (ns == 1) return 0;
  return (size_t)(ns * B * Hq * Nq * (d + 1) * (int64_t)sizeof(float));
}

size_t fa_fwd_mask_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t d, int n_splits,
                                   int64_t mask_b_stride, int64_t mask_h_stride) {
  int64_t nq = 0, grid = 0;
  if (n_splits < 0 || n_splits > kMaxSplits || mask_b_stride < 0 || mask_h_stride < 0) return 0;
  if (check_problem(B, Hq, 1, Nq, Nk, d, FA_F16, &nq, &grid) != FA_OK) return 0;
  int ns = 1, kc = 0;
  split_plan(grid, Nk, n_splits, &ns, &kc);
  return (size_t)fa::mask_layout(ns > 1 ? ns * B * Hq * Nq * (d + 1) * 4 : 0, B, Hq, Nq, Nk, mask_b_stride,
                                 mask_h_stride, false)
      .bytes;
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, float* workspace,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                       int64_t window_left, int64_t window_right, int n_splits, fa_dtype in_dtype,
                       fa_dtype out_dtype, void* stream) {
  return fwd_run(q, k, v, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d, scale, window_left, window_right, n_splits,
                 MaskArg{}, in_dtype, out_dtype, stream);
}

fa_status fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                         int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int64_t window_left,
                         int64_t window_right, float keep_prob, uint64_t seed, uint32_t offset, fa_dtype in_dtype,
                         fa_dtype out_dtype, void* stream) {
  if (!(keep_prob > 0.0f && keep_prob <= 1.0f)) return FA_ERR_SHAPE;
  DropArg dr;
  dr.keep_t = std::min(256, std::max(1, (int)std::lround(256.0 * (double)keep_prob)));
  dr.seed = seed;
  dr.offset = offset;
  return fwd_run(q, k, v, o, lse, nullptr, B, Hq, Hkv, Nq, Nk, d, scale, window_left, window_right, 1, MaskArg{},
                 in_dtype, out_dtype, stream, dr);
}

fa_status fa_fwd_float_mask(const void* q, const void* k, const void* v, void* o, float* lse, const void* mask,
                            fa_dtype mask_dtype, int64_t mask_b_stride, int64_t mask_h_stride,
                            int64_t mask_row_stride, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                            int64_t d, float scale, int64_t window_left, int64_t window_right, fa_dtype in_dtype,
                            fa_dtype out_dtype, void* stream) {
  if (!mask) return FA_ERR_NULLPTR;
  if (mask_dtype != FA_F16 && mask_dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  FloatMaskArg fmk;
  fmk.data = mask;
  fmk.bytes = mask_dtype == FA_F16 ? 2 : 4;
  fmk.b_stride = mask_b_stride;
  fmk.h_stride = mask_h_stride;
  fmk.row_stride = mask_row_stride;
  return fwd_run(q, k, v, o, lse, nullptr, B, Hq, Hkv, Nq, Nk, d, scale, window_left, window_right, 1, MaskArg{},
                 in_dtype, out_dtype, stream, DropArg{}, fmk);
}

fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                               int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                               int64_t window_left, int64_t window_right, int n_splits, fa_dtype in_dtype,
                               fa_dtype out_dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
  // 0 for a problem that does not split (or invalid arguments, which fwd_run reports)
  const size_t need = fa_fwd_split_workspace_bytes(B, Hq, Nq, Nk, d, n_splits);
  if (need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  float* ws = nullptr;
  if (need > 0) {
    const fa_status st = device_scratch(stream, &ws);
    if (st != FA_OK) return st;
  }
  return fwd_run(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, d, scale, window_left, window_right, n_splits, MaskArg{},
                 in_dtype, out_dtype, stream);
}

fa_status fa_fwd_mask(const void* q, const void* k, const void* v, void* o, float* lse, const void* mask,
                      int64_t mask_b_stride, int64_t mask_h_stride, int64_t mask_row_stride, float* workspace,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                      int64_t window_left, int64_t window_right, int n_splits, fa_dtype in_dtype,
                      fa_dtype out_dtype, void* stream) {
  if (!mask) return FA_ERR_NULLPTR;
  MaskArg m;
  m.data = mask;
  m.b_stride = mask_b_stride;
  m.h_stride = mask_h_stride;
  m.row_stride = mask_row_stride;
  return fwd_run(q, k, v, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d, scale, window_left, window_right, n_splits, m,
                 in_dtype, out_dtype, stream);
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float* o, float* lse, float descale_q,
                     float descale_k, float descale_v, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                     int64_t d, float scale, int64_t window_left, int64_t window_right, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
  int64_t nq = 0, grid = 0;
  const fa_status st = check_problem(B, Hq, Hkv, Nq, Nk, d, FA_F16, &nq, &grid);
  if (st != FA_OK) return st;
  const double c = (double)scale * descale_q * descale_k * 1.4426950408889634074;
  if (!(std::isfinite(scale) && scale > 0.0f) || !(std::isfinite(descale_q) && descale_q > 0.0f) ||
      !(std::isfinite(descale_k) && descale_k > 0.0f) || !(std::isfinite(descale_v) && descale_v > 0.0f) ||
      !(std::isfinite(c) && c > 0.0 && c < 3.0e38))
    return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  fa::Params p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.off = (int)(Nk - Nq);
  p.left = window_left < 0 || window_left >= kUnlimited ? kUnlimited : (int)window_left;
  p.right = window_right < 0 || window_right >= kUnlimited ? kUnlimited : (int)window_right;
  p.group = (int)(Hq / Hkv);
  p.n_qtiles = (int)nq;
  p.nsplit = 1;
  p.kchunk = (int)(((Nk + 63) / 64) * 64);
  p.total_wg = (int)grid;
  p.ilv = 1;
  p.c = (float)c;
  p.vscale = descale_v;
  const bool band = p.left != kUnlimited || p.right != kUnlimited;
  return fa::fwd_dispatch_fp8(p, (int)d, band, reinterpret_cast<hipStream_t>(stream));
}

fa_status fa_fwd_tile(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal, fa_dtype in_dtype,
                      int* block_m, int* block_n, int64_t* grid) {
  if (!block_m || !block_n || !grid) return FA_ERR_NULLPTR;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  int64_t nq = 0, g = 0;
  const fa_status st = check_problem(B, Hq, Hkv, N, N, d, in_dtype, &nq, &g);
  if (st != FA_OK) return st;
  *block_m = kBlockM;
  *block_n = in_dtype == FA_F32 ? 32 : 32 * key_blocks(d, g);
  *grid = g;
  return FA_OK;
}

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULLPTR: return "FA_ERR_NULLPTR: a pointer argument is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid sizes, head grouping, scale or causal flag";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim must be a multiple of 16 from 32 to 128, inputs fp16/bf16 (or fp32 without split keys or mask, fp32 output), output fp32 or the input type";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: every pointer must be 16-byte aligned";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error (see fa_last_hip_error)";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: the split partials exceed the 64 MiB static scratch of fa_fwd_split_noalloc "
             "(use fa_fwd_split with a workspace)";
  }
  return "unknown fa_status";
}

int fa_last_hip_error(void) { return fa::last_hip_error; }

}  // extern "C"
