// fa_fwd_launch.hpp — launches of the forward kernels, one (input type, head dimension) slice at
// a time. Each slice's kernel instances live in their own object, built from fa_fwd_inst.hip with
// FA_INST_BF16 and FA_INST_D defined, so the slices compile in parallel; the host code in
// fa_fwd.hip reaches them through fwd_dispatch and merge_dispatch.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_fwd_kernel.hpp"
#include "fa_status.hpp"

namespace fa {

// Waves per work-group: 4, 32 query rows each, so a work-group takes BM = 128 rows.
constexpr int kFwdWaves = 4;

// The attention kernel for one problem (p filled by the host), after its argument checks.
// fm: the additive mask's element bytes (0: none, 2: fp16, 4: fp32).
fa_status fwd_dispatch(const Params& p, bool bf16, int d, bool band, bool am, bool drop, int fm, bool out_f32, int kb,
                       hipStream_t s);
// The fp32-input kernel (fa_fwd_f32.hip): no split keys, no mask input, fp32 O.
fa_status fwd_dispatch_f32(const Params& p, int d, bool band, hipStream_t s);
// The fp8-input kernel (fa_fwd_fp8.hip): e4m3 Q, K, V with descales folded into p.c and
// p.vscale; no split keys, no mask input, fp32 O.
fa_status fwd_dispatch_fp8(const Params& p, int d, bool band, hipStream_t s);
// The merge of split-key partials (fa_merge_kernel) on grid mg.
void merge_dispatch(bool bf16, int d, bool out_f32, dim3 mg, const float* ow, const float* lw, void* o, float* lse,
                    int64_t rows, int nsplit, hipStream_t s);

// One slice: defined in the slice's object only.
template <bool BF16, int D>
fa_status fwd_dispatch_slice(const Params& p, bool band, bool am, bool drop, int fm, bool out_f32, int kb,
                             hipStream_t s);
template <bool BF16, int D>
void merge_dispatch_slice(bool out_f32, dim3 mg, const float* ow, const float* lw, void* o, float* lse, int64_t rows,
                          int nsplit, hipStream_t s);

#define FA_FWD_SLICE_DECL(BF, D)                                                                              \
  template <>                                                                                                 \
  fa_status fwd_dispatch_slice<BF, D>(const Params& p, bool band, bool am, bool drop, int fm, bool out_f32, int kb, \
                                      hipStream_t s);                                                           \
  template <>                                                                                                 \
  void merge_dispatch_slice<BF, D>(bool out_f32, dim3 mg, const float* ow, const float* lw, void* o, float* lse,  \
                                   int64_t rows, int nsplit, hipStream_t s);
#define FA_FWD_SLICE_DECL_D(D) FA_FWD_SLICE_DECL(false, D) FA_FWD_SLICE_DECL(true, D)
FA_FWD_SLICE_DECL_D(32)
FA_FWD_SLICE_DECL_D(48)
FA_FWD_SLICE_DECL_D(64)
FA_FWD_SLICE_DECL_D(80)
FA_FWD_SLICE_DECL_D(96)
FA_FWD_SLICE_DECL_D(112)
FA_FWD_SLICE_DECL_D(128)
#undef FA_FWD_SLICE_DECL_D
#undef FA_FWD_SLICE_DECL

#ifdef FA_INST_D
// ---- kernel launches, compiled in the slice objects only
template <bool BF16, int D, bool BAND, bool OUT_F32, int KB, bool AM, bool DROP, int FM>
fa_status launch(const Params& p, hipStream_t stream) {
  // The K/V double buffer is static LDS inside the kernel (4 tiles of 32*KB rows).
  auto kern = fa_fwd_kernel<BF16, D, BAND, OUT_F32, kFwdWaves, KB, AM, DROP, FM>;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.total_wg), dim3(kFwdWaves * 64), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    last_hip_error = (int)e;
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// The additive mask takes one key block per step (its tile is staged through LDS).
template <bool BF16, int D, bool BAND, bool OUT_F32, bool AM, bool DROP, int FM>
fa_status dispatch_kb(const Params& p, int kb, hipStream_t s) {
  if constexpr (FM != 0) {
    return launch<BF16, D, BAND, OUT_F32, 1, AM, DROP, FM>(p, s);
  } else {
    if constexpr (D > 64) {
      if (kb == 1) return launch<BF16, D, BAND, OUT_F32, 1, AM, DROP, FM>(p, s);
    }
    return launch<BF16, D, BAND, OUT_F32, 2, AM, DROP, FM>(p, s);
  }
}
template <bool BF16, int D, bool BAND, bool AM, bool DROP = false, int FM = 0>
fa_status dispatch_out(const Params& p, bool out_f32, int kb, hipStream_t s) {
  return out_f32 ? dispatch_kb<BF16, D, BAND, true, AM, DROP, FM>(p, kb, s)
                 : dispatch_kb<BF16, D, BAND, false, AM, DROP, FM>(p, kb, s);
}
#endif

}  // namespace fa
