// fa_fwd_inst.hip — the forward kernel instances of one (input type, head dimension) slice.
// Built once per slice with FA_INST_BF16 (0 or 1) and FA_INST_D (a head dimension: 32, 48, 64,
// 80, 96, 112 or 128) defined
// (exact_attention_114_amd/build.py); fa_fwd.hip's host code calls them through
// fa::fwd_dispatch and fa::merge_dispatch.
#include "fa_fwd_launch.hpp"

#if !defined(FA_INST_BF16) || !defined(FA_INST_D)
#error "build one slice per (FA_INST_BF16, FA_INST_D)"
#endif

namespace fa {

// A mask runs on the banded kernel (with unlimited edges when there is no band).
template <>
fa_status fwd_dispatch_slice<(bool)FA_INST_BF16, FA_INST_D>(const Params& p, bool band, bool am, bool drop, int fm,
                                                            bool out_f32, int kb, hipStream_t s) {
  constexpr bool BF = (bool)FA_INST_BF16;
  constexpr int D = FA_INST_D;
  // the additive mask runs on the banded kernel, alone
  if (fm == 2) return dispatch_out<BF, D, true, false, false, 2>(p, out_f32, kb, s);
  if (fm == 4) return dispatch_out<BF, D, true, false, false, 4>(p, out_f32, kb, s);
  // dropout has its own instances (no mask input with it)
  if (drop)
    return band ? dispatch_out<BF, D, true, false, true>(p, out_f32, kb, s)
                : dispatch_out<BF, D, false, false, true>(p, out_f32, kb, s);
  if (am) return dispatch_out<BF, D, true, true>(p, out_f32, kb, s);
  return band ? dispatch_out<BF, D, true, false>(p, out_f32, kb, s) : dispatch_out<BF, D, false, false>(p, out_f32, kb, s);
}

template <>
void merge_dispatch_slice<(bool)FA_INST_BF16, FA_INST_D>(bool out_f32, dim3 mg, const float* ow, const float* lw,
                                                         void* o, float* lse, int64_t rows, int nsplit,
                                                         hipStream_t s) {
  constexpr bool BF = (bool)FA_INST_BF16;
  constexpr int D = FA_INST_D;
  if (out_f32)
    hipLaunchKernelGGL((fa_merge_kernel<BF, D, true>), mg, dim3(256), 0, s, ow, lw, o, lse, rows, nsplit);
  else
    hipLaunchKernelGGL((fa_merge_kernel<BF, D, false>), mg, dim3(256), 0, s, ow, lw, o, lse, rows, nsplit);
}

}  // namespace fa
