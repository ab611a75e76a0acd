// fa_bwd_inst.hip — the backward kernel instances of one (input type, head dimension) slice.
// Built once per slice with FA_INST_BF16 (0 or 1) and FA_INST_D (a head dimension: 32, 48, 64,
// 80, 96, 112 or 128) defined (exact_attention_114_amd/build.py); fa_bwd.hip's host code calls
// them through fa::bwd_dispatch_slice.
#include "fa_bwd_launch.hpp"

#if !defined(FA_INST_BF16) || !defined(FA_INST_D)
#error "build one slice per (FA_INST_BF16, FA_INST_D)"
#endif

namespace fa {
namespace {

fa_status launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    last_hip_error = (int)e;
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// The row statistics, then dK/dV over 32 * kBwdWaves keys per work-group, then dQ over as many
// query rows.
template <bool BF16, int D, bool BAND, bool AM, bool DROP, int FM = 0>
fa_status launch_all(BwdParams p, bool o_f32, int64_t prep_rows, int64_t grid_kv, int64_t grid_q, hipStream_t s) {
  constexpr int RPB = 256 / prep_lanes(D);  // the prep kernel's rows per work-group
  constexpr int kTile = 32 * kBwdWaves;
  const unsigned prep_grid = (unsigned)((prep_rows + RPB - 1) / RPB);
  if (o_f32)
    hipLaunchKernelGGL((fa_bwd_prep_kernel<BF16, D, true>), dim3(prep_grid), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((fa_bwd_prep_kernel<BF16, D, false>), dim3(prep_grid), dim3(256), 0, s, p);
  fa_status st = launched();
  if (st != FA_OK) return st;
  p.n_tiles = (int)((p.Nk + kTile - 1) / kTile);
  p.total_wg = (int)grid_kv;
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<BF16, D, BAND, kBwdWaves, AM, DROP, FM>), dim3((unsigned)grid_kv),
                     dim3(kBwdWaves * 64), 0, s, p);
  st = launched();
  if (st != FA_OK) return st;
  p.n_tiles = (int)((p.Nq + kTile - 1) / kTile);
  p.total_wg = (int)grid_q;
  hipLaunchKernelGGL((fa_bwd_dq_kernel<BF16, D, BAND, kBwdWaves, AM, DROP, FM>), dim3((unsigned)grid_q),
                     dim3(kBwdWaves * 64), 0, s, p);
  return launched();
}

}  // namespace

// A mask runs on the banded kernels (with unlimited edges when there is no band); dropout has its
// own instances (no mask input with it); the additive mask runs on the banded kernels, alone.
template <>
fa_status bwd_dispatch_slice<(bool)FA_INST_BF16, FA_INST_D>(const BwdParams& p, bool band, bool am, bool drop, int fm,
                                                            bool o_f32, int64_t pr, int64_t gkv, int64_t gq,
                                                            hipStream_t s) {
  constexpr bool BF = (bool)FA_INST_BF16;
  constexpr int D = FA_INST_D;
  if (fm == 2) return launch_all<BF, D, true, false, false, 2>(p, o_f32, pr, gkv, gq, s);
  if (fm == 4) return launch_all<BF, D, true, false, false, 4>(p, o_f32, pr, gkv, gq, s);
  if (drop)
    return band ? launch_all<BF, D, true, false, true>(p, o_f32, pr, gkv, gq, s)
                : launch_all<BF, D, false, false, true>(p, o_f32, pr, gkv, gq, s);
  if (am) return launch_all<BF, D, true, true, false>(p, o_f32, pr, gkv, gq, s);
  return band ? launch_all<BF, D, true, false, false>(p, o_f32, pr, gkv, gq, s)
              : launch_all<BF, D, false, false, false>(p, o_f32, pr, gkv, gq, s);
}

}  // namespace fa
