// fa_bwd_launch.hpp — launches of the backward kernels, one (input type, head dimension) slice at
// a time. Each slice's kernel instances live in their own object, built from fa_bwd_inst.hip with
// FA_INST_BF16 and FA_INST_D defined, so the slices compile in parallel; the host code in
// fa_bwd.hip reaches them through bwd_dispatch_slice.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_bwd_kernel.hpp"
#include "fa_status.hpp"

namespace fa {

// Waves per work-group of the dK/dV and dQ kernels: 4, 32 keys or query rows each.
constexpr int kBwdWaves = 4;

// The three kernels of one backward problem (p filled by the host, after its argument checks):
// the row statistics over prep_rows rows, dK/dV on grid_kv work-groups and dQ on grid_q.
// fm: the additive mask's element bytes (0: none, 2: fp16, 4: fp32). One slice: defined in the
// slice's object only.
template <bool BF16, int D>
fa_status bwd_dispatch_slice(const BwdParams& p, bool band, bool am, bool drop, int fm, bool o_f32, int64_t prep_rows,
                             int64_t grid_kv, int64_t grid_q, hipStream_t s);

#define FA_BWD_SLICE_DECL(BF, D)                                                                                 \
  template <>                                                                                                    \
  fa_status bwd_dispatch_slice<BF, D>(const BwdParams& p, bool band, bool am, bool drop, int fm, bool o_f32,     \
                                      int64_t prep_rows, int64_t grid_kv, int64_t grid_q, hipStream_t s);
#define FA_BWD_SLICE_DECL_D(D) FA_BWD_SLICE_DECL(false, D) FA_BWD_SLICE_DECL(true, D)
FA_BWD_SLICE_DECL_D(32)
FA_BWD_SLICE_DECL_D(48)
FA_BWD_SLICE_DECL_D(64)
FA_BWD_SLICE_DECL_D(80)
FA_BWD_SLICE_DECL_D(96)
FA_BWD_SLICE_DECL_D(112)
FA_BWD_SLICE_DECL_D(128)
#undef FA_BWD_SLICE_DECL_D
#undef FA_BWD_SLICE_DECL

}  // namespace fa
