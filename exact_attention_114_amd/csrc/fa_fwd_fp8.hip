// fa_fwd_fp8.hip — the fp8-input forward kernels (fa_fwd_fp8_kernel.hpp), one per head dimension
// and band flag, reached from fa_fwd.hip's host code through fa::fwd_dispatch_fp8.
#include "fa_fwd_fp8_kernel.hpp"
#include "fa_fwd_launch.hpp"

namespace fa {

template <int D>
fa_status launch_fp8(const Params& p, bool band, hipStream_t s) {
  if (band)
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, true>), dim3((unsigned)p.total_wg), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, false>), dim3((unsigned)p.total_wg), dim3(256), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    last_hip_error = (int)e;
    return FA_ERR_HIP;
  }
  return FA_OK;
}

fa_status fwd_dispatch_fp8(const Params& p, int d, bool band, hipStream_t s) {
  switch (d) {
    case 32: return launch_fp8<32>(p, band, s);
    case 48: return launch_fp8<48>(p, band, s);
    case 64: return launch_fp8<64>(p, band, s);
    case 80: return launch_fp8<80>(p, band, s);
    case 96: return launch_fp8<96>(p, band, s);
    case 112: return launch_fp8<112>(p, band, s);
    case 128: return launch_fp8<128>(p, band, s);
  }
  return FA_ERR_UNSUPPORTED;
}

}  // namespace fa
