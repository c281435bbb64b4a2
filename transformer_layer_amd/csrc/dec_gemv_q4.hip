// GEMV-core instantiations for q4 weights.
#include "dec_gemv.h"

namespace dec {

template <int NJ, int KS>
static hipError_t go_q4(int epi, const GemvArgs& a, hipStream_t s) {
  const int tpw = kWaves / KS;
  const int grid = (a.ntask + tpw - 1) / tpw;
  if (grid <= 0) return hipSuccess;
  switch (epi) {
    case kEpiStore:
      hipLaunchKernelGGL((gemv_kernel<WQ4, NJ, KS, EPI_STORE>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    case kEpiResidual:
      hipLaunchKernelGGL((gemv_kernel<WQ4, NJ, KS, EPI_RESIDUAL>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    case kEpiQkv:
      hipLaunchKernelGGL((gemv_kernel<WQ4, NJ, KS, EPI_QKV>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    case kEpiSwiglu:
      hipLaunchKernelGGL((gemv_kernel<WQ4, NJ, KS, EPI_SWIGLU>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    case kEpiStore2:
      hipLaunchKernelGGL((gemv_kernel<WQ4, NJ, KS, EPI_STORE2>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_q4(int epi, const GemvArgs& a, hipStream_t s) {
  const int ks = gemv_ks(a.cols, 32);
  const int nj = gemv_nj(a.cols, 32, ks);
  if (ks == 1) {
    if (nj <= 1) return go_q4<1, 1>(epi, a, s);
    if (nj <= 2) return go_q4<2, 1>(epi, a, s);
  }
  if (ks == 4) {
    if (nj <= 1) return go_q4<1, 4>(epi, a, s);
    if (nj <= 2) return go_q4<2, 4>(epi, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dec
