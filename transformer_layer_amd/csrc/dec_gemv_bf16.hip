// GEMV-core instantiations for bf16 weights.
#include "dec_gemv.h"

namespace dec {

template <int NJ, int KS>
static hipError_t go_bf16(int epi, const GemvArgs& a, hipStream_t s) {
  const int tpw = kWaves / KS;
  const int grid = (a.ntask + tpw - 1) / tpw;
  if (grid <= 0) return hipSuccess;
  switch (epi) {
    case kEpiStore:
      hipLaunchKernelGGL((gemv_kernel<WBF16, NJ, KS, EPI_STORE>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    case kEpiResidual:
      hipLaunchKernelGGL((gemv_kernel<WBF16, NJ, KS, EPI_RESIDUAL>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    case kEpiQkv:
      hipLaunchKernelGGL((gemv_kernel<WBF16, NJ, KS, EPI_QKV>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    case kEpiSwiglu:
      hipLaunchKernelGGL((gemv_kernel<WBF16, NJ, KS, EPI_SWIGLU>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    case kEpiStore2:
      hipLaunchKernelGGL((gemv_kernel<WBF16, NJ, KS, EPI_STORE2>), dim3(grid), dim3(kBlock), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_bf16(int epi, const GemvArgs& a, hipStream_t s) {
  const int ks = gemv_ks(a.cols, 8);
  const int nj = gemv_nj(a.cols, 8, ks);
  if (ks == 1) {
    if (nj <= 2) return go_bf16<2, 1>(epi, a, s);
    if (nj <= 4) return go_bf16<4, 1>(epi, a, s);
    if (nj <= 8) return go_bf16<8, 1>(epi, a, s);
  }
  if (ks == 4) {
    if (nj <= 2) return go_bf16<2, 4>(epi, a, s);
    if (nj <= 4) return go_bf16<4, 4>(epi, a, s);
    if (nj <= 8) return go_bf16<8, 4>(epi, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dec
