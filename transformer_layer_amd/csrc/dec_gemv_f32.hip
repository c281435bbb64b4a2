// GEMV-core instantiations for f32 weights.
#include "dec_gemv.h"

namespace dec {

// Row pairs per task: two when a lane holds few granules of a row, so that a
// wave still has several 16-byte loads in flight; one otherwise (fewer
// registers, higher occupancy). Measured on the 7B/9B layer shapes, fetching
// the next task ahead (PF) did not help once occupancy was high.
template <int NJ>
constexpr int pairs_per_task() { return NJ <= 2 ? 2 : 1; }

template <int NJ, int KS, int EPI>
static hipError_t go_f32_epi(GemvArgs a, hipStream_t s) {
  constexpr int NP = pairs_per_task<NJ>();
  auto kernel = gemv_kernel<WF32, NJ, KS, EPI, NP, false>;
  a.ntask = (a.ntask + NP - 1) / NP;  // row pairs -> tasks
  const int tpw = kWaves / KS;
  const int groups = (a.ntask + tpw - 1) / tpw;
  if (groups <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(gemv_grid(kernel, groups, gemv_per_cu<EPI>(a.cols))), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <int NJ, int KS>
static hipError_t go_f32(int epi, const GemvArgs& a, hipStream_t s) {
  switch (epi) {
    case kEpiStore: return go_f32_epi<NJ, KS, EPI_STORE>(a, s);
    case kEpiResidual: return go_f32_epi<NJ, KS, EPI_RESIDUAL>(a, s);
    case kEpiQkv: return go_f32_epi<NJ, KS, EPI_QKV>(a, s);
    case kEpiSwiglu: return go_f32_epi<NJ, KS, EPI_SWIGLU>(a, s);
    case kEpiStore2: return go_f32_epi<NJ, KS, EPI_STORE2>(a, s);
    case kEpiNormStore: return go_f32_epi<NJ, KS, EPI_NORM_STORE>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_f32(int epi, const GemvArgs& a, hipStream_t s) {
  constexpr int GE = 4;
  const int ks = gemv_ks(a.cols, GE);
  const int nj = gemv_nj(a.cols, GE, ks);
  if (ks == 1) {
    if (nj <= 1) return go_f32<1, 1>(epi, a, s);
    if (nj <= 4) return go_f32<4, 1>(epi, a, s);
    if (nj <= 8) return go_f32<8, 1>(epi, a, s);
    if (nj <= 16) return go_f32<16, 1>(epi, a, s);
  }
  if (ks == 2) {
    if (nj <= 1) return go_f32<1, 2>(epi, a, s);
    if (nj <= 4) return go_f32<4, 2>(epi, a, s);
    if (nj <= 8) return go_f32<8, 2>(epi, a, s);
    if (nj <= 16) return go_f32<16, 2>(epi, a, s);
  }
  if (ks == 4) {
    if (nj <= 1) return go_f32<1, 4>(epi, a, s);
    if (nj <= 4) return go_f32<4, 4>(epi, a, s);
    if (nj <= 8) return go_f32<8, 4>(epi, a, s);
    if (nj <= 16) return go_f32<16, 4>(epi, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dec
