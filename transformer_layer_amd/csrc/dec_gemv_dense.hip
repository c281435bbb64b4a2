// GEMV-core launches for f32 and bf16 weights (one template for both).
#include "dec_gemv.h"

namespace dec {

// Row pairs per task: two when a lane holds few granules of a row, so that a
// wave still has several 16-byte loads in flight; one otherwise (fewer
// registers, higher occupancy). Measured on the 7B/9B layer shapes, fetching
// the next task ahead (PF) did not help once occupancy was high.
template <int NJ>
constexpr int pairs_per_task() { return NJ <= 2 ? 2 : 1; }

template <class T, int NJ, int KS, int EPI>
static hipError_t go_epi(GemvArgs a, hipStream_t s) {
  constexpr int NP = pairs_per_task<NJ>();
  auto kernel = gemv_kernel<T, NJ, KS, EPI, NP, false>;
  a.ntask = (a.ntask + NP - 1) / NP;  // row pairs -> tasks
  const int tpw = kWaves / KS;
  const int groups = (a.ntask + tpw - 1) / tpw;
  if (groups <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(gemv_grid(kernel, groups, gemv_per_cu<EPI>(a.cols))), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <class T, int NJ, int KS>
static hipError_t go_nj(int epi, const GemvArgs& a, hipStream_t s) {
  switch (epi) {
    case kEpiStore: return go_epi<T, NJ, KS, EPI_STORE>(a, s);
    case kEpiResidual: return go_epi<T, NJ, KS, EPI_RESIDUAL>(a, s);
    case kEpiQkv: return go_epi<T, NJ, KS, EPI_QKV>(a, s);
    case kEpiSwiglu: return go_epi<T, NJ, KS, EPI_SWIGLU>(a, s);
    case kEpiStore2: return go_epi<T, NJ, KS, EPI_STORE2>(a, s);
    case kEpiNormStore: return go_epi<T, NJ, KS, EPI_NORM_STORE>(a, s);
    default: return hipErrorInvalidValue;
  }
}

// Granules per lane are rounded up to one of four instantiated counts: the
// lane's input slice (NJ granules of GE values) stays within 16 registers
// for the column split gemv_ks picks, and 64 for the longest rows.
template <class T, int KS, int N0, int N1, int N2, int N3>
static hipError_t go_ks(int nj, int epi, const GemvArgs& a, hipStream_t s) {
  if (nj <= N0) return go_nj<T, N0, KS>(epi, a, s);
  if (nj <= N1) return go_nj<T, N1, KS>(epi, a, s);
  if (nj <= N2) return go_nj<T, N2, KS>(epi, a, s);
  if (nj <= N3) return go_nj<T, N3, KS>(epi, a, s);
  return hipErrorInvalidValue;
}

template <class T, int N0, int N1, int N2, int N3>
static hipError_t launch_dense(int epi, const GemvArgs& a, hipStream_t s) {
  const int ks = gemv_ks(a.cols, T::GE);
  const int nj = gemv_nj(a.cols, T::GE, ks);
  switch (ks) {
    case 1: return go_ks<T, 1, N0, N1, N2, N3>(nj, epi, a, s);
    case 2: return go_ks<T, 2, N0, N1, N2, N3>(nj, epi, a, s);
    case 4: return go_ks<T, 4, N0, N1, N2, N3>(nj, epi, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemv_f32(int epi, const GemvArgs& a, hipStream_t s) {
  return launch_dense<WF32, 1, 4, 8, 16>(epi, a, s);
}

hipError_t launch_gemv_bf16(int epi, const GemvArgs& a, hipStream_t s) {
  return launch_dense<WBF16, 2, 4, 6, 8>(epi, a, s);
}

}  // namespace dec
