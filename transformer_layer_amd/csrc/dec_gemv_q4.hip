// Launches of the four-bit GEMV (matrix-core kernel).
#include "dec_q4mfma.h"

namespace dec {

template <int EPI, int NW, int SPW>
static hipError_t go_q4mfma(const GemvArgs& a, int ntiles, hipStream_t s) {
  // one tile per workgroup when every tile's workgroup fits on the chip at
  // once; otherwise two adjacent tiles per workgroup, or three for a gated
  // FFN of 1536+ tiles (the 9B-shaped layer: 512 workgroups, two per CU;
  // each re-quantizes the input once for three tiles, +0.15% tokens/s in a
  // same-box A/B; each tile's weights are still requested only once the
  // previous tile runs: requesting the second and third together lost 3.5%)
  // (16 steps per wave, rows above 12288 columns: one tile per workgroup,
  // since two tiles' weights in flight would not fit in registers)
  constexpr bool kMulti = SPW <= 12;
  auto one = q4mfma_kernel<EPI, NW, SPW, 1>;
  const int lds1 = q4mfma_lds_bytes(a.cols, NW, SPW, 1);
  const int lds2 = q4mfma_lds_bytes(a.cols, NW, SPW, 2);
  const int lds3 = q4mfma_lds_bytes(a.cols, NW, SPW, 3);
  if (lds1 > 65536) return hipErrorInvalidValue;
  if constexpr (EPI == EPI_SWIGLU && kMulti) {
    if (ntiles >= 1536 && lds3 <= 65536) {
      auto three = q4mfma_kernel<EPI, NW, SPW, 3>;
      hipLaunchKernelGGL(three, dim3((ntiles + 2) / 3), dim3(NW * 64), lds3, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (kMulti) {
    if (ntiles > resident_blocks(one, NW * 64, lds1) && lds2 <= 65536) {
      auto two = q4mfma_kernel<EPI, NW, SPW, 2>;
      hipLaunchKernelGGL(two, dim3((ntiles + 1) / 2), dim3(NW * 64), lds2, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL(one, dim3(ntiles), dim3(NW * 64), lds1, s, a);
  return hipGetLastError();
}

template <int EPI, int NW>
static hipError_t go_q4mfma_spw(const GemvArgs& a, int ntiles, int spw, hipStream_t s) {
  switch (spw) {
    case 4: return go_q4mfma<EPI, NW, 4>(a, ntiles, s);
    case 8: return go_q4mfma<EPI, NW, 8>(a, ntiles, s);
    case 12: return go_q4mfma<EPI, NW, 12>(a, ntiles, s);
    case 16: return go_q4mfma<EPI, NW, 16>(a, ntiles, s);
    default: return hipErrorInvalidValue;
  }
}

template <int EPI>
static hipError_t go_q4mfma_epi(const GemvArgs& a, hipStream_t s) {
  // row pairs -> tiles of eight pairs
  const int ntiles = (a.ntask + 7) / 8;
  if (ntiles <= 0) return hipSuccess;
  int nw = 0, spw = 0;
  if (!q4mfma_plan(a.cols, ntiles, &nw, &spw)) return hipErrorInvalidValue;
  return nw == 8 ? go_q4mfma_spw<EPI, 8>(a, ntiles, spw, s) : go_q4mfma_spw<EPI, 4>(a, ntiles, spw, s);
}

hipError_t launch_gemv_q4(int epi, const GemvArgs& a, hipStream_t s) {
  switch (epi) {
    case kEpiStore: return go_q4mfma_epi<EPI_STORE>(a, s);
    case kEpiResidual: return go_q4mfma_epi<EPI_RESIDUAL>(a, s);
    case kEpiQkv: return go_q4mfma_epi<EPI_QKV>(a, s);
    case kEpiSwiglu: return go_q4mfma_epi<EPI_SWIGLU>(a, s);
    case kEpiStore2: return go_q4mfma_epi<EPI_STORE2>(a, s);
    case kEpiNormStore: return go_q4mfma_epi<EPI_NORM_STORE>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dec
