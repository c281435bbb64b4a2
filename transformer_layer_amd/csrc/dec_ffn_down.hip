// Gated FFN with the down projection folded in, 4-bit weights: the layer's
// last two steps as one launch ("RDNA4 Decode Kernel Fusion: Pipeline
// Barriers, Not Launches, Are the Win", section "Fusion removes the barrier
// by removing the write": its four-kernel row folds down into the FFN).
//
// One workgroup of eight waves per 16-row tile of the down projection (256
// on the 9B-shaped layer), all resident at once. A workgroup first computes
// TTF tiles of h = silu(Wg u) * (Wu u), u = RMSNorm(x) g (the gated FFN's
// steps; h stored with agent-scope stores), then arrives at a grid-wide
// counter, requests its down tile's scales and weights (they do not depend
// on h, so they stream while it waits), waits until every workgroup has
// arrived, reads all of h with agent-scope loads, turns it into digits and
// adds Wd h to its 16 rows of x.
//
// The wait is bounded: a workgroup that gives up sets DEC_ERR_SYNC in the
// error word and skips its down tile; its launch still completes. Words 2
// and 3 of the first counter line count arrivals and departures; the last
// workgroup to leave clears both, so the next launch starts from zero (graph
// replay safe).
//
// Against the two-kernel form the arithmetic differs only in the gate/up
// sums: their steps are split over eight waves instead of four, so h may
// differ in the last bits; the down products and the residual are the same.
#include "dec_q4mfma.h"

namespace dec {

constexpr unsigned kGridSpinMax = 1u << 16;   // polls of the arrival counter before a workgroup gives up

template <int SPWF, int TTF, int SPWD>
__global__ __launch_bounds__(512) void q4_ffn_down_kernel(GemvArgs f, GemvArgs dn, uint32_t* bar, int no_wait) {
  constexpr int NW = 8;
  using FT = Q4Tiles<EPI_SWIGLU_PUB, NW, SPWF, TTF>;
  using DT = Q4Tiles<EPI_RESIDUAL, NW, SPWD, 1>;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int gave_up;

  if (f.null_kernel) return;

  // ---- gate/up + SwiGLU: tiles blockIdx.x * TTF .. + TTF - 1 (eight h
  // elements each), as the gated FFN kernel computes them
  {
    const FT q(f, smem);
    float4 xv[FT::GQ];
    uint4 gv[FT::GQ];
    if (q.quant()) q.load_input(xv, gv);
    const int tile0 = blockIdx.x * TTF;
    uint32_t sv[TTF][FT::NSL];
#pragma unroll
    for (int t = 0; t < TTF; ++t) q.load_scales(tile0 + t, sv[t]);
    u32x4 wq[TTF][SPWF];
    q.load_tile(tile0, wq[0]);
    q.prologue(xv, gv, sv);
#pragma unroll
    for (int t = 0; t < TTF; ++t) {
      if (t + 1 < TTF) q.load_tile(tile0 + t + 1, wq[t + 1]);
      q.run_tile(tile0 + t, t, wq[t], sv[t], 0);
    }
  }

  // ---- arrival: this workgroup's h stores have completed
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- the down tile's scales and weights, requested before the wait
  const DT p(dn, smem);
  uint32_t svd[1][DT::NSL];
  u32x4 wd[1][SPWD];
  p.load_scales(blockIdx.x, svd[0]);
  p.load_tile(blockIdx.x, wd[0]);

  // ---- every workgroup has arrived (bounded wait), then departure
  if (threadIdx.x == 0) {
    const uint32_t all = gridDim.x;
    int late = 0;
    unsigned spins = 0;
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < all) {
      if (no_wait || ++spins > kGridSpinMax) {
        late = 1;
        atomicOr(f.err, kErrSync);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    gave_up = late;
    const uint32_t prev = __hip_atomic_fetch_add(bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == all - 1) {   // every workgroup has arrived and left: clear both words
      __hip_atomic_store(bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(bar + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (gave_up) return;

  // ---- down: all of h as digits (agent-scope loads: other workgroups wrote
  // it), then x += Wd h for this workgroup's 16 rows
  float4 hv[DT::GQ];
  uint4 unused[DT::GQ];
  if (p.quant()) p.template load_input<true>(hv, unused);
  p.prologue(hv, unused, svd);
  p.run_tile(blockIdx.x, 0, wd[0], svd[0], 0);
}

namespace {

int pick_ttf(int need) {
  for (int c : {1, 2, 3, 4, 6, 8})
    if (c >= need) return c;
  return 0;
}

template <int SPWF, int TTF, int SPWD>
hipError_t go(const GemvArgs& f, const GemvArgs& dn, uint32_t* bar, int no_wait, int nblk, int lds, bool check_only,
              bool* fits, hipStream_t s) {
  auto k = q4_ffn_down_kernel<SPWF, TTF, SPWD>;
  *fits = nblk <= resident_blocks(k, 512, lds);
  if (check_only) return hipSuccess;
  if (!*fits) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(k, dim3(nblk), dim3(512), lds, s, f, dn, bar, no_wait);
  return hipGetLastError();
}

template <int SPWF, int TTF>
hipError_t go_spwd(int spwd, const GemvArgs& f, const GemvArgs& dn, uint32_t* bar, int no_wait, int nblk, int lds,
                   bool check_only, bool* fits, hipStream_t s) {
  switch (spwd) {
    case 4: return go<SPWF, TTF, 4>(f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    case 8: return go<SPWF, TTF, 8>(f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    case 12: return go<SPWF, TTF, 12>(f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    case 16: return go<SPWF, TTF, 16>(f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    default: return hipErrorInvalidValue;
  }
}

template <int SPWF>
hipError_t go_ttf(int ttf, int spwd, const GemvArgs& f, const GemvArgs& dn, uint32_t* bar, int no_wait, int nblk,
                  int lds, bool check_only, bool* fits, hipStream_t s) {
  switch (ttf) {
    case 1: return go_spwd<SPWF, 1>(spwd, f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    case 2: return go_spwd<SPWF, 2>(spwd, f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    case 3: return go_spwd<SPWF, 3>(spwd, f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    case 4: return go_spwd<SPWF, 4>(spwd, f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    case 6: return go_spwd<SPWF, 6>(spwd, f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    case 8: return go_spwd<SPWF, 8>(spwd, f, dn, bar, no_wait, nblk, lds, check_only, fits, s);
    default: return hipErrorInvalidValue;
  }
}

// Plan and (unless check_only) launch. Returns hipErrorInvalidValue for a
// shape outside the kernel's templates and hipErrorInvalidConfiguration when
// its workgroups would not all be resident at once.
hipError_t plan_and_go(const GemvArgs& f, const GemvArgs& dn, uint32_t* bar, int no_wait, bool check_only,
                       hipStream_t s) {
  const int H = f.cols, F = dn.cols;
  const int nblk = (dn.ntask + 7) / 8;   // down tiles of 16 rows (8 row pairs)
  const int ntf = (f.ntask + 7) / 8;     // gate/up tiles of 8 h elements
  const int pf = ((H / 32 + 3) / 4 + 7) / 8;   // gate/up steps per wave
  const int pd = ((F / 32 + 3) / 4 + 7) / 8;   // down steps per wave
  if (nblk < 1 || pf > 8 || pd > 16) return hipErrorInvalidValue;
  const int spwf = pf <= 4 ? 4 : 8;
  const int spwd = pd <= 4 ? 4 : pd <= 8 ? 8 : pd <= 12 ? 12 : 16;
  const int ttf = pick_ttf((ntf + nblk - 1) / nblk);
  if (!ttf) return hipErrorInvalidValue;
  const int lf = q4mfma_lds_bytes(H, 8, spwf, ttf), ld = q4mfma_lds_bytes(F, 8, spwd, 1);
  const int lds = lf > ld ? lf : ld;
  if (lds > 65536) return hipErrorInvalidValue;
  bool fits = false;
  const hipError_t e = spwf == 4 ? go_ttf<4>(ttf, spwd, f, dn, bar, no_wait, nblk, lds, check_only, &fits, s)
                                 : go_ttf<8>(ttf, spwd, f, dn, bar, no_wait, nblk, lds, check_only, &fits, s);
  if (e != hipSuccess) return e;
  return fits ? hipSuccess : hipErrorInvalidConfiguration;
}

}  // namespace

hipError_t ffn_down_q4_check(const GemvArgs& f, const GemvArgs& dn) {
  return plan_and_go(f, dn, nullptr, 0, true, nullptr);
}

hipError_t launch_ffn_down_q4(const GemvArgs& f, const GemvArgs& dn, uint32_t* bar, int no_wait, hipStream_t s) {
  if (f.ntask <= 0 || dn.ntask <= 0) return hipSuccess;
  return plan_and_go(f, dn, bar, no_wait, false, s);
}

}  // namespace dec
