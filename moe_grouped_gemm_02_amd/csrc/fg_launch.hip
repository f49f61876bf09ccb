// fg_launch.hip -- kernel instantiations and launchers for one layout and one
// scale kind (both epilogues). Built once per part: FG_LAUNCH_PART =
// 2 * layout + pow2 (layout 0 dense, 1 contiguous, 2 masked).
#include <hip/hip_runtime.h>

#include "fg_tiles.hpp"

#ifndef FG_LAUNCH_PART
#error "FG_LAUNCH_PART selects the layout and scale kind of this object"
#endif

namespace fg {

namespace {
// One tile configuration; the fused epilogue exists only for 256-column tiles.
template <int LAYOUT, bool POW2, int EPI, class C>
hipError_t launch_tile(const Params& p, int grid, hipStream_t s) {
  if constexpr (EPI == kEpiSwigluQuant && C::BN != 256) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((fp8_bs_gemm<LAYOUT, C, POW2, EPI>), dim3(grid), dim3(C::THREADS), 0, s, p);
    return hipGetLastError();
  }
}
}  // namespace

template <int LAYOUT, bool POW2, int EPI>
hipError_t launch_layout(int tile, const Params& p, int grid, hipStream_t s) {
  using namespace tiles;
  switch (tile) {
    case 0: return launch_tile<LAYOUT, POW2, EPI, Cfg0>(p, grid, s);
    case 1: return launch_tile<LAYOUT, POW2, EPI, Cfg1>(p, grid, s);
    case 2: return launch_tile<LAYOUT, POW2, EPI, Cfg2>(p, grid, s);
    case 3: return launch_tile<LAYOUT, POW2, EPI, Cfg3>(p, grid, s);
    case 4: return launch_tile<LAYOUT, POW2, EPI, Cfg4>(p, grid, s);
    case 5: return launch_tile<LAYOUT, POW2, EPI, Cfg5>(p, grid, s);
    case 6: return launch_tile<LAYOUT, POW2, EPI, Cfg6>(p, grid, s);
    case kSplitTile:
      if constexpr (LAYOUT == kDense && EPI == kEpiBf16) {
        hipLaunchKernelGGL((fp8_bs_gemm_split<SplitWide, SplitNarrow, POW2>), dim3(grid),
                           dim3(SplitWide::THREADS), 0, s, p);
        return hipGetLastError();
      } else {
        return hipErrorInvalidValue;
      }
    case kRunsTile:
      if constexpr (LAYOUT == kContiguous) {
        hipLaunchKernelGGL((fp8_bs_gemm_runs<RunsFull, RunsHalf, POW2, EPI>), dim3(grid),
                           dim3(RunsFull::THREADS), 0, s, p);
        return hipGetLastError();
      } else {
        return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
}

constexpr int kPartLayout = FG_LAUNCH_PART / 2;
constexpr bool kPartPow2 = (FG_LAUNCH_PART % 2) != 0;
template hipError_t launch_layout<kPartLayout, kPartPow2, kEpiBf16>(int, const Params&, int, hipStream_t);
template hipError_t launch_layout<kPartLayout, kPartPow2, kEpiSwigluQuant>(int, const Params&, int, hipStream_t);

}  // namespace fg
