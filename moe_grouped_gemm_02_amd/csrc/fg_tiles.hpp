// fg_tiles.hpp -- the compiled tile configurations of the FP8 block-scaled
// GEMM and the launcher of one (layout, scale kind, epilogue) combination.
// Each combination's kernels are instantiated in its own object (fg_launch.hip
// built once per layout and scale kind), so the library compiles in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "fg_kernel.hpp"

namespace fg {
namespace tiles {
// rows x cols of D per workgroup; the host's tile table lists them in this order
using Cfg0 = TileCfg<256, 256, 4, 2, 2, false, 2, false, 3>;   // large dense / grouped
using Cfg1 = TileCfg<256, 128, 4, 2, 3, false, 2, false, 3>;
using Cfg2 = TileCfg<128, 256, 2, 4, 3, false, 2, false, 3>;   // contiguous (BM | 128)
using Cfg3 = TileCfg<128, 128, 2, 2, 4, false, 3, false, 3>;
using Cfg4 = TileCfg<64, 112, 4, 1, 4, true, 3, true, 3, 4>;     // skinny M, HBM-bound
using Cfg5 = TileCfg<256, 112, 4, 1, 3, true, 2, false, 3>;    // masked decode, HBM-bound
using Cfg6 = TileCfg<256, 224, 4, 2, 2, true, 2, false, 3>;    // N = 7168: 32 column tiles
// Dense problems whose wide-tile count leaves a partial last round: whole
// rounds of 256x256 tiles, the remaining columns on 256x128 tiles
// (fp8_bs_gemm_split); launched as tile index kSplitTile
using SplitWide = Cfg0;
using SplitNarrow = Cfg1;
constexpr int kSplitTile = 7;
// Contiguous layout: run-following 256x256 tiles with the single-block and
// tail work on 128x256 tiles (fp8_bs_gemm_runs); launched as tile index kRunsTile
using RunsFull = Cfg0;
using RunsHalf = Cfg2;
constexpr int kRunsTile = 8;
}  // namespace tiles

// Launches tile configuration `tile` (the index of its Cfg above) with `grid`
// workgroups on stream s. Defined for every LAYOUT x POW2 x EPI in
// fg_launch.hip.
template <int LAYOUT, bool POW2, int EPI>
hipError_t launch_layout(int tile, const Params& p, int grid, hipStream_t s);

#define FG_DECLARE_LAUNCH(L, P, E) extern template hipError_t launch_layout<L, P, E>(int, const Params&, int, hipStream_t);
#define FG_FOR_EACH_LAUNCH(X)                                                    \
  X(kDense, false, kEpiBf16) X(kDense, false, kEpiSwigluQuant)                   \
  X(kDense, true, kEpiBf16) X(kDense, true, kEpiSwigluQuant)                     \
  X(kContiguous, false, kEpiBf16) X(kContiguous, false, kEpiSwigluQuant)         \
  X(kContiguous, true, kEpiBf16) X(kContiguous, true, kEpiSwigluQuant)           \
  X(kMasked, false, kEpiBf16) X(kMasked, false, kEpiSwigluQuant)                 \
  X(kMasked, true, kEpiBf16) X(kMasked, true, kEpiSwigluQuant)
#ifndef FG_LAUNCH_PART
FG_FOR_EACH_LAUNCH(FG_DECLARE_LAUNCH)
#endif

}  // namespace fg
