// fg_host.hip -- host side of the FP8 block-scaled GEMM library: argument
// validation, device checks, tile selection and kernel launch behind the C ABI
// declared in include/fg.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "fg.h"
#include "fg_tiles.hpp"

namespace {

using fg::Params;

// ---------------------------------------------------------------- devices
constexpr int kMaxDevices = 64;
// largest N (a multiple of 8) whose 256-row output tile, 256 x N bf16, stays
// below 2^31 bytes
constexpr int kMaxN = 4194296;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
std::atomic<int> g_dev_cus[kMaxDevices];

// Checks that the current device is gfx950; caches its CU count.
int current_device(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FG_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return FG_EDEVICE;
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FG_EDEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    st = ok ? 1 : -1;
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  if (st < 0) return FG_EUNSUPPORTED;
  if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return FG_OK;
}

// ---------------------------------------------------------------- tiles
struct Tile {
  int bm, bn, waves;
  double eff;   // fraction of the matrix-core rate the tile's K loop sustains
};
// The compiled tile shapes (fg_tiles.hpp), in the order of its launch switch.
using namespace fg::tiles;
constexpr Tile kTiles[] = {{256, 256, Cfg0::W, 0.75}, {256, 128, Cfg1::W, 0.75},
                           {128, 256, Cfg2::W, 0.75}, {128, 128, Cfg3::W, 0.70},
                           {64, 112, Cfg4::W, 0.60},  {256, 112, Cfg5::W, 0.70},
                           {256, 224, Cfg6::W, 0.70}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int kDefaultCUs = 256;

#ifdef FG_TESTING
// Test-only build (libfg_testing.so): a per-thread tile override that the
// test suite sets around a call to run one compiled tile on a problem the
// cost model would give another. The product library has no such state.
thread_local int t_forced_tile = -1;
#endif

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Contiguous layout: tiles of at most 128 rows sit on the aligned 128-row
// expert blocks; 256-row tiles follow each expert's run of blocks, from a tile
// list the kernel derives from m_indices (at most kRunMaxBlocks blocks).
bool run_path(int layout, const Tile& t) { return layout == FG_LAYOUT_CONTIGUOUS && t.bm == 256; }
bool tile_allowed(int layout, int M, int G, const Tile& t) {
  if (layout != FG_LAYOUT_CONTIGUOUS || 128 % t.bm == 0) return true;
  return run_path(layout, t) && ceil_div(M, 128) <= fg::kRunMaxBlocks && G <= fg::kRunMaxExperts;
}
// 256-row contiguous tiles per column: a run of r blocks takes ceil(r/2), so
// with at most G runs (one per expert) there are at most ceil((blocks+G)/2);
// the cost model takes half of the runs as odd.
long run_tiles_m(int M, int G, bool bound) {
  const long nblk = ceil_div(M, 128);
  const long m = bound ? (nblk + G + 1) / 2 : (2 * nblk + G + 3) / 4;
  return m < nblk ? m : nblk;
}

// Number of tiles a problem splits into with a given tile shape (the
// contiguous 256-row case: the cost model's estimate).
long count_tiles(int layout, int M, int N, int G, const Tile& t) {
  const long tn = ceil_div(N, t.bn);
  if (layout == FG_LAYOUT_MASKED) return (long)G * ceil_div(M, t.bm) * tn;
  if (run_path(layout, t)) return run_tiles_m(M, G, false) * tn;
  return (long)ceil_div(M, t.bm) * tn;
}

// Workgroups a launch uses: one per tile, except the contiguous 256-row case,
// whose workgroups walk the tile list persistently (at most one per CU, as
// many as the largest possible list needs).
long launch_grid(int layout, int M, int N, int G, const Tile& t, int cus) {
  if (!run_path(layout, t)) return count_tiles(layout, M, N, G, t);
  const long most = run_tiles_m(M, G, true) * ceil_div(N, t.bn);
  return most < cus ? most : cus;
}

// Estimated cycles of one tile over kblocks K-blocks: the larger of its
// matrix-core time (BM*BN*256 FLOP at 8192 FLOP/clk per CU, derated by the
// tile's sustained fraction) and its global->LDS time ((BM+BN)*128 bytes at
// the per-CU rate the GEMM sustains: ~24 B/clk with 4 issuing waves, ~30 with
// 8) per K-block, plus a fixed prologue/epilogue cost.
constexpr double kTileFixedCycles = 4000.0;
double tile_cycles(const Tile& t, double kblocks) {
  const double t_mfma = (double)t.bm * t.bn * 256.0 / (8192.0 * t.eff);
  const double t_mem = (double)(t.bm + t.bn) * 128.0 / (t.waves >= 8 ? 30.0 : 24.0);
  return kblocks * (t_mfma > t_mem ? t_mfma : t_mem) + kTileFixedCycles;
}

// A launch plan: one compiled tile shape (index ti), or (split) the dense
// two-shape kernel -- columns [0, n_split) on SplitWide tiles in whole rounds
// (tiles_a of them), the rest on SplitNarrow tiles (tiles_b), walked by at
// most one workgroup per CU.
struct Plan {
  int ti = -1;
  bool split = false;
  bool runs = false;   // contiguous: fp8_bs_gemm_runs (RunsFull + RunsHalf tiles)
  int n_split = 0;
  long tiles_a = 0, tiles_b = 0;
  long grid = 0;
};
constexpr int kWide = 0, kNarrow = 1;   // kTiles indices of SplitWide / SplitNarrow
static_assert(SplitWide::BM == 256 && SplitWide::BN == 256 && SplitNarrow::BM == 256 && SplitNarrow::BN == 128,
              "kTiles[kWide] / kTiles[kNarrow] describe the split kernel's tile shapes");
constexpr int kRunsFull = 0, kRunsHalf = 2;   // kTiles indices of RunsFull / RunsHalf
static_assert(RunsFull::BM == 256 && RunsFull::BN == 256 && RunsHalf::BM == 128 && RunsHalf::BN == 256,
              "kTiles[kRunsFull] / kTiles[kRunsHalf] describe the runs kernel's tile shapes");

// The contiguous runs kernel: one workgroup per CU at most (the workgroups
// walk the work items), and no more than there can be 128-row items.
Plan runs_plan(int M, int N, int cus) {
  Plan p;
  p.runs = true;
  p.ti = kRunsFull;
  const long most = (long)ceil_div(M, 128) * ceil_div(N, kTiles[kRunsFull].bn);
  p.grid = most < cus ? most : cus;
  return p;
}

// Estimated cycles of the runs kernel. The tile list depends on m_indices
// (device memory), so the host takes the expected shape: G runs (one per
// expert, at most one per block), half of them odd, i.e. S = runs / 2
// single-block tiles and F = (blocks - S) / 2 two-block tiles per column; the
// kernel's own rule then decides how the two-block tiles' last round runs.
double runs_cycles(int M, int N, int G, int grid, double kblocks) {
  const long nblk = ceil_div(M, 128);
  const long runs = G < nblk ? G : nblk;
  const long S = runs / 2, F = (nblk - S) / 2;
  const long tn = ceil_div(N, kTiles[kRunsFull].bn);
  const double tf = tile_cycles(kTiles[kRunsFull], kblocks), th = tile_cycles(kTiles[kRunsHalf], kblocks);
  const long full_items = F * tn, rounds = full_items / grid, rest = full_items - rounds * grid;
  if (rest && 2 * rest + S * tn <= grid) return (double)rounds * tf + th;
  return (double)((full_items + grid - 1) / grid) * tf + (double)((S * tn + grid - 1) / grid) * th;
}

// The dense split for columns [0, nc) on wide tiles and [nc, N) on narrow ones.
Plan split_plan(int M, int N, int nc, int cus) {
  Plan p;
  p.split = true;
  p.ti = kWide;
  p.n_split = nc;
  p.tiles_a = (long)ceil_div(M, kTiles[kWide].bm) * (nc / kTiles[kWide].bn);
  p.tiles_b = (long)ceil_div(M, kTiles[kNarrow].bm) * ceil_div(N - nc, kTiles[kNarrow].bn);
  const long most = p.tiles_a > p.tiles_b ? p.tiles_a : p.tiles_b;
  p.grid = most < cus ? most : cus;
  return p;
}

#ifdef FG_TESTING
thread_local int t_forced_split = -1;   // test build: force the dense split at this column
thread_local int t_forced_grid = 0;     // test build: cap on the workgroups of the tile-walking kernels
thread_local bool t_forced_runs = false;   // test build: force the contiguous runs kernel
#endif

// Picks the launch for a problem: the compiled shape with the smallest
// estimated time, in CU cycles (tile_cycles per tile, tiles in rounds over the
// CUs, which carries the wave-quantisation loss the zwzgs.cn DeepGEMM page
// describes under "non-standard block sizes": a tile count just above a
// multiple of the SM count leaves most of the last round idle; partial tiles
// carry their padding), or for the dense layout the split onto two tile
// shapes: the widest column range whose 256x256 tiles make whole rounds, the
// remaining columns on 256x128 tiles. Contiguous tiles must not straddle an
// aligned 128-row expert block. The fused SiLU-gate epilogue needs 256-column
// tiles (one gate and one up block per row); bn256 restricts the choice to
// those (and rules out the split).
Plan pick_plan(int layout, int M, int N, int K, int G, int cus, bool bn256 = false) {
  Plan best;
#ifdef FG_TESTING
  const int forced = t_forced_tile;
  if (forced >= 0) {
    if ((!bn256 || kTiles[forced].bn == 256) && tile_allowed(layout, M, G, kTiles[forced])) {
      best.ti = forced;
      best.grid = launch_grid(layout, M, N, G, kTiles[forced], cus);
    }
    return best;
  }
  if (t_forced_split >= 0) {
    if (layout == FG_LAYOUT_DENSE && !bn256 && t_forced_split < N) best = split_plan(M, N, t_forced_split, cus);
    return best;
  }
  if (t_forced_runs) {
    if (layout == FG_LAYOUT_CONTIGUOUS && tile_allowed(layout, M, G, kTiles[kRunsFull])) best = runs_plan(M, N, cus);
    return best;
  }
#endif
  double best_cost = 0.0;
  const double kblocks = K / 128;
  for (int i = 0; i < kNumTiles; ++i) {
    const Tile& t = kTiles[i];
    if (!tile_allowed(layout, M, G, t)) continue;
    if (bn256 && t.bn != 256) continue;
    const long tiles = count_tiles(layout, M, N, G, t);
    const long rounds = (tiles + cus - 1) / cus;
    const double cost = (double)rounds * tile_cycles(t, kblocks);
    if (best.ti < 0 || cost < best_cost * (1.0 - 1e-9)) {
      best.ti = i;
      best.grid = launch_grid(layout, M, N, G, t, cus);
      best_cost = cost;
    }
  }
  if (layout == FG_LAYOUT_CONTIGUOUS && tile_allowed(layout, M, G, kTiles[kRunsFull])) {
    const Plan rp = runs_plan(M, N, cus);
    const double cost = runs_cycles(M, N, G, (int)rp.grid, kblocks);
    if (cost < best_cost * (1.0 - 1e-9)) {
      best = rp;
      best_cost = cost;
    }
  }
  if (layout == FG_LAYOUT_DENSE && !bn256) {
    const Tile& w = kTiles[kWide];
    const long tm = ceil_div(M, w.bm);
    for (long nc = (N / w.bn) * w.bn; nc >= w.bn; nc -= w.bn) {
      const long a = tm * (nc / w.bn);
      if (a % cus) continue;
      if (nc == N) break;   // whole rounds on the wide tile alone
      const Plan sp = split_plan(M, N, (int)nc, cus);
      const long b = sp.tiles_b;
      const double cost = (double)(a / cus) * tile_cycles(w, kblocks) +
                          (double)((b + cus - 1) / cus) * tile_cycles(kTiles[kNarrow], kblocks);
      if (cost < best_cost * (1.0 - 1e-9)) best = sp;
      break;
    }
  }
  return best;
}

template <bool POW2, int EPI>
hipError_t launch(int layout, int tile, const Params& p, int grid, hipStream_t s) {
  switch (layout) {
    case FG_LAYOUT_DENSE: return fg::launch_layout<fg::kDense, POW2, EPI>(tile, p, grid, s);
    case FG_LAYOUT_CONTIGUOUS: return fg::launch_layout<fg::kContiguous, POW2, EPI>(tile, p, grid, s);
    default: return fg::launch_layout<fg::kMasked, POW2, EPI>(tile, p, grid, s);
  }
}

// Outputs of the fused SiLU-gate + re-quantisation epilogue (all null: the
// plain bf16 D epilogue).
struct FusedOut {
  void* Q = nullptr;
  float* sq = nullptr;
  float* act = nullptr;
};

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// pow2: every sa and sb is a power of two, applied by the matrix core as an
// E8M0 block scale (no separate promotion). fused: write the SiLU-gated,
// re-quantised activation (out.Q / out.sq / out.act) instead of D.
int run(int layout, const void* A, const float* sa, const void* B, const float* sb, void* D,
        const int32_t* m_indices, const int32_t* masked_m, int M, int N, int K, int G,
        hipStream_t stream, bool pow2, const FusedOut* fused = nullptr) {
  // N: whole 16-byte pieces of bf16 output rows; K: whole 128-wide K-blocks
  if (M < 0 || N < 0 || K < 128 || (K % 128) != 0 || (N % 8) != 0) return FG_EINVAL;
  if (fused && (N % 256) != 0) return FG_EINVAL;
  if (layout != FG_LAYOUT_DENSE && G < 1) return FG_EINVAL;
  if (M == 0 || N == 0) return FG_OK;
  if (!A || !sa || !B || !sb) return FG_EINVAL;
  if (fused) {
    if (!fused->Q || !fused->sq || !aligned(fused->Q, 16) || !aligned(fused->sq, 4)) return FG_EINVAL;
    if (fused->act && !aligned(fused->act, 16)) return FG_EINVAL;
  } else if (!D || !aligned(D, 16)) {
    return FG_EINVAL;
  }
  if (layout == FG_LAYOUT_CONTIGUOUS && !m_indices) return FG_EINVAL;
  if (layout == FG_LAYOUT_MASKED && !masked_m) return FG_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sa, 4) || !aligned(sb, 4)) return FG_EINVAL;
  if (m_indices && !aligned(m_indices, 4)) return FG_EINVAL;
  if (masked_m && !aligned(masked_m, 4)) return FG_EINVAL;
  // 32-bit byte offsets: operand rows (M x K, N x K per expert) and the output
  // rows of one 256-row tile (256 x N bf16)
  if ((long long)M * K > 0x7fffffffLL || (long long)N * K > 0x7fffffffLL || N > kMaxN) return FG_EINVAL;

  int cus = 0;
  const int st = current_device(&cus);
  if (st != FG_OK) return st;

  const Plan plan = pick_plan(layout, M, N, K, G, cus, fused != nullptr);
  if (plan.ti < 0) return FG_EINVAL;   // (test build) a forced tile this call cannot use
  const int ti = plan.split ? fg::tiles::kSplitTile : plan.runs ? fg::tiles::kRunsTile : plan.ti;
  const Tile& t = kTiles[plan.ti];
  Params p;
  p.A = static_cast<const uint8_t*>(A);
  p.sa = sa;
  p.B = static_cast<const uint8_t*>(B);
  p.sb = sb;
  p.D = static_cast<uint16_t*>(D);
  p.Q = fused ? static_cast<uint8_t*>(fused->Q) : nullptr;
  p.sq = fused ? fused->sq : nullptr;
  p.act = fused ? fused->act : nullptr;
  p.m_indices = m_indices;
  p.masked_m = masked_m;
  p.M = M;
  p.N = N;
  p.K = K;
  p.G = layout == FG_LAYOUT_DENSE ? 1 : G;
  p.KB = K / 128;
  p.tiles_m = ceil_div(M, t.bm);   // the contiguous run-following kernels count their own
  p.tiles_n = ceil_div(N, t.bn);
  p.n_split = plan.n_split;
  p.tiles_a = (int)plan.tiles_a;
  if (plan.grid > 0x7fffffffL) return FG_EINVAL;
  int grid = (int)plan.grid;
#ifdef FG_TESTING
  // the kernels whose workgroups walk their tiles cover every tile with any
  // number of workgroups
  if (t_forced_grid > 0 && (plan.split || plan.runs || run_path(layout, t)) && grid > t_forced_grid)
    grid = t_forced_grid;
#endif

  hipError_t e;
  if (fused)
    e = pow2 ? launch<true, fg::kEpiSwigluQuant>(layout, ti, p, grid, stream)
             : launch<false, fg::kEpiSwigluQuant>(layout, ti, p, grid, stream);
  else
    e = pow2 ? launch<true, fg::kEpiBf16>(layout, ti, p, grid, stream)
             : launch<false, fg::kEpiBf16>(layout, ti, p, grid, stream);
  return e == hipSuccess ? FG_OK : FG_ELAUNCH;
}

// Tile index and grid for a problem, from sizes only.
int select_tile(int M, int N, int K, int G, int layout, int num_cus, int* ti, long* grid) {
  const bool fused = (layout & FG_SELECT_SWIGLU_QUANT) != 0;
  layout &= ~FG_SELECT_SWIGLU_QUANT;
  if (layout < FG_LAYOUT_DENSE || layout > FG_LAYOUT_MASKED) return FG_EINVAL;
  if (M < 0 || N < 0 || K < 0 || (layout != FG_LAYOUT_DENSE && G < 1)) return FG_EINVAL;
  if (layout == FG_LAYOUT_DENSE) G = 1;
  const int cus = num_cus > 0 ? num_cus : kDefaultCUs;
  const Plan plan = pick_plan(layout, M, N, K, G, cus, fused);
  if (plan.ti < 0) return FG_EINVAL;
  *ti = plan.ti;   // the split plan reports its wide tile
  *grid = plan.grid;
  return FG_OK;
}

}  // namespace

extern "C" {

int fg_gemm_fp8_nt(const void* A, const float* sa, const void* B, const float* sb, void* D,
                   int M, int N, int K, hipStream_t stream) {
  return run(FG_LAYOUT_DENSE, A, sa, B, sb, D, nullptr, nullptr, M, N, K, 1, stream, false);
}

int fg_grouped_contiguous(const void* A, const float* sa, const void* B, const float* sb,
                          void* D, const int32_t* m_indices, int M, int N, int K, int G,
                          hipStream_t stream) {
  return run(FG_LAYOUT_CONTIGUOUS, A, sa, B, sb, D, m_indices, nullptr, M, N, K, G, stream, false);
}

int fg_grouped_masked(const void* A, const float* sa, const void* B, const float* sb,
                      void* D, const int32_t* masked_m, int G, int M_max, int N, int K,
                      hipStream_t stream) {
  if (G < 1) return FG_EINVAL;
  return run(FG_LAYOUT_MASKED, A, sa, B, sb, D, nullptr, masked_m, M_max, N, K, G, stream, false);
}

int fg_gemm_fp8_nt_pow2(const void* A, const float* sa, const void* B, const float* sb, void* D,
                        int M, int N, int K, hipStream_t stream) {
  return run(FG_LAYOUT_DENSE, A, sa, B, sb, D, nullptr, nullptr, M, N, K, 1, stream, true);
}

int fg_grouped_contiguous_pow2(const void* A, const float* sa, const void* B, const float* sb,
                               void* D, const int32_t* m_indices, int M, int N, int K, int G,
                               hipStream_t stream) {
  return run(FG_LAYOUT_CONTIGUOUS, A, sa, B, sb, D, m_indices, nullptr, M, N, K, G, stream, true);
}

int fg_grouped_masked_pow2(const void* A, const float* sa, const void* B, const float* sb,
                           void* D, const int32_t* masked_m, int G, int M_max, int N, int K,
                           hipStream_t stream) {
  if (G < 1) return FG_EINVAL;
  return run(FG_LAYOUT_MASKED, A, sa, B, sb, D, nullptr, masked_m, M_max, N, K, G, stream, true);
}

int fg_gemm_fp8_nt_swiglu_quant(const void* A, const float* sa, const void* B, const float* sb,
                                void* Q, float* sq, float* act, int M, int N, int K, int scales,
                                hipStream_t stream) {
  if (scales != FG_SCALES_FP32 && scales != FG_SCALES_POW2) return FG_EINVAL;
  FusedOut out;
  out.Q = Q;
  out.sq = sq;
  out.act = act;
  return run(FG_LAYOUT_DENSE, A, sa, B, sb, nullptr, nullptr, nullptr, M, N, K, 1, stream,
             scales == FG_SCALES_POW2, &out);
}

int fg_grouped_contiguous_swiglu_quant(const void* A, const float* sa, const void* B, const float* sb,
                                       void* Q, float* sq, float* act, const int32_t* m_indices,
                                       int M, int N, int K, int G, int scales, hipStream_t stream) {
  if (scales != FG_SCALES_FP32 && scales != FG_SCALES_POW2) return FG_EINVAL;
  FusedOut out;
  out.Q = Q;
  out.sq = sq;
  out.act = act;
  return run(FG_LAYOUT_CONTIGUOUS, A, sa, B, sb, nullptr, m_indices, nullptr, M, N, K, G, stream,
             scales == FG_SCALES_POW2, &out);
}

int fg_grouped_masked_swiglu_quant(const void* A, const float* sa, const void* B, const float* sb,
                                   void* Q, float* sq, float* act, const int32_t* masked_m, int G,
                                   int M_max, int N, int K, int scales, hipStream_t stream) {
  if (scales != FG_SCALES_FP32 && scales != FG_SCALES_POW2) return FG_EINVAL;
  if (G < 1) return FG_EINVAL;
  FusedOut out;
  out.Q = Q;
  out.sq = sq;
  out.act = act;
  return run(FG_LAYOUT_MASKED, A, sa, B, sb, nullptr, nullptr, masked_m, M_max, N, K, G, stream,
             scales == FG_SCALES_POW2, &out);
}

int fg_select_config(int M, int N, int K, int G, int layout, int num_cus, int* bm, int* bn) {
  int ti = -1;
  long grid = 0;
  const int rc = select_tile(M, N, K, G, layout, num_cus, &ti, &grid);
  if (rc != FG_OK) return rc;
  if (bm) *bm = kTiles[ti].bm;
  if (bn) *bn = kTiles[ti].bn;
  return FG_OK;
}

int fg_select_grid(int M, int N, int K, int G, int layout, int num_cus, int* grid) {
  int ti = -1;
  long g = 0;
  const int rc = select_tile(M, N, K, G, layout, num_cus, &ti, &g);
  if (rc != FG_OK) return rc;
  if (grid) *grid = g > 0x7fffffffL ? 0x7fffffff : (int)g;
  return FG_OK;
}

#ifdef FG_TESTING
// Test build only: force tile bm x bn (one of the compiled tiles) for this
// thread's later calls, or restore the automatic choice with bm = bn = 0. A
// call that cannot use the forced tile returns FG_EINVAL.
int fgt_force_tile(int bm, int bn) {
  t_forced_split = -1;
  t_forced_runs = false;
  if (bm == 0 && bn == 0) {
    t_forced_tile = -1;
    return FG_OK;
  }
  for (int i = 0; i < kNumTiles; ++i) {
    if (kTiles[i].bm == bm && kTiles[i].bn == bn) {
      t_forced_tile = i;
      return FG_OK;
    }
  }
  return FG_EINVAL;
}

// Test build only: run this thread's later dense calls on the two-shape split
// kernel with columns [0, n_split) on 256x256 tiles (n_split a positive
// multiple of 256 below N; otherwise the call returns FG_EINVAL), or restore
// the automatic choice with n_split = -1.
int fgt_force_split(int n_split) {
  if (n_split != -1 && (n_split <= 0 || n_split % 256)) return FG_EINVAL;
  t_forced_tile = -1;
  t_forced_runs = false;
  t_forced_split = n_split;
  return FG_OK;
}

// Test build only: launch at most `grid` workgroups for this thread's later
// calls on the kernels whose workgroups walk their tiles (the dense two-shape
// kernel, the contiguous 256-row kernels), so that each workgroup walks many
// tiles; 0 restores the automatic grid. Other calls are unaffected.
int fgt_force_grid(int grid) {
  if (grid < 0) return FG_EINVAL;
  t_forced_grid = grid;
  return FG_OK;
}

// Test build only: run this thread's later contiguous calls on the runs
// kernel (256x256 run-following tiles, 128x256 single-block and tail tiles)
// whenever its tile list fits, or restore the automatic choice with on = 0.
int fgt_force_runs(int on) {
  t_forced_tile = -1;
  t_forced_split = -1;
  t_forced_runs = on != 0;
  return FG_OK;
}
#endif

const char* fg_strerror(int code) {
  switch (code) {
    case FG_OK: return "success";
    case FG_EINVAL: return "invalid argument (null pointer, negative size, K not a multiple of 128, N not a multiple of 8 (256 for the fused epilogue), K < 128, misaligned pointer, G < 1, unknown layout or scale kind, an operand of 2^31 bytes or more, N > 4194296)";
    case FG_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case FG_ELAUNCH: return "kernel launch failed";
    case FG_EDEVICE: return "HIP device query failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
