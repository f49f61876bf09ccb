// fg_host.hip -- host side of the FP8 block-scaled GEMM library: argument
// validation, device checks, tile selection and kernel launch behind the C ABI
// declared in include/fg.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "fg.h"
#include "fg_kernel.hpp"

namespace {

using fg::Params;

// ---------------------------------------------------------------- devices
constexpr int kMaxDevices = 64;
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
// Compiled tile shapes (rows x cols of D per workgroup), in the order of the
// launch switch below.
using Cfg0 = fg::TileCfg<256, 256, 4, 2, 2, false, 2, false, 3>;   // large dense / grouped
using Cfg1 = fg::TileCfg<256, 128, 4, 2, 3, false, 2, false, 3>;
using Cfg2 = fg::TileCfg<128, 256, 2, 4, 3, false, 2, false, 3>;   // contiguous (BM | 128)
using Cfg3 = fg::TileCfg<128, 128, 2, 2, 4, false, 3, false, 3>;
using Cfg4 = fg::TileCfg<64, 112, 4, 1, 6, true, 6, true, 3, 3>;     // skinny M, HBM-bound
using Cfg5 = fg::TileCfg<256, 112, 4, 1, 3, true, 2, false, 3>;    // masked decode, HBM-bound
constexpr Tile kTiles[] = {{256, 256, Cfg0::W, 0.70}, {256, 128, Cfg1::W, 0.75},
                           {128, 256, Cfg2::W, 0.75}, {128, 128, Cfg3::W, 0.70},
                           {64, 112, Cfg4::W, 0.60},  {256, 112, Cfg5::W, 0.70}};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
constexpr int kDefaultCUs = 256;

std::atomic<int> g_forced_tile{-1};

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Number of tiles a problem splits into with a given tile shape.
long count_tiles(int layout, int M, int N, int G, const Tile& t) {
  const long tn = ceil_div(N, t.bn);
  if (layout == FG_LAYOUT_MASKED) return (long)G * ceil_div(M, t.bm) * tn;
  return (long)ceil_div(M, t.bm) * tn;
}

// Picks the tile for a problem: the compiled shape with the smallest
// estimated time, in CU cycles. One K-block of a tile costs the larger of its
// matrix-core time (BM*BN*256 FLOP at 8192 FLOP/clk per CU, derated by the
// tile's sustained fraction) and its global->LDS time ((BM+BN)*128 bytes at
// the per-CU rate the GEMM sustains: ~24 B/clk with 4 issuing waves, ~30 with
// 8); each tile adds a fixed prologue/epilogue cost. Tiles run in rounds over
// the CUs, which carries the wave-quantisation loss the zwzgs.cn DeepGEMM
// page describes ("non-standard block sizes": a tile count just above a
// multiple of the SM count leaves most of the last round idle); partial tiles
// carry their padding. Contiguous tiles must not straddle an aligned 128-row
// expert block.
constexpr double kTileFixedCycles = 4000.0;
int pick_tile(int layout, int M, int N, int K, int G, int cus) {
  const int forced = g_forced_tile.load(std::memory_order_relaxed);
  if (forced >= 0) return forced;
  int best = -1;
  double best_cost = 0.0;
  const double kblocks = K / 128;
  for (int i = 0; i < kNumTiles; ++i) {
    const Tile& t = kTiles[i];
    if (layout == FG_LAYOUT_CONTIGUOUS && 128 % t.bm != 0) continue;
    const long tiles = count_tiles(layout, M, N, G, t);
    const long rounds = (tiles + cus - 1) / cus;
    const double t_mfma = (double)t.bm * t.bn * 256.0 / (8192.0 * t.eff);
    const double t_mem = (double)(t.bm + t.bn) * 128.0 / (t.waves >= 8 ? 30.0 : 24.0);
    const double cost = (double)rounds * (kblocks * (t_mfma > t_mem ? t_mfma : t_mem) + kTileFixedCycles);
    if (best < 0 || cost < best_cost * (1.0 - 1e-9)) {
      best = i;
      best_cost = cost;
    }
  }
  return best;
}

template <int LAYOUT, bool POW2>
hipError_t launch_layout(int tile, const Params& p, int grid, hipStream_t s) {
  switch (tile) {
    case 0: hipLaunchKernelGGL((fg::fp8_bs_gemm<LAYOUT, Cfg0, POW2>), dim3(grid), dim3(Cfg0::THREADS), 0, s, p); break;
    case 1: hipLaunchKernelGGL((fg::fp8_bs_gemm<LAYOUT, Cfg1, POW2>), dim3(grid), dim3(Cfg1::THREADS), 0, s, p); break;
    case 2: hipLaunchKernelGGL((fg::fp8_bs_gemm<LAYOUT, Cfg2, POW2>), dim3(grid), dim3(Cfg2::THREADS), 0, s, p); break;
    case 3: hipLaunchKernelGGL((fg::fp8_bs_gemm<LAYOUT, Cfg3, POW2>), dim3(grid), dim3(Cfg3::THREADS), 0, s, p); break;
    case 4: hipLaunchKernelGGL((fg::fp8_bs_gemm<LAYOUT, Cfg4, POW2>), dim3(grid), dim3(Cfg4::THREADS), 0, s, p); break;
    case 5: hipLaunchKernelGGL((fg::fp8_bs_gemm<LAYOUT, Cfg5, POW2>), dim3(grid), dim3(Cfg5::THREADS), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool POW2>
hipError_t launch(int layout, int tile, const Params& p, int grid, hipStream_t s) {
  switch (layout) {
    case FG_LAYOUT_DENSE: return launch_layout<fg::kDense, POW2>(tile, p, grid, s);
    case FG_LAYOUT_CONTIGUOUS: return launch_layout<fg::kContiguous, POW2>(tile, p, grid, s);
    default: return launch_layout<fg::kMasked, POW2>(tile, p, grid, s);
  }
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// pow2: every sa and sb is a power of two, applied by the matrix core as an
// E8M0 block scale (no separate promotion)
int run(int layout, const void* A, const float* sa, const void* B, const float* sb, void* D,
        const int32_t* m_indices, const int32_t* masked_m, int M, int N, int K, int G,
        hipStream_t stream, bool pow2) {
  if (M < 0 || N < 0 || K < 128 || (K % 128) != 0 || (N % 128) != 0) return FG_EINVAL;
  if (layout != FG_LAYOUT_DENSE && G < 1) return FG_EINVAL;
  if (M == 0 || N == 0) return FG_OK;
  if (!A || !sa || !B || !sb || !D) return FG_EINVAL;
  if (layout == FG_LAYOUT_CONTIGUOUS && !m_indices) return FG_EINVAL;
  if (layout == FG_LAYOUT_MASKED && !masked_m) return FG_EINVAL;
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || !aligned(sa, 4) || !aligned(sb, 4))
    return FG_EINVAL;
  if (m_indices && !aligned(m_indices, 4)) return FG_EINVAL;
  if (masked_m && !aligned(masked_m, 4)) return FG_EINVAL;
  // the kernels address one expert's A or B with 32-bit byte offsets
  if ((long long)M * K > 0x7fffffffLL || (long long)N * K > 0x7fffffffLL) return FG_EINVAL;

  int cus = 0;
  const int st = current_device(&cus);
  if (st != FG_OK) return st;

  const int ti = pick_tile(layout, M, N, K, G, cus);
  const Tile& t = kTiles[ti];
  // contiguous tiles must not straddle an aligned 128-row expert block
  if (layout == FG_LAYOUT_CONTIGUOUS && 128 % t.bm != 0) return FG_EINVAL;
  Params p;
  p.A = static_cast<const uint8_t*>(A);
  p.sa = sa;
  p.B = static_cast<const uint8_t*>(B);
  p.sb = sb;
  p.D = static_cast<uint16_t*>(D);
  p.m_indices = m_indices;
  p.masked_m = masked_m;
  p.M = M;
  p.N = N;
  p.K = K;
  p.G = layout == FG_LAYOUT_DENSE ? 1 : G;
  p.KB = K / 128;
  p.tiles_m = ceil_div(M, t.bm);
  p.tiles_n = ceil_div(N, t.bn);
  const long tiles = count_tiles(layout, M, N, p.G, t);
  if (tiles > 0x7fffffffL) return FG_EINVAL;
  const int grid = (int)tiles;

  const hipError_t e = pow2 ? launch<true>(layout, ti, p, grid, stream) : launch<false>(layout, ti, p, grid, stream);
  return e == hipSuccess ? FG_OK : FG_ELAUNCH;
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

int fg_select_config(int layout, int M, int N, int K, int G, int num_cus, int* bm, int* bn,
                     int* grid) {
  if (layout < FG_LAYOUT_DENSE || layout > FG_LAYOUT_MASKED) return FG_EINVAL;
  if (M < 0 || N < 0 || K < 0 || (layout != FG_LAYOUT_DENSE && G < 1)) return FG_EINVAL;
  if (layout == FG_LAYOUT_DENSE) G = 1;
  const int cus = num_cus > 0 ? num_cus : kDefaultCUs;
  const int ti = pick_tile(layout, M, N, K, G, cus);
  if (bm) *bm = kTiles[ti].bm;
  if (bn) *bn = kTiles[ti].bn;
  if (grid) *grid = (int)count_tiles(layout, M, N, G, kTiles[ti]);
  return FG_OK;
}

int fg_force_tile(int bm, int bn) {
  if (bm == 0 && bn == 0) {
    g_forced_tile.store(-1);
    return FG_OK;
  }
  for (int i = 0; i < kNumTiles; ++i) {
    if (kTiles[i].bm == bm && kTiles[i].bn == bn) {
      g_forced_tile.store(i);
      return FG_OK;
    }
  }
  return FG_EINVAL;
}

const char* fg_strerror(int code) {
  switch (code) {
    case FG_OK: return "success";
    case FG_EINVAL: return "invalid argument (null pointer, negative size, K or N not a multiple of 128, K < 128, misaligned pointer, G < 1 or unknown tile)";
    case FG_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case FG_ELAUNCH: return "kernel launch failed";
    case FG_EDEVICE: return "HIP device query failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
