// fg_kernel.hpp -- gfx950 kernel for the FP8 (OCP E4M3) block-scaled GEMM
// D = A . B^T with per-1x128 (A) and per-128x128 (B) fp32 scales and
// two-level FP32 accumulation, in the dense, MoE-contiguous and MoE-masked
// layouts.
//
// Method: the zwzgs.cn page "DeepGEMM: an open-source FP8 GEMM library",
// "Technical details > two-level accumulation": the matrix-core FP8 partial
// sums are accumulated a second time in FP32 on the general-purpose ALUs.
// Here every 128-wide K-block is one v_mfma_f32_16x16x128_f8f6f4 per 16x16
// sub-tile with a zero C operand (a fresh FP32 partial covering exactly one
// scale block), followed by one v_fma_f32 per output element that adds
// partial * (sa * sb) into the master accumulator held in VGPRs. Each MFMA's
// promotion is issued after the next MFMA, so the VALU work overlaps the
// matrix core instead of waiting on it.
//
// Data movement (the pages' "data movement / compute / epilogue" overlap,
// "Technical details > thread specialisation", done the gfx950 way): every
// wave issues direct global->LDS loads (global_load_lds_dwordx4, no VGPR
// staging) for its share of the next K-blocks into an S-stage ring of LDS
// buffers, so there are no producer waves; one workgroup barrier per K-block
// both publishes the next stage and frees the stage just consumed. The
// barrier sits before the last column of MFMAs, so the next K-block's
// fragments are read from LDS while those MFMAs run.
//
// LDS layout of a stage: A tile [BM rows][128 B], B tile [BN rows][128 B],
// then BM activation scales and the weight scales of the tile's 128-column
// blocks (fp32), so every operand of a K-block arrives through the same
// counted DMA stream. A 16-byte chunk c of tile row r is stored
// at chunk position c ^ (r & 7) (XOR swizzle): the 16 rows a quarter-wave
// reads for one chunk index hit distinct bank groups. The swizzle is applied
// by choosing which global chunk each DMA lane fetches, since a DMA lane's LDS
// destination is fixed (lane * 16 bytes after the wave's base).
//
// Operand roles. The MFMA's first operand is fed with rows of B (output
// columns n), its second with rows of A (output rows m). The 16x16 result then
// gives each lane four consecutive n for a single m, so a lane needs one
// activation scale per sub-tile row and its four results form one 8-byte bf16
// store.
//
// K order inside a fragment. The hardware sums a 128-long dot product; which
// lane/byte holds which k does not change the sum as long as both operands use
// the same placement. Lane l (row l % 16, quarter q = l / 16) holds bytes
// [16q, 16q+16) and [64+16q, 64+16q+16) of its row's K-block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg {

typedef int   i32x4 __attribute__((ext_vector_type(4)));
typedef int   i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(1))) const uint8_t gbl_u8;
typedef __attribute__((address_space(3))) const float lds_f32;

enum Layout { kDense = 0, kContiguous = 1, kMasked = 2 };

constexpr int kKBlock = 128;   // scale block along K (elements == bytes)
constexpr int kXCDs = 8;       // MI355X: workgroups go round-robin to 8 XCDs
constexpr int kGroupM = 4;     // m-blocks per rasterisation group

struct Params {
  const uint8_t* A;       // E4M3 [rows][K] (masked: [G][M][K])
  const float* sa;        // [K/128][rows] (masked: [G][K/128][M])
  const uint8_t* B;       // E4M3 [N][K] (grouped: [G][N][K])
  const float* sb;        // [N/128][K/128] (grouped: [G][N/128][K/128])
  uint16_t* D;            // bf16 bits [rows][N] (masked: [G][M][N])
  const int32_t* m_indices;  // contiguous: expert per row, -1 = padding
  const int32_t* masked_m;   // masked: valid rows per expert
  int M;                  // rows (dense/contiguous) or M_max (masked)
  int N, K, G;
  int KB;                 // K / 128
  int tiles_m, tiles_n;   // tile grid of one group
};

// Compile-time tile configuration.
//   BM x BN   output tile per workgroup
//   WGM x WGN waves per workgroup (each wave owns a (BM/WGM) x (BN/WGN) block)
//   STAGES    depth of the LDS ring
//   STRADDLE  a wave's columns may span two 128-wide scale blocks of B
template <int BM_, int BN_, int WGM_, int WGN_, int STAGES_, bool STRADDLE_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, STAGES = STAGES_;
  static constexpr bool STRADDLE = STRADDLE_;
  static constexpr int W = WGM * WGN;
  static constexpr int THREADS = 64 * W;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 16, TN = WN / 16;
  // DMA instructions per wave per stage; padding slots load a clamped row.
  static constexpr int A_INSTR = (BM * 8 + 64 * W - 1) / (64 * W);
  static constexpr int B_INSTR = (BN * 8 + 64 * W - 1) / (64 * W);
  static constexpr int SB_SLOTS = 4;   // weight scales of the tile's (up to 3) 128-column blocks
  static constexpr int SA_INSTR = (BM + SB_SLOTS + 64 * W - 1) / (64 * W);
  static constexpr int A_BYTES = A_INSTR * W * 1024;
  static constexpr int B_BYTES = B_INSTR * W * 1024;
  static constexpr int SA_BYTES = SA_INSTR * W * 256;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
  static constexpr int ROWB = BN * 2 + 16;   // staged bf16 output row (+16 B against bank conflicts)
  static constexpr int LDS_BYTES = RING_BYTES > BM * ROWB ? RING_BYTES : BM * ROWB;
  static constexpr int DMA_PER_STAGE = A_INSTR + B_INSTR + SA_INSTR;
  static_assert(WM % 16 == 0 && WN % 16 == 0 && TM >= 1 && TN >= 1, "wave tile must be 16-aligned");
  static_assert(BM % WGM == 0 && BN % WGN == 0, "waves must split the tile evenly");
  static_assert(STAGES >= 2, "need at least double buffering");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS ring exceeds 160 KB");
  static_assert(WN <= 128, "a wave's columns may touch at most two scale blocks");
  static_assert(TN >= 2, "the B-fragment ring needs at least two sub-tile columns per wave");
  static_assert(STRADDLE || 128 % WN == 0, "non-straddling waves must tile the 128-wide scale blocks");
};

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kKBlock + ((chunk ^ (row & 7)) << 4);
}

// Wait until at most N of this wave's vector-memory operations are in flight
// (the LDS-DMA loads complete in issue order), then stop the compiler from
// moving LDS accesses across the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Target builtins live in __device__ helpers: the lambdas below are
// host+device, and a gfx950 builtin inside one would make the host-side
// instantiation of the kernel (its launch stub) silently fail.
//
// The LDS-DMA loads are issued through inline asm. When the compiler sees an
// LDS-DMA in flight it can no longer count LDS reads precisely and waits for
// all of them (lgkmcnt(0)) before every fragment use; hidden from it, the DMA
// is tracked only by this kernel's explicit vmcnt waits, and the compiler's
// lgkmcnt waits cover exactly the fragment reads. M0 holds the wave-uniform
// LDS destination; one wait state separates its write from the DMA.
__device__ __forceinline__ void dma16(const uint8_t* sbase, uint32_t voff, lds_u8* dst) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"((uint32_t)(uintptr_t)dst) : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* addr, lds_u8* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(addr), "s"((uint32_t)(uintptr_t)dst) : "memory");
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// Keep one pipeline step's order -- the MFMA first, then its LDS reads, then
// the VALU promotion of the previous partial -- and let nothing cross steps.
__device__ __forceinline__ void step_fence() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ i32x8 frag_read(const lds_u8* tile, int row, int lq) {
  const i32x4 lo = *(const __attribute__((address_space(3))) i32x4*)(tile + swz(row, lq));
  const i32x4 hi = *(const __attribute__((address_space(3))) i32x4*)(tile + swz(row, lq + 4));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ f32x4 mfma_e4m3(const i32x8& b_rows, const i32x8& a_rows) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // cbsz = blgp = 0 selects E4M3 for both operands; C = 0 starts a fresh partial
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b_rows, a_rows, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ void promote(f32x4& acc, const f32x4& part, float s) {
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(part[r], s, acc[r]);
}

template <int LAYOUT, class T>
__global__ __launch_bounds__(T::THREADS) void fp8_bs_gemm(Params p) {
  constexpr int BM = T::BM, BN = T::BN, W = T::W, WM = T::WM, WN = T::WN;
  constexpr int TM = T::TM, TN = T::TN, S = T::STAGES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
  __shared__ int s_group;
  lds_u8* const lds = (lds_u8*)smem;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = uniform(t >> 6);
  const int wm = wave / T::WGN, wn = wave % T::WGN;
  const int lr = lane & 15, lq = lane >> 4;

  // ---- workgroup -> tile. Consecutive tile ids are placed on the same XCD
  // (workgroups are dealt round-robin to the XCDs), then tiles are walked in
  // groups of kGroupM m-blocks so the tiles resident on one XCD share A rows
  // and B columns in its L2.
  int tile;
  {
    const int b = blockIdx.x, nwg = gridDim.x;
    const int x = b % kXCDs, l = b / kXCDs;
    const int per = nwg / kXCDs, rem = nwg % kXCDs;
    tile = x * per + (x < rem ? x : rem) + l;
  }
  int g = 0;
  if (LAYOUT == kMasked) {
    const int per = p.tiles_m * p.tiles_n;
    g = tile / per;
    tile -= g * per;
  }
  int mb, nbk;
  {
    const int span = kGroupM * p.tiles_n;
    const int grp = tile / span;
    const int first = grp * kGroupM;
    const int gsz = min(kGroupM, p.tiles_m - first);
    const int in = tile - grp * span;
    mb = first + in % gsz;
    nbk = in / gsz;
  }
  const int m0 = mb * BM, n0 = nbk * BN;

  int rows_valid = p.M;  // rows of this slab that have an output
  if (LAYOUT == kMasked) {
    int mm = p.masked_m[g];
    mm = mm < 0 ? 0 : (mm > p.M ? p.M : mm);
    if (m0 >= mm) return;  // uniform over the workgroup
    rows_valid = mm;
  }
  if (LAYOUT == kContiguous) {
    if (t == 0) s_group = -1;
    __syncthreads();
    if (t < BM && m0 + t < p.M) {
      const int id = p.m_indices[m0 + t];
      if (id >= 0 && id < p.G) atomicMax(&s_group, id);
    }
    __syncthreads();
    g = s_group;
    if (g < 0) return;  // all-padding block
  }
  g = uniform(g);

  const int K = p.K, KB = p.KB, M = p.M;
  const uint8_t* Ag = p.A + (LAYOUT == kMasked ? (size_t)g * M * K : 0);
  const float* sag = p.sa + (LAYOUT == kMasked ? (size_t)g * KB * M : 0);
  const uint8_t* Bg = p.B + (LAYOUT != kDense ? (size_t)g * p.N * K : 0);
  const float* sbg = p.sb + (LAYOUT != kDense ? (size_t)g * (p.N / 128) * KB : 0);
  uint16_t* Dg = p.D + (LAYOUT == kMasked ? (size_t)g * M * p.N : 0);

  // ---- per-lane DMA sources (byte offsets within one K-block column).
  // Slot s of a region is the 16-byte LDS chunk s; it holds row s/8, chunk
  // position s%8, i.e. global chunk (s%8) ^ (row%8). Rows past the tile
  // (padding slots) and past the matrix are clamped to a valid row.
  uint32_t a_off[T::A_INSTR], b_off[T::B_INSTR], sa_off[T::SA_INSTR];
#pragma unroll
  for (int q = 0; q < T::A_INSTR; ++q) {
    const int slot = (q * W + wave) * 64 + lane;
    const int row = slot >> 3, chunk = (slot & 7) ^ (row & 7);
    const int m = min(m0 + min(row, BM - 1), M - 1);
    a_off[q] = (uint32_t)m * (uint32_t)K + chunk * 16;
  }
#pragma unroll
  for (int q = 0; q < T::B_INSTR; ++q) {
    const int slot = (q * W + wave) * 64 + lane;
    const int row = slot >> 3, chunk = (slot & 7) ^ (row & 7);
    const int n = min(n0 + min(row, BN - 1), p.N - 1);
    b_off[q] = (uint32_t)n * (uint32_t)K + chunk * 16;
  }
  // scale slots: [0, BM) activation rows, [BM, BM+4) weight blocks from the
  // tile's first 128-column block on (clamped), the rest duplicate a row
  const int nb_tile = n0 >> 7;
  bool sa_is_sb[T::SA_INSTR];
#pragma unroll
  for (int q = 0; q < T::SA_INSTR; ++q) {
    const int idx = (q * W + wave) * 64 + lane;
    sa_is_sb[q] = idx >= BM && idx < BM + T::SB_SLOTS;
    sa_off[q] = sa_is_sb[q] ? (uint32_t)min(nb_tile + idx - BM, p.N / 128 - 1) * (uint32_t)KB * 4u
                            : (uint32_t)min(m0 + min(idx, BM - 1), M - 1) * 4u;
  }

  // One DMA instruction d (0 .. DMA_PER_STAGE-1) of K-block kb into a stage:
  // A chunks first, then B chunks, then the scale slots.
  auto issue_one = [&](int kb, int stage, int d) {
    lds_u8* const base = lds + stage * T::STAGE_BYTES;
    if (d < T::A_INSTR) {
      dma16(Ag + (size_t)kb * kKBlock, a_off[d], base + (d * W + wave) * 1024);
    } else if (d < T::A_INSTR + T::B_INSTR) {
      const int q = d - T::A_INSTR;
      dma16(Bg + (size_t)kb * kKBlock, b_off[q], base + T::A_BYTES + (q * W + wave) * 1024);
    } else {
      const int q = d - T::A_INSTR - T::B_INSTR;
      const uint8_t* const src = sa_is_sb[q] ? (const uint8_t*)(sbg + kb) : (const uint8_t*)(sag + (size_t)kb * M);
      dma4(src + sa_off[q], base + T::A_BYTES + T::B_BYTES + (q * W + wave) * 256);
    }
  };

  // ---- scale blocks of B covered by this wave's columns (at most two)
  const int wn0 = n0 + wn * WN;
  const int nb_lo = uniform(min(wn0 >> 7, p.N / 128 - 1));
  const int nb_hi = uniform(min(nb_lo + 1, p.N / 128 - 1));
  // first sub-tile column whose scale block is nb_hi
  const int j_switch = T::STRADDLE ? uniform(((nb_lo + 1) * 128 - wn0) >> 4) : TN;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- DMA schedule. K-block x lands in stage x % S.
  //
  // S >= 3: x's stage is freed at the barrier of K-block x-S and must be
  // complete at the barrier of K-block x-1. Its instructions are spread one per
  // pipeline step over the K-block after the freeing barrier ("head" after that
  // barrier, "tail" before the next one), leaving a further full K-block for
  // the loads to land.
  //
  // S == 2: each K-block takes two barriers. The A fragments are held in
  // registers for the whole K-block, so a stage's A half is free once column 0
  // has consumed them: a first barrier after column 0 releases it, and the A
  // half of K-block kb+2 is spread over the rest of K-block kb (almost two
  // K-blocks to land). The B half (and the scales) is freed by the main
  // barrier before column TN-2 and spread over the last two columns.
  //
  // Spreading keeps the MFMA pipe fed instead of stalling every wave on a
  // burst of DMA issue. K-block indices past the end are clamped (those repeat
  // loads hit L2), which keeps every wave's DMA count a compile-time constant
  // for the vmcnt waits.
  constexpr int STEPS = TM * TN;
  constexpr int JB = TN - 2;          // the main barrier precedes sub-tile column JB
  constexpr int PRE = JB * TM;        // pipeline steps before it
  constexpr int POST = STEPS - PRE;   // pipeline steps after it
  constexpr int D = T::DMA_PER_STAGE;
  constexpr bool SPLIT = S == 2;
  constexpr int NA = T::A_INSTR, NBS = D - T::A_INSTR;
  // pipeline step at which DMA instruction d is issued (S >= 3: position in the
  // head/tail window of STEPS steps that starts after the freeing barrier)
  auto dma_slot = [](int d) constexpr {
    if (SPLIT) return d < NA ? TM + d * (STEPS - TM) / NA : PRE + (d - NA) * POST / NBS;
    return d * STEPS / D;
  };
  constexpr int N_HEAD = [] {   // S >= 3: instructions issued after the freeing barrier
    int n = 0;
    for (int d = 0; d < D; ++d) n += d * STEPS / D < POST;
    return n;
  }();
  constexpr int N_EARLY = [] {  // S == 2: A instructions issued before the main barrier
    int n = 0;
    if (SPLIT)
      for (int d = 0; d < NA; ++d) n += TM + d * (STEPS - TM) / NA < PRE;
    return n;
  }();
  static_assert((S - 2) * D + N_HEAD < 64 && D + N_EARLY < 64, "vmcnt counter range");

  // ---- prologue: wait for K-block 0 with the later ones in flight
  //   S >= 3: K-blocks 1 .. S-2 and the head of K-block S-1
  //   S == 2: K-block 1
#pragma unroll
  for (int x = 0; x < S - 1; ++x)
#pragma unroll
    for (int d = 0; d < D; ++d) issue_one(min(x, KB - 1), x, d);
  if (SPLIT) {
#pragma unroll
    for (int d = 0; d < D; ++d) issue_one(min(1, KB - 1), 1, d);
    wait_vm<D>();
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (dma_slot(d) < POST) issue_one(min(S - 1, KB - 1), S - 1, d);
    wait_vm<(S - 2) * D + N_HEAD>();
  }
  block_barrier();

  // B fragments live in a ring of three: column j+2 is read while column j
  // computes. A fragments are held for the whole K-block.
  i32x8 fa[TM], fbr[3];
  float s_lo[TM], s_hi[TM];
  // activation scales of this lane's rows and the weight scale(s) of the
  // wave's columns, all from the stage's LDS copy (sb at a wave-uniform address)
  auto scale_read = [&](const lds_u8* st, float (&a)[TM], float& b0, float& b1) {
    lds_f32* sas = (lds_f32*)(st + T::A_BYTES + T::B_BYTES);
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = sas[wm * WM + i * 16 + lr];
    b0 = sas[BM + nb_lo - nb_tile];
    b1 = sas[BM + nb_hi - nb_tile];
  };
  auto set_scales = [&](const float (&a)[TM], float b0, float b1) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      s_lo[i] = a[i] * b0;
      s_hi[i] = T::STRADDLE ? a[i] * b1 : 0.f;
    }
  };
#pragma unroll
  for (int i = 0; i < TM; ++i) fa[i] = frag_read(lds, wm * WM + i * 16 + lr, lq);
  fbr[0] = frag_read(lds + T::A_BYTES, wn * WN + lr, lq);
  if (TN > 1) fbr[1] = frag_read(lds + T::A_BYTES, wn * WN + 16 + lr, lq);
  {
    float a0[TM], b0, b1;
    scale_read(lds, a0, b0, b1);
    set_scales(a0, b0, b1);
  }

  // One K-block: TM x TN MFMAs in column order. Step u issues MFMA u and then
  // promotes MFMA u-1 (complete by then), so the FMAs run under the next
  // MFMA. The barrier sits before column JB = TN-2, when every read of the
  // current stage has been issued; after it the next stage's first two B
  // fragments and its scales are read into free ring slots, and each fa[i] is
  // replaced by the next stage's fragment right after its last MFMA.
  int stage = 0;
  for (int kb = 0; kb < KB; ++kb) {
    const int nstage = stage + 1 == S ? 0 : stage + 1;
    const int pstage = stage == 0 ? S - 1 : stage - 1;   // stage of K-block kb+S-1
    const int kb_head = min(kb + S, KB - 1), kb_tail = min(kb + S - 1, KB - 1);
    const lds_u8* cur = lds + stage * T::STAGE_BYTES;
    const lds_u8* nxt = lds + nstage * T::STAGE_BYTES;
    f32x4 part[2];
    float sa_next[TM], sb_next0 = 0.f, sb_next1 = 0.f;
#pragma unroll
    for (int u = 0; u < STEPS; ++u) {
      const int j = u / TM, i = u % TM;
      if (SPLIT && u == TM && TM < PRE) block_barrier();   // A half of this stage is free
      if (u == PRE) {
        // every read of the current stage has been issued; the next stage (and,
        // for S == 2, every DMA older than this K-block's early A loads) is in
        wait_lgkm0();
        wait_vm<(S - 2) * D + N_EARLY>();
        block_barrier();
        scale_read(nxt, sa_next, sb_next0, sb_next1);
      }
      part[u & 1] = mfma_e4m3(fbr[j % 3], fa[i]);
      if (i == 0) {
        // column j+2 of this stage, or (past the end) column j+2-TN of the next
        const int jn = j + 2;
        if (jn < TN) fbr[jn % 3] = frag_read(cur + T::A_BYTES, wn * WN + jn * 16 + lr, lq);
        else fbr[jn % 3] = frag_read(nxt + T::A_BYTES, wn * WN + (jn - TN) * 16 + lr, lq);
      }
      if (j == TN - 1) fa[i] = frag_read(nxt, wm * WM + i * 16 + lr, lq);
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (SPLIT) {
          if (dma_slot(d) == u) issue_one(kb_head, stage, d);   // K-block kb+2 into this stage
        } else {
          if (u >= PRE && dma_slot(d) == u - PRE) issue_one(kb_head, stage, d);
          if (u < PRE && dma_slot(d) == POST + u) issue_one(kb_tail, pstage, d);
        }
      }
      if (u > 0) {
        const int pj = (u - 1) / TM, pi = (u - 1) % TM;
        const float s = (!T::STRADDLE || pj < j_switch) ? s_lo[pi] : s_hi[pi];
        promote(acc[pi][pj], part[(u - 1) & 1], s);
      }
      step_fence();
    }
    {
      const float s = (!T::STRADDLE || TN - 1 < j_switch) ? s_lo[TM - 1] : s_hi[TM - 1];
      promote(acc[TM - 1][TN - 1], part[(STEPS - 1) & 1], s);
    }
    // the next stage's first columns sit in ring slots TN % 3 and (TN+1) % 3
    if (TN % 3 != 0) {
      const i32x8 c0 = fbr[TN % 3];
      const i32x8 c1 = fbr[(TN + 1) % 3];
      fbr[0] = c0;
      fbr[1] = c1;
    }
    set_scales(sa_next, sb_next0, sb_next1);
    stage = nstage;
  }

  // ---- epilogue: bf16 RNE, staged through LDS so that every global store is
  // a full 16-byte piece of a contiguous output row
  wait_vm<0>();          // the clamped tail DMAs must land before LDS is reused
  wait_lgkm0();
  block_barrier();
  constexpr int ROWB = T::ROWB;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int ml = wm * WM + i * 16 + lr;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int nl = wn * WN + j * 16 + 4 * lq;
      const uint32_t lo = bf16_rne_bits(acc[i][j][0]) | (bf16_rne_bits(acc[i][j][1]) << 16);
      const uint32_t hi = bf16_rne_bits(acc[i][j][2]) | (bf16_rne_bits(acc[i][j][3]) << 16);
      *(__attribute__((address_space(3))) u32x2*)(lds + ml * ROWB + nl * 2) = u32x2{lo, hi};
    }
  }
  wait_lgkm0();
  block_barrier();
  constexpr int CPR = BN * 2 / 16;   // 16-byte pieces per output row
#pragma unroll 4
  for (int c = t; c < BM * CPR; c += T::THREADS) {
    const int row = c / CPR, cc = c - row * CPR;
    const int m = m0 + row, n = n0 + cc * 8;
    bool ok = m < rows_valid && n < p.N;
    if (LAYOUT == kContiguous && ok) ok = p.m_indices[m] == g;
    if (ok) {
      const i32x4 v = *(const __attribute__((address_space(3))) i32x4*)(lds + row * ROWB + cc * 16);
      *(i32x4*)(Dg + (size_t)m * p.N + n) = v;
    }
  }
}

}  // namespace fg
