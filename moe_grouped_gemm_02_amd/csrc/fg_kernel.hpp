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
// promotion is issued a few MFMAs after it, so the VALU work overlaps the
// matrix core instead of waiting on its result.
//
// Data movement (the pages' "data movement / compute / epilogue" overlap,
// "Technical details > thread specialisation", done the gfx950 way): every
// wave issues direct global->LDS loads (buffer_load ... lds, no VGPR staging)
// for its share of later K-blocks, so there are no producer waves. A tiles
// and scales go into one ring of LDS stages, B tiles into a second ring that
// may run further ahead (B streams from HBM; A is re-read from L2 by every
// N-tile). One workgroup barrier per K-block both publishes the next stage
// and frees the stages just consumed (two with a two-stage ring, which frees
// its A half earlier). The barrier sits before the last columns of MFMAs, so
// the next K-block's fragments are read from LDS while those MFMAs run. A
// workgroup may compute several tiles one after another (gemm_tiles); each
// tile addresses its operands through buffer resources of its own.
//
// LDS layout: the scale blocks of all A stages (BM activation scales and the
// weight scales of the tile's 128-column blocks, fp32), then the A tiles
// [BM rows][128 B], then the B tiles [BN rows][128 B]. A 16-byte chunk c of
// tile row r is stored at chunk position c ^ (r & 7) (XOR swizzle): the 16
// rows a quarter-wave reads for one chunk index hit distinct bank groups. The
// swizzle is applied by choosing which global chunk each DMA lane fetches,
// since a DMA lane's LDS destination is fixed (lane * 16 bytes after M0).
//
// Operand roles. The MFMA's first operand is fed with rows of B (output
// columns n), its second with rows of A (output rows m). The 16x16 result then
// gives each lane four consecutive n for a single m, so a lane needs one
// activation scale per sub-tile row. Loading the B rows of two neighbouring
// sub-tiles in pair_column order makes a lane's eight results of the pair
// eight consecutive columns: one 16-byte bf16 store straight from registers.
//
// Fused epilogue (EPI = kEpiSwigluQuant), for an MoE expert's first
// projection whose weight interleaves gate and up rows every 128: the 2kiu.com
// explainer, section 7, names fusing the activation around a GEMM as the way
// to save its memory round trips. A 256-column tile holds gate block j and up
// block j for its rows; the waves holding the gate half stage silu(gate) in
// LDS, the up waves form act = silu(gate) * up in FP32 from it and their
// accumulators, and a 16-lane group per row then takes the row's amax over its
// 128 columns, the 1x128 scale and 8 codes per lane -- the next GEMM's A operand and its
// K-block-major scales, with no bf16 D written or re-read.
//
// Power-of-two variant (POW2). The 2kiu.com DeepGEMM explainer, section 7,
// points to MX / micro-scaling formats, whose block scales are powers of two
// (E8M0). gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 applies such a scale per
// lane -- to that lane's row of each operand and its 32-wide K chunk -- inside
// the matrix core and adds the result to C. When every sa and sb is a power
// of two, the scale of a K-block is therefore taken by the MFMA itself: each
// 16x16 sub-tile accumulates straight into its master accumulator (C = acc),
// and the partial ring and the VALU promotion disappear. The scales arrive in
// the same fp32 layout; the exponent field of a normal fp32 power of two is
// its E8M0 code (bias 127 in both).
//
// K order inside a fragment. The hardware sums a 128-long dot product; which
// lane/byte holds which k does not change the sum as long as both operands use
// the same placement. Lane l (row l % 16, quarter q = l / 16) holds bytes
// [16q, 16q+16) and [64+16q, 64+16q+16) of its row's K-block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fg_e4m3.hpp"

namespace fg {

typedef int   i32x4 __attribute__((ext_vector_type(4)));
typedef int   i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(1))) const uint8_t gbl_u8;
typedef __attribute__((address_space(3))) const float lds_f32;

enum Layout { kDense = 0, kContiguous = 1, kMasked = 2 };
// What the epilogue writes: D in bf16, or the SiLU-gated activation of D
// re-quantised to E4M3 with 1x128 scales (gate/up interleaved every 128 columns)
enum Epilogue { kEpiBf16 = 0, kEpiSwigluQuant = 1 };

constexpr int kKBlock = 128;   // scale block along K (elements == bytes)
constexpr int kXCDs = 8;       // MI355X: workgroups go round-robin to 8 XCDs
constexpr int kGroupM = 4;     // m-blocks per rasterisation group
// A DMA lane offset past every operand's buffer (the host keeps one expert's
// A and B below 2^31 bytes): the buffer range check turns the load into zeros.
constexpr uint32_t kNoRow = 0x80000000u;

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
  // dense on two tile shapes (fp8_bs_gemm_split): columns [0, n_split) on the
  // wide tiles, tiles_a of them; the rest on the narrow tiles
  int n_split, tiles_a;
  // kEpiSwigluQuant outputs (I = N / 2 columns): codes [rows][I] (masked
  // [G][M][I]), scales [I/128][rows] (masked [G][I/128][M]), and optionally
  // the fp32 activation [rows][I] (masked [G][M][I]; null: not written)
  uint8_t* Q;
  float* sq;
  float* act;
};

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }
constexpr int lcm_c(int a, int b) { return a / gcd_c(a, b) * b; }

// Compile-time tile configuration.
//   BM x BN   output tile per workgroup
//   WGM x WGN waves per workgroup (each wave owns a (BM/WGM) x (BN/WGN) block)
//   STAGES    depth of the LDS ring of B tiles
//   ASTAGES   depth of the LDS ring of A tiles and scales (<= STAGES): the A
//             operand is re-read from L2 by every N-tile and needs less
//             buffering than B, which streams from HBM
//   STRADDLE  a wave's columns may span two 128-wide scale blocks of B
//   PD        B fragments are read PD sub-tile columns ahead of their MFMAs
//             (a register ring of PD+1 fragments)
//   FA2       the next K-block's A fragments are read into a second register
//             set right after the barrier instead of after each one's last use
//   PL        each MFMA's partial is promoted PL MFMAs after it was issued
//             (a ring of PL+1 partials, slot = MFMA number modulo PL+1)
template <int BM_, int BN_, int WGM_, int WGN_, int STAGES_, bool STRADDLE_, int PD_ = 2,
          bool FA2_ = false, int PL_ = 1, int ASTAGES_ = STAGES_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_, STAGES = STAGES_;
  static constexpr int ASTAGES = ASTAGES_;
  static constexpr bool STRADDLE = STRADDLE_;
  static constexpr int PD = PD_, RING = PD_ + 1;
  static constexpr bool FA2 = FA2_;
  static constexpr int PL = PL_, PARTS = PL_ + 1;
  static constexpr int W = WGM * WGN;
  static constexpr int THREADS = 64 * W;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int TM = WM / 16, TN = WN / 16;
  // DMA instructions per wave per stage (16 bytes per lane); padding slots
  // load a clamped row.
  static constexpr int A_INSTR = (BM * 8 + 64 * W - 1) / (64 * W);
  static constexpr int B_INSTR = (BN * 8 + 64 * W - 1) / (64 * W);
  // scale DMAs (4 bytes per lane): one per 64 activation rows plus one for
  // the weight scales of the tile's (up to 3) 128-column blocks, dealt
  // round-robin to the waves; a wave with a spare slot repeats a load
  static constexpr int SC_LOADS = BM / 64 + 1;
  static constexpr int SC_INSTR = (SC_LOADS + W - 1) / W;
  static constexpr int A_BYTES = A_INSTR * W * 1024;
  static constexpr int B_BYTES = B_INSTR * W * 1024;
  static constexpr int SC_BYTES = BM * 4 + 256;
  // LDS rings: the scale blocks of all A stages, then the A tiles, then the B
  // tiles (scale reads then always fall within the first 64 KB)
  static constexpr int SC_BASE = 0;
  static constexpr int A_BASE = ASTAGES * SC_BYTES;
  static constexpr int B_BASE = A_BASE + ASTAGES * A_BYTES;
  static constexpr int RING_BYTES = B_BASE + STAGES * B_BYTES;
  static constexpr int ROWB = BN * 2 + 16;   // staged bf16 output row (+16 B against bank conflicts)
  static constexpr int LDS_BYTES = RING_BYTES > BM * ROWB ? RING_BYTES : BM * ROWB;
  // DMA instructions per wave per K-block, in the order A chunks, scale loads,
  // B chunks
  static constexpr int DMA_PER_STAGE = A_INSTR + B_INSTR + SC_INSTR;
  // K-blocks per main-loop iteration: every per-K-block choice (ring stage,
  // B-ring slots, A-fragment set, scale set) repeats with this period, so each
  // copy of the K-block body works with compile-time registers and offsets
  static constexpr int UNROLL =
      lcm_c(lcm_c(lcm_c(lcm_c(STAGES, ASTAGES), RING / gcd_c(TN, RING)), PARTS / gcd_c(TM * TN, PARTS)), 2);
  static_assert(WM % 16 == 0 && WN % 16 == 0 && TM >= 1 && TN >= 1, "wave tile must be 16-aligned");
  static_assert(BM % WGM == 0 && BN % WGN == 0, "waves must split the tile evenly");
  static_assert(BM % 64 == 0, "activation scales are loaded 64 rows at a time");
  static_assert(ASTAGES >= 2 && ASTAGES <= STAGES, "need at least double buffering, A ring no deeper than B");
  static_assert(STAGES != 2 || ASTAGES == 2, "the two-stage schedule uses one ring depth");
  // a wave never has more loads in flight than the 6-bit vmcnt counter holds
  static_assert(STAGES * DMA_PER_STAGE <= 63, "too many DMA instructions in flight per wave");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS ring exceeds 160 KB");
  static_assert(WN <= 128, "a wave's columns may touch at most two scale blocks");
  static_assert(PD >= 1 && PD <= TN - 1, "prefetch distance must leave the barrier inside the K-block");
  static_assert(PL >= 1 && PL < TM * TN, "promotion lag must stay within one K-block");
  static_assert(STRADDLE || 128 % WN == 0, "non-straddling waves must tile the 128-wide scale blocks");
};

// Pipeline-step schedule of one K-block (see the kernel for its meaning).
template <class T>
struct Sched {
  static constexpr int STEPS = T::TM * T::TN;
  static constexpr int JB = T::TN - T::PD;     // the main barrier precedes sub-tile column JB
  static constexpr int PRE = JB * T::TM;       // pipeline steps before it
  static constexpr int POST = STEPS - PRE;     // pipeline steps after it
  static constexpr int D = T::DMA_PER_STAGE;
  static constexpr bool SPLIT = T::STAGES == 2;
  static constexpr int NA = T::A_INSTR, NBS = D - T::A_INSTR;
  // pipeline step at which DMA instruction d is issued (S >= 3: position in the
  // head/tail window of STEPS steps that starts after the freeing barrier)
  static constexpr int slot(int d) {
    if (SPLIT) return d < NA ? T::TM + d * (STEPS - T::TM) / NA : PRE + (d - NA) * POST / NBS;
    return d * STEPS / D;
  }
  // S >= 3: instructions issued after the freeing barrier
  static constexpr int n_head() {
    int n = 0;
    for (int d = 0; d < D; ++d) n += slot(d) < POST;
    return n;
  }
  // S == 2: A instructions issued before the main barrier
  static constexpr int n_early() {
    int n = 0;
    if (SPLIT)
      for (int d = 0; d < NA; ++d) n += slot(d) < PRE;
    return n;
  }
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
// The LDS-DMA loads (buffer_load ... lds) are issued through inline asm. When
// the compiler sees an LDS-DMA in flight it can no longer count LDS reads
// precisely and waits for all of them (lgkmcnt(0)) before every fragment use;
// hidden from it, the DMA is tracked only by this kernel's explicit vmcnt
// waits, and the compiler's lgkmcnt waits cover exactly the fragment reads.
// Each operand is addressed through a buffer resource (base and byte size; the
// hardware range check keeps every load inside the operand), a loop-invariant
// per-lane offset and one scalar offset per K-block. M0 holds the wave-uniform
// LDS destination; one wait state separates its write from the DMA.
// (A resource is uniform over the wave; readfirstlane states it for the
// compiler, which keeps the resource in scalar registers as the instructions
// need.)
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
               __builtin_amdgcn_readfirstlane((int)((uint32_t)(b >> 32) & 0xffffu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x20000};
}
template <int IMM>
__device__ __forceinline__ void dma16(const i32x4& rs, uint32_t voff, uint32_t soff, uint32_t lds_at) {
  asm volatile("s_add_u32 m0, %3, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "s"(lds_at), "n"(IMM) : "memory", "scc");
}
template <int IMM>
__device__ __forceinline__ void dma4(const i32x4& rs, uint32_t voff, uint32_t soff, uint32_t lds_at) {
  asm volatile("s_add_u32 m0, %3, %4\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "s"(lds_at), "n"(IMM) : "memory", "scc");
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// Keep one pipeline step's order -- the MFMA first, then its LDS reads, then
// the VALU promotion of an earlier partial -- and let nothing cross steps.
__device__ __forceinline__ void step_fence() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// A per-lane LDS byte address with one copy per 64 KB window, hidden from the
// compiler so that an access at base + OFF (OFF a compile-time constant)
// becomes one DS instruction with the 16-bit immediate OFF % 65536.
template <int NWIN>
struct LdsAddr {
  uint32_t w[NWIN];
  __device__ __forceinline__ void init(uint32_t a) {
#pragma unroll
    for (int k = 0; k < NWIN; ++k) {
      w[k] = a + (uint32_t)k * 65536u;
      asm("" : "+v"(w[k]));
    }
  }
  template <int OFF>
  __device__ __forceinline__ const lds_u8* at() const {
    static_assert(OFF >= 0 && (OFF >> 16) < NWIN, "LDS window");
    return (const lds_u8*)(size_t)w[OFF >> 16] + (OFF & 0xffff);
  }
};
template <int OFF, int NWIN>
__device__ __forceinline__ i32x8 frag_at(const LdsAddr<NWIN>& lo, const LdsAddr<NWIN>& hi) {
  const i32x4 a = *(const __attribute__((address_space(3))) i32x4*)lo.template at<OFF>();
  const i32x4 b = *(const __attribute__((address_space(3))) i32x4*)hi.template at<OFF>();
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <int OFF, int NWIN>
__device__ __forceinline__ float f32_at(const LdsAddr<NWIN>& b) {
  return *(const lds_f32*)b.template at<OFF>();
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>)
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <class F, int... I>
__device__ __forceinline__ bool static_any_impl(F&& f, std::integer_sequence<int, I...>) {
  return (f(std::integral_constant<int, I>{}) || ...);
}
// f(0) || f(1) || ... || f(N-1), evaluated in order, stopping at the first true
template <int N, class F>
__device__ __forceinline__ bool static_any(F&& f) {
  return static_any_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ f32x4 mfma_e4m3(const i32x8& b_rows, const i32x8& a_rows) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // cbsz = blgp = 0 selects E4M3 for both operands; C = 0 starts a fresh partial
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b_rows, a_rows, zero, 0, 0, 0, 0, 0, 0);
}

// acc + 2^(eb-127) * 2^(ea-127) * (B rows . A rows): eb scales the lane's row
// of the first operand, ea the lane's row of the second
__device__ __forceinline__ f32x4 mfma_e4m3_pow2(const i32x8& b_rows, const i32x8& a_rows, const f32x4& acc,
                                               int eb, int ea) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b_rows, a_rows, acc, 0, 0, 0, eb, 0, ea);
}

// E8M0 code of a positive normal fp32 power of two: its exponent field
__device__ __forceinline__ int e8m0_of(float s) { return (int)((__float_as_uint(s) >> 23) & 0xffu); }

// x * sigmoid(x) in FP32 with the hardware exp2 and reciprocal (about 1e-6
// relative, far below the error of one E4M3 matrix-core dot product); exp
// overflows to +inf for very negative x, and x * rcp(inf) gives -0
__device__ __forceinline__ float silu_f32(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ void promote(f32x4& acc, const f32x4& part, float s) {
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(part[r], s, acc[r]);
}

// Fused SiLU-gate + E4M3 re-quantisation epilogue (see the header comment).
// acc holds this wave's (BM/WGM) x (BN/WGN) block: sub-tile (i, j) row
// wm*WM + 16i + lr, columns wn*WN + 16j + 4lq + 0..3. Every ring stage is free
// (the caller has drained the DMAs and passed a barrier).
template <int LAYOUT, class T, bool POW2>
__device__ __forceinline__ void swiglu_quant_epilogue(const Params& p, const f32x4 (&acc)[T::TM][T::TN],
                                                      lds_u8* lds, int g, int m0, int n0, int rows_valid,
                                                      int wm, int wn, int lr, int lq, int t) {
  constexpr int BM = T::BM, BN = T::BN, WM = T::WM, WN = T::WN, TM = T::TM, TN = T::TN;
  static_assert(BN == 256 && 128 % WN == 0, "fused epilogue: 256-column tiles, each wave inside one half");
  constexpr int UROW = 128 * 4 + 16;   // fp32 row of one 128-column half (+16 B against bank conflicts)
  static_assert(BM * UROW <= T::LDS_BYTES, "fused epilogue staging exceeds the tile's LDS");
  constexpr int RPP = T::THREADS / 16;   // rows per pass of the quantiser (16 lanes per row)
  static_assert(BM % RPP == 0, "every lane takes the same number of rows");
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

  const int M = p.M, I = p.N / 2;
  const int qc0 = n0 / 2;               // first activation column of this tile
  uint8_t* Qg = p.Q + (LAYOUT == kMasked ? (size_t)g * M * I : 0);
  float* sqg = p.sq + (LAYOUT == kMasked ? (size_t)g * (I / 128) * M : 0);
  float* actg = p.act ? p.act + (LAYOUT == kMasked ? (size_t)g * M * I : 0) : nullptr;
  auto row_ok = [&](int m) {
    bool ok = m < rows_valid;
    if (LAYOUT == kContiguous && ok) ok = p.m_indices[m] == g;
    return ok;
  };

  // Gate waves store silu(gate) in LDS [BM][128] fp32; after the barrier the
  // up waves form act = silu(gate) * up in place (and write act if asked).
  // (Staging the raw up accumulators instead makes the register allocator
  // spill the main loop's DMA offsets in the FP32-scale instantiations.) One
  // sub-tile row of LDS reads at a time in the second pass: hoisting all of
  // them would keep TM*TN more fragments live next to the accumulators.
  const bool up_wave = wn * WN >= 128;
  if (!up_wave) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int ml = wm * WM + i * 16 + lr, c = wn * WN + j * 16 + 4 * lq;
        f32x4 sg;
#pragma unroll
        for (int r = 0; r < 4; ++r) sg[r] = silu_f32(acc[i][j][r]);
        *(lds_f32x4*)(lds + ml * UROW + c * 4) = sg;
      }
  }
  wait_lgkm0();
  block_barrier();
  if (up_wave) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int ml = wm * WM + i * 16 + lr, c = wn * WN - 128 + j * 16 + 4 * lq;
        lds_f32x4* at = (lds_f32x4*)(lds + ml * UROW + c * 4);
        const f32x4 sg = *at;
        f32x4 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = sg[r] * acc[i][j][r];
        *at = a;
        if (actg) {
          const int m = m0 + ml;
          if (row_ok(m)) *(f32x4*)(actg + (size_t)m * I + qc0 + c) = a;
        }
        if (j == TN - 1) __builtin_amdgcn_sched_barrier(0);
      }
  }
  wait_lgkm0();
  block_barrier();
  // quantise: a 16-lane group per row, 8 columns per lane
  const int c8 = (t & 15) * 8;
  const size_t kbq = (size_t)(qc0 / 128);
#pragma unroll 2
  for (int rr = t >> 4; rr < BM; rr += RPP) {
    const lds_f32x4* at = (const lds_f32x4*)(lds + rr * UROW + c8 * 4);
    const f32x4 v0 = at[0], v1 = at[1];
    float am = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) am = fmaxf(am, fmaxf(fabsf(v0[r]), fabsf(v1[r])));
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) am = fmaxf(am, __shfl_xor(am, d, 16));
    float s = block_scale(am);
    uint32_t lo, hi;
    if constexpr (POW2) {
      s = pow2_up(s);
      const float inv = 1.0f / s;   // exact: s is a power of two
      lo = e4m3x4_mul(v0[0], v0[1], v0[2], v0[3], inv);
      hi = e4m3x4_mul(v1[0], v1[1], v1[2], v1[3], inv);
    } else {
      lo = e4m3x4_div(v0[0], v0[1], v0[2], v0[3], s);
      hi = e4m3x4_div(v1[0], v1[1], v1[2], v1[3], s);
    }
    const int m = m0 + rr;
    if (row_ok(m)) {
      *(u32x2*)(Qg + (size_t)m * I + qc0 + c8) = u32x2{lo, hi};
      if ((t & 15) == 0) sqg[kbq * M + m] = s;
    }
  }
}

// Column order of the B tile for the direct-store epilogue. The matrix core
// gives lane (lr, lq) of a 16x16 sub-tile four consecutive columns 4lq..4lq+3;
// loading the 32 weight rows of two neighbouring sub-tiles in the order
// below makes that lane's columns of the pair 8lq..8lq+7 instead, one 16-byte
// piece of an output row. LDS row R of a 32-row group (sub-tile R / 16, its
// row R % 16) holds group column 8 * ((R % 16) / 4) + 4 * (R / 16) + R % 4.
__device__ __forceinline__ int pair_column(int row) {
  const int r = row & 31;
  return (row & ~31) | (((r & 15) >> 2) << 3) | ((r >> 4) << 2) | (r & 3);
}
template <class T, int EPI>
struct DirectStore {
  // bf16 output written from the accumulators as 16-byte row pieces, without
  // staging through LDS (needs whole sub-tile pairs within 32-column groups)
  static constexpr bool value = EPI == kEpiBf16 && T::TN % 2 == 0 && T::WN % 32 == 0;
};

// One output tile: expert g (dense: 0), first row m0, first column n0, and
// the bound on rows that have an output.
struct TileDesc {
  int g, m0, n0, rows_valid;
};

// The tiles a workgroup computes one after another: next(d) fills the next
// tile and returns true, or returns false when the workgroup has no more
// (uniform over the workgroup). Every tile sums K-blocks [kb0, kb0 + nkb)
// (nkb = 0: all of them, K / 128).
//
// With the direct-store epilogue (DirectStore) the LDS ring is free once a
// tile's K loop has ended, so the next tile's first stages are issued before
// this tile's output stores: the loads' latency overlaps the stores, and the
// stores drain while the next tile starts. Otherwise the epilogue stages the
// output through LDS and the next tile starts after it.
template <int LAYOUT, class T, bool POW2, int EPI, class Next>
__device__ __forceinline__ void gemm_tiles(const Params& p, lds_u8* const lds, Next&& next, const int kb0 = 0,
                                           int nkb = 0) {
  constexpr int BM = T::BM, BN = T::BN, W = T::W, WM = T::WM, WN = T::WN;
  constexpr int TM = T::TM, TN = T::TN, PD = T::PD, R = T::RING;
  constexpr int PL = T::PL, P = T::PARTS;
  constexpr bool DIRECT = DirectStore<T, EPI>::value;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = uniform(t >> 6);
  // Waves w and w+4 share a SIMD. The fused epilogue gives the gate and the
  // up half of the tile different work, so there the column half is the high
  // part of the wave number and every SIMD holds one wave of each half.
  const int wm = EPI == kEpiSwigluQuant ? wave % T::WGM : wave / T::WGN;
  const int wn = EPI == kEpiSwigluQuant ? wave / T::WGM : wave % T::WGN;
  const int lr = lane & 15, lq = lane >> 4;

  const int K = p.K, KB = p.KB, M = p.M;
  if (nkb == 0) nkb = KB;
  const int NB128 = (p.N + 127) / 128;   // weight-scale row blocks (the last may be partial)
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  const uint32_t wave_at = lds_addr + wave * 1024;   // this wave's 1 KB DMA slot in a tile region

  // tile descriptors and the loop's branches are uniform over the workgroup
  // (made explicit: a descriptor read from LDS would otherwise count as
  // per-lane, and so would every buffer resource derived from it)
  auto next_tile = [&](TileDesc& d) {
    const bool more = uniform(next(d) ? 1 : 0) != 0;
    d = TileDesc{uniform(d.g), uniform(d.m0), uniform(d.n0), uniform(d.rows_valid)};
    return more;
  };
  TileDesc cur;
  if (!next_tile(cur)) return;

  // ---- DMA sources. Each tile gets a buffer resource per operand whose base
  // is the tile's first row (A, B) or first scale (sa, sb) and whose size
  // ends at the tile's last row with an output (A: rows_valid, B: N); the
  // per-lane byte offsets within one K-block column are then the same for
  // every tile. Slot s of a tile region is the 16-byte LDS chunk s; it holds
  // row s/8, chunk position s%8, i.e. global chunk (s%8) ^ (row%8). Rows that
  // have no output -- padding slots past the tile, A rows past M, masked rows
  // at or beyond masked_m[g], contiguous rows of padding or of another
  // expert, B rows past N -- fall past the resource's end (or get the offset
  // kNoRow): the range check returns zeros for them without a memory access,
  // so they cost no traffic and their MFMAs multiply zeros (the matrix core
  // draws less power on them).
  constexpr int NA = T::A_INSTR, NSC = T::SC_INSTR, NB = T::B_INSTR;
  struct Srd {
    i32x4 a, b, s[NSC];
  };
  uint32_t a_off[NA], b_off[NB], sc_off[NSC];
  int nb_lo, nb_hi, j_switch;
  // Scale loads: load i = q*W + wave brings activation rows [64i, 64i+64)
  // (i < BM/64) or the weight scales of the tile's 128-column blocks
  // (i == BM/64); a wave without a load of its own repeats load 0.
  int sc_row[NSC];   // i * 64, or -1 for the weight-scale load
  uint32_t sc_stride[NSC], sc_dst[NSC];
#pragma unroll
  for (int q = 0; q < NSC; ++q) {
    int i = q * W + wave;
    if (i >= T::SC_LOADS) i = 0;
    const bool is_b = i == BM / 64;
    sc_row[q] = is_b ? -1 : i * 64;
    sc_stride[q] = is_b ? 4u : (uint32_t)M * 4u;
    sc_dst[q] = lds_addr + T::SC_BASE + (is_b ? BM * 4 : i * 256);
    // weight scales: a tile reads at most the blocks nb_tile .. nb_tile+2, so
    // lanes past 3 repeat lane 3's row (one cache line instead of one per lane)
    sc_off[q] = is_b ? (uint32_t)min(lane, 3) * (uint32_t)KB * 4u : (uint32_t)(i * 64 + lane) * 4u;
  }
  auto a_slot = [&](int q, int& row, int& chunk) {
    const int slot = (q * W + wave) * 64 + lane;
    row = slot >> 3;
    chunk = (slot & 7) ^ (row & 7);
  };
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    int row, chunk;
    a_slot(q, row, chunk);
    a_off[q] = row < BM ? (uint32_t)row * (uint32_t)K + chunk * 16 : kNoRow;
  }
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const int slot = (q * W + wave) * 64 + lane;
    const int row = slot >> 3, chunk = (slot & 7) ^ (row & 7);
    b_off[q] = row < BN ? (uint32_t)(DIRECT ? pair_column(row) : row) * (uint32_t)K + chunk * 16 : kNoRow;
  }
  // the buffer resources of tile d (sizes clamp at 0: a tile past every row
  // with an output reads zeros only)
  auto srd_of = [&](const TileDesc& d) {
    const int g = d.g, m0 = d.m0, n0 = d.n0;
    const uint8_t* Ag = p.A + (LAYOUT == kMasked ? (size_t)g * M * K : 0);
    const float* sag = p.sa + (LAYOUT == kMasked ? (size_t)g * KB * M : 0);
    const uint8_t* Bg = p.B + (LAYOUT != kDense ? (size_t)g * p.N * K : 0);
    const float* sbg = p.sb + (LAYOUT != kDense ? (size_t)g * NB128 * KB : 0);
    const int rows = max(0, min(d.rows_valid - m0, BM)), cols = max(0, min(p.N - n0, BN));
    const int nb_tile = n0 >> 7;
    Srd r;
    r.a = buffer_rsrc(Ag + (size_t)m0 * K, (uint32_t)rows * (uint32_t)K);
    r.b = buffer_rsrc(Bg + (size_t)n0 * K, (uint32_t)cols * (uint32_t)K);
    // activation scales: rows past M read the next K-block's first rows (or
    // zeros past the end); those rows have no output
    const i32x4 rsSA = buffer_rsrc(sag + m0, (uint32_t)(KB * M - m0) * 4u);
    const i32x4 rsSB = buffer_rsrc(sbg + (size_t)nb_tile * KB, (uint32_t)(NB128 - nb_tile) * (uint32_t)KB * 4u);
#pragma unroll
    for (int q = 0; q < NSC; ++q) r.s[q] = sc_row[q] < 0 ? rsSB : rsSA;
    return r;
  };
  Srd rs;   // this tile's resources
  // ---- per-lane LDS addresses of this wave's fragments and scales. Chunk c
  // of tile row r sits at r*128 + ((c ^ (r & 7)) << 4); a wave's fragments
  // start at multiples of 16 rows, so r & 7 == lr & 7 and every fragment is
  // one of four per-lane bases plus a compile-time offset.
  constexpr int NWIN = (T::RING_BYTES + 65535) >> 16;
  LdsAddr<NWIN> aLo, aHi, bLo, bHi, sA, sB0, sB1;
  {
    const uint32_t lane_lo = lr * 128 + ((lq ^ (lr & 7)) << 4);
    const uint32_t lane_hi = lr * 128 + (((lq + 4) ^ (lr & 7)) << 4);
    aLo.init(lds_addr + wm * WM * 128 + lane_lo);
    aHi.init(lds_addr + wm * WM * 128 + lane_hi);
    bLo.init(lds_addr + wn * WN * 128 + lane_lo);
    bHi.init(lds_addr + wn * WN * 128 + lane_hi);
    sA.init(lds_addr + (wm * WM + lr) * 4);
  }
  auto setup = [&](const TileDesc& d) {
    const int g = d.g, m0 = d.m0, n0 = d.n0;
    rs = srd_of(d);
    if constexpr (LAYOUT == kContiguous) {
      // rows of padding or of another expert load nothing
#pragma unroll
      for (int q = 0; q < NA; ++q) {
        int row, chunk;
        a_slot(q, row, chunk);
        const int m = m0 + row;
        const bool live = row < BM && m < M && p.m_indices[m] == g;
        a_off[q] = live ? (uint32_t)row * (uint32_t)K + chunk * 16 : kNoRow;
      }
    }
    // scale blocks of B covered by this wave's columns (at most two) and the
    // first sub-tile column whose scale block is nb_hi
    const int nb_tile = n0 >> 7;
    const int wn0 = n0 + wn * WN;
    nb_lo = uniform(min(wn0 >> 7, NB128 - 1));
    nb_hi = uniform(min(nb_lo + 1, NB128 - 1));
    j_switch = T::STRADDLE ? uniform(((nb_lo + 1) * 128 - wn0) >> 4) : TN;
    sB0.init(lds_addr + (BM + nb_lo - nb_tile) * 4);
    sB1.init(lds_addr + (BM + nb_hi - nb_tile) * 4);
  };

  // Scalar offsets of one DMA group: the A tile and scales of K-block ka and
  // the B tile of K-block kbb (the two rings run different distances ahead).
  struct Soff {
    uint32_t a, b, sc[T::SC_INSTR];
  };
  auto soff_of = [&](int ka, int kbb) {
    Soff o;
    o.a = (uint32_t)(kb0 + ka) * (uint32_t)kKBlock;
    o.b = (uint32_t)(kb0 + kbb) * (uint32_t)kKBlock;
#pragma unroll
    for (int q = 0; q < T::SC_INSTR; ++q) o.sc[q] = (uint32_t)(kb0 + ka) * sc_stride[q];
    return o;
  };
  // DMA instruction d of a group (A chunks, then scale loads, then B chunks)
  // of the tile with resources r into A-ring stage AST and B-ring stage BST
  auto issue = [&](auto d_c, auto ast_c, auto bst_c, const Soff& o, const Srd& r) {
    constexpr int d = decltype(d_c)::value, AST = decltype(ast_c)::value, BST = decltype(bst_c)::value;
    if constexpr (d < NA) {
      dma16<T::A_BASE + AST * T::A_BYTES + d * W * 1024>(r.a, a_off[d], o.a, wave_at);
    } else if constexpr (d < NA + NSC) {
      constexpr int q = d - NA;
      dma4<AST * T::SC_BYTES>(r.s[q], sc_off[q], o.sc[q], sc_dst[q]);
    } else {
      constexpr int q = d - NA - NSC;
      dma16<T::B_BASE + BST * T::B_BYTES + q * W * 1024>(r.b, b_off[q], o.b, wave_at);
    }
  };

  // A fragment i / B fragment j of ring stage ST
  auto fragA = [&](auto st_c, auto i_c) {
    return frag_at<T::A_BASE + decltype(st_c)::value * T::A_BYTES + decltype(i_c)::value * 2048>(aLo, aHi);
  };
  auto fragB = [&](auto st_c, auto j_c) {
    return frag_at<T::B_BASE + decltype(st_c)::value * T::B_BYTES + decltype(j_c)::value * 2048>(bLo, bHi);
  };

  // ---- DMA schedule. The A tile and scales of K-block x land in A-ring
  // stage x % SA, its B tile in B-ring stage x % SB.
  //
  // SB >= 3: DMA group g(kb) holds the A tile and scales of K-block kb+SA and
  // the B tile of K-block kb+SB, whose stages the barrier of K-block kb has
  // just freed. Its instructions are spread one per pipeline step over the
  // K-block after that barrier ("head" after it, "tail" before the next one).
  // Groups are issued in order and loads complete in issue order, so at the
  // barrier of K-block kb, which needs K-block kb+1, everything issued after
  // the A part of group g(kb+1-SA) may still be in flight: its B part (the B
  // tile of an older K-block is already complete when SB > SA) and the
  // groups g(kb+2-SA) .. g(kb-1).
  //
  // S == 2: each K-block takes two barriers. The A fragments are held in
  // registers for the whole K-block, so a stage's A half is free once column 0
  // has consumed them: a first barrier after column 0 releases it, and the A
  // half of K-block kb+2 is spread over the rest of K-block kb (almost two
  // K-blocks to land). The B half (and the scales) is freed by the main
  // barrier before column TN-PD and spread over the last PD columns.
  //
  // Spreading keeps the MFMA pipe fed instead of stalling every wave on a
  // burst of DMA issue. K-block indices past the end are clamped (those repeat
  // loads hit L2), which keeps every wave's DMA count a compile-time constant
  // for the vmcnt waits.
  using SCH = Sched<T>;
  constexpr int STEPS = SCH::STEPS, PRE = SCH::PRE, POST = SCH::POST, D = SCH::D;
  constexpr bool SPLIT = SCH::SPLIT;
  constexpr int N_HEAD = SCH::n_head(), N_EARLY = SCH::n_early();
  constexpr int SA = T::ASTAGES, SB = T::STAGES;
  constexpr int B_AFTER_A = SA == SB ? 0 : NB;   // a group's loads that may trail its A part
  constexpr int WAIT_LOOP = SPLIT ? N_EARLY : B_AFTER_A + (SA - 2) * D;
  constexpr int WAIT_PRO = SPLIT ? D : B_AFTER_A + (SA - 2) * D + N_HEAD;
  static_assert(WAIT_PRO < 64 && WAIT_LOOP < 64, "vmcnt counter range");

  // ---- prologue: the groups g(-SB) .. g(-1) (the last one only its head),
  // i.e. the B tiles of K-blocks 0 .. SB-1 and the A tiles of 0 .. SA-1, then
  // wait for K-block 0 (after the previous tile's output stores, if they were
  // issued after this prologue)
  auto prologue = [&]() {
    if constexpr (SPLIT) {
      static_for<2>([&](auto x_c) {
        constexpr int x = decltype(x_c)::value;
        const Soff o = soff_of(min(x, nkb - 1), min(x, nkb - 1));
        static_for<D>([&](auto d_c) { issue(d_c, x_c, x_c, o, rs); });
      });
    } else {
      static_for<SB>([&](auto x_c) {
        constexpr int x = decltype(x_c)::value;       // group g(x - SB)
        constexpr int ka = x - SB + SA;               // its A K-block (< 0: none)
        const Soff o = soff_of(min(ka < 0 ? 0 : ka, nkb - 1), min(x, nkb - 1));
        static_for<D>([&](auto d_c) {
          constexpr int d = decltype(d_c)::value;
          constexpr bool a_part = d < NA + NSC;
          if constexpr (!(a_part && ka < 0) && !(x == SB - 1 && SCH::slot(d) >= POST))
            issue(d_c, std::integral_constant<int, (ka < 0 ? 0 : ka)>{}, x_c, o, rs);
        });
      });
    }
  };
  constexpr int NST = DIRECT ? TM * (TN / 2) : 0;   // output stores per wave and tile (direct epilogue)
  static_assert(WAIT_PRO + NST < 64, "vmcnt counter range");
  setup(cur);
  prologue();
  TileDesc nx = cur;
  bool after_stores = false;   // the previous tile's NST stores were issued after this tile's first loads
  for (;;) {
    if (after_stores) {
      wait_vm<WAIT_PRO + NST>();
    } else {
      wait_vm<WAIT_PRO>();
    }
    block_barrier();
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Register state. B fragments live in a ring of R = PD+1 (column g of the
    // K-block sequence, counting columns across K-blocks, in slot g % R); column
    // j+PD is read while column j computes. A fragments are held for the whole
    // K-block; with FA2 the K-blocks alternate between two sets and the next
    // K-block's set is read right after the barrier. Scales alternate between
    // two sets as well: a K-block's own and its predecessor's, which the first
    // PL steps still need for the carried promotions.
    i32x8 fbr[R], fa[T::FA2 ? 2 : 1][TM];
    float sc_lo[2][TM], sc_hi[2][TM];
    int ea[2][TM], eb_lo[2], eb_hi[2];   // POW2: E8M0 codes of the two scale sets
    f32x4 part[P];
    auto scale_read = [&](auto st_c, float (&a)[TM], float& b0, float& b1) {
      constexpr int ST = decltype(st_c)::value;
      static_for<TM>([&](auto i_c) {
        a[decltype(i_c)::value] = f32_at<T::SC_BASE + ST * T::SC_BYTES + decltype(i_c)::value * 64>(sA);
      });
      b0 = f32_at<T::SC_BASE + ST * T::SC_BYTES>(sB0);
      b1 = f32_at<T::SC_BASE + ST * T::SC_BYTES>(sB1);
    };
    auto set_scales = [&](auto set_c, const float (&a)[TM], float b0, float b1) {
      constexpr int SET = decltype(set_c)::value;
      if constexpr (POW2) {
  #pragma unroll
        for (int i = 0; i < TM; ++i) ea[SET][i] = e8m0_of(a[i]);
        eb_lo[SET] = e8m0_of(b0);
        eb_hi[SET] = T::STRADDLE ? e8m0_of(b1) : 0;
      } else {
  #pragma unroll
        for (int i = 0; i < TM; ++i) {
          sc_lo[SET][i] = a[i] * b0;
          sc_hi[SET][i] = T::STRADDLE ? a[i] * b1 : 0.f;
        }
      }
    };
    // scale of sub-tile (pi, pj) from scale set SET (a value select: selecting
    // between the two array elements themselves would keep the arrays in memory)
    auto scale_of = [&](auto set_c, auto pi_c, auto pj_c) {
      constexpr int SET = decltype(set_c)::value, pi = decltype(pi_c)::value, pj = decltype(pj_c)::value;
      const float lo = sc_lo[SET][pi];
      if constexpr (!T::STRADDLE) return lo;
      const float hi = sc_hi[SET][pi];
      return pj >= j_switch ? hi : lo;
    };

    // Stage 0's reads are issued in the order in which the loop itself leaves
    // the next stage's reads in flight (scales, then FA2 ? A, B : B, A). The
    // compiler places one LDS wait at the loop head that must hold for both the
    // entry and the back edge; with matching orders it is the steady-state wait
    // instead of a full drain on every K-block.
    {
      using Z = std::integral_constant<int, 0>;
      float a0[TM], b0, b1;
      scale_read(Z{}, a0, b0, b1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (T::FA2) {
        static_for<TM>([&](auto i_c) {
          fa[0][decltype(i_c)::value] = fragA(Z{}, i_c);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      static_for<PD>([&](auto c_c) {
        fbr[decltype(c_c)::value] = fragB(Z{}, c_c);
        __builtin_amdgcn_sched_barrier(0);
      });
      if constexpr (!T::FA2) {
        static_for<TM>([&](auto i_c) {
          fa[0][decltype(i_c)::value] = fragA(Z{}, i_c);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      set_scales(std::integral_constant<int, 0>{}, a0, b0, b1);
    }
    // before K-block 0 nothing is pending: zero partials promoted with zero
    // scales leave the (zero) accumulators unchanged
    if constexpr (!POW2) {
  #pragma unroll
      for (int c = 0; c < P; ++c) part[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int i = 0; i < TM; ++i) sc_lo[1][i] = sc_hi[1][i] = 0.f;
    }

    // promotion of MFMA u - PL of a K-block with phase PH (for u < PL: MFMA
    // STEPS + u - PL of the previous K-block, with the previous scale set)
    auto promote_step = [&](auto ph_c, auto u_c) {
      constexpr int PH = decltype(ph_c)::value, u = decltype(u_c)::value;
      constexpr int v = u - PL;
      constexpr int w = v >= 0 ? v : v + STEPS;
      constexpr int pj = w / TM, pi = w % TM;
      constexpr int set = v >= 0 ? (PH & 1) : ((PH + 1) & 1);
      promote(acc[pi][pj], part[(PH * STEPS + v + T::UNROLL * STEPS) % P],
              scale_of(std::integral_constant<int, set>{}, std::integral_constant<int, pi>{},
                       std::integral_constant<int, pj>{}));
    };

    // One K-block with compile-time phase PH = kb % U: TM x TN MFMAs in column
    // order. Step u issues MFMA u and then promotes MFMA u-PL. An MFMA's result
    // arrives well after the next MFMA could issue; waiting PL MFMAs before
    // reading it keeps the VALU work off the matrix core's critical path even
    // with a single wave per SIMD. The barrier sits before column JB = TN-PD,
    // when every read of the current stage has been issued; after it the next
    // stage's scales, first PD B fragments and (FA2) A fragments are read, or
    // (otherwise) each fa[i] is replaced right after its last MFMA.
    int kb = 0;
    auto kblock = [&](auto ph_c) -> bool {
      constexpr int PH = decltype(ph_c)::value;
      constexpr int U = T::UNROLL;
      constexpr int CA = PH % SA, NXA = (PH + 1) % SA, TA = (PH + U - 1) % SA;   // A ring: this, next, tail group
      constexpr int CB = PH % SB, NXB = (PH + 1) % SB, TB = (PH + U - 1) % SB;   // B ring
      constexpr int FSET = T::FA2 ? (PH & 1) : 0, NFSET = T::FA2 ? ((PH + 1) & 1) : 0;
      using CurA = std::integral_constant<int, CA>;
      using NxtA = std::integral_constant<int, NXA>;
      using CurB = std::integral_constant<int, CB>;
      using NxtB = std::integral_constant<int, NXB>;
      const Soff head = soff_of(min(kb + SA, nkb - 1), min(kb + SB, nkb - 1));           // group g(kb)
      const Soff tail = soff_of(min(kb - 1 + SA, nkb - 1), min(kb - 1 + SB, nkb - 1));   // group g(kb-1)
      (void)tail;
      float sa_next[TM], sb_next0 = 0.f, sb_next1 = 0.f;
      static_for<STEPS>([&](auto u_c) {
        constexpr int u = decltype(u_c)::value;
        constexpr int j = u / TM, i = u % TM;
        if constexpr (SPLIT && u == TM && TM < PRE) block_barrier();   // A half of this stage is free
        if constexpr (u == PRE) {
          // every read of the current stage has been issued; the next stage (and,
          // for S == 2, every DMA older than this K-block's early A loads) is in
          wait_lgkm0();
          wait_vm<WAIT_LOOP>();
          block_barrier();
          scale_read(NxtA{}, sa_next, sb_next0, sb_next1);
          if constexpr (T::FA2) {
            static_for<TM>([&](auto ii_c) { fa[NFSET][decltype(ii_c)::value] = fragA(NxtA{}, ii_c); });
          }
        }
        if constexpr (POW2) {
          // this K-block's scales are set PH & 1 (K-blocks alternate sets)
          constexpr int SET = PH & 1;
          int eb = eb_lo[SET];
          if constexpr (T::STRADDLE) eb = j >= j_switch ? eb_hi[SET] : eb_lo[SET];
          acc[i][j] = mfma_e4m3_pow2(fbr[(PH * TN + j) % R], fa[FSET][i], acc[i][j], eb, ea[SET][i]);
        } else {
          part[(PH * STEPS + u) % P] = mfma_e4m3(fbr[(PH * TN + j) % R], fa[FSET][i]);
        }
        if constexpr (i == 0) {
          // column j+PD of this stage, or (past the end) column j+PD-TN of the next
          constexpr int jn = j + PD;
          constexpr int slot = (PH * TN + jn) % R;
          if constexpr (jn < TN) fbr[slot] = fragB(CurB{}, std::integral_constant<int, jn>{});
          else fbr[slot] = fragB(NxtB{}, std::integral_constant<int, jn - TN>{});
        }
        if constexpr (!T::FA2 && j == TN - 1) fa[0][i] = fragA(NxtA{}, std::integral_constant<int, i>{});
        static_for<D>([&](auto d_c) {
          constexpr int d = decltype(d_c)::value;
          if constexpr (SPLIT) {
            if constexpr (SCH::slot(d) == u) issue(d_c, CurA{}, CurB{}, head, rs);   // K-block kb+2
          } else {
            if constexpr (u >= PRE && SCH::slot(d) == u - PRE) issue(d_c, CurA{}, CurB{}, head, rs);
            if constexpr (u < PRE && SCH::slot(d) == POST + u)
              issue(d_c, std::integral_constant<int, TA>{}, std::integral_constant<int, TB>{}, tail, rs);
          }
        });
        if constexpr (!POW2) promote_step(ph_c, u_c);
        step_fence();
      });
      set_scales(std::integral_constant<int, (PH + 1) & 1>{}, sa_next, sb_next0, sb_next1);
      return ++kb == nkb;
    };
    bool done = false;
    for (;;) {
      static_for<T::UNROLL>([&](auto ph_c) {
        if (!done) done = kblock(ph_c);
      });
      if (done) break;
    }
    // The last K-block's final PL partials, promoted once after the loop (an
    // exit path per phase that did this work would keep the register allocator
    // from holding each accumulator in one register across the phases).
    if constexpr (!POW2) {
      const int last = (nkb - 1) % T::UNROLL;
      static_for<T::UNROLL>([&](auto ph_c) {
        constexpr int PH = decltype(ph_c)::value;
        if (last == PH) {
          static_for<PL>([&](auto c_c) {
            constexpr int w = STEPS - PL + decltype(c_c)::value;
            promote(acc[w % TM][w / TM], part[(PH * STEPS + w) % P],
                    scale_of(std::integral_constant<int, PH & 1>{}, std::integral_constant<int, w % TM>{},
                             std::integral_constant<int, w / TM>{}));
          });
        }
      });
    }

    const int g = cur.g, m0 = cur.m0, n0 = cur.n0, rows_valid = cur.rows_valid;
    uint16_t* Dg = p.D + (LAYOUT == kMasked ? (size_t)g * M * p.N : 0);
    wait_vm<0>();          // the clamped tail DMAs must land before LDS is reused
    wait_lgkm0();
    block_barrier();
    if constexpr (DIRECT) {
      // bf16 RNE straight from the accumulators: sub-tiles 2q and 2q+1 hold
      // columns 32q + 8lq .. 32q + 8lq + 7 of row 16i + lr (the B tile was
      // loaded in pair_column order). Stores go through a buffer resource
      // over this tile's output rows, so a row or column without an output
      // gets an offset past it and its store is dropped: every wave issues
      // exactly NST stores, which the next tile's first wait counts. N is a
      // multiple of 8, so a 16-byte piece is wholly inside or wholly past N.
      const int rows_here = max(0, min(rows_valid - m0, BM));
      const __amdgpu_buffer_rsrc_t rsD =
          __builtin_amdgcn_make_buffer_rsrc(Dg + (size_t)m0 * p.N, 0, rows_here * p.N * 2, 0x20000);
      uint32_t roff[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int m = m0 + wm * WM + i * 16 + lr;
        bool ok = m < rows_valid;
        if (LAYOUT == kContiguous && ok) ok = p.m_indices[m] == g;
        roff[i] = ok ? (uint32_t)(m - m0) * (uint32_t)p.N * 2u : kNoRow;
        // any m_indices load completes here, before the next tile's DMAs are
        // in flight (a later wait for it would also wait for them)
        asm volatile("" : "+v"(roff[i]));
      }
      const bool more = next_tile(nx);
      if (more) {
        setup(nx);
        prologue();
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < TN / 2; ++q) {
          const int n = n0 + wn * WN + q * 32 + lq * 8;
          const uint32_t off = n < p.N ? roff[i] + (uint32_t)n * 2u : kNoRow;
          const f32x4& x = acc[i][2 * q];
          const f32x4& y = acc[i][2 * q + 1];
          const i32x4 v = {(int)(bf16_rne_bits(x[0]) | (bf16_rne_bits(x[1]) << 16)),
                           (int)(bf16_rne_bits(x[2]) | (bf16_rne_bits(x[3]) << 16)),
                           (int)(bf16_rne_bits(y[0]) | (bf16_rne_bits(y[1]) << 16)),
                           (int)(bf16_rne_bits(y[2]) | (bf16_rne_bits(y[3]) << 16))};
          __builtin_amdgcn_raw_buffer_store_b128(v, rsD, off, 0, 0);
        }
      if (!more) break;
      cur = nx;
      after_stores = true;
    } else {
      if constexpr (EPI == kEpiSwigluQuant) {
        swiglu_quant_epilogue<LAYOUT, T, POW2>(p, acc, lds, g, m0, n0, rows_valid, wm, wn, lr, lq, t);
      } else {
        // ---- epilogue: bf16 RNE, staged through LDS so that every global store is
        // a full 16-byte piece of a contiguous output row
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
      if (!next_tile(nx)) break;
      wait_vm<0>();        // this tile's stores and LDS reads are done
      wait_lgkm0();
      block_barrier();
      cur = nx;
      setup(cur);
      prologue();
    }
  }
}

// One BM x BN output tile of expert g (dense: g = 0) whose first row is m0
// and first column n0; rows_valid bounds the rows that have an output (see
// gemm_tiles).
template <int LAYOUT, class T, bool POW2, int EPI>
__device__ __forceinline__ void gemm_tile(const Params& p, lds_u8* const lds, int g, const int m0,
                                          const int n0, const int rows_valid, const int kb0 = 0,
                                          int nkb = 0) {
  bool done = false;
  gemm_tiles<LAYOUT, T, POW2, EPI>(
      p, lds,
      [&](TileDesc& d) {
        if (done) return false;
        d = TileDesc{g, m0, n0, rows_valid};
        done = true;
        return true;
      },
      kb0, nkb);
}

// Contiguous layout with 256-row tiles. Experts' row segments are padded only
// to 128 rows, so 256-row tiles on a fixed 256-row grid would straddle two
// experts wherever a segment starts at an odd 128-row block. A tile instead
// starts at the first 128-row block of each run of blocks that belong to one
// expert, and at every second block after it. The last tile of a run with an
// odd number of blocks covers one block of the run; its other 128 rows
// (another expert's, padding, or past M) are computed with this expert's
// weight and never stored, since rows are stored only where m_indices names
// the tile's expert. The runs depend on m_indices, which lives in device
// memory, so every workgroup derives the tile list itself and the workgroups
// walk it persistently (a fixed grid; tile i goes to workgroup i mod grid).
constexpr int kRunMaxBlocks = 2048;    // 128-row blocks one list holds (M <= 262144)
constexpr int kRunMaxExperts = 32767;  // experts a packed list entry can name
template <int LAYOUT, class T>
constexpr bool run_tiles() {
  return LAYOUT == kContiguous && T::BM == 256;
}

// The tile list of the 256-row contiguous layout. Pass 1 (all threads, 32
// lanes per block): the expert of each 128-row block -- the largest valid id
// among its rows, -1 if it has none, the rule the 128-row tiles use -- into
// blk[]. Pass 2 (wave 0, 64 blocks at a time, one lane each): a block starts
// a run when its expert differs from the previous block's, and starts a tile
// when it lies an even number of blocks after its run's start. Entries are
// (block | expert << 16) in row order. Without SINGLES every tile goes to
// list[0 ..) and s_count[0] is their number. With SINGLES the last tile of a
// run with an odd number of blocks (it covers a single block of the run) goes
// to the back, list[kRunMaxBlocks - 1], list[kRunMaxBlocks - 2], ..., the
// two-block tiles to the front; s_count[0] / s_count[1] are their numbers.
// Every thread of the workgroup must call it.
template <int THREADS, bool SINGLES>
__device__ __forceinline__ void contiguous_run_tiles(const Params& p, int* blk, int* list, int* s_count) {
  const int t = threadIdx.x, lane = t & 63;
  const int nblk = (p.M + 127) / 128;
  constexpr int BPI = THREADS / 32;   // blocks per pass-1 iteration
  const int iters = (nblk + BPI - 1) / BPI;
  // Lane h of a block's 32 reads rows 4h .. 4h+3 (one 16-byte load through a
  // buffer resource over m_indices: rows past M read zeros, masked below);
  // the loads of BATCH iterations are in flight together.
  constexpr int BATCH = 8;
  const __amdgpu_buffer_rsrc_t rsI =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.m_indices, 0, p.M * 4, 0x20000);
  for (int it0 = 0; it0 < iters; it0 += BATCH) {   // same trip counts for every lane (shuffles below)
    i32x4 ids[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int bk = (it0 + b) * BPI + (t >> 5), h = t & 31;
      ids[b] = __builtin_amdgcn_raw_buffer_load_b128(rsI, (uint32_t)(bk * 128 + h * 4) * 4u, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int bk = (it0 + b) * BPI + (t >> 5), h = t & 31;
      int v = -1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = bk * 128 + h * 4 + r, id = ids[b][r];
        if (m < p.M && id >= 0 && id < p.G) v = max(v, id);
      }
#pragma unroll
      for (int d = 16; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, 32));
      if (h == 0 && bk < nblk) blk[bk] = v;
    }
  }
  __syncthreads();
  if (t < 64) {
    int prev_e = -1, prev_rs = 0, count = 0, singles = 0;
    const unsigned long long lt = (1ull << lane) - 1ull, le = lt | (1ull << lane);
    for (int c0 = 0; c0 < nblk; c0 += 64) {
      const int bk = c0 + lane;
      const int e = bk < nblk ? blk[bk] : -1;
      int before = __shfl_up(e, 1);
      if (lane == 0) before = prev_e;
      const unsigned long long starts = __ballot(e >= 0 && e != before) & le;
      const int rs = starts ? c0 + 63 - __clzll((long long)starts) : prev_rs;   // start of this block's run
      const bool first = e >= 0 && ((bk - rs) & 1) == 0;
      // the tile's second block is outside the run: a single-block tile
      const bool single = SINGLES && first && (bk + 1 >= nblk || blk[bk + 1] != e);
      const unsigned long long fulls = __ballot(first && !single);
      const unsigned long long ones = __ballot(single);
      if (first && !single) list[count + __popcll(fulls & lt)] = bk | (e << 16);
      if (single) list[kRunMaxBlocks - 1 - (singles + __popcll(ones & lt))] = bk | (e << 16);
      count += __popcll(fulls);
      singles += __popcll(ones);
      prev_e = __shfl(e, 63);
      prev_rs = __shfl(rs, 63);
    }
    if (t == 0) {
      s_count[0] = count;
      if (SINGLES) s_count[1] = singles;
    }
  }
  __syncthreads();
}

// Position of workgroup b among nwg: consecutive positions are placed on the
// same XCD (workgroups are dealt round-robin to the XCDs).
__device__ __forceinline__ int xcd_position(int b, int nwg) {
  const int x = b % kXCDs, l = b / kXCDs;
  const int per = nwg / kXCDs, rem = nwg % kXCDs;
  return x * per + (x < rem ? x : rem) + l;
}

// Tile position -> (m-block, n-block) of a tiles_m x tiles_n grid, walked in
// groups of kGroupM m-blocks so the tiles resident on one XCD share A rows and
// B columns in its L2.
__device__ __forceinline__ void raster(int tile, int tiles_m, int tiles_n, int& mb, int& nbk) {
  const int span = kGroupM * tiles_n;
  const int grp = tile / span;
  const int first = grp * kGroupM;
  const int gsz = min(kGroupM, tiles_m - first);
  const int in = tile - grp * span;
  mb = first + in % gsz;
  nbk = in / gsz;
}

template <int LAYOUT, class T, bool POW2 = false, int EPI = kEpiBf16>
__global__ __launch_bounds__(T::THREADS) void fp8_bs_gemm(Params p) {
  constexpr int BM = T::BM, BN = T::BN;
  constexpr bool RUNS = run_tiles<LAYOUT, T>();
  constexpr int LIST_BYTES = RUNS ? kRunMaxBlocks * 4 : 0;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES + LIST_BYTES];
  __shared__ int s_group;
  lds_u8* const lds = (lds_u8*)smem;
  const int t = threadIdx.x;

  const int pos = xcd_position(blockIdx.x, gridDim.x);

  if constexpr (RUNS) {
    int* list = (int*)(smem + T::LDS_BYTES);
    contiguous_run_tiles<T::THREADS, false>(p, (int*)smem, list, &s_group);
    const int ntm = s_group;
    const int total = ntm * p.tiles_n;
    int tile = pos;
    gemm_tiles<LAYOUT, T, POW2, EPI>(p, lds, [&](TileDesc& d) {
      if (tile >= total) return false;
      int mb, nbk;
      raster(tile, ntm, p.tiles_n, mb, nbk);
      const int e = list[mb];
      d = TileDesc{e >> 16, (e & 0xffff) * 128, nbk * BN, p.M};
      tile += gridDim.x;
      return true;
    });
  } else {
    int tile = pos;
    int g = 0;
    if (LAYOUT == kMasked) {
      const int per = p.tiles_m * p.tiles_n;
      g = tile / per;
      tile -= g * per;
    }
    int mb, nbk;
    raster(tile, p.tiles_m, p.tiles_n, mb, nbk);
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
    gemm_tile<LAYOUT, T, POW2, EPI>(p, lds, g, m0, n0, rows_valid);
  }
}


// Dense layout on two tile shapes in one launch. A problem whose tile count on
// the wide tile TA leaves a partial last round (the wave quantisation the
// zwzgs.cn DeepGEMM page describes under "non-standard block sizes") puts
// columns [0, n_split) on TA tiles -- tiles_a of them, whole rounds over the
// CUs -- and the remaining columns on the narrower TB tiles, which fill the
// last round. The workgroups (one per CU) walk the TA tiles persistently, then
// the TB tiles; tile i of either kind goes to workgroup i mod grid, and the
// tiles are XCD-grouped and rasterised like the single-shape kernel's.
template <class TA, class TB, bool POW2>
__global__ __launch_bounds__(TA::THREADS) void fp8_bs_gemm_split(Params p) {
  static_assert(TA::THREADS == TB::THREADS, "both tile shapes run with the same workgroup size");
  constexpr int LDS = TA::LDS_BYTES > TB::LDS_BYTES ? TA::LDS_BYTES : TB::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
  lds_u8* const lds = (lds_u8*)smem;
  const int grid = gridDim.x, na = p.tiles_a;
  const int tma = (p.M + TA::BM - 1) / TA::BM, tna = p.n_split / TA::BN;
  const int tmb = (p.M + TB::BM - 1) / TB::BM, tnb = (p.N - p.n_split + TB::BN - 1) / TB::BN;
  const int nb = tmb * tnb;
  int k = blockIdx.x;
  gemm_tiles<kDense, TA, POW2, kEpiBf16>(p, lds, [&](TileDesc& d) {
    if (k >= na) return false;
    int mb, nbk;
    raster(xcd_position(k, na), tma, tna, mb, nbk);
    d = TileDesc{0, mb * TA::BM, nbk * TA::BN, p.M};
    k += grid;
    return true;
  });
  wait_lgkm0();
  block_barrier();   // no wave still reads the TA ring when the TB tiles' DMAs start
  k = blockIdx.x;
  gemm_tiles<kDense, TB, POW2, kEpiBf16>(p, lds, [&](TileDesc& d) {
    if (k >= nb) return false;
    int mb, nbk;
    raster(xcd_position(k, nb), tmb, tnb, mb, nbk);
    d = TileDesc{0, mb * TB::BM, p.n_split + nbk * TB::BN, p.M};
    k += grid;
    return true;
  });
}

// Contiguous layout on run-following 256-row tiles (TF, 256 x BN) with the
// work the 256-row tiles would waste put on 128-row tiles (TH, 128 x BN):
//  * the last tile of a run with an odd number of 128-row blocks covers one
//    block of the run, so it runs as a 128-row tile (the 256-row kernel
//    computes another expert's block, or padding, beside it and discards it);
//  * the two-block tiles fill whole rounds over the workgroups; if the rest
//    of them, split into 128-row halves, fits one round together with the
//    single-block tiles, it runs that way (the wave-quantisation tail the
//    zwzgs.cn DeepGEMM page describes under "non-standard block sizes"),
//    otherwise every two-block tile runs whole.
// The workgroups walk the work items persistently: two-block tiles first,
// then the 128-row items. The tile list comes from m_indices (device memory),
// so every workgroup derives it and the split itself.
template <class TF, class TH, bool POW2, int EPI>
__global__ __launch_bounds__(TF::THREADS) void fp8_bs_gemm_runs(Params p) {
  static_assert(TF::BM == 256 && TH::BM == 128 && TF::BN == TH::BN && TF::THREADS == TH::THREADS,
                "two-block tiles of 256 rows, single-block tiles of 128 rows, same columns and workgroup");
  constexpr int LDS = TF::LDS_BYTES > TH::LDS_BYTES ? TF::LDS_BYTES : TH::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS + kRunMaxBlocks * 4];
  __shared__ int s_count[2];
  lds_u8* const lds = (lds_u8*)smem;
  int* list = (int*)(smem + LDS);
  contiguous_run_tiles<TF::THREADS, true>(p, (int*)smem, list, s_count);
  const int F = s_count[0], S = s_count[1], tn = p.tiles_n;
  const long grid = gridDim.x;
  const long full_items = (long)F * tn;
  long whole = full_items;   // two-block tiles that run as 256-row tiles
  {
    const long rounds = full_items / grid, rest = full_items - rounds * grid;
    if (rest && 2 * rest + (long)S * tn <= grid) whole = rounds * grid;
  }
  const long halves = 2 * (full_items - whole);
  const long items = whole + halves + (long)S * tn;
  long w = xcd_position(blockIdx.x, gridDim.x);
  gemm_tiles<kContiguous, TF, POW2, EPI>(p, lds, [&](TileDesc& d) {
    if (w >= whole) return false;
    int mb, nbk;
    raster((int)w, F, tn, mb, nbk);
    const int e = list[mb];
    d = TileDesc{e >> 16, (e & 0xffff) * 128, nbk * TF::BN, p.M};
    w += grid;
    return true;
  });
  wait_lgkm0();
  block_barrier();   // no wave still reads LDS of the 256-row tiles when the 128-row ones start
  gemm_tiles<kContiguous, TH, POW2, EPI>(p, lds, [&](TileDesc& d) {
    if (w >= items) return false;
    const long h = w - whole;
    int mb, nbk, e, m0;
    if (h < halves) {   // one 128-row half of a two-block tile
      raster((int)(whole + h / 2), F, tn, mb, nbk);
      e = list[mb];
      m0 = (e & 0xffff) * 128 + (int)(h & 1) * 128;
    } else {            // a single-block tile
      raster((int)(h - halves), S, tn, mb, nbk);
      e = list[kRunMaxBlocks - 1 - mb];
      m0 = (e & 0xffff) * 128;
    }
    d = TileDesc{e >> 16, m0, nbk * TH::BN, p.M};
    w += grid;
    return true;
  });
}

}  // namespace fg
