/*
 * fg.h -- FP8 (OCP E4M3) GEMM with fine-grained fp32 block scales, for AMD
 * MI355X (gfx950). C ABI.
 *
 * Every GEMM entry point computes D = A . B^T with
 *
 *     D[m, n] = sum_kb  sa[m, kb] * sb[n / 128, kb] * P_kb[m, n]
 *     P_kb[m, n] = sum_{k in K-block kb} e4m3(A[m, k]) * e4m3(B[n, k])
 *
 * i.e. A is scaled per 1x128 block (one fp32 per row and 128-wide K-block) and
 * B per 128x128 block, each 128-wide K-block partial is formed in a fresh FP32
 * accumulator on the matrix cores and then multiplied by sa*sb and added into
 * a master FP32 accumulator ("two-level accumulation"), and the result is
 * rounded once to bf16 (round to nearest even).
 *
 * Sources: the zwzgs.cn page "DeepGEMM: an open-source FP8 GEMM library",
 * sections "Features > fine-grained scaling" (DeepSeek-V3 style per-block
 * scales), "Features > layouts" (normal, MoE contiguous, MoE masked) and
 * "Technical details > two-level accumulation"; the 2kiu.com DeepGEMM
 * explainer, section 3.3 (FP8 inputs, FP32 accumulation, conversion to the
 * output type at the end). The 1x128 / 128x128 granularity and the E4M3
 * variant (bias 7, max 448, NaN = S.1111.111, no infinities) are the readings
 * taken where the pages only say "fine-grained" and "E4M3".
 *
 * Conventions shared by all calls
 *   - All pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory and keeps no reference after returning.
 *   - A, B: E4M3 bytes, K contiguous ("NT": B is given as N x K).
 *   - sa: fp32, K-block-major: sa[kb * M + m] (masked: [G][K/128][M_max]).
 *   - sb: fp32, row-major [ceil(N/128)][K/128] (grouped: [G][ceil(N/128)][K/128]);
 *     when N is not a multiple of 128 the last row block of B covers the
 *     remaining N mod 128 rows.
 *   - D: bf16 bit patterns, row-major [M][N] (masked: [G][M_max][N]).
 *   - K must be a multiple of 128 and N a multiple of 8 (whole 16-byte pieces
 *     of a bf16 output row; the fused calls need N % 256 == 0); M is
 *     arbitrary (>= 0). The boundary handling the 2kiu.com explainer
 *     discusses in section 4.3 is done in one code path: loads of rows past N
 *     (and of A rows without an output) read zeros through the buffer range
 *     check, and the stores of columns >= N are skipped.
 *   - A, B and D base pointers must be 16-byte aligned, sa and sb 4-byte.
 *   - Calls are asynchronous on `stream` (0 = null stream), never synchronise
 *     and never read device data on the host, so they can be captured in a
 *     HIP graph. Rows the call has no output for are never written.
 *   - Kernels run on the current device (hipGetDevice); `stream` and every
 *     pointer must belong to it.
 *   - Results are bitwise reproducible (no atomics, no split-K), and do not
 *     depend on the tile configuration or the layout either: every output
 *     element takes the same K-block dot products and the same FP32
 *     promotion sequence whichever tile, kernel or layout computes it.
 *   - Return value: FG_OK or a negative FG_E* code; no exception crosses the
 *     ABI. fg_strerror() gives a static description.
 */
#ifndef FG_H
#define FG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FG_OK = 0,
  FG_EINVAL = -1,        /* bad argument: null pointer, negative size,
                            K not a multiple of 128, N not a multiple of
                            8, misalignment,
                            G < 1 for a grouped call, unknown
                            layout or scale kind; N not a multiple
                            of 256 for the fused calls; an operand
                            (M x K or N x K bytes, per expert) of
                            2^31 bytes or more, or N > 4194296 (the
                            kernels address these with 32-bit byte
                            offsets) */
  FG_EUNSUPPORTED = -2,  /* current device is not gfx950 */
  FG_ELAUNCH = -3,       /* the kernel launch failed (hipGetLastError) */
  FG_EDEVICE = -4        /* a HIP runtime query failed */
};

enum { FG_LAYOUT_DENSE = 0, FG_LAYOUT_CONTIGUOUS = 1, FG_LAYOUT_MASKED = 2 };

/* Block-scale kinds of the fused calls below. */
enum { FG_SCALES_FP32 = 0, FG_SCALES_POW2 = 1 };

/* OR-ed into fg_select_config's layout: the tile the fused SiLU-gate
 * epilogue would use. */
enum { FG_SELECT_SWIGLU_QUANT = 0x100 };

/*
 * Dense ("normal") layout. zwzgs.cn DeepGEMM page, "Features > layouts".
 *   A  [M][K] E4M3, sa [K/128][M] fp32, B [N][K] E4M3, sb [ceil(N/128)][K/128] fp32,
 *   D  [M][N] bf16 (written in full).
 * M == 0 (or N == 0) returns FG_OK without launching anything.
 */
int fg_gemm_fp8_nt(const void* A, const float* sa, const void* B, const float* sb,
                   void* D, int M, int N, int K, hipStream_t stream);

/*
 * MoE grouped, contiguous layout (training / prefill). zwzgs.cn DeepGEMM
 * page, "Features > layouts" and "Applications > MoE".
 *   A  [M][K] E4M3: the rows of all G experts concatenated along M,
 *   sa [K/128][M], B [G][N][K] E4M3 (one weight per expert),
 *   sb [G][ceil(N/128)][K/128], D [M][N] bf16,
 *   m_indices [M] int32 (device): expert id of each row, or -1 for a padding
 *   row. Every aligned 128-row block of A must hold rows of at most one expert
 *   (plus padding rows); experts' segments are therefore padded to multiples
 *   of 128 rows. Rows with m_indices = -1 are not written. Ids >= G are
 *   treated as padding (never read out of bounds).
 */
int fg_grouped_contiguous(const void* A, const float* sa, const void* B, const float* sb,
                          void* D, const int32_t* m_indices, int M, int N, int K, int G,
                          hipStream_t stream);

/*
 * MoE grouped, masked layout (decode). zwzgs.cn DeepGEMM page, "Features >
 * layouts" and "Applications > MoE".
 *   A  [G][M_max][K] E4M3, sa [G][K/128][M_max], B [G][N][K] E4M3,
 *   sb [G][ceil(N/128)][K/128], D [G][M_max][N] bf16,
 *   masked_m [G] int32 (device): number of valid rows of each expert, clamped
 *   to [0, M_max] by the kernel. Only rows r < masked_m[g] of expert g are
 *   written; the rest of D keeps its prior content. masked_m is read only by
 *   the kernel (no host synchronisation).
 */
int fg_grouped_masked(const void* A, const float* sa, const void* B, const float* sb,
                      void* D, const int32_t* masked_m, int G, int M_max, int N, int K,
                      hipStream_t stream);

/*
 * Power-of-two block scales on the matrix core (E8M0). The 2kiu.com DeepGEMM
 * explainer, section 7, names MX / micro-scaling formats as the next step
 * beyond per-block FP8 scaling; their block scales are pure powers of two.
 * These three calls compute the same D as fg_gemm_fp8_nt /
 * fg_grouped_contiguous / fg_grouped_masked -- same arguments, layouts,
 * ownership, row rules and error codes -- under one more precondition: every
 * sa and sb entry must be a power of two between 2^-126 and 2^127 (a normal
 * fp32 value with a zero mantissa; fg_quant_*_pow2 produce such scales). Its
 * exponent field is then the E8M0 code (2^(e-127)) that gfx950's
 * v_mfma_scale_f32_16x16x128_f8f6f4 applies per row and K-block inside the
 * matrix core, accumulating every K-block straight into the FP32 master
 * accumulator; no promotion step runs on the vector ALUs. Accumulation is
 * FP32 throughout, as in the two-level form. A scale that is not such a power
 * of two is not detected: its mantissa is ignored (the result is then that of
 * the scale rounded down to a power of two); memory safety is unaffected.
 */
int fg_gemm_fp8_nt_pow2(const void* A, const float* sa, const void* B, const float* sb,
                        void* D, int M, int N, int K, hipStream_t stream);
int fg_grouped_contiguous_pow2(const void* A, const float* sa, const void* B, const float* sb,
                               void* D, const int32_t* m_indices, int M, int N, int K, int G,
                               hipStream_t stream);
int fg_grouped_masked_pow2(const void* A, const float* sa, const void* B, const float* sb,
                           void* D, const int32_t* masked_m, int G, int M_max, int N, int K,
                           hipStream_t stream);

/*
 * Fused first projection of an MoE expert FFN: GEMM, SiLU gate and FP8
 * re-quantisation in one kernel. The 2kiu.com DeepGEMM explainer, section 7,
 * names fusing the activation functions around a GEMM, to save memory round
 * trips, as the next optimisation; sections 4.4 and the zwzgs.cn page
 * ("Features > fine-grained scaling") give the 1x128 quantisation the next
 * GEMM consumes. Readings taken (the pages name neither the activation nor a
 * weight layout): the activation is SiLU-gated, and B's rows interleave gate
 * and up every 128 rows, so with H = A . B^T as computed by fg_gemm_fp8_nt
 * (FP32, before bf16 rounding), I = N / 2 and j = 0 .. I/128 - 1,
 *
 *     act[m, 128j + c] = silu(H[m, 256j + c]) * H[m, 256j + 128 + c],
 *     silu(x) = x / (1 + exp(-x))   (FP32),
 *
 * and act is quantised per 1x128 block exactly as fg_quant_act_1x128 (scales
 * = FG_SCALES_FP32) or fg_quant_act_1x128_pow2 (FG_SCALES_POW2) would
 * quantise it. With FG_SCALES_POW2 the input scales sa, sb must also be
 * powers of two (as for the fg_*_pow2 calls).
 *   A, sa, B, sb, m_indices, masked_m, M, M_max, G, K: as for the plain calls.
 *   N: columns of H, a multiple of 256.
 *   Q   [M][I] E4M3 (masked [G][M_max][I]), 16-byte aligned: the codes.
 *   sq  [I/128][M] fp32 (masked [G][I/128][M_max]): the scales, K-block-major
 *       as the next GEMM's sa (its K is I).
 *   act [M][I] fp32 (masked [G][M_max][I]), 16-byte aligned, or NULL: the
 *       activation before quantisation (for callers that keep it, and for
 *       checking the quantisation bit for bit).
 * Rows without output (M tail, masked rows >= masked_m[g], contiguous rows
 * with m_indices = -1) are not written in Q, sq or act. No bf16 H is written.
 * The call uses 256-column tiles only (fg_select_config with
 * FG_SELECT_SWIGLU_QUANT).
 */
int fg_gemm_fp8_nt_swiglu_quant(const void* A, const float* sa, const void* B, const float* sb,
                                void* Q, float* sq, float* act, int M, int N, int K, int scales,
                                hipStream_t stream);
int fg_grouped_contiguous_swiglu_quant(const void* A, const float* sa, const void* B, const float* sb,
                                       void* Q, float* sq, float* act, const int32_t* m_indices,
                                       int M, int N, int K, int G, int scales, hipStream_t stream);
int fg_grouped_masked_swiglu_quant(const void* A, const float* sa, const void* B, const float* sb,
                                   void* Q, float* sq, float* act, const int32_t* masked_m, int G,
                                   int M_max, int N, int K, int scales, hipStream_t stream);

/*
 * Tile configuration the library would launch for a problem, computed on the
 * host from sizes only (pure: no device access, no state; usable without a
 * GPU). Tiles are chosen from a fixed table to minimise wave quantisation
 * over `num_cus` compute units, the point the zwzgs.cn DeepGEMM page makes in
 * "Technical details > non-standard block sizes" (M=256, N=7168 on 132 SMs:
 * 112 tiles of 128x128 versus 128 of 128x112), weighed against each tile's
 * per-K-block cost.
 *   M       total rows (dense, contiguous) or M_max (masked);
 *   N, K    as for the GEMM calls (N % 8 == 0, K % 128 == 0 need not hold
 *           here: the choice is made for any non-negative sizes);
 *   G       experts (ignored for dense; >= 1 for the grouped layouts);
 *   layout  FG_LAYOUT_*, optionally | FG_SELECT_SWIGLU_QUANT for the tile the
 *           fused SiLU-gate epilogue would use;
 *   num_cus compute units to fill; <= 0 means the library's default (256,
 *           MI355X).
 * Writes the tile's rows / columns to *bm / *bn (either may be NULL).
 * Returns FG_OK, or FG_EINVAL for an unknown layout, a negative size or
 * G < 1 with a grouped layout.
 */
int fg_select_config(int M, int N, int K, int G, int layout, int num_cus, int* bm, int* bn);

/*
 * Number of workgroups the launch for the same problem would use (same
 * arguments and errors as fg_select_config): one per output tile, except
 * the contiguous layout on 256-row tiles, whose workgroups walk a tile list
 * persistently (at most one per compute unit).
 */
int fg_select_grid(int M, int N, int K, int G, int layout, int num_cus, int* grid);

/*
 * fp32 -> E4M3 quantisation producing this library's operand layouts
 * (2kiu.com DeepGEMM explainer, section 4.4: scales from the data's
 * statistics, saturation of out-of-range values; zwzgs.cn DeepGEMM page,
 * "Features > fine-grained scaling"). Per block: amax = max |x|;
 * scale = amax / 448 (1 if amax == 0); code = nearest E4M3 of
 * clamp(x / scale, -448, 448), ties to even, sign kept (so -tiny -> 0x80).
 * Inputs must be finite. Asynchronous on `stream`; caller owns all buffers.
 *
 * Activations, 1x128 blocks: x [batch][M][K] fp32 (16-byte aligned),
 *   q [batch][M][K] E4M3, sa [batch][K/128][M] fp32 (the GEMM's sa layout;
 *   batch = 1 for dense/contiguous, G for masked). K % 128 == 0.
 */
int fg_quant_act_1x128(const float* x, void* q, float* sa, int batch, int M, int K,
                       hipStream_t stream);

/* Weights, 128x128 blocks: w [G][N][K] fp32 (16-byte aligned; G = 1 for a
 *   dense weight), q [G][N][K] E4M3, sb [G][ceil(N/128)][K/128] fp32 (the
 *   GEMM's sb layout). K % 128 == 0; N >= 0 is arbitrary: when N is not a
 *   multiple of 128 the last row block of each expert holds the remaining
 *   N mod 128 rows, its amax and scale come from those rows alone (the same
 *   block the GEMM scales with the last sb row), and nothing past row N is
 *   read or written. The 2kiu.com explainer, section 4.3, names boundary
 *   handling for shapes that do not fill a block. */
int fg_quant_weight_128x128(const float* w, void* q, float* sb, int G, int N, int K,
                            hipStream_t stream);

/* Power-of-two variants of the two quantisers (same arguments, layouts and
 * errors): each block's scale amax / 448 (1 for an all-zero block) is rounded
 * up to the next power of two and floored at 2^-126, so x / scale is exact and
 * lies within [-448, 448]. Their scales satisfy the precondition of the
 * fg_*_pow2 GEMM calls. Reading taken for the MX scale rule, which the pages
 * name (2kiu.com explainer, section 7) without defining. */
int fg_quant_act_1x128_pow2(const float* x, void* q, float* sa, int batch, int M, int K,
                            hipStream_t stream);
int fg_quant_weight_128x128_pow2(const float* w, void* q, float* sb, int G, int N, int K,
                                 hipStream_t stream);

/* Static, human-readable description of a return code. */
const char* fg_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* FG_H */
