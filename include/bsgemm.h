/*
 * bsgemm -- block-scaled low-precision GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the library.  Plain pointers and sizes only.
 *
 * The operation is C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k]:
 *   - A is [M][K] and B is [N][K], both K-contiguous;
 *   - FP32 accumulation;
 *   - C is [M][N] BF16, rounded to nearest-even.
 * Sources:
 *   - "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera Rubin NVL72",
 *     section "Building the GEMM": block-scaled NVFP4 and FP8 E4M3 GEMMs; M x N
 *     output tiles sharing B along M; a K loop over staged operand chunks.
 *   - "Triton #11171 -- Why Two New NVFP4 Test Cases Produced Twelve
 *     Tensor-Memory Failures", sections "The missing case was defined by shape,
 *     layout, and execution mode together" and "Ragged mode added routing rather
 *     than a plain matrix": NVFP4 activations x a dense BF16 operand, ragged
 *     (routed) rows, BF16 output.
 *   - "Add sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic" (bitsandbytes
 *     PR #2030), sections "Methodology" and "The SIMT / MMA layer": a fused
 *     small-M GEMM with 4-bit weights and BF16 activations.
 *
 * Formats (bit layouts per the OCP Microscaling Formats (MX) v1.0 spec):
 *   NVFP4 operand [R][K], K % 32 == 0:
 *     codes  uint8 [R][K/2]   E2M1 values; element 2j in the low nibble of byte j
 *     scales uint8 [R][K/16]  E4M3 (FN) scale of each 16-element block along K
 *     tscale float            FP32 per-tensor decode scale
 *     value  = e2m1(code) * e4m3(scale) * tscale
 *              e4m3(scale) keeps its sign bit; a NaN scale code (0x7F, 0xFF)
 *              makes every output its block contributes to NaN
 *   MXFP8 operand [R][K], K % 32 == 0:
 *     codes  uint8 [R][K]     E4M3 (FN) values
 *     scales uint8 [R][K/32]  E8M0 scale of each 32-element block along K
 *     value  = e4m3(code) * 2^(scale - 127)
 *   MXFP4 operand [R][K], K % 32 == 0:
 *     codes  uint8 [R][K/2]   E2M1 values; element 2j in the low nibble of byte j
 *     scales uint8 [R][K/32]  E8M0 scale of each 32-element block along K
 *     value  = e2m1(code) * 2^(scale - 127)
 *   BF16 operands and outputs are uint16 bit patterns, row-major.
 *
 * Conventions common to every call:
 *   - Pointers are DEVICE pointers (visible to the current HIP device), unless
 *     noted.  The caller allocates and owns every buffer.  The library never
 *     allocates, frees or keeps a pointer after the call returns.
 *   - Buffers are dense and row-major; pitches are implied by the sizes.  Code
 *     buffers, scale buffers, x, w_bf16, x_bf16 and c_bf16 must be 16-byte
 *     aligned (the kernels fetch scales in 4- and 16-byte pieces).  Scalar
 *     slots (tensor scales, group offsets) need only their natural alignment.
 *   - Work is queued on `stream` (a hipStream_t; NULL = the null stream).  The
 *     call returns without waiting.  Keep the buffers alive until the stream
 *     has finished.
 *   - Every call returns a bsgemm_status.  All arguments are validated before
 *     anything is launched: a failing call launches nothing, and a passing call
 *     always launches its work (never a silent no-op).  bsgemm_last_error()
 *     gives a message for the last failure on the calling thread.
 *   - Preconditions that are documented but not checked on the device: inputs
 *     are finite, and group offsets are monotone.
 *   - Accuracy.  Quantizers are bit-exact.  The GEMMs accumulate in FP32 and
 *     round C once to BF16.  For BSGEMM_NVFP4, BSGEMM_MXFP8_EXACT, BSGEMM_MXFP4
 *     and every grouped and W4A16 call, every product is exact and the result
 *     differs from the exact sum only by FP32 summation order and the final
 *     rounding: |C - C_exact| <= 2^-8 |C_exact| + 1e-5 sum_k |a_k b_k| per
 *     element, for operands whose products and sums stay in FP32's normal
 *     range.  BSGEMM_MXFP8 is the exception; see bsgemm_run.
 *   - Results do not depend on the launch configuration chosen internally
 *     beyond FP32 summation order.
 */
#ifndef BSGEMM_H
#define BSGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bsgemm_status {
  BSGEMM_OK = 0,
  BSGEMM_ERR_INVALID_ARG = 1,   /* null pointer, negative size, num_groups < 1 */
  BSGEMM_ERR_UNSUPPORTED = 2,   /* k % 32 != 0, unknown format, bad format/scale combination */
  BSGEMM_ERR_BAD_ALIGNMENT = 3, /* a pointer is not aligned as its call requires */
  BSGEMM_ERR_DEVICE = 4,        /* no HIP device, or the current device is not gfx950 */
  BSGEMM_ERR_RESOURCE = 5,      /* no kernel configuration fits the problem */
  BSGEMM_ERR_LAUNCH = 6         /* the HIP runtime reported a launch failure */
};

enum bsgemm_format {
  BSGEMM_NVFP4 = 1,
  BSGEMM_MXFP8 = 2,        /* native scaled FP8 MFMA; see the accuracy note at bsgemm_run */
  BSGEMM_MXFP4 = 3,
  BSGEMM_MXFP8_EXACT = 4   /* MXFP8 operands, exact products on the BF16 MFMA */
};

/*
 * NVFP4 quantizer: x[rows][k] (FP32) -> codes, scales, *tensor_scale.
 *
 *   1. amax = max |x| over the whole tensor;
 *      s_t  = fl32(amax / 2688), where 2688 = 6 * 448.
 *   2. For each 16-element block along k:
 *        bamax  = max |x|;
 *        s_real = fl32(fl32(bamax / 6) / s_t);
 *        scale  = E4M3_RNE_satfinite(s_real).  Subnormal scales are kept.
 *        If s_t == 0, scale = 0.
 *   3. S = fl32(e4m3(scale) * s_t).  For each element:
 *        code = signbit(x) << 3 | E2M1_RNE_satfinite(|fl32(x / S)|).
 *      If S == 0, code = signbit(x) << 3.
 * Every FP32 step is IEEE round-to-nearest-even.  The output is bit-exact.
 *
 * Scale recipe: "scale = block absmax / 6, over the tensor scale"; "tensor
 * scale = absmax / (6 * 448)".  The pages name the format ("Together AI Ports
 * ThunderKittens ...", section "Building the GEMM"; "Triton #11171 ...",
 * section "The existing tests already mentioned NVFP4") but do not print the
 * recipe.
 *
 * Arguments:
 *   x            device float[rows][k], 16-byte aligned
 *   codes        device uint8[rows][k/2], 16-byte aligned (written)
 *   scales       device uint8[rows][k/16], 16-byte aligned (written)
 *   tensor_scale device float[1] (written).  Used as the amax slot during the
 *                call: it holds amax bits until the call's last kernel has run.
 * Sizes: rows >= 0, k >= 0, k % 32 == 0.
 * With rows * k == 0, *tensor_scale is set to 0.
 * Launches 4 kernels on `stream`: reset slot, amax, finalize, encode.
 */
int bsgemm_quantize_nvfp4(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                          uint8_t* scales, float* tensor_scale, void* stream);

/*
 * MXFP8 quantizer: x[rows][k] (FP32) -> codes uint8[rows][k], scales uint8[rows][k/32].
 *
 *   For each 32-element block along k:
 *     bamax = max |x|;
 *     e     = ceil(log2(bamax / 448)), computed exactly as
 *             min{e : 448 * 2^e >= bamax}, clamped to [-127, 127]
 *             (bamax == 0 gives -127);
 *     scale = e + 127 (E8M0);
 *     code  = signbit(x) << 7 | E4M3_RNE_satfinite(|x * 2^-e|).
 * The output is bit-exact.  Format named on the pages: "MXFP" ("Triton
 * #11171 ...", section "The broader related matrix protected neighboring
 * policy"); "FP8 E4M3" ("Together AI Ports ThunderKittens ...", section
 * "Building the GEMM").
 *
 * Arguments:
 *   x      device float[rows][k], 16-byte aligned
 *   codes  device uint8[rows][k], 16-byte aligned (written)
 *   scales device uint8[rows][k/32], 16-byte aligned (written)
 * Sizes: rows >= 0, k >= 0, k % 32 == 0.
 */
int bsgemm_quantize_mxfp8(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                          uint8_t* scales, void* stream);

/*
 * MXFP4 quantizer: x[rows][k] (FP32) -> codes uint8[rows][k/2], scales uint8[rows][k/32].
 *
 *   For each 32-element block along k:
 *     bamax = max |x|;
 *     e     = ceil(log2(bamax / 6)), computed exactly as
 *             min{e : 6 * 2^e >= bamax}, clamped to [-127, 127]
 *             (bamax == 0 gives -127);
 *     scale = e + 127 (E8M0);
 *     code  = signbit(x) << 3 | E2M1_RNE(|x * 2^-e|)  (never saturates:
 *             |x * 2^-e| <= 6 by the choice of e).
 *   Element 2j of a row goes to the low nibble of byte j.
 * This is the MXFP8 rule with E2M1's largest value (6) in place of E4M3's
 * (448).  The output is bit-exact.  Format family named on the pages:
 * "MXFP" ("Triton #11171 ...", section "The broader related matrix protected
 * neighboring policy"); the 4-bit E2M1 element is the one of NVFP4 ("Together
 * AI Ports ThunderKittens ...", section "Building the GEMM").
 *
 * Arguments:
 *   x      device float[rows][k], 16-byte aligned
 *   codes  device uint8[rows][k/2], 16-byte aligned (written)
 *   scales device uint8[rows][k/32], 16-byte aligned (written)
 * Sizes: rows >= 0, k >= 0, k % 32 == 0.
 */
int bsgemm_quantize_mxfp4(int64_t rows, int64_t k, const float* x, uint8_t* codes,
                          uint8_t* scales, void* stream);

/*
 * Dense block-scaled GEMM with both operands in format `fmt`:
 *   C[m][n] = bf16_RNE( sum_k deq(A)[m][k] * deq(B)[n][k] )
 * with FP32 accumulation.  For NVFP4 the sum runs over
 * (e2m1 * e4m3)_A * (e2m1 * e4m3)_B and is then multiplied by
 * (*a_tscale) * (*b_tscale).  MXFP8 and MXFP4 apply their E8M0 block scales
 * inside the matrix-core product.
 *
 * MXFP8 accuracy.  The two MXFP8 paths take the same operands:
 *   BSGEMM_MXFP8        the native scaled FP8 MFMA, at the FP8 rate.  It sums
 *                       each aligned group of 8 products to about 14 bits
 *                       below the group's largest product (measured on
 *                       gfx950; the groups are then combined in FP32).  The
 *                       per-element bound is therefore
 *                         2^-8 |C| + 1e-5 sum_k |a_k b_k| + 2^-10 sum_groups max |a_k b_k|.
 *                       The last term matters only where one 32-element block
 *                       holds values ~2^10 or more apart next to each other.
 *                       On quantizer output of data without such spread
 *                       (e.g. N(0,1)), the plain bound holds.
 *   BSGEMM_MXFP8_EXACT  every e4m3(code) * 2^(scale - 127) expanded exactly to
 *                       BF16 and multiplied on the BF16 MFMA: the plain bound
 *                       (FP32 summation order only) on every operand whose
 *                       products stay in FP32's normal range, at half the FP8
 *                       rate.
 * Source: "Together AI Ports ThunderKittens GEMM Kernels to NVIDIA Vera Rubin
 * NVL72", section "Building the GEMM" (NVFP4 and FP8 E4M3 GEMMs, 16k square);
 * MXFP4 is the MX member with the E2M1 element ("Triton #11171 ...", section
 * "The broader related matrix protected neighboring policy").
 *
 * Arguments:
 *   fmt                 BSGEMM_NVFP4, BSGEMM_MXFP8, BSGEMM_MXFP8_EXACT or
 *                       BSGEMM_MXFP4
 *   a, a_scales         operand A [m][k] in the layout of `fmt`
 *   a_tscale, b_tscale  device float[1] for NVFP4; must be NULL for the MX
 *                       formats
 *   b, b_scales         operand B [n][k], in the same format
 *   c_bf16              device uint16[m][n] (written)
 * Sizes: m, n, k >= 0, k % 32 == 0.
 *   m == 0 or n == 0: returns BSGEMM_OK and launches nothing.
 *   k == 0: C is all zeros.
 */
int bsgemm_run(int fmt, int64_t m, int64_t n, int64_t k,
               const uint8_t* a, const uint8_t* a_scales, const float* a_tscale,
               const uint8_t* b, const uint8_t* b_scales, const float* b_tscale,
               uint16_t* c_bf16, void* stream);

/*
 * Ragged grouped GEMM: NVFP4 activations x dense BF16 weights.
 * Rows off[g] .. off[g+1]-1 of A belong to group g and are multiplied with
 * W[g]:
 *   C[r][n] = bf16_RNE( s_t * sum_k (e2m1 * e4m3)(A)[r][k] * W[g][n][k] )
 * Source: "Triton #11171 -- Why Two New NVFP4 Test Cases Produced Twelve
 * Tensor-Memory Failures", sections "Ragged mode added routing rather than a
 * plain matrix" and "NVFP4 x dense matmul": routed per-slice activations meet
 * their slice's dense RHS, BF16 output.
 *
 * Arguments:
 *   num_groups    G >= 1
 *   m_total       total rows of A and C
 *   a, a_scales, a_tscale
 *                 NVFP4 activations [m_total][k], one tensor scale for all rows
 *   group_offsets device int32[G+1], with off[0] = 0, off[G] = m_total, and
 *                 non-decreasing.  Empty groups are allowed.  Read on the
 *                 device; the host never waits for it.
 *   w_bf16        device uint16[G][n][k]
 *   c_bf16        device uint16[m_total][n] (written)
 * Sizes: m_total, n, k >= 0, k % 32 == 0.
 *   m_total == 0 or n == 0: BSGEMM_OK and nothing is launched.
 */
int bsgemm_grouped_run(int num_groups, int64_t m_total, int64_t n, int64_t k,
                       const uint8_t* a, const uint8_t* a_scales, const float* a_tscale,
                       const int32_t* group_offsets, const uint16_t* w_bf16,
                       uint16_t* c_bf16, void* stream);

/* Element type of the dense grouped operand. */
enum bsgemm_wtype {
  BSGEMM_W_BF16 = 1,
  BSGEMM_W_F16 = 2
};

/*
 * Ragged grouped GEMM with the routing and epilogue variants: NVFP4
 * activations x dense BF16 or FP16 weights.  For logical row r of group g
 * (off[g] <= r < off[g+1]):
 *   src(r)  = gather_idx[r] if gather_idx is given, else r   (row of A read)
 *   y[r][n] = (s_t * sum_k (e2m1 * e4m3)(A)[src(r)][k] * W[g][n][k] + bias[g][n]) * gamma[r]
 *   C[dst(r)][n] = bf16_RNE(y[r][n]),  dst(r) = scatter_idx[r] if given, else r
 * with FP32 accumulation and FP32 epilogue arithmetic; an absent bias adds 0
 * and an absent gamma multiplies by 1.  Bias is added to the scaled product
 * and gamma multiplies the sum: the order in which the page lists them.
 * Source: "Triton #11171 -- Why Two New NVFP4 Test Cases Produced Twelve
 * Tensor-Memory Failures", sections "Scatter changes where output rows are
 * written" (a permutation of output rows), "Gamma adds a per-row scaling
 * input", "The ordinary variants also exercise the shared bias route"
 * (matmul + bias + optional gamma + optional scatter), "Filter 3: gather
 * variants are excluded" (gathered activation rows) and the rhs_dtype sweep
 * over bfloat16 and float16 in "The missing case was defined by shape,
 * layout, and execution mode together".
 *
 * Arguments (as bsgemm_grouped_run, plus):
 *   a_rows       rows of A (and of a_scales).  Must equal m_total when
 *                gather_idx is NULL.
 *   w_dtype      BSGEMM_W_BF16 or BSGEMM_W_F16: the bit patterns in w
 *   w            device uint16[G][n][k], 16-byte aligned
 *   bias         device float[G][n] or NULL
 *   gamma        device float[m_total] or NULL
 *   gather_idx   device int32[m_total] or NULL; entries in [0, a_rows)
 *   scatter_idx  device int32[m_total] or NULL; a permutation of
 *                [0, m_total), so every row of C is written once
 *   bias, gamma and the index arrays need 4-byte alignment.
 * Device-side preconditions (documented, not checked on the host): offsets
 * as for bsgemm_grouped_run; index entries in range.  A gather entry out of
 * range reads a zero row and a scatter entry out of range skips its store,
 * so bad indices never touch memory outside the buffers; a scatter that is
 * not a permutation leaves some rows of C unwritten.
 * Sizes: m_total, n, k, a_rows >= 0, k % 32 == 0, a_rows * k / 2 < 2^31.
 *   m_total == 0 or n == 0: BSGEMM_OK and nothing is launched.
 * With all four of bias, gamma, gather_idx and scatter_idx NULL and
 * w_dtype BSGEMM_W_BF16 this is bsgemm_grouped_run.
 */
int bsgemm_grouped_run_ex(int num_groups, int64_t m_total, int64_t n, int64_t k, int64_t a_rows,
                          const uint8_t* a, const uint8_t* a_scales, const float* a_tscale,
                          const int32_t* group_offsets, int w_dtype, const uint16_t* w,
                          const float* bias, const float* gamma, const int32_t* gather_idx,
                          const int32_t* scatter_idx, uint16_t* c_bf16, void* stream);

/*
 * Inner-expert (K-ragged) grouped GEMM: the groups split the contraction
 * dimension K instead of the rows.  For each group g:
 *   C[g][m][n] = bf16_RNE( s_t * sum_{k_offsets[g] <= k < k_offsets[g+1]}
 *                                  (e2m1 * e4m3)(A)[m][k] * W[n][k] )
 * with FP32 accumulation.  Each group's K slice is padded in A and W to a
 * multiple of 256 elements (16 E4M3 scale bytes per row); the padding takes
 * part in the sum like any other element, so zero padding (what quantizing
 * zero-padded data gives) contributes nothing.  An empty slice gives C[g] = 0.
 * Source: "Triton #11171 -- Why Two New NVFP4 Test Cases Produced Twelve
 * Tensor-Memory Failures", sections "Why `pad_a` represents the K-ragged
 * boundary" (the activation is ragged along dimension 1, K, with ragged
 * padding on A) and "The skip logic is part of the regression contract"
 * (a microscaled activation in inner-expert mode requires that padding).
 *
 * Arguments:
 *   num_groups   G >= 1
 *   a, a_scales, a_tscale  NVFP4 activations [m][k], one tensor scale
 *   k_offsets    device int32[G+1]: k_offsets[0] = 0, k_offsets[G] = k,
 *                non-decreasing multiples of 256.  Read on the device; an
 *                offset that breaks this is clamped to [0, k] and rounded
 *                down to a multiple of 256 (documented, not an error).
 *   w_dtype      BSGEMM_W_BF16 or BSGEMM_W_F16
 *   w            device uint16[n][k] (the dense operand, same K layout)
 *   c_bf16       device uint16[G][m][n] (written)
 * Sizes: m, n, k >= 0; k % 256 == 0 (else BSGEMM_ERR_UNSUPPORTED).
 *   m == 0 or n == 0: BSGEMM_OK and nothing is launched.
 */
int bsgemm_grouped_kragged_run(int num_groups, int64_t m, int64_t n, int64_t k, const uint8_t* a,
                               const uint8_t* a_scales, const float* a_tscale, const int32_t* k_offsets,
                               int w_dtype, const uint16_t* w, uint16_t* c_bf16, void* stream);

/*
 * Small-M weight-only 4-bit GEMM: BF16 activations x NVFP4 weights.
 *   C[m][n] = bf16_RNE( s_tW * sum_k X[m][k] * (e2m1 * e4m3)(W)[n][k] )
 * Each weight byte is read from HBM once.  The kernel family is chosen by m:
 *   - VALU dot products for the smallest m;
 *   - BF16 MFMA tiles for larger m.
 * Source: "Add sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic",
 * sections "Methodology", "The SIMT / MMA layer" and the tile-selection
 * follow-up: a fused dequant + GEMM for small M, choosing SIMT vs matrix-core
 * kernels and the tile width along N by M.
 *
 * Arguments:
 *   x_bf16                device uint16[m][k]
 *   w, w_scales, w_tscale NVFP4 weights [n][k]
 *   c_bf16                device uint16[m][n] (written)
 * Sizes: m, n, k >= 0, k % 32 == 0.
 *   m == 0 or n == 0: BSGEMM_OK and nothing is launched.
 */
int bsgemm_w4a16_run(int64_t m, int64_t n, int64_t k, const uint16_t* x_bf16,
                     const uint8_t* w, const uint8_t* w_scales, const float* w_tscale,
                     uint16_t* c_bf16, void* stream);

/*
 * W4A16 configurations and a forced path, for calibrating the selector the
 * way "Add sm121 (GB10) tier to the 4-bit GEMM dispatch heuristic",
 * tile-selection follow-up, does: one build runs every legal configuration
 * on every shape through the same forced path, the selector's decisions can
 * be enumerated exhaustively on the host, and no configuration id launches
 * nothing (an invalid one is an error, never a silent no-op).
 *
 * Configurations (ids 0 .. bsgemm_w4a16_num_configs() - 1):
 *   "valu_gemv"          vector-ALU dot products, one X row per grid row
 *                        (re-reads W once per row; m <= 65535);
 *   "mfma_m{16,32,64}_n{fit,16,32,64}"
 *                        BF16 MFMA kernel with that m tile and that many W
 *                        rows per workgroup (the tile width along N); "fit"
 *                        takes the narrowest width (16..64) whose grid fits
 *                        in one wave of 256 workgroups; further variants of
 *                        it differ in ring depth and K split (suffixes);
 *   "tile_m16_n64", "tile_m64_n64", "tile_m128_n128"
 *                        BF16 MFMA tile kernel, one workgroup per m x n
 *                        output tile over all of K; k must be a multiple of
 *                        512, 256 and 128 respectively, otherwise the call
 *                        fails with BSGEMM_ERR_UNSUPPORTED.
 * bsgemm_w4a16_run runs bsgemm_w4a16_select(m, n, k), unless the environment
 * variable BSGEMM_W4A16_FORCE_CONFIG holds a configuration id or name; a
 * value that names none makes the call fail with BSGEMM_ERR_UNSUPPORTED.
 * Every configuration computes the same C within the documented tolerance.
 */
int bsgemm_w4a16_num_configs(void);

/* Static name of configuration `config`; NULL if there is none. */
const char* bsgemm_w4a16_config_name(int config);

/* The configuration bsgemm_w4a16_run picks for (m, n, k) without an
 * override; host-only, no device needed.  -1 for negative sizes or
 * k % 32 != 0. */
int bsgemm_w4a16_select(int64_t m, int64_t n, int64_t k);

/* bsgemm_w4a16_run with configuration `config` forced (the environment
 * override is ignored).  BSGEMM_ERR_UNSUPPORTED for an unknown id or a k the
 * configuration does not take; BSGEMM_ERR_RESOURCE when m exceeds what the
 * configuration takes. */
int bsgemm_w4a16_run_config(int config, int64_t m, int64_t n, int64_t k, const uint16_t* x_bf16,
                            const uint8_t* w, const uint8_t* w_scales, const float* w_tscale,
                            uint16_t* c_bf16, void* stream);

/* Static name of a status code ("BSGEMM_OK", ...); "unknown status" otherwise. */
const char* bsgemm_status_string(int status);

/* Message of the last failing call on this thread ("" if none).  Valid until
 * the next call into the library on this thread. */
const char* bsgemm_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int bsgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSGEMM_H */
