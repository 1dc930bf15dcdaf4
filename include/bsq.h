/*
 * bsq.h -- C ABI of libbsq, the block-scaled quantized linear-layer hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * Operations: NVFP4 quantization (rowwise / columnwise, round-to-nearest-even or
 * Philox-keyed stochastic rounding, optional 16-point random Hadamard transform),
 * NVFP4 dequantization, the MXFP8 cast, the standalone Hadamard transform, and the
 * block-scaled GEMM C = A * B^T that consumes the quantized operands with fp32
 * accumulation.
 *
 * Conventions shared by every entry point:
 *   - Tensors are row-major and contiguous.  A bf16 tensor x has shape [rows][cols].
 *   - "Rowwise" blocks run along cols; "columnwise" blocks run along rows and are
 *     stored as the rowwise quantization of x^T, i.e. with shape [cols][...].  A GEMM
 *     operand is always the direction whose blocks run along the contraction dim,
 *     so every GEMM here is C[M][N] = A[M][K] * B[N][K]^T with both operands stored
 *     along K (fprop: X and W rowwise; dgrad: dY rowwise, W columnwise; wgrad: dY
 *     and X columnwise).  This is the per-direction operand choice of the GEMM
 *     dispatch on the page "[Pytorch][Common] Hybrid quantization"
 *     (TransformerEngine PR #2817, Description and dispatch flowchart).
 *   - Every pointer argument that names tensor data is a DEVICE pointer; every
 *     device pointer must be 16-byte aligned.  The caller allocates and owns all
 *     buffers, scratch space included (the `workspace` arguments); the library allocates
 *     no device memory and keeps no state between calls besides the thread-local error
 *     message.
 *   - Work is enqueued asynchronously on hip_stream (a hipStream_t; NULL is the
 *     null stream).  Return values report argument validation and launch errors
 *     only; faults during kernel execution surface at the next synchronisation.
 *   - Status codes: 0 (BSQ_OK) or one of the BSQ_ERR_* values; validation happens
 *     on the host before any HIP call, so a rejected call touches no device state.
 *     bsq_last_error() returns a message for the last failing call of the thread.
 */
#ifndef BSQ_H
#define BSQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bsq_status {
    BSQ_OK = 0,
    BSQ_ERR_NULL = 1,        /* a required pointer is NULL                          */
    BSQ_ERR_SHAPE = 2,       /* a dimension is negative or not a required multiple  */
    BSQ_ERR_ARG = 3,         /* an enum/flag value is out of range                  */
    BSQ_ERR_UNSUPPORTED = 4, /* a valid combination this library does not implement */
    BSQ_ERR_HIP = 5,         /* a HIP runtime call (launch) failed                  */
    BSQ_ERR_ALIGN = 6        /* a device pointer is not 16-byte aligned            */
};

/* direction bitmask: which quantizations to produce (the usage flags of a quantizer). */
#define BSQ_ROW 1
#define BSQ_COL 2
/* OR'ed into an MXFP8 cast's direction: the codes it writes are in the slab layout */
#define BSQ_MX_SLAB 4
/* element rounding */
#define BSQ_RNE 0
#define BSQ_SR 1
/* GEMM operand formats */
#define BSQ_FMT_NVFP4 0
#define BSQ_FMT_MXFP8 1
/* flags OR'ed into BSQ_FMT_NVFP4: that operand's tensor scale is one float per row */
#define BSQ_FMT_A_ROWSCALED 0x10
#define BSQ_FMT_B_ROWSCALED 0x20
/* flags OR'ed into BSQ_FMT_MXFP8: that operand's codes are in the slab layout */
#define BSQ_FMT_MX_SLAB_A 0x40
#define BSQ_FMT_MX_SLAB_B 0x80
#define BSQ_FMT_MX_SLAB (BSQ_FMT_MX_SLAB_A | BSQ_FMT_MX_SLAB_B)

/*
 * The slab layout of an MXFP8 code matrix [rows][K] (K % 64 == 0): a layout of the same
 * rows * K bytes for the GEMM, not part of the format.  Rows are taken in bands of 256 (the
 * last band holds the remaining n = rows - 256 b); band b starts at byte 256 b K and holds
 * its n rows as K/64 consecutive slabs of n x 64 bytes, so byte k of row r is at
 *   256 b K + (k / 64) n 64 + (r - 256 b) 64 + k % 64,   b = r / 256.
 * A GEMM tile's rows are one band and each 64-element K slice of them one contiguous
 * block, which the GEMM's loads fill LDS from at about 1.6 times the rate of 64-byte pieces
 * of row-major rows.  Scales keep their row-major layout.
 */
/* grouped GEMM modes */
#define BSQ_GROUP_M 1   /* groups split the rows of A and C (per-expert fprop / dgrad) */
#define BSQ_GROUP_K 2   /* groups split the contraction (per-expert wgrad)             */
/* GEMM output types */
#define BSQ_OUT_BF16 0
#define BSQ_OUT_F32 1

/*
 * nvfp4_quantize -- NVFP4 quantization of a bf16 tensor.
 *
 * Defines: the recipe of the page "Add an NVFP4 quantization converter"
 * (torchtitan PR #3914): 16-element blocks with one inner scale each and one outer
 * per-tensor scale (review thread on the recipe's inner 1x16 scale), stochastic
 * rounding keyed by a Philox seed and an RHT whose +-1 sign vector both GEMM
 * operands share (Summary, "What changed").  Numerics, per block of 16 values v:
 *   A     = max |v| over the tensor (over the transformed values when RHT is on,
 *           separately per direction),
 *   S     = 2688 / A in fp32 (6 * 448: the largest E2M1 code times the largest E4M3
 *           value); A = 0 gives S = 1; an infinite S is clamped to FLT_MAX,
 *   s_b   = E4M3_RNE_saturating((blockmax * S) / 6)  -- the block scale byte,
 *   codes = E2M1(v * (S / fp32(s_b))), RNE or SR; all zero when s_b == 0.
 * With SR, element i (linear index in the OUTPUT layout of its direction) is
 * rounded up with probability equal to its position between the two neighbouring
 * E2M1 values, using word i%4 of Philox4x32-10(counter = (lo32(i/4), hi32(i/4),
 * sr_stream, d), key = (lo32(sr_seed), hi32(sr_seed))), d = 0 rowwise, 1
 * columnwise; it is compared as (word >> 8) * 2^-24 < p.  Block scales are always RNE.
 *
 * Arguments:
 *   x          [rows][cols] bf16 (device).
 *   direction  BSQ_ROW, BSQ_COL or both.  BSQ_ROW needs cols % 16 == 0; BSQ_COL
 *              needs rows % 16 == 0; in every case cols % 8 == 0.
 *   rounding   BSQ_RNE or BSQ_SR (sr_seed/sr_stream are ignored under BSQ_RNE).
 *   rht_signs  NULL, or 16 int8 values each +1 or -1 (device): apply the 16-point
 *              random Hadamard transform y = x diag(d) H16 / 4 (Sylvester order,
 *              fp32 butterfly with strides 1, 2, 4, 8) to each 16-block along the
 *              blocked dimension before quantizing; the transformed values are
 *              not rounded to bf16.
 *   row_codes  [rows][cols/2] uint8: element 2j in bits 3:0 of byte j, 2j+1 in
 *              bits 7:4 (sign in bit 3 of a nibble); row_scales [rows][cols/16]
 *              E4M3 bytes.  Required iff BSQ_ROW.
 *   col_codes  [cols][rows/2], col_scales [cols][rows/16]; required iff BSQ_COL.
 *   amax_out   float[2] (device): [0] the rowwise amax A, [1] the columnwise one.
 *              Required.
 *   s_enc_out  float[2] (device): the matching tensor scales S.  Required.
 *              Slots of an unrequested direction are left unspecified.
 *   workspace  BSQ_NVFP4_QUANTIZE_WORKSPACE_BYTES of device scratch (16-byte aligned),
 *              owned by the caller: the amax pass stores per-workgroup partial maxima there
 *              and the encode pass reads them.  No initial contents are needed and the
 *              contents afterwards are unspecified; each call writes every slot it reads, so
 *              a call never depends on an earlier one (graph replays included).  The
 *              workspace must not overlap another argument, and two calls that may run at
 *              the same time (on different streams) need different workspaces.  Required
 *              unless the tensor is empty.
 */
#define BSQ_NVFP4_QUANTIZE_WORKSPACE_BYTES 8192
int nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int direction, int rounding,
                   uint64_t sr_seed, uint32_t sr_stream, const int8_t* rht_signs,
                   uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                   uint8_t* col_scales, float* amax_out, float* s_enc_out, void* workspace,
                   void* hip_stream);

/*
 * nvfp4_quantize_fprop_wgrad -- one bf16 activation quantized for both of its GEMMs in one
 * amax pass and one encode pass: rowwise NVFP4 with RNE and no transform (the forward operand,
 * exactly nvfp4_quantize with direction BSQ_ROW, rounding BSQ_RNE, rht_signs NULL) and
 * columnwise NVFP4 with the given rounding and transform (the wgrad operand, exactly
 * nvfp4_quantize with direction BSQ_COL and these rounding, sr_seed, sr_stream and rht_signs).
 *
 * Defines: the recipe of the page "Add an NVFP4 quantization converter" (Summary: the random
 * Hadamard transform and stochastic rounding apply to the backward operands only) applied to
 * the activation X, whose columnwise quantization is made in the forward pass and saved for
 * wgrad (Table 1 takeaway: quantized activations are what is saved).
 *
 * Arguments: as for nvfp4_quantize with direction BSQ_ROW | BSQ_COL (rows % 16 == 0,
 * cols % 16 == 0); amax_out[0] / s_enc_out[0] are the rowwise amax and tensor scale of the
 * untransformed values, [1] the columnwise ones (of the transformed values with RHT).
 * Errors: those of nvfp4_quantize for these arguments.
 */
int nvfp4_quantize_fprop_wgrad(const void* x, int64_t rows, int64_t cols, int rounding,
                               uint64_t sr_seed, uint32_t sr_stream, const int8_t* rht_signs,
                               uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                               uint8_t* col_scales, float* amax_out, float* s_enc_out,
                               void* workspace, void* hip_stream);

/*
 * nvfp4_col_mxfp8_row_quantize -- one bf16 tensor quantized to two formats, one per direction,
 * in one pass over it: NVFP4 columnwise (exactly nvfp4_quantize with direction BSQ_COL) and
 * MXFP8 rowwise (exactly mxfp8_quantize with direction BSQ_ROW).
 *
 * Defines: hybrid (per-direction) quantization, page "[Pytorch][Common] Hybrid quantization"
 * (Description: rowwise and columnwise operands of one tensor may use different formats).
 * This pairing serves the backward operand dY in the per-direction recipe of this library:
 * rowwise MXFP8 for the dgrad GEMM, columnwise NVFP4 (with RHT and SR) for the wgrad GEMM.  The NVFP4 part's
 * amax pass still reads x; the MXFP8 codes come from the encode pass's read, so x is read twice
 * in all instead of three times.
 *
 * Arguments: x, rows, cols, rounding, sr_seed, sr_stream, rht_signs, col_codes, col_scales,
 * amax_out, s_enc_out and workspace as for nvfp4_quantize with direction BSQ_COL (rows % 16 ==
 * 0; amax_out / s_enc_out slots as nvfp4_quantize writes them for BSQ_COL); the RHT and
 * SR apply to the NVFP4 part only.  mx_layout 0 (row-major codes) or BSQ_MX_SLAB;
 * mx_row_codes [rows][cols] E4M3 bytes (row-major, or the slab layout, which needs cols % 64
 * == 0) and mx_row_scales [rows][cols/32] E8M0 bytes as mxfp8_quantize writes them (cols % 32
 * == 0); required unless the tensor is empty.
 * Errors: those of nvfp4_quantize and mxfp8_quantize for these arguments; BSQ_ERR_ARG for
 * another mx_layout.
 */
int nvfp4_col_mxfp8_row_quantize(const void* x, int64_t rows, int64_t cols, int rounding,
                                 uint64_t sr_seed, uint32_t sr_stream, const int8_t* rht_signs,
                                 uint8_t* col_codes, uint8_t* col_scales, float* amax_out,
                                 float* s_enc_out, void* workspace, int mx_layout,
                                 uint8_t* mx_row_codes, uint8_t* mx_row_scales, void* hip_stream);

/*
 * nvfp4_quantize_noalloc -- nvfp4_quantize without the workspace argument, for callers that
 * cannot allocate device memory or pass scratch: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, numerics, outputs and errors are those
 * of nvfp4_quantize; the partial maxima go to a fixed device array inside the library instead
 * (BSQ_NVFP4_QUANTIZE_WORKSPACE_BYTES per GPU, set aside when the library is loaded and held
 * until the process ends; its device address is looked up on the first call on each GPU).
 * The array's size does not depend on the tensor, so every size nvfp4_quantize accepts is
 * accepted.  Every call on a GPU shares that GPU's array: calls that may run at the same time
 * on one GPU (on different streams, or from threads that do not order their calls) race and
 * give unspecified results.  The array needs no initial contents (each call writes every
 * slot it reads), so nothing carries over from one call to the next.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 */
int nvfp4_quantize_noalloc(const void* x, int64_t rows, int64_t cols, int direction, int rounding,
                           uint64_t sr_seed, uint32_t sr_stream, const int8_t* rht_signs,
                           uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                           uint8_t* col_scales, float* amax_out, float* s_enc_out, void* hip_stream);

/*
 * nvfp4_quantize_rowscaled -- rowwise NVFP4 quantization with one outer fp32 scale per
 * row instead of one per tensor.
 *
 * Defines: the "row_scaled_nvfp4" rowwise quantizer of the Composer-style recipe on the
 * page "[Pytorch][Common] Hybrid quantization" (TransformerEngine PR #2817, Description),
 * and the recipe with "outer scale rowwise, inner scale 1x16" raised in the review of "Add
 * an NVFP4 quantization converter" (torchtitan PR #3914).  Row r is quantized exactly as
 * nvfp4_quantize(direction = BSQ_ROW) quantizes a tensor, with A replaced by the row's amax
 * A_r (over the transformed values when RHT is on) and S by S_r = 2688 / A_r (A_r = 0 gives
 * S_r = 1; infinite S_r is clamped to FLT_MAX).  SR draws use the element's linear index
 * r * cols + c and d = 0, as in the per-tensor rowwise quantization.
 *
 * Arguments:
 *   x          [rows][cols] bf16 (device); cols % 16 == 0.
 *   rounding, sr_seed, sr_stream, rht_signs: as for nvfp4_quantize.
 *   codes      [rows][cols/2] uint8, scales [rows][cols/16] E4M3 (device), laid out as the
 *              rowwise outputs of nvfp4_quantize.
 *   amax_rows  float[rows] (device): A_r.  s_enc_rows float[rows] (device): S_r.
 * A row is read from memory once when cols <= 8192 and twice otherwise.  The call uses no
 * memory beyond its arguments.
 */
int nvfp4_quantize_rowscaled(const void* x, int64_t rows, int64_t cols, int rounding,
                             uint64_t sr_seed, uint32_t sr_stream, const int8_t* rht_signs,
                             uint8_t* codes, uint8_t* scales, float* amax_rows,
                             float* s_enc_rows, void* hip_stream);

/*
 * nvfp4_dequantize -- bf16 value of an NVFP4 tensor: out = bf16_RNE((E2M1(code) *
 * fp32(s_b)) / S) (the product is exact).  This is the "rowwise_dequantized"
 * columnwise source of the hybrid quantizer on the page "[Pytorch][Common] Hybrid
 * quantization" (TransformerEngine PR #2817, "Enable columnwise_source and hybrid
 * recipes"): the backward operand is re-quantized from dequantize(rowwise(x)).
 *   codes [rows][cols/2], scales [rows][cols/16], s_enc float[1] (all device);
 *   out [rows][cols] bf16 (device).  cols % 16 == 0.
 */
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s_enc,
                     int64_t rows, int64_t cols, void* out, void* hip_stream);

/*
 * mxfp8_quantize -- MXFP8 cast of a bf16 tensor: 32-element blocks, one E8M0 scale
 * per block, E4M3 codes (block size and per-block scale count: page "[Pytorch]
 * [Common] Hybrid quantization", review thread on MXFP8_BLOCK_SCALING_SIZE and the
 * columnwise scale count; scale rule: the OCP MX shared exponent, from the MX
 * paper cited in the TorchAO review page's references).  Per block:
 *   X = floor(log2 blockmax) - 8 clamped to [-127, 127], scale byte X + 127,
 *   codes = E4M3_RNE_saturating(v * 2^-X) (values above 448 clip);
 *   an all-zero block gives scale byte 0 and codes 0.
 * Arguments: x [rows][cols] bf16; BSQ_ROW needs cols % 32 == 0, BSQ_COL needs
 * rows % 32 == 0, always cols % 8 == 0.  row_codes [rows][cols], row_scales
 * [rows][cols/32]; col_codes [cols][rows], col_scales [cols][rows/32] (required
 * iff the direction is requested).  direction | BSQ_MX_SLAB writes the requested codes in
 * the slab layout (rowwise: cols % 64 == 0; columnwise: rows % 64 == 0), the scales as
 * before.
 */
int mxfp8_quantize(const void* x, int64_t rows, int64_t cols, int direction,
                   uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                   uint8_t* col_scales, void* hip_stream);

/*
 * mxfp8_requantize_nvfp4 -- MXFP8 cast (as mxfp8_quantize) of the bf16 tensor
 * nvfp4_dequantize(codes, scales, s_enc), computed from the NVFP4 rowwise codes and scales
 * without materialising the bf16 tensor: the "rowwise_dequantized" columnwise source of the
 * hybrid quantizer (page "[Pytorch][Common] Hybrid quantization", TransformerEngine PR
 * #2817, commit note "Enable columnwise_source and hybrid recipes": the backward operand is
 * built from dequantize(rowwise(x))), fused.  Bit-identical to nvfp4_dequantize followed by
 * mxfp8_quantize.
 *   codes [rows][cols/2], scales [rows][cols/16], s_enc float[1]: an NVFP4 rowwise tensor
 *              (device).  cols % 16 == 0.
 *   direction, outputs and their preconditions as for mxfp8_quantize.
 */
int mxfp8_requantize_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* s_enc,
                           int64_t rows, int64_t cols, int direction, uint8_t* row_codes,
                           uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales,
                           void* hip_stream);

/*
 * rht_apply -- the 16-point random Hadamard transform on its own: out = fp32 of
 * each 16-block of x times diag(d) H16 / 4 (same definition and evaluation order as
 * in nvfp4_quantize; page "Add an NVFP4 quantization converter", Summary: the
 * transform cancels in a GEMM only when both operands share the sign vector).
 *   x [rows][cols] bf16; axis 1: blocks of 16 consecutive elements of a row
 *   (cols % 16 == 0); axis 0: blocks of 16 consecutive elements of a column
 *   (rows % 16 == 0).  cols % 8 == 0.  signs: 16 int8 +-1 (device).
 *   out [rows][cols] fp32 (device).
 */
int rht_apply(const void* x, int64_t rows, int64_t cols, int axis, const int8_t* signs,
              float* out, void* hip_stream);

/*
 * blockscaled_gemm -- C[M][N] = alpha * sum_k A[m][k] B[n][k] on block-scaled
 * operands with fp32 accumulation (the fprop / dgrad / wgrad GEMM of a quantized
 * linear layer; page "Add an NVFP4 quantization converter", Design notes: the
 * GEMM on low-precision operands is what the recipe buys).
 *   fmt BSQ_FMT_NVFP4: a_codes [M][K/2], a_scales [M][K/16] (E4M3), a_s_enc float[1]
 *       (device, the operand's tensor scale S), likewise for B; alpha =
 *       1/(S_a * S_b).  K % 32 == 0.
 *   fmt BSQ_FMT_NVFP4 | BSQ_FMT_A_ROWSCALED and/or BSQ_FMT_B_ROWSCALED: that operand is
 *       row-scaled (nvfp4_quantize_rowscaled) and its s_enc pointer is float[M] (A) or
 *       float[N] (B); alpha(m, n) = 1/(S_a[m] * S_b[n]).  With one row-scaled operand the
 *       factor is the binary64 quotient rounded once to fp32, as in the per-tensor case;
 *       with two it is the fp32 product of 1/S_a[m] and 1/S_b[n], each so rounded.
 *   fmt BSQ_FMT_MXFP8: a_codes [M][K] (E4M3), a_scales [M][K/32] (E8M0); s_enc
 *       pointers are ignored (may be NULL); alpha = 1.  K % 32 == 0.
 *   fmt BSQ_FMT_MXFP8 | BSQ_FMT_MX_SLAB_A and/or BSQ_FMT_MX_SLAB_B (BSQ_FMT_MX_SLAB: both):
 *       that operand's codes are in the slab layout (as an MXFP8 cast with BSQ_MX_SLAB
 *       writes them), scales as for BSQ_FMT_MXFP8; K % 512 == 0, else BSQ_ERR_SHAPE.
 *       blockscaled_grouped_gemm accepts BSQ_FMT_MX_SLAB_B with BSQ_GROUP_M, B being G
 *       slab-layout matrices [N][K] one after the other, and either flag with BSQ_GROUP_K,
 *       where A [M][K] and B [N][K] are whole slab-layout matrices over all groups (K the
 *       grouped extent, e.g. the columnwise casts of dY and X with BSQ_MX_SLAB).
 *   c [M][N], c_dtype BSQ_OUT_BF16 (RNE) or BSQ_OUT_F32.
 *   M, N >= 0 arbitrary; M, N or K == 0 are valid (K == 0 writes zeros).  K is below 2^24
 *   (NVFP4) or 2^23 (MXFP8), so that a 256-row operand tile stays below 2 GiB.
 */
int blockscaled_gemm(int fmt, int64_t M, int64_t N, int64_t K,
                     const uint8_t* a_codes, const uint8_t* a_scales, const float* a_s_enc,
                     const uint8_t* b_codes, const uint8_t* b_scales, const float* b_s_enc,
                     void* c, int c_dtype, void* hip_stream);

/*
 * blockscaled_grouped_gemm -- one block-scaled GEMM per group in a single launch: the
 * grouped GEMM of a mixture-of-experts linear layer ("general_grouped_gemm" of the
 * GroupedLinear path in the dispatch flowchart of the page "[Pytorch][Common] Hybrid
 * quantization", TransformerEngine PR #2817, whose Composer-style grouped recipe quantizes
 * the expert inputs as row-scaled NVFP4 for fprop and uses MXFP8 for the backward GEMMs).
 * Each group's GEMM computes exactly what blockscaled_gemm computes on that group's operands.
 *
 *   offsets  int64[groups + 1] (device, 8-byte aligned): group g covers indices
 *            offsets[g] .. offsets[g+1] of the grouped dimension.  Read on the device, so the
 *            routing that produces them needs no host synchronisation.  A group's start is
 *            clamped to [0, extent] and its end to [start, extent], so no group ever touches
 *            memory outside the tensors.  Groups must not overlap: with overlapping
 *            BSQ_GROUP_M groups the output is unspecified (still within C).
 *   mode BSQ_GROUP_M (fprop, dgrad): extent = M.  A [M][K] holds the groups' rows one after
 *            another (tokens sorted by expert); B [groups][N][K] stacks one operand per
 *            group; C [M][N]: rows offsets[g] .. offsets[g+1] = A_g B_g^T.  Rows outside
 *            every group are not written.  Any group sizes (zero included).
 *   mode BSQ_GROUP_K (wgrad): extent = K.  A [M][K] and B [N][K] are whole-tensor operands
 *            stored along the grouped dimension (e.g. the columnwise quantization of dY and X
 *            over all tokens); C [groups][M][N]: C_g = A[:, offsets[g]..offsets[g+1]) *
 *            B[:, same]^T.  Boundaries must be multiples of 32 (where per-group and
 *            whole-tensor MXFP8 blocks coincide); a group whose boundaries are not is
 *            computed as empty (C_g = 0), as is an empty group.
 *   fmt, codes, scales, c, c_dtype: as for blockscaled_gemm, with K % 32 == 0.
 *   NVFP4 tensor scales: a_s_enc float[groups] and b_s_enc float[groups] (one per group's
 *            operand); with BSQ_FMT_A_ROWSCALED (BSQ_GROUP_M only) a_s_enc is float[M], one
 *            per row of A, and with BSQ_FMT_B_ROWSCALED b_s_enc is float[groups * N].
 *            alpha follows blockscaled_gemm.  MXFP8 ignores them.
 * The launch covers an upper bound of the groups' tiles computed on the host from M, N and
 * groups; workgroups past the tiles that the device-side offsets produce exit at once.
 */
int blockscaled_grouped_gemm(int fmt, int mode, int64_t groups, const int64_t* offsets,
                             int64_t M, int64_t N, int64_t K,
                             const uint8_t* a_codes, const uint8_t* a_scales, const float* a_s_enc,
                             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_s_enc,
                             void* c, int c_dtype, void* hip_stream);

/*
 * The NVFP4 linear layer, forward and backward, as two calls over the kernels above: the
 * quantized linear of the page "Add an NVFP4 quantization converter" (torchtitan PR #3914:
 * Summary / "What changed" -- forward operands in NVFP4, the backward GEMMs' operands with
 * the 16-point RHT under a shared sign vector along their contraction dimension and
 * stochastic rounding keyed by a seed; "Numerical and performance validation", Table 1 and
 * its takeaway -- the layer keeps quantized activations and their scales for the backward
 * pass instead of bf16, which is where its memory saving comes from).
 *
 *   forward:  Y[T][N] (bf16) = NVFP4_row_RNE(X) * NVFP4_row_RNE(W)^T, and `saved` receives
 *             X's columnwise NVFP4 along tokens with RHT + SR (SR stream 1) -- the wgrad
 *             operand, 0.5625 bytes per element instead of the 2 of bf16 X.
 *   backward: dY is quantized once in both directions with RHT + SR (SR stream 0; rowwise
 *             along N for dgrad, columnwise along tokens for wgrad); W columnwise along N with
 *             RHT + SR (SR stream 2);
 *             dW[N][K] (fp32) = dY_col * X_col^T  (contraction over tokens, X from `saved`),
 *             dX[T][K] (bf16) = dY_row * W_col^T  (contraction over N).
 * Each step is exactly the corresponding nvfp4_quantize / blockscaled_gemm call (X's two
 * casts are one nvfp4_quantize_fprop_wgrad call); the intermediate quantized operands live in
 * `workspace`.
 *
 *   x [T][K], w [N][K], dy [T][N] bf16 (device); T = tokens, K = in_features,
 *   N = out_features, all multiples of 32, non-zero and below 2^24 (each is the contraction
 *   length of one of the three GEMMs).
 *   sr_seed, rht_signs: as for nvfp4_quantize (rht_signs required); the same values must be
 *   passed to forward and backward (the saved operand was drawn with them).
 *   saved      device buffer of nvfp4_linear_saved_bytes(T, K) bytes, written by forward and
 *              read by backward (layout private to the library).
 *   workspace  device buffer of nvfp4_linear_workspace_bytes(T, K, N) bytes, scratch for
 *              either call (contents not preserved).
 *   y [T][N] bf16; dx [T][K] bf16; dw [N][K] fp32 (device).
 * Work is enqueued on hip_stream; a failed launch returns BSQ_ERR_HIP with the steps before
 * it already enqueued.  The size queries return -1 for negative sizes.
 */
int64_t nvfp4_linear_workspace_bytes(int64_t tokens, int64_t in_features, int64_t out_features);
int64_t nvfp4_linear_saved_bytes(int64_t tokens, int64_t in_features);
int nvfp4_linear_forward(const void* x, const void* w, int64_t tokens, int64_t in_features,
                         int64_t out_features, uint64_t sr_seed, const int8_t* rht_signs,
                         void* saved, void* workspace, void* y, void* hip_stream);
int nvfp4_linear_backward(const void* dy, const void* w, const void* saved, int64_t tokens,
                          int64_t in_features, int64_t out_features, uint64_t sr_seed,
                          const int8_t* rht_signs, void* workspace, void* dx, float* dw,
                          void* hip_stream);

/* Message of the last failing call on this thread ("" if none).  Host memory owned
 * by the library; valid until the thread's next call. */
const char* bsq_last_error(void);

/* Library ABI version (major * 100 + minor): 200 (nvfp4_quantize takes a caller workspace). */
int bsq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_H */
