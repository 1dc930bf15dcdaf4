/*
 * oracle.c -- plain, slow CPU reference of block-scaled quantization (NVFP4, MXFP8),
 * the 16-point random Hadamard transform and the block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no source, header, table or
 * helper with the HIP library; the two meet only in the seeded inputs.
 *
 * Arithmetic rules: every floating-point step below is one IEEE-754 binary32
 * operation in round-to-nearest-even, in the order written (the build uses
 * -ffp-contract=off and no fast-math), except the GEMM, which is the textbook
 * sum in binary64.  Element encoders are nearest-value searches over the code
 * tables, not bit tricks, so that they can be checked by eye against the format
 * definitions.
 *
 * Sources.  The quantization recipe (16-element blocks with an inner scale and a
 * per-tensor outer scale, Philox-keyed stochastic rounding, a random Hadamard
 * transform whose sign vector both GEMM operands share) is the one described on
 * the page "Add an NVFP4 quantization converter" (torchtitan PR #3914), in its
 * Summary ("What changed") and in the review thread about the recipe's inner
 * 1x16 scale and outer scale.  Rowwise/columnwise directions, the MXFP8 block
 * size of 32 and the rowwise-dequantized columnwise source come from the page
 * "[Pytorch][Common] Hybrid quantization" (TransformerEngine PR #2817),
 * Description and the review thread on columnwise scale truncation.  The pages
 * define neither the code points nor the scale formulas; those follow the
 * public OCP Microscaling (MX) format definitions (the MX paper the TorchAO
 * review page cites in its references) and the readings listed in the design
 * notes of this repository (tensor scale 6*448/amax, scale op order, Philox
 * counter layout).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ bf16 ---- */

/* bf16 is the top half of a binary32; widening is exact. */
float or_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even (finite inputs). */
uint16_t or_f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ E2M1 ---- */

/* FP4 E2M1 magnitudes, indexed by the low three code bits (1 sign, 2 exponent,
 * 1 mantissa bit, exponent bias 1, one subnormal value 0.5). */
static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float or_e2m1_decode(uint8_t code)
{
    float m = E2M1_MAG[code & 7u];
    return (code & 8u) ? -m : m;
}

/* Nearest E2M1 value, ties to the even code; magnitudes above 6 saturate to 6.
 * The sign bit is copied from the input, including for -0. */
uint8_t or_e2m1_encode_rne(float v)
{
    uint8_t sign = signbit(v) ? 8u : 0u;
    double a = fabs((double)v);
    if (a >= 6.0) return (uint8_t)(sign | 7u);
    int best = 0;
    double bestd = a;                       /* distance to E2M1_MAG[0] = 0 */
    for (int i = 1; i < 8; ++i) {
        double d = fabs(a - (double)E2M1_MAG[i]);
        if (d < bestd || (d == bestd && (i % 2) == 0)) {
            best = i;
            bestd = d;
        }
    }
    return (uint8_t)(sign | (uint8_t)best);
}

/* Stochastic rounding onto the E2M1 grid.  With lo <= |v| < hi the neighbouring
 * grid magnitudes, the result is hi with probability p = (|v|-lo)/(hi-lo) and lo
 * otherwise; u is a uniform 32-bit word of which the top 24 bits are used:
 * round up iff (u >> 8) * 2^-24 < p.  Magnitudes at or above 6 saturate to 6.
 * p is exact in binary32: |v|-lo is exact (Sterbenz, hi <= 2*lo or lo = 0) and
 * hi-lo is a power of two. */
uint8_t or_e2m1_encode_sr(float v, uint32_t u)
{
    uint8_t sign = signbit(v) ? 8u : 0u;
    float a = fabsf(v);
    if (a >= 6.0f) return (uint8_t)(sign | 7u);
    int lo = 0;
    while (lo < 6 && E2M1_MAG[lo + 1] <= a) ++lo;
    float lov = E2M1_MAG[lo];
    float hiv = E2M1_MAG[lo + 1];
    float num = a - lov;
    float den = hiv - lov;
    float p = num / den;
    float r = (float)(u >> 8) * 0x1p-24f;
    int code = (r < p) ? lo + 1 : lo;
    return (uint8_t)(sign | (uint8_t)code);
}

/* ------------------------------------------------------------------ E4M3 ---- */

/* OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities; max 448. */
float or_e4m3_decode(uint8_t code)
{
    int s = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    float v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexpf((float)m / 8.0f, -6);
    else
        v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -v : v;
}

/* Nearest E4M3 value (ties to the even code), finite overflow saturating to
 * +-448, sign (including -0) preserved.  Codes 0x00..0x7E are the non-negative
 * finite values in increasing order; binary search for the bracket. */
uint8_t or_e4m3_encode_rne_sat(float v)
{
    uint8_t sign = signbit(v) ? 0x80u : 0u;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
    int lo = 0, hi = 0x7E;                  /* invariant: val(lo) <= a < val(hi) */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if ((double)or_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - (double)or_e4m3_decode((uint8_t)lo);
    double dhi = (double)or_e4m3_decode((uint8_t)hi) - a;
    int code;
    if (dlo < dhi)
        code = lo;
    else if (dhi < dlo)
        code = hi;
    else
        code = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | (uint8_t)code);
}

/* ------------------------------------------------------------------ E8M0 ---- */

/* E8M0 scale byte: 2^(byte-127); 0xFF is NaN. */
float or_e8m0_decode(uint8_t b)
{
    if (b == 0xFF) return NAN;
    return ldexpf(1.0f, (int)b - 127);
}

/* ------------------------------------------------------------ Philox4x32-10 - */

/* Philox4x32 with 10 rounds, as published by Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11): each round multiplies
 * counter words 0 and 2 by the two round constants, and the new counter is
 * (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); the key is
 * bumped by the two Weyl constants between rounds. */
void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c[0];
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c[2];
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c[1] ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c[3] ^ k1;
        uint32_t n3 = lo0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* Uniform word for output element i (linear index in the output layout) of a
 * quantization in direction dir (0 rowwise, 1 columnwise):
 * key = (lo32(seed), hi32(seed)), counter = (lo32(i/4), hi32(i/4), stream, dir),
 * word i mod 4 of the Philox output. */
uint32_t or_sr_word(uint64_t seed, uint32_t stream, uint32_t dir, uint64_t i)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint64_t q = i >> 2;
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), stream, dir};
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    return out[i & 3u];
}

/* ------------------------------------------------------------- RHT (16) ---- */

/* Random Hadamard transform of one 16-vector: y = x * diag(d) * H16 / 4, H16 the
 * Sylvester Hadamard matrix in natural order, H[i][j] = (-1)^popcount(i & j).
 * Evaluated as: sign flip (exact), the fast Walsh-Hadamard butterfly with
 * strides 1, 2, 4, 8 where each pair (a, b) becomes (a + b, a - b) in binary32,
 * then the exact multiplication by 1/4.  The transform is orthogonal
 * (R R^T = I), so it cancels in a product when both operands use the same d. */
void or_rht16(const float x[16], const int8_t d[16], float y[16])
{
    float v[16];
    for (int i = 0; i < 16; ++i) v[i] = x[i] * (float)d[i];
    for (int h = 1; h < 16; h *= 2) {
        for (int i = 0; i < 16; i += 2 * h) {
            for (int j = i; j < i + h; ++j) {
                float a = v[j];
                float b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
    for (int i = 0; i < 16; ++i) y[i] = v[i] * 0.25f;
}

/* ------------------------------------------------------------ helpers ---- */

enum { OR_ROW = 1, OR_COL = 2 };
enum { OR_RNE = 0, OR_SR = 1 };

/* Widen a bf16 [R][C] matrix to binary32, either as is (transpose = 0, result
 * [R][C]) or transposed (result [C][R]).  Columnwise quantization is the
 * rowwise quantization of the transpose. */
static float* widen(const uint16_t* x, int64_t R, int64_t C, int transpose)
{
    float* v = (float*)malloc(sizeof(float) * (size_t)(R * C > 0 ? R * C : 1));
    if (!v) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            float f = or_bf16_to_f32(x[r * C + c]);
            if (transpose)
                v[c * R + r] = f;
            else
                v[r * C + c] = f;
        }
    return v;
}

/* Apply the 16-point RHT to every consecutive 16-block of every row of v[rows][cols]. */
static void rht_rows(float* v, int64_t rows, int64_t cols, const int8_t* d)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < cols / 16; ++b) {
            float y[16];
            or_rht16(v + r * cols + 16 * b, d, y);
            memcpy(v + r * cols + 16 * b, y, sizeof y);
        }
}

static float amax_of(const float* v, int64_t n)
{
    float m = 0.0f;
#pragma omp parallel for reduction(max : m) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > m) m = a;
    }
    return m;
}

/* Per-tensor (outer) scale: S = 6*448 / A in binary32, so that the block holding
 * the tensor's amax gets the largest E4M3 scale.  A = 0 gives S = 1; an
 * overflow to infinity is clamped to FLT_MAX. */
float or_nvfp4_tensor_scale(float amax)
{
    if (amax == 0.0f) return 1.0f;
    float s = 2688.0f / amax;
    if (isinf(s)) s = FLT_MAX;
    return s;
}

/* Block (inner) scale byte for a 16-block with amax b: E4M3 of (b * S) / 6,
 * two binary32 operations in this order, RNE, saturating at 448. */
uint8_t or_nvfp4_block_scale(float block_amax, float s_enc)
{
    float t = block_amax * s_enc;
    t = t / 6.0f;
    return or_e4m3_encode_rne_sat(t);
}

/* NVFP4 quantization of every row of v[rows][cols] (cols % 16 == 0) with tensor
 * scale s_tensor, or with row r's own scale s_rows[r] when s_rows is given.  Writes codes [rows][cols/2] (element 2j in the low nibble of
 * byte j, element 2j+1 in the high nibble) and scales [rows][cols/16].  For a
 * nonzero block scale s_b the elements are multiplied by S / fp32(s_b) (one
 * division, then one multiplication per element) and rounded onto E2M1; a zero
 * block scale gives all-zero codes.  Under SR, element i (linear index in this
 * [rows][cols] output) draws its word from or_sr_word(seed, stream, dir, i). */
static void quantize_rows_nvfp4(const float* v, int64_t rows, int64_t cols, float s_tensor,
                                const float* s_rows, int rounding, uint64_t seed, uint32_t stream,
                                uint32_t dir, uint8_t* codes, uint8_t* scales)
{
    const int64_t nb = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float s_enc = s_rows ? s_rows[r] : s_tensor;
        for (int64_t b = 0; b < nb; ++b) {
            const float* blk = v + r * cols + 16 * b;
            float bmax = 0.0f;
            for (int j = 0; j < 16; ++j)
                if (fabsf(blk[j]) > bmax) bmax = fabsf(blk[j]);
            uint8_t sb = or_nvfp4_block_scale(bmax, s_enc);
            scales[r * nb + b] = sb;
            uint8_t q[16];
            if (sb == 0) {
                memset(q, 0, sizeof q);
            } else {
                float enc = s_enc / or_e4m3_decode(sb);
                for (int j = 0; j < 16; ++j) {
                    float xs = blk[j] * enc;
                    if (rounding == OR_SR) {
                        uint64_t i = (uint64_t)(r * cols + 16 * b + j);
                        q[j] = or_e2m1_encode_sr(xs, or_sr_word(seed, stream, dir, i));
                    } else {
                        q[j] = or_e2m1_encode_rne(xs);
                    }
                }
            }
            uint8_t* out = codes + r * (cols / 2) + 8 * b;
            for (int j = 0; j < 8; ++j) out[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
        }
    }
}

/* ------------------------------------------------------------ NVFP4 ---- */

/* NVFP4 quantization of a bf16 tensor x[R][C], in the requested directions
 * (bit 1 rowwise: 16-blocks along C; bit 2 columnwise: 16-blocks along R,
 * stored as the rowwise quantization of x^T, i.e. codes [C][R/2], scales
 * [C][R/16]).  With a sign vector, each direction first applies the 16-point
 * RHT along its own blocked dimension, and its tensor amax is taken over the
 * transformed values.  amax_out[0] / s_enc_out[0] are the rowwise values,
 * [1] the columnwise ones (both equal without RHT).  Returns 0, or -1 on a
 * shape error, -2 on allocation failure. */
int or_nvfp4_quantize(const uint16_t* x, int64_t R, int64_t C, int direction, int rounding,
                      uint64_t seed, uint32_t stream, const int8_t* signs,
                      uint8_t* row_codes, uint8_t* row_scales,
                      uint8_t* col_codes, uint8_t* col_scales,
                      float* amax_out, float* s_enc_out)
{
    for (int dir = 0; dir < 2; ++dir) {
        if (!(direction & (dir == 0 ? OR_ROW : OR_COL))) continue;
        int64_t rows = dir == 0 ? R : C;
        int64_t cols = dir == 0 ? C : R;
        if (cols % 16 != 0) return -1;
        float* v = widen(x, R, C, dir);
        if (!v) return -2;
        if (signs) rht_rows(v, rows, cols, signs);
        float a = amax_of(v, rows * cols);
        float s = or_nvfp4_tensor_scale(a);
        quantize_rows_nvfp4(v, rows, cols, s, NULL, rounding, seed, stream, (uint32_t)dir,
                            dir == 0 ? row_codes : col_codes,
                            dir == 0 ? row_scales : col_scales);
        amax_out[dir] = a;
        s_enc_out[dir] = s;
        free(v);
    }
    return 0;
}

/* Row-scaled NVFP4 (the "row_scaled_nvfp4" rowwise quantizer of the Composer-style recipe
 * on the page "[Pytorch][Common] Hybrid quantization"; outer scale per row, inner scale
 * 1x16, as asked in the review of "Add an NVFP4 quantization converter"): the rowwise
 * quantization above with each row's own amax A_r and tensor scale S_r = f(A_r) (same
 * rule as the per-tensor scale) in place of the tensor's.  With a sign vector the RHT is
 * applied along the rows first and A_r is taken over the transformed row.  Writes codes
 * [R][C/2], scales [R][C/16], amax_rows[R], s_enc_rows[R].  SR words are drawn exactly
 * as for the rowwise per-tensor quantization (direction 0, linear output index). */
int or_nvfp4_quantize_rowscaled(const uint16_t* x, int64_t R, int64_t C, int rounding,
                                uint64_t seed, uint32_t stream, const int8_t* signs,
                                uint8_t* codes, uint8_t* scales, float* amax_rows,
                                float* s_enc_rows)
{
    if (C % 16 != 0) return -1;
    float* v = widen(x, R, C, 0);
    if (!v) return -2;
    if (signs) rht_rows(v, R, C, signs);
    for (int64_t r = 0; r < R; ++r) {
        float a = amax_of(v + r * C, C);
        amax_rows[r] = a;
        s_enc_rows[r] = or_nvfp4_tensor_scale(a);
    }
    quantize_rows_nvfp4(v, R, C, 0.0f, s_enc_rows, rounding, seed, stream, 0u, codes, scales);
    free(v);
    return 0;
}

/* Dequantized value of one NVFP4 element, rounded to bf16:
 * bf16_RNE((E2M1(code) * fp32(s_b)) / S); the product is exact. */
static uint16_t nvfp4_deq_bf16(uint8_t code, uint8_t sb, float s_enc)
{
    float p = or_e2m1_decode(code) * or_e4m3_decode(sb);
    float q = p / s_enc;
    return or_f32_to_bf16_rne(q);
}

/* Rowwise-dequantized tensor: out[rows][cols] bf16 from NVFP4 codes [rows][cols/2],
 * scales [rows][cols/16] and tensor scale s_enc (the "rowwise_dequantized"
 * columnwise source of the hybrid quantizer, TransformerEngine PR #2817,
 * "Enable columnwise_source and hybrid recipes"). */
void or_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, float s_enc,
                         int64_t rows, int64_t cols, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[r * (cols / 2) + c / 2];
            uint8_t code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            out[r * cols + c] = nvfp4_deq_bf16(code, scales[r * (cols / 16) + c / 16], s_enc);
        }
}

/* ------------------------------------------------------------ MXFP8 ---- */

/* MXFP8 scale byte of a 32-block with amax b > 0 (OCP MX rule): the shared
 * exponent is X = floor(log2 b) - 8 (8 = largest E4M3 exponent), clamped to
 * [-127, 127]; the byte is X + 127.  floor(log2 b) is read exactly from frexp. */
uint8_t or_mxfp8_scale_byte(float block_amax)
{
    if (block_amax == 0.0f) return 0;
    int e;
    frexpf(block_amax, &e);                 /* b = m * 2^e, m in [0.5, 1) */
    int X = (e - 1) - 8;
    if (X < -127) X = -127;
    if (X > 127) X = 127;
    return (uint8_t)(X + 127);
}

static void quantize_rows_mxfp8(const float* v, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales)
{
    const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            const float* blk = v + r * cols + 32 * b;
            float bmax = 0.0f;
            for (int j = 0; j < 32; ++j)
                if (fabsf(blk[j]) > bmax) bmax = fabsf(blk[j]);
            uint8_t* out = codes + r * cols + 32 * b;
            if (bmax == 0.0f) {
                scales[r * nb + b] = 0;
                memset(out, 0, 32);
                continue;
            }
            uint8_t sb = or_mxfp8_scale_byte(bmax);
            scales[r * nb + b] = sb;
            int X = (int)sb - 127;
            for (int j = 0; j < 32; ++j) out[j] = or_e4m3_encode_rne_sat(ldexpf(blk[j], -X));
        }
}

/* MXFP8 cast of a bf16 tensor x[R][C]: 32-blocks along the blocked dimension,
 * one E8M0 scale per block and E4M3 codes.  Rowwise: codes [R][C], scales
 * [R][C/32].  Columnwise (of x^T): codes [C][R], scales [C][R/32].  Returns 0,
 * -1 on a shape error, -2 on allocation failure. */
int or_mxfp8_quantize(const uint16_t* x, int64_t R, int64_t C, int direction,
                      uint8_t* row_codes, uint8_t* row_scales,
                      uint8_t* col_codes, uint8_t* col_scales)
{
    for (int dir = 0; dir < 2; ++dir) {
        if (!(direction & (dir == 0 ? OR_ROW : OR_COL))) continue;
        int64_t rows = dir == 0 ? R : C;
        int64_t cols = dir == 0 ? C : R;
        if (cols % 32 != 0) return -1;
        float* v = widen(x, R, C, dir);
        if (!v) return -2;
        quantize_rows_mxfp8(v, rows, cols, dir == 0 ? row_codes : col_codes,
                            dir == 0 ? row_scales : col_scales);
        free(v);
    }
    return 0;
}

/* ------------------------------------------------------------ RHT apply ---- */

/* Standalone RHT of a bf16 tensor x[R][C] into binary32 out[R][C], along C
 * (axis 1: blocks of 16 consecutive elements of a row) or along R (axis 0:
 * blocks of 16 consecutive elements of a column). */
int or_rht_apply(const uint16_t* x, int64_t R, int64_t C, int axis, const int8_t* d, float* out)
{
    if (axis == 1) {
        if (C % 16 != 0) return -1;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < R; ++r)
            for (int64_t b = 0; b < C / 16; ++b) {
                float in[16];
                for (int j = 0; j < 16; ++j) in[j] = or_bf16_to_f32(x[r * C + 16 * b + j]);
                or_rht16(in, d, out + r * C + 16 * b);
            }
    } else {
        if (R % 16 != 0) return -1;
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < C; ++c)
            for (int64_t b = 0; b < R / 16; ++b) {
                float in[16], y[16];
                for (int j = 0; j < 16; ++j) in[j] = or_bf16_to_f32(x[(16 * b + j) * C + c]);
                or_rht16(in, d, y);
                for (int j = 0; j < 16; ++j) out[(16 * b + j) * C + c] = y[j];
            }
    }
    return 0;
}

/* ------------------------------------------------------------ GEMM ---- */

/* Dequantized binary64 value of element k of row r of an operand [rows][K].
 * fmt 0 (NVFP4): E2M1(code) * E4M3(scale) / S.  fmt 1 (MXFP8): E4M3(code) * 2^(byte-127). */
static double deq_elem(int fmt, const uint8_t* codes, const uint8_t* scales, double s_enc,
                       int64_t K, int64_t r, int64_t k)
{
    if (fmt == 0) {
        uint8_t byte = codes[r * (K / 2) + k / 2];
        uint8_t code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        double v = (double)or_e2m1_decode(code) * (double)or_e4m3_decode(scales[r * (K / 16) + k / 16]);
        return v / s_enc;
    }
    double v = (double)or_e4m3_decode(codes[r * K + k]);
    return v * (double)or_e8m0_decode(scales[r * (K / 32) + k / 32]);
}

/* Block-scaled GEMM C = A * B^T on the dequantized operands, A [M][K], B [N][K]
 * (both stored along K), in binary64: C[m][n] = sum_k A[m][k] * B[n][k].  Only
 * the rows mi[0..nm) and columns ni[0..nn) of C are computed, into
 * out[nm][nn]; pass every index for the full product.  NVFP4 tensor scales:
 * a_s[0] for every row of A, or a_s[m] for row m when a_per_row (row-scaled
 * operand); likewise b_s for the rows of B.  Ignored for MXFP8.  When out_abs is
 * not NULL it receives sum_k |A[m][k] * B[n][k]| for the same outputs (the scale
 * of the rounding-error bound of any finite-precision evaluation of C). */
int or_blockscaled_gemm_rows(int fmt, int64_t M, int64_t N, int64_t K,
                             const uint8_t* a_codes, const uint8_t* a_scales, const float* a_s,
                             int a_per_row, const uint8_t* b_codes, const uint8_t* b_scales,
                             const float* b_s, int b_per_row,
                             const int64_t* mi, int64_t nm, const int64_t* ni, int64_t nn,
                             double* out, double* out_abs)
{
    if (fmt == 0 && K % 16 != 0) return -1;
    if (fmt == 1 && K % 32 != 0) return -1;
    for (int64_t i = 0; i < nm; ++i)
        if (mi[i] < 0 || mi[i] >= M) return -1;
    for (int64_t j = 0; j < nn; ++j)
        if (ni[j] < 0 || ni[j] >= N) return -1;
    double* a = (double*)malloc(sizeof(double) * (size_t)(nm * K > 0 ? nm * K : 1));
    double* b = (double*)malloc(sizeof(double) * (size_t)(nn * K > 0 ? nn * K : 1));
    if (!a || !b) {
        free(a);
        free(b);
        return -2;
    }
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nm; ++i)
        for (int64_t k = 0; k < K; ++k)
            a[i * K + k] = deq_elem(fmt, a_codes, a_scales, (double)a_s[a_per_row ? mi[i] : 0], K, mi[i], k);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < nn; ++j)
        for (int64_t k = 0; k < K; ++k)
            b[j * K + k] = deq_elem(fmt, b_codes, b_scales, (double)b_s[b_per_row ? ni[j] : 0], K, ni[j], k);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nm; ++i)
        for (int64_t j = 0; j < nn; ++j) {
            double s = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = a[i * K + k] * b[j * K + k];
                s += p;
                t += fabs(p);
            }
            out[i * nn + j] = s;
            if (out_abs) out_abs[i * nn + j] = t;
        }
    free(a);
    free(b);
    return 0;
}

/* The same with one tensor scale per operand. */
int or_blockscaled_gemm(int fmt, int64_t M, int64_t N, int64_t K,
                        const uint8_t* a_codes, const uint8_t* a_scales, float a_s_enc,
                        const uint8_t* b_codes, const uint8_t* b_scales, float b_s_enc,
                        const int64_t* mi, int64_t nm, const int64_t* ni, int64_t nn,
                        double* out)
{
    return or_blockscaled_gemm_rows(fmt, M, N, K, a_codes, a_scales, &a_s_enc, 0, b_codes, b_scales,
                                    &b_s_enc, 0, mi, nm, ni, nn, out, NULL);
}

/* Number of OpenMP threads the oracle uses. */
int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads of later oracle calls (n >= 1). */
void or_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
