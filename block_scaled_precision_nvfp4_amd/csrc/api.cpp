// api.cpp -- the C ABI of libbsq (declared in include/bsq.h): argument validation on the
// host, then one launcher call.  Validation runs before any HIP call, so a rejected call
// never touches the device and works on a machine without a GPU.
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/bsq.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return BSQ_OK;
}

bool misaligned(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// Largest K of a GEMM: a 256-row operand tile (codes) must stay below 2^31 bytes, the range of
// one buffer resource: 8 Mi elements for MXFP8 (1 byte each), 16 Mi for NVFP4.
// Exclusive bound on K: a 256-row operand tile of K-element rows (K/2 bytes NVFP4, K bytes
// MXFP8) must span fewer than 2^31 bytes, the largest range a buffer resource covers.
int64_t gemm_k_limit(int fmt) { return fmt == BSQ_FMT_MXFP8 ? (int64_t)1 << 23 : (int64_t)1 << 24; }

int launched(int hip_code, const char* what) {
    if (hip_code != 0)
        return fail(BSQ_ERR_HIP, "%s: kernel launch failed: %s", what, bsq::hip_error_string(hip_code));
    return ok();
}

}  // namespace

extern "C" {

int bsq_version(void) { return 200; }

const char* bsq_last_error(void) { return g_last_error.c_str(); }

// Argument checks shared by nvfp4_quantize and nvfp4_quantize_noalloc (need_ws: the call takes
// a workspace argument).
static int nvfp4_quantize_check(const char* fn, const void* x, int64_t rows, int64_t cols, int direction,
                                int rounding, const int8_t* rht_signs, uint8_t* row_codes, uint8_t* row_scales,
                                uint8_t* col_codes, uint8_t* col_scales, float* amax_out, float* s_enc_out,
                                bool need_ws, void* workspace) {
    if (direction < 1 || direction > 3) return fail(BSQ_ERR_ARG, "%s: direction must be 1 (row), 2 (col) or 3, got %d", fn, direction);
    if (rounding != BSQ_RNE && rounding != BSQ_SR) return fail(BSQ_ERR_ARG, "%s: rounding must be 0 (RNE) or 1 (SR), got %d", fn, rounding);
    if (rows < 0 || cols < 0) return fail(BSQ_ERR_SHAPE, "%s: negative shape [%lld, %lld]", fn, (long long)rows, (long long)cols);
    if (cols % 8 != 0) return fail(BSQ_ERR_SHAPE, "%s: cols (%lld) must be a multiple of 8", fn, (long long)cols);
    if ((direction & BSQ_ROW) && cols % 16 != 0) return fail(BSQ_ERR_SHAPE, "%s: rowwise needs cols %% 16 == 0, got %lld", fn, (long long)cols);
    if ((direction & BSQ_COL) && rows % 16 != 0) return fail(BSQ_ERR_SHAPE, "%s: columnwise needs rows %% 16 == 0, got %lld", fn, (long long)rows);
    if (!amax_out || !s_enc_out) return fail(BSQ_ERR_NULL, "%s: amax_out and s_enc_out are required", fn);
    const bool empty = rows == 0 || cols == 0;
    if (!empty && !x) return fail(BSQ_ERR_NULL, "%s: x is NULL", fn);
    if ((direction & BSQ_ROW) && !empty && (!row_codes || !row_scales)) return fail(BSQ_ERR_NULL, "%s: rowwise outputs are NULL", fn);
    if ((direction & BSQ_COL) && !empty && (!col_codes || !col_scales)) return fail(BSQ_ERR_NULL, "%s: columnwise outputs are NULL", fn);
    if (need_ws && !empty && !workspace) return fail(BSQ_ERR_NULL, "%s: workspace is NULL", fn);
    if (misaligned(x) || misaligned(row_codes) || misaligned(col_codes) || misaligned(rht_signs) || misaligned(workspace))
        return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return BSQ_OK;
}

int nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int direction, int rounding, uint64_t sr_seed,
                   uint32_t sr_stream, const int8_t* rht_signs, uint8_t* row_codes, uint8_t* row_scales,
                   uint8_t* col_codes, uint8_t* col_scales, float* amax_out, float* s_enc_out, void* workspace,
                   void* hip_stream) {
    static const char* fn = "nvfp4_quantize";
    if (const int st = nvfp4_quantize_check(fn, x, rows, cols, direction, rounding, rht_signs, row_codes, row_scales,
                                            col_codes, col_scales, amax_out, s_enc_out, true, workspace))
        return st;
    return launched(bsq::launch_nvfp4_quantize(x, rows, cols, direction, rounding, sr_seed, sr_stream, rht_signs,
                                               row_codes, row_scales, col_codes, col_scales, amax_out, s_enc_out,
                                               static_cast<float*>(workspace), hip_stream), fn);
}

int nvfp4_quantize_fprop_wgrad(const void* x, int64_t rows, int64_t cols, int rounding, uint64_t sr_seed,
                               uint32_t sr_stream, const int8_t* rht_signs, uint8_t* row_codes, uint8_t* row_scales,
                               uint8_t* col_codes, uint8_t* col_scales, float* amax_out, float* s_enc_out,
                               void* workspace, void* hip_stream) {
    static const char* fn = "nvfp4_quantize_fprop_wgrad";
    if (const int st = nvfp4_quantize_check(fn, x, rows, cols, BSQ_ROW | BSQ_COL, rounding, rht_signs, row_codes,
                                            row_scales, col_codes, col_scales, amax_out, s_enc_out, true, workspace))
        return st;
    return launched(bsq::launch_nvfp4_quantize_fprop_wgrad(x, rows, cols, rounding, sr_seed, sr_stream, rht_signs,
                                                           row_codes, row_scales, col_codes, col_scales, amax_out,
                                                           s_enc_out, static_cast<float*>(workspace), hip_stream),
                    fn);
}

int nvfp4_quantize_noalloc(const void* x, int64_t rows, int64_t cols, int direction, int rounding, uint64_t sr_seed,
                           uint32_t sr_stream, const int8_t* rht_signs, uint8_t* row_codes, uint8_t* row_scales,
                           uint8_t* col_codes, uint8_t* col_scales, float* amax_out, float* s_enc_out,
                           void* hip_stream) {
    static const char* fn = "nvfp4_quantize_noalloc";
    if (const int st = nvfp4_quantize_check(fn, x, rows, cols, direction, rounding, rht_signs, row_codes, row_scales,
                                            col_codes, col_scales, amax_out, s_enc_out, false, nullptr))
        return st;
    return launched(bsq::launch_nvfp4_quantize_noalloc(x, rows, cols, direction, rounding, sr_seed, sr_stream,
                                                       rht_signs, row_codes, row_scales, col_codes, col_scales,
                                                       amax_out, s_enc_out, hip_stream), fn);
}

int nvfp4_col_mxfp8_row_quantize(const void* x, int64_t rows, int64_t cols, int rounding, uint64_t sr_seed,
                                 uint32_t sr_stream, const int8_t* rht_signs, uint8_t* col_codes,
                                 uint8_t* col_scales, float* amax_out, float* s_enc_out, void* workspace,
                                 int mx_layout, uint8_t* mx_row_codes, uint8_t* mx_row_scales, void* hip_stream) {
    static const char* fn = "nvfp4_col_mxfp8_row_quantize";
    if (mx_layout != 0 && mx_layout != BSQ_MX_SLAB)
        return fail(BSQ_ERR_ARG, "%s: mx_layout must be 0 or BSQ_MX_SLAB, got %d", fn, mx_layout);
    if (const int st = nvfp4_quantize_check(fn, x, rows, cols, BSQ_COL, rounding, rht_signs, nullptr, nullptr,
                                            col_codes, col_scales, amax_out, s_enc_out, true, workspace))
        return st;
    if (cols % 32 != 0) return fail(BSQ_ERR_SHAPE, "%s: MXFP8 rowwise needs cols %% 32 == 0, got %lld", fn, (long long)cols);
    if (mx_layout && cols % 64 != 0)
        return fail(BSQ_ERR_SHAPE, "%s: rowwise slab codes need cols %% 64 == 0, got %lld", fn, (long long)cols);
    const bool empty = rows == 0 || cols == 0;
    if (!empty && (!mx_row_codes || !mx_row_scales)) return fail(BSQ_ERR_NULL, "%s: MXFP8 rowwise outputs are NULL", fn);
    if (misaligned(mx_row_codes)) return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return launched(bsq::launch_nvfp4_quantize(x, rows, cols, BSQ_COL, rounding, sr_seed, sr_stream, rht_signs, nullptr,
                                               nullptr, col_codes, col_scales, amax_out, s_enc_out,
                                               static_cast<float*>(workspace), hip_stream, mx_row_codes,
                                               mx_row_scales, mx_layout ? 1 : 0), fn);
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s_enc, int64_t rows, int64_t cols,
                     void* out, void* hip_stream) {
    static const char* fn = "nvfp4_dequantize";
    if (rows < 0 || cols < 0) return fail(BSQ_ERR_SHAPE, "%s: negative shape", fn);
    if (cols % 16 != 0) return fail(BSQ_ERR_SHAPE, "%s: cols (%lld) must be a multiple of 16", fn, (long long)cols);
    if (rows * cols == 0) return ok();
    if (!codes || !scales || !s_enc || !out) return fail(BSQ_ERR_NULL, "%s: NULL argument", fn);
    if (misaligned(codes) || misaligned(out)) return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return launched(bsq::launch_nvfp4_dequantize(codes, scales, s_enc, rows, cols, out, hip_stream), fn);
}

// MXFP8 cast directions, optionally with BSQ_MX_SLAB (the codes' contraction length, cols for
// rowwise and rows for columnwise codes, must then be a multiple of 64)
static int mx_direction_check(const char* fn, int direction, int64_t rows, int64_t cols) {
    const int dirs = direction & ~BSQ_MX_SLAB;
    if (dirs < 1 || dirs > 3)
        return fail(BSQ_ERR_ARG, "%s: direction must be 1 (row), 2 (col) or 3, optionally with BSQ_MX_SLAB, got %d", fn, direction);
    if (rows < 0 || cols < 0) return fail(BSQ_ERR_SHAPE, "%s: negative shape", fn);
    if (direction & BSQ_MX_SLAB) {
        if ((dirs & BSQ_ROW) && cols % 64 != 0)
            return fail(BSQ_ERR_SHAPE, "%s: rowwise slab codes need cols %% 64 == 0, got %lld", fn, (long long)cols);
        if ((dirs & BSQ_COL) && rows % 64 != 0)
            return fail(BSQ_ERR_SHAPE, "%s: columnwise slab codes need rows %% 64 == 0, got %lld", fn, (long long)rows);
    }
    return BSQ_OK;
}

int mxfp8_quantize(const void* x, int64_t rows, int64_t cols, int direction, uint8_t* row_codes,
                   uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, void* hip_stream) {
    static const char* fn = "mxfp8_quantize";
    if (const int st = mx_direction_check(fn, direction, rows, cols)) return st;
    if (cols % 8 != 0) return fail(BSQ_ERR_SHAPE, "%s: cols (%lld) must be a multiple of 8", fn, (long long)cols);
    if ((direction & BSQ_ROW) && cols % 32 != 0) return fail(BSQ_ERR_SHAPE, "%s: rowwise needs cols %% 32 == 0, got %lld", fn, (long long)cols);
    if ((direction & BSQ_COL) && rows % 32 != 0) return fail(BSQ_ERR_SHAPE, "%s: columnwise needs rows %% 32 == 0, got %lld", fn, (long long)rows);
    if (rows == 0 || cols == 0) return ok();
    if (!x) return fail(BSQ_ERR_NULL, "%s: x is NULL", fn);
    if ((direction & BSQ_ROW) && (!row_codes || !row_scales)) return fail(BSQ_ERR_NULL, "%s: rowwise outputs are NULL", fn);
    if ((direction & BSQ_COL) && (!col_codes || !col_scales)) return fail(BSQ_ERR_NULL, "%s: columnwise outputs are NULL", fn);
    if (misaligned(x) || misaligned(row_codes) || misaligned(col_codes))
        return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return launched(bsq::launch_mxfp8_quantize(x, rows, cols, direction, row_codes, row_scales, col_codes,
                                               col_scales, hip_stream), fn);
}

int mxfp8_requantize_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* s_enc, int64_t rows,
                           int64_t cols, int direction, uint8_t* row_codes, uint8_t* row_scales,
                           uint8_t* col_codes, uint8_t* col_scales, void* hip_stream) {
    static const char* fn = "mxfp8_requantize_nvfp4";
    if (const int st = mx_direction_check(fn, direction, rows, cols)) return st;
    if (cols % 16 != 0) return fail(BSQ_ERR_SHAPE, "%s: cols (%lld) must be a multiple of 16", fn, (long long)cols);
    if ((direction & BSQ_ROW) && cols % 32 != 0) return fail(BSQ_ERR_SHAPE, "%s: rowwise needs cols %% 32 == 0, got %lld", fn, (long long)cols);
    if ((direction & BSQ_COL) && rows % 32 != 0) return fail(BSQ_ERR_SHAPE, "%s: columnwise needs rows %% 32 == 0, got %lld", fn, (long long)rows);
    if (rows == 0 || cols == 0) return ok();
    if (!codes || !scales || !s_enc) return fail(BSQ_ERR_NULL, "%s: NVFP4 input is NULL", fn);
    if ((direction & BSQ_ROW) && (!row_codes || !row_scales)) return fail(BSQ_ERR_NULL, "%s: rowwise outputs are NULL", fn);
    if ((direction & BSQ_COL) && (!col_codes || !col_scales)) return fail(BSQ_ERR_NULL, "%s: columnwise outputs are NULL", fn);
    if (misaligned(codes) || misaligned(row_codes) || misaligned(col_codes))
        return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return launched(bsq::launch_mxfp8_requantize_nvfp4(codes, scales, s_enc, rows, cols, direction, row_codes,
                                                       row_scales, col_codes, col_scales, hip_stream), fn);
}

int rht_apply(const void* x, int64_t rows, int64_t cols, int axis, const int8_t* signs, float* out,
              void* hip_stream) {
    static const char* fn = "rht_apply";
    if (axis != 0 && axis != 1) return fail(BSQ_ERR_ARG, "%s: axis must be 0 or 1, got %d", fn, axis);
    if (rows < 0 || cols < 0) return fail(BSQ_ERR_SHAPE, "%s: negative shape", fn);
    if (cols % 8 != 0) return fail(BSQ_ERR_SHAPE, "%s: cols (%lld) must be a multiple of 8", fn, (long long)cols);
    if (axis == 1 && cols % 16 != 0) return fail(BSQ_ERR_SHAPE, "%s: axis 1 needs cols %% 16 == 0", fn);
    if (axis == 0 && rows % 16 != 0) return fail(BSQ_ERR_SHAPE, "%s: axis 0 needs rows %% 16 == 0", fn);
    if (!signs) return fail(BSQ_ERR_NULL, "%s: signs is NULL", fn);
    if (rows == 0 || cols == 0) return ok();
    if (!x || !out) return fail(BSQ_ERR_NULL, "%s: NULL argument", fn);
    if (misaligned(x) || misaligned(out) || misaligned(signs)) return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return launched(bsq::launch_rht_apply(x, rows, cols, axis, signs, out, hip_stream), fn);
}

int nvfp4_quantize_rowscaled(const void* x, int64_t rows, int64_t cols, int rounding, uint64_t sr_seed,
                             uint32_t sr_stream, const int8_t* rht_signs, uint8_t* codes, uint8_t* scales,
                             float* amax_rows, float* s_enc_rows, void* hip_stream) {
    static const char* fn = "nvfp4_quantize_rowscaled";
    if (rounding != BSQ_RNE && rounding != BSQ_SR) return fail(BSQ_ERR_ARG, "%s: rounding must be 0 (RNE) or 1 (SR), got %d", fn, rounding);
    if (rows < 0 || cols < 0) return fail(BSQ_ERR_SHAPE, "%s: negative shape [%lld, %lld]", fn, (long long)rows, (long long)cols);
    if (cols % 16 != 0) return fail(BSQ_ERR_SHAPE, "%s: cols (%lld) must be a multiple of 16", fn, (long long)cols);
    if (rows == 0) return ok();
    if (!amax_rows || !s_enc_rows) return fail(BSQ_ERR_NULL, "%s: amax_rows and s_enc_rows are required", fn);
    if (cols > 0 && (!x || !codes || !scales)) return fail(BSQ_ERR_NULL, "%s: x, codes or scales is NULL", fn);
    if (misaligned(x) || misaligned(codes) || misaligned(rht_signs))
        return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return launched(bsq::launch_nvfp4_quantize_rowscaled(x, rows, cols, rounding, sr_seed, sr_stream, rht_signs,
                                                         codes, scales, amax_rows, s_enc_rows, hip_stream), fn);
}

int blockscaled_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes, const uint8_t* a_scales,
                     const float* a_s_enc, const uint8_t* b_codes, const uint8_t* b_scales, const float* b_s_enc,
                     void* c, int c_dtype, void* hip_stream) {
    static const char* fn = "blockscaled_gemm";
    const int a_rows = (fmt & BSQ_FMT_A_ROWSCALED) != 0, b_rows = (fmt & BSQ_FMT_B_ROWSCALED) != 0;
    const int slab = ((fmt & BSQ_FMT_MX_SLAB_A) ? 1 : 0) | ((fmt & BSQ_FMT_MX_SLAB_B) ? 2 : 0);
    const int flags = fmt & (BSQ_FMT_A_ROWSCALED | BSQ_FMT_B_ROWSCALED | BSQ_FMT_MX_SLAB);
    fmt &= ~(BSQ_FMT_A_ROWSCALED | BSQ_FMT_B_ROWSCALED | BSQ_FMT_MX_SLAB);
    if (fmt != BSQ_FMT_NVFP4 && fmt != BSQ_FMT_MXFP8) return fail(BSQ_ERR_ARG, "%s: fmt must be 0 (NVFP4) or 1 (MXFP8), optionally with the row-scaled or slab flags, got %d", fn, fmt | flags);
    if ((a_rows || b_rows) && fmt != BSQ_FMT_NVFP4) return fail(BSQ_ERR_ARG, "%s: the row-scaled flags apply to NVFP4 operands only", fn);
    if (slab && fmt != BSQ_FMT_MXFP8) return fail(BSQ_ERR_ARG, "%s: the slab flags apply to MXFP8 operands only", fn);
    if (slab && K % 512 != 0) return fail(BSQ_ERR_SHAPE, "%s: slab operands need K %% 512 == 0, got %lld", fn, (long long)K);
    if (c_dtype != BSQ_OUT_BF16 && c_dtype != BSQ_OUT_F32) return fail(BSQ_ERR_ARG, "%s: c_dtype must be 0 (bf16) or 1 (f32), got %d", fn, c_dtype);
    if (M < 0 || N < 0 || K < 0) return fail(BSQ_ERR_SHAPE, "%s: negative shape", fn);
    if (K % 32 != 0) return fail(BSQ_ERR_SHAPE, "%s: K (%lld) must be a multiple of 32", fn, (long long)K);
    if (K >= gemm_k_limit(fmt))
        return fail(BSQ_ERR_SHAPE, "%s: K (%lld) exceeds %lld", fn, (long long)K, (long long)gemm_k_limit(fmt) - 1);
    if (M == 0 || N == 0) return ok();
    if (!c) return fail(BSQ_ERR_NULL, "%s: c is NULL", fn);
    if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales)) return fail(BSQ_ERR_NULL, "%s: operand pointer is NULL", fn);
    if (fmt == BSQ_FMT_NVFP4 && (!a_s_enc || !b_s_enc)) return fail(BSQ_ERR_NULL, "%s: NVFP4 needs both tensor scales", fn);
    if (misaligned(a_codes) || misaligned(b_codes) || misaligned(c) || misaligned(a_scales) || misaligned(b_scales))
        return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return launched(bsq::launch_blockscaled_gemm(fmt, M, N, K, a_codes, a_scales, a_s_enc, b_codes, b_scales,
                                                 b_s_enc, a_rows, b_rows, c, c_dtype, hip_stream, slab), fn);
}

int blockscaled_grouped_gemm(int fmt, int mode, int64_t groups, const int64_t* offsets, int64_t M, int64_t N,
                             int64_t K, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_s_enc,
                             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_s_enc, void* c,
                             int c_dtype, void* hip_stream) {
    static const char* fn = "blockscaled_grouped_gemm";
    const int a_rows = (fmt & BSQ_FMT_A_ROWSCALED) != 0, b_rows = (fmt & BSQ_FMT_B_ROWSCALED) != 0;
    const int slab = ((fmt & BSQ_FMT_MX_SLAB_A) ? 1 : 0) | ((fmt & BSQ_FMT_MX_SLAB_B) ? 2 : 0);
    const int flags = fmt & (BSQ_FMT_A_ROWSCALED | BSQ_FMT_B_ROWSCALED);
    fmt &= ~(BSQ_FMT_A_ROWSCALED | BSQ_FMT_B_ROWSCALED | BSQ_FMT_MX_SLAB);
    if (slab && fmt != BSQ_FMT_MXFP8) return fail(BSQ_ERR_ARG, "%s: the slab flags apply to MXFP8 only", fn);
    if ((slab & 1) && mode != BSQ_GROUP_K)
        return fail(BSQ_ERR_ARG, "%s: BSQ_FMT_MX_SLAB_A applies with BSQ_GROUP_K only (M-grouped A is cut by the groups)", fn);
    if (slab && K % 512 != 0) return fail(BSQ_ERR_SHAPE, "%s: slab operands need K %% 512 == 0, got %lld", fn, (long long)K);
    if (fmt != BSQ_FMT_NVFP4 && fmt != BSQ_FMT_MXFP8) return fail(BSQ_ERR_ARG, "%s: fmt must be 0 (NVFP4) or 1 (MXFP8), optionally with the row-scaled flags, got %d", fn, fmt | flags);
    if (flags && fmt != BSQ_FMT_NVFP4) return fail(BSQ_ERR_ARG, "%s: the row-scaled flags apply to NVFP4 operands only", fn);
    if (mode != BSQ_GROUP_M && mode != BSQ_GROUP_K) return fail(BSQ_ERR_ARG, "%s: mode must be 1 (BSQ_GROUP_M) or 2 (BSQ_GROUP_K), got %d", fn, mode);
    if (flags && mode != BSQ_GROUP_M) return fail(BSQ_ERR_ARG, "%s: row-scaled operands are supported with BSQ_GROUP_M only", fn);
    if (c_dtype != BSQ_OUT_BF16 && c_dtype != BSQ_OUT_F32) return fail(BSQ_ERR_ARG, "%s: c_dtype must be 0 (bf16) or 1 (f32), got %d", fn, c_dtype);
    if (groups < 0 || M < 0 || N < 0 || K < 0) return fail(BSQ_ERR_SHAPE, "%s: negative size", fn);
    if (K % 32 != 0) return fail(BSQ_ERR_SHAPE, "%s: K (%lld) must be a multiple of 32", fn, (long long)K);
    if (K >= gemm_k_limit(fmt))
        return fail(BSQ_ERR_SHAPE, "%s: K (%lld) exceeds %lld", fn, (long long)K, (long long)gemm_k_limit(fmt) - 1);
    if (groups == 0 || M == 0 || N == 0) return ok();
    if (groups > (int64_t)1 << 24) return fail(BSQ_ERR_SHAPE, "%s: too many groups (%lld)", fn, (long long)groups);
    if (bsq::grouped_gemm_workgroups(mode, groups, M, N) > 0x7FFFFFFF) return fail(BSQ_ERR_SHAPE, "%s: problem too large for one launch", fn);
    if (!offsets) return fail(BSQ_ERR_NULL, "%s: offsets is NULL", fn);
    if (!c) return fail(BSQ_ERR_NULL, "%s: c is NULL", fn);
    if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales)) return fail(BSQ_ERR_NULL, "%s: operand pointer is NULL", fn);
    if (fmt == BSQ_FMT_NVFP4 && (!a_s_enc || !b_s_enc)) return fail(BSQ_ERR_NULL, "%s: NVFP4 needs both tensor-scale arrays", fn);
    if ((reinterpret_cast<uintptr_t>(offsets) & 7u) != 0) return fail(BSQ_ERR_ALIGN, "%s: offsets must be 8-byte aligned", fn);
    if (misaligned(a_codes) || misaligned(b_codes) || misaligned(c) || misaligned(a_scales) || misaligned(b_scales))
        return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    return launched(bsq::launch_blockscaled_grouped_gemm(fmt, mode, groups, offsets, M, N, K, a_codes, a_scales,
                                                         a_s_enc, b_codes, b_scales, b_s_enc, a_rows, b_rows, c,
                                                         c_dtype, hip_stream, slab), fn);
}

}  // extern "C"

// ---------------------------------------------------------------- the linear layer

namespace {

constexpr int64_t kAlign = 256;

int64_t up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// One NVFP4 operand inside a caller buffer: codes, scales, then amax[2] and s_enc[2].
struct Nv {
    int64_t codes, scales, amax, s_enc, end;
};

Nv nv_at(int64_t base, int64_t elems) {
    Nv o;
    o.codes = base;
    o.scales = up(o.codes + elems / 2);
    o.amax = up(o.scales + elems / 16);
    o.s_enc = o.amax + 8;
    o.end = up(o.s_enc + 8);
    return o;
}

struct LinearLayout {
    int64_t qws;                // the quantize calls' scratch (partial maxima), both phases
    Nv x_row, w_row;            // forward workspace
    Nv dy, w_col;               // backward workspace (dy holds both directions' codes)
    int64_t dy_col_codes, dy_col_scales;
    int64_t fwd_bytes, bwd_bytes;
    Nv x_col;                   // the saved activation
    int64_t saved_bytes;
};

LinearLayout linear_layout(int64_t T, int64_t K, int64_t N) {
    LinearLayout L;
    L.qws = 0;
    const int64_t q0 = up(BSQ_NVFP4_QUANTIZE_WORKSPACE_BYTES);
    L.x_row = nv_at(q0, T * K);
    L.w_row = nv_at(L.x_row.end, N * K);
    L.fwd_bytes = L.w_row.end;
    L.dy = nv_at(q0, T * N);
    L.dy_col_codes = L.dy.end;
    L.dy_col_scales = up(L.dy_col_codes + T * N / 2);
    L.w_col = nv_at(up(L.dy_col_scales + T * N / 16), K * N);
    L.bwd_bytes = L.w_col.end;
    L.x_col = nv_at(0, K * T);
    L.saved_bytes = L.x_col.end;
    return L;
}

template <typename T>
T* at(void* base, int64_t off) { return reinterpret_cast<T*>(static_cast<uint8_t*>(base) + off); }

int linear_shape_check(const char* fn, int64_t T, int64_t K, int64_t N) {
    if (T < 0 || K < 0 || N < 0) return fail(BSQ_ERR_SHAPE, "%s: negative shape", fn);
    if (T % 32 != 0 || K % 32 != 0 || N % 32 != 0)
        return fail(BSQ_ERR_SHAPE, "%s: tokens, in_features and out_features must be multiples of 32, got %lld, %lld, %lld",
                    fn, (long long)T, (long long)K, (long long)N);
    // each is the contraction length of one of the three NVFP4 GEMMs (wgrad contracts over tokens)
    const int64_t lim = gemm_k_limit(BSQ_FMT_NVFP4);
    if (T >= lim || K >= lim || N >= lim)
        return fail(BSQ_ERR_SHAPE, "%s: tokens, in_features and out_features must be below %lld", fn, (long long)lim);
    return BSQ_OK;
}

}  // namespace

extern "C" {

int64_t nvfp4_linear_workspace_bytes(int64_t tokens, int64_t in_features, int64_t out_features) {
    if (tokens < 0 || in_features < 0 || out_features < 0) return -1;
    const LinearLayout L = linear_layout(tokens, in_features, out_features);
    return L.fwd_bytes > L.bwd_bytes ? L.fwd_bytes : L.bwd_bytes;
}

int64_t nvfp4_linear_saved_bytes(int64_t tokens, int64_t in_features) {
    if (tokens < 0 || in_features < 0) return -1;
    return linear_layout(tokens, in_features, 0).saved_bytes;
}

int nvfp4_linear_forward(const void* x, const void* w, int64_t tokens, int64_t in_features, int64_t out_features,
                         uint64_t sr_seed, const int8_t* rht_signs, void* saved, void* workspace, void* y,
                         void* hip_stream) {
    static const char* fn = "nvfp4_linear_forward";
    const int64_t T = tokens, K = in_features, N = out_features;
    int st = linear_shape_check(fn, T, K, N);
    if (st) return st;
    if (T == 0 || K == 0 || N == 0) return fail(BSQ_ERR_SHAPE, "%s: empty layer", fn);
    if (!x || !w || !rht_signs || !saved || !workspace || !y) return fail(BSQ_ERR_NULL, "%s: NULL argument", fn);
    if (misaligned(x) || misaligned(w) || misaligned(rht_signs) || misaligned(saved) || misaligned(workspace) ||
        misaligned(y))
        return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    const LinearLayout L = linear_layout(T, K, N);
    void* ws = workspace;
    // X for both of its GEMMs in one pass: rowwise RNE (the fprop operand, in the workspace) and
    // columnwise along tokens with RHT + SR (the saved activation for wgrad); slot 0 of the saved
    // tensor scales holds the rowwise one
    st = bsq::launch_nvfp4_quantize_fprop_wgrad(x, T, K, BSQ_SR, sr_seed, 1, rht_signs, at<uint8_t>(ws, L.x_row.codes),
                                                at<uint8_t>(ws, L.x_row.scales), at<uint8_t>(saved, L.x_col.codes),
                                                at<uint8_t>(saved, L.x_col.scales), at<float>(saved, L.x_col.amax),
                                                at<float>(saved, L.x_col.s_enc), at<float>(ws, L.qws), hip_stream);
    if (st) return launched(st, fn);
    // W rowwise, RNE
    st = bsq::launch_nvfp4_quantize(w, N, K, BSQ_ROW, BSQ_RNE, 0, 0, nullptr, at<uint8_t>(ws, L.w_row.codes),
                                    at<uint8_t>(ws, L.w_row.scales), nullptr, nullptr, at<float>(ws, L.w_row.amax),
                                    at<float>(ws, L.w_row.s_enc), at<float>(ws, L.qws), hip_stream);
    if (st) return launched(st, fn);
    st = bsq::launch_blockscaled_gemm(BSQ_FMT_NVFP4, T, N, K, at<uint8_t>(ws, L.x_row.codes),
                                      at<uint8_t>(ws, L.x_row.scales), at<float>(saved, L.x_col.s_enc),
                                      at<uint8_t>(ws, L.w_row.codes), at<uint8_t>(ws, L.w_row.scales),
                                      at<float>(ws, L.w_row.s_enc), 0, 0, y, BSQ_OUT_BF16, hip_stream);
    return launched(st, fn);
}

int nvfp4_linear_backward(const void* dy, const void* w, const void* saved, int64_t tokens, int64_t in_features,
                          int64_t out_features, uint64_t sr_seed, const int8_t* rht_signs, void* workspace, void* dx,
                          float* dw, void* hip_stream) {
    static const char* fn = "nvfp4_linear_backward";
    const int64_t T = tokens, K = in_features, N = out_features;
    int st = linear_shape_check(fn, T, K, N);
    if (st) return st;
    if (T == 0 || K == 0 || N == 0) return fail(BSQ_ERR_SHAPE, "%s: empty layer", fn);
    if (!dy || !w || !saved || !rht_signs || !workspace || !dx || !dw) return fail(BSQ_ERR_NULL, "%s: NULL argument", fn);
    if (misaligned(dy) || misaligned(w) || misaligned(saved) || misaligned(rht_signs) || misaligned(workspace) ||
        misaligned(dx) || misaligned(dw))
        return fail(BSQ_ERR_ALIGN, "%s: device pointers must be 16-byte aligned", fn);
    const LinearLayout L = linear_layout(T, K, N);
    void* ws = workspace;
    void* sv = const_cast<void*>(saved);
    // dY in both directions in one pass (RHT + SR; rowwise along out_features for dgrad,
    // columnwise along tokens for wgrad)
    st = bsq::launch_nvfp4_quantize(dy, T, N, BSQ_ROW | BSQ_COL, BSQ_SR, sr_seed, 0, rht_signs,
                                    at<uint8_t>(ws, L.dy.codes), at<uint8_t>(ws, L.dy.scales),
                                    at<uint8_t>(ws, L.dy_col_codes), at<uint8_t>(ws, L.dy_col_scales),
                                    at<float>(ws, L.dy.amax), at<float>(ws, L.dy.s_enc), at<float>(ws, L.qws), hip_stream);
    if (st) return launched(st, fn);
    // wgrad: dW[N][K] = dY^T X over tokens
    st = bsq::launch_blockscaled_gemm(BSQ_FMT_NVFP4, N, K, T, at<uint8_t>(ws, L.dy_col_codes),
                                      at<uint8_t>(ws, L.dy_col_scales), at<float>(ws, L.dy.s_enc) + 1,
                                      at<uint8_t>(sv, L.x_col.codes), at<uint8_t>(sv, L.x_col.scales),
                                      at<float>(sv, L.x_col.s_enc) + 1, 0, 0, dw, BSQ_OUT_F32, hip_stream);
    if (st) return launched(st, fn);
    // dgrad operand W columnwise along out_features, RHT + SR
    st = bsq::launch_nvfp4_quantize(w, N, K, BSQ_COL, BSQ_SR, sr_seed, 2, rht_signs, nullptr, nullptr,
                                    at<uint8_t>(ws, L.w_col.codes), at<uint8_t>(ws, L.w_col.scales),
                                    at<float>(ws, L.w_col.amax), at<float>(ws, L.w_col.s_enc), at<float>(ws, L.qws),
                                    hip_stream);
    if (st) return launched(st, fn);
    // dgrad: dX[T][K] = dY W over out_features
    st = bsq::launch_blockscaled_gemm(BSQ_FMT_NVFP4, T, K, N, at<uint8_t>(ws, L.dy.codes),
                                      at<uint8_t>(ws, L.dy.scales), at<float>(ws, L.dy.s_enc),
                                      at<uint8_t>(ws, L.w_col.codes), at<uint8_t>(ws, L.w_col.scales),
                                      at<float>(ws, L.w_col.s_enc) + 1, 0, 0, dx, BSQ_OUT_BF16, hip_stream);
    return launched(st, fn);
}

}  // extern "C"
