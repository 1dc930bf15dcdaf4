// launch.hpp -- internal host-side launchers of the HIP kernels.  The C ABI (api.cpp)
// validates every argument before calling one of these; the launchers only enqueue
// kernels and return 0 or a hipError_t code.  Streams travel as void* so that api.cpp
// needs no HIP header.
#pragma once

#include <stdint.h>

namespace bsq {

// With mx_codes (direction == BSQ_COL only): also the MXFP8 rowwise cast of x into mx_codes /
// mx_scales (row-major, or the slab layout when mx_slab), from the same pass over x.
int launch_nvfp4_quantize(const void* x, int64_t R, int64_t C, int direction, int rounding, uint64_t seed,
                          uint32_t stream, const int8_t* signs, uint8_t* row_codes, uint8_t* row_scales,
                          uint8_t* col_codes, uint8_t* col_scales, float* amax, float* s_enc, float* workspace,
                          void* hip_stream, uint8_t* mx_codes = nullptr, uint8_t* mx_scales = nullptr,
                          int mx_slab = 0);
int launch_nvfp4_quantize_fprop_wgrad(const void* x, int64_t R, int64_t C, int rounding, uint64_t seed,
                                      uint32_t stream, const int8_t* signs, uint8_t* row_codes, uint8_t* row_scales,
                                      uint8_t* col_codes, uint8_t* col_scales, float* amax, float* s_enc,
                                      float* workspace, void* hip_stream);
int launch_nvfp4_quantize_noalloc(const void* x, int64_t R, int64_t C, int direction, int rounding, uint64_t seed,
                                  uint32_t stream, const int8_t* signs, uint8_t* row_codes, uint8_t* row_scales,
                                  uint8_t* col_codes, uint8_t* col_scales, float* amax, float* s_enc,
                                  void* hip_stream);
int launch_mxfp8_quantize(const void* x, int64_t R, int64_t C, int direction, uint8_t* row_codes,
                          uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, void* hip_stream);
int launch_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s_enc, int64_t rows,
                            int64_t cols, void* out, void* hip_stream);
int launch_mxfp8_requantize_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* s_enc, int64_t R,
                                  int64_t C, int direction, uint8_t* row_codes, uint8_t* row_scales,
                                  uint8_t* col_codes, uint8_t* col_scales, void* hip_stream);
int launch_rht_apply(const void* x, int64_t R, int64_t C, int axis, const int8_t* signs, float* out,
                     void* hip_stream);
int launch_blockscaled_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const uint8_t* a_scales, const float* a_s_enc, const uint8_t* b_codes,
                            const uint8_t* b_scales, const float* b_s_enc, int a_rows, int b_rows, void* c,
                            int c_dtype, void* hip_stream, int slab = 0);
int64_t grouped_gemm_workgroups(int mode, int64_t groups, int64_t M, int64_t N);
int launch_blockscaled_grouped_gemm(int fmt, int mode, int64_t groups, const int64_t* offsets, int64_t M, int64_t N,
                                    int64_t K, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_s_enc,
                                    const uint8_t* b_codes, const uint8_t* b_scales, const float* b_s_enc,
                                    int a_rows, int b_rows, void* c, int c_dtype, void* hip_stream, int slab = 0);
int launch_nvfp4_quantize_rowscaled(const void* x, int64_t R, int64_t C, int rounding, uint64_t seed,
                                    uint32_t stream, const int8_t* signs, uint8_t* codes, uint8_t* scales,
                                    float* amax_rows, float* s_enc_rows, void* hip_stream);
const char* hip_error_string(int e);

}  // namespace bsq
