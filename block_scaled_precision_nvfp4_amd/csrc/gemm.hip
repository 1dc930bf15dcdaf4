// gemm.hip -- block-scaled GEMM C[M][N] = alpha * A[M][K] * B[N][K]^T on gfx950 MFMA.
//
// NVFP4 operands (E2M1 codes, one E4M3 scale per 16 K-elements, fp32 tensor scale): the
// gfx950 block-scaled MFMA takes one power-of-two (E8M0) scale per 32 K-elements, which
// can express neither an E4M3 mantissa nor a 16-element block.  Each element is therefore
// dequantized in registers to f16 -- E2M1 value times E4M3 scale has at most 6 significant
// bits and lies in [2^-10, 2688], so the f16 value is exact -- and contracted with the
// f16 MFMA (v_mfma_f32_32x32x16_f16).  One 32x32x16 MFMA covers exactly one 16-block of K
// per lane half, and each lane's 8 operand values share one block scale.  The tensor
// scales enter once, in the epilogue: alpha = 1 / (S_a * S_b).
//
// MXFP8 operands (E4M3 codes, one E8M0 scale per 32 K-elements) map one-to-one onto the
// scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4: each lane holds the 32 codes of one
// 32-block and passes that block's scale byte.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of C; wave w computes the
// 64 x 64 quadrant (w >> 1, w & 1) as 2 x 2 MFMA tiles of 32 x 32.  The K loop stages
// 64-element slices of both operands (codes + scales) in LDS, with the next slice's
// global loads in flight while the current one is contracted.
#include "device_common.hpp"
#include "launch.hpp"

namespace bsq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));

constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GTHREADS = 256;

// ---------------------------------------------------------------- NVFP4

// LDS row strides (bytes): 32 code bytes per row padded to 36 so that the 32 rows read by a
// half-wave fall into distinct banks.
constexpr int NV_CODE_STRIDE = 36;
constexpr int NV_SC_STRIDE = 4;

struct GemmArgs {
    int64_t M, N, K;
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const float* a_s_enc;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* b_s_enc;
    void* c;
};

// Exact value of a 4-bit E2M1 code times a binary32 scale.  The code's exponent and
// mantissa bits placed at binary32 bits 24:22 form the value times 2^-126 (exponent field
// 0 gives the subnormal 0.5 case), so one multiplication by 2^126 rebiases it exactly.
__device__ __forceinline__ float e2m1_times(uint32_t c, float sc) {
    const float v = __uint_as_float(((c & 7u) << 22) | ((c & 8u) << 28)) * 0x1p126f;
    return v * sc;
}

__device__ __forceinline__ half8_t nv_dequant8(uint32_t codes8, float sc) {
    half8_t h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (_Float16)e2m1_times((codes8 >> (4 * j)) & 0xFu, sc);
    return h;
}

template <int OUT_F32>
__global__ __launch_bounds__(GTHREADS, 2) void gemm_nvfp4_kernel(GemmArgs g) {
    __shared__ uint8_t sA[GBM * NV_CODE_STRIDE];
    __shared__ uint8_t sB[GBN * NV_CODE_STRIDE];
    __shared__ uint8_t sAs[GBM * NV_SC_STRIDE];
    __shared__ uint8_t sBs[GBN * NV_SC_STRIDE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * GBM, n0 = (int64_t)blockIdx.x * GBN;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int64_t kb2 = K / 2, kb16 = K / 16;

    // global -> register staging: thread loads 16 code bytes of row (tid >> 1), half (tid & 1)
    const int lrow = tid >> 1, lhalf = tid & 1;
    const int64_t arow = m0 + lrow, brow = n0 + lrow;
    uint4 ra, rb;
    uint32_t ras, rbs;

    auto gload = [&](int64_t k0) {
        const int64_t kc = k0 + 32 * lhalf;             // first element of this 16-byte chunk
        ra = (arow < M && kc < K) ? *(const uint4*)(g.a_codes + arow * kb2 + kc / 2) : make_uint4(0, 0, 0, 0);
        rb = (brow < N && kc < K) ? *(const uint4*)(g.b_codes + brow * kb2 + kc / 2) : make_uint4(0, 0, 0, 0);
        // scales: 4 bytes per row per slice; lanes with lhalf == 0 take A, lhalf == 1 take B
        const int64_t srow = lhalf ? brow : arow;
        const int64_t slim = lhalf ? N : M;
        const uint8_t* sp = (lhalf ? g.b_scales : g.a_scales) + srow * kb16 + k0 / 16;
        uint32_t s = 0;
        if (srow < slim) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (k0 + 16 * i < K) s |= (uint32_t)sp[i] << (8 * i);
        }
        if (lhalf) rbs = s; else ras = s;
    };
    auto sstore = [&]() {
        uint32_t* pa = (uint32_t*)(sA + lrow * NV_CODE_STRIDE + 16 * lhalf);
        uint32_t* pb = (uint32_t*)(sB + lrow * NV_CODE_STRIDE + 16 * lhalf);
        pa[0] = ra.x; pa[1] = ra.y; pa[2] = ra.z; pa[3] = ra.w;
        pb[0] = rb.x; pb[1] = rb.y; pb[2] = rb.z; pb[3] = rb.w;
        if (lhalf) *(uint32_t*)(sBs + lrow * NV_SC_STRIDE) = rbs;
        else *(uint32_t*)(sAs + lrow * NV_SC_STRIDE) = ras;
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int frow = lane & 31, khalf = lane >> 5;
    const int64_t nk = (K + GBK - 1) / GBK;

    if (nk > 0) gload(0);
    for (int64_t kt = 0; kt < nk; ++kt) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (kt + 1 < nk) gload((kt + 1) * GBK);
#pragma unroll
        for (int ks = 0; ks < GBK / 16; ++ks) {
            half8_t af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = wm + 32 * i + frow;
                const uint32_t cw = *(const uint32_t*)(sA + r * NV_CODE_STRIDE + 8 * ks + 4 * khalf);
                const float sc = e4m3_decode_nonneg(sAs[r * NV_SC_STRIDE + ks] & 0x7Fu);
                af[i] = nv_dequant8(cw, sc);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wn + 32 * j + frow;
                const uint32_t cw = *(const uint32_t*)(sB + r * NV_CODE_STRIDE + 8 * ks + 4 * khalf);
                const float sc = e4m3_decode_nonneg(sBs[r * NV_SC_STRIDE + ks] & 0x7Fu);
                bf[j] = nv_dequant8(cw, sc);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }

    // epilogue: alpha = 1 / (S_a * S_b), one rounding (the product is formed in binary64)
    const float alpha = (float)(1.0 / ((double)g.a_s_enc[0] * (double)g.b_s_enc[0]));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * khalf + (r & 3);
                const int64_t col = n0 + wn + 32 * j + frow;
                if (row < M && col < N) {
                    const float v = acc[i][j][r] * alpha;
                    if (OUT_F32) ((float*)g.c)[row * N + col] = v;
                    else ((uint16_t*)g.c)[row * N + col] = (uint16_t)f32_to_bf16_rne(v);
                }
            }
}

// ---------------------------------------------------------------- MXFP8

constexpr int MX_CODE_STRIDE = 80;   // 64 code bytes per row + 16 bytes of padding
constexpr int MX_SC_STRIDE = 2;

template <int OUT_F32>
__global__ __launch_bounds__(GTHREADS, 2) void gemm_mxfp8_kernel(GemmArgs g) {
    __shared__ uint8_t sA[GBM * MX_CODE_STRIDE];
    __shared__ uint8_t sB[GBN * MX_CODE_STRIDE];
    __shared__ uint8_t sAs[GBM * MX_SC_STRIDE];
    __shared__ uint8_t sBs[GBN * MX_SC_STRIDE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * GBM, n0 = (int64_t)blockIdx.x * GBN;
    const int64_t M = g.M, N = g.N, K = g.K;
    const int64_t kb32 = K / 32;

    // staging: per operand 128 rows x 64 bytes = 512 chunks of 16 bytes, 2 per thread
    uint4 ra[2], rb[2];
    uint32_t rs;   // threads 0..127: A scales of row tid; 128..255: B scales of row tid - 128
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int ch = tid + GTHREADS * p;
            const int row = ch >> 2, c16 = ch & 3;
            const int64_t kc = k0 + 16 * c16;
            const int64_t ar = m0 + row, br = n0 + row;
            ra[p] = (ar < M && kc < K) ? *(const uint4*)(g.a_codes + ar * K + kc) : make_uint4(0, 0, 0, 0);
            rb[p] = (br < N && kc < K) ? *(const uint4*)(g.b_codes + br * K + kc) : make_uint4(0, 0, 0, 0);
        }
        const int srow = tid & 127;
        const bool isb = tid >= 128;
        const int64_t gr = (isb ? n0 : m0) + srow;
        const uint8_t* sp = (isb ? g.b_scales : g.a_scales) + gr * kb32 + k0 / 32;
        uint32_t s = 0;
        if (gr < (isb ? N : M)) {
            if (k0 < K) s |= sp[0];
            if (k0 + 32 < K) s |= (uint32_t)sp[1] << 8;
        }
        rs = s;
    };
    auto sstore = [&]() {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int ch = tid + GTHREADS * p;
            const int row = ch >> 2, c16 = ch & 3;
            *(uint4*)(sA + row * MX_CODE_STRIDE + 16 * c16) = ra[p];
            *(uint4*)(sB + row * MX_CODE_STRIDE + 16 * c16) = rb[p];
        }
        const int srow = tid & 127;
        uint8_t* d = (tid >= 128 ? sBs : sAs) + srow * MX_SC_STRIDE;
        d[0] = (uint8_t)(rs & 0xFF);
        d[1] = (uint8_t)(rs >> 8);
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int frow = lane & 31, khalf = lane >> 5;
    const int64_t nk = (K + GBK - 1) / GBK;

    if (nk > 0) gload(0);
    for (int64_t kt = 0; kt < nk; ++kt) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (kt + 1 < nk) gload((kt + 1) * GBK);
        intx8 af[2], bf[2];
        int as[2], bs[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = wm + 32 * i + frow;
            const uint4 lo = *(const uint4*)(sA + r * MX_CODE_STRIDE + 32 * khalf);
            const uint4 hi = *(const uint4*)(sA + r * MX_CODE_STRIDE + 32 * khalf + 16);
            af[i] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            as[i] = sAs[r * MX_SC_STRIDE + khalf];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = wn + 32 * j + frow;
            const uint4 lo = *(const uint4*)(sB + r * MX_CODE_STRIDE + 32 * khalf);
            const uint4 hi = *(const uint4*)(sB + r * MX_CODE_STRIDE + 32 * khalf + 16);
            bf[j] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            bs[j] = sBs[r * MX_SC_STRIDE + khalf];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0,
                                                                             as[i], 0, bs[j]);
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * khalf + (r & 3);
                const int64_t col = n0 + wn + 32 * j + frow;
                if (row < M && col < N) {
                    const float v = acc[i][j][r];
                    if (OUT_F32) ((float*)g.c)[row * N + col] = v;
                    else ((uint16_t*)g.c)[row * N + col] = (uint16_t)f32_to_bf16_rne(v);
                }
            }
}

int launch_blockscaled_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const uint8_t* a_scales, const float* a_s_enc, const uint8_t* b_codes,
                            const uint8_t* b_scales, const float* b_s_enc, void* c, int c_dtype, void* hip_stream) {
    if (M == 0 || N == 0) return 0;
    hipStream_t s = (hipStream_t)hip_stream;
    GemmArgs g{M, N, K, a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc, c};
    const dim3 grid((unsigned)((N + GBN - 1) / GBN), (unsigned)((M + GBM - 1) / GBM), 1);
    if (fmt == 0) {
        if (c_dtype == 1) hipLaunchKernelGGL(gemm_nvfp4_kernel<1>, grid, dim3(GTHREADS), 0, s, g);
        else hipLaunchKernelGGL(gemm_nvfp4_kernel<0>, grid, dim3(GTHREADS), 0, s, g);
    } else {
        if (c_dtype == 1) hipLaunchKernelGGL(gemm_mxfp8_kernel<1>, grid, dim3(GTHREADS), 0, s, g);
        else hipLaunchKernelGGL(gemm_mxfp8_kernel<0>, grid, dim3(GTHREADS), 0, s, g);
    }
    return (int)hipGetLastError();
}

}  // namespace bsq
