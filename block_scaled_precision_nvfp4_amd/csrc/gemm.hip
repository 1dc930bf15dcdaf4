// gemm.hip -- block-scaled GEMM C[M][N] = alpha * A[M][K] * B[N][K]^T on gfx950 MFMA.
//
// NVFP4 operands (E2M1 codes, one E4M3 scale per 16 K-elements, fp32 tensor scale).  The
// gfx950 block-scaled MFMA takes one power-of-two (E8M0) scale per 32 K-elements, which
// can express neither an E4M3 mantissa nor a 16-element block.  Each element is therefore
// dequantized in registers to f16 -- E2M1 value times E4M3 scale has at most 6 significant
// bits and lies in [2^-10, 2688], so the f16 value is exact -- and contracted with the
// f16 MFMA v_mfma_f32_32x32x16_f16.  Dequantization per pair of codes is one
// v_cvt_scalef32_pk_f16_fp4 (hardware E2M1 -> f16; its scale operand contributes only its
// exponent, here 2^8) and one packed f16 multiply by the block scale, held as the f16
// whose bit pattern is (E4M3 byte << 7): for every E4M3 code, normal or subnormal, that
// f16 equals the E4M3 value times 2^-8, so the product is exactly code * scale.  The
// tensor scales enter once, in the epilogue: alpha = 1 / (S_a * S_b).
//
// MXFP8 operands (E4M3 codes, one E8M0 scale per 32 K-elements) map one-to-one onto the
// scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4.  Its K layout: in lane (row, g), bytes
// 0-15 of the 32-byte operand are K-elements 16g..16g+15 of the step and bytes 16-31 are
// K-elements 32+16g..32+16g+15; the scale of K-block 0 (elements 0-31) comes from lanes
// 0-31, that of K-block 1 from lanes 32-63.
//
// Tiling (both formats): a 256-thread workgroup computes a 256 x 256 tile of C; wave w
// computes the 128 x 128 quadrant (w >> 1, w & 1) as 4 x 4 MFMA tiles of 32 x 32 (256
// fp32 accumulators per lane).  Each K slice (128 elements for NVFP4, 64 for MXFP8) of
// both operands is 64 bytes of codes per row, staged through registers into one of two
// LDS buffers (one barrier per slice); 16-byte chunks are XOR-swizzled by row so that the
// fragment reads (ds_read_b128) of 8 consecutive rows hit distinct banks.  Ragged M, N
// and a K tail (K % 32 == 0) are handled by zero-filling the staged slice.  Workgroups
// are renumbered so that each of the 8 XCDs (which take workgroups round-robin) works on
// a contiguous band of output tiles and reuses operand rows from its own L2.
#include "device_common.hpp"
#include "launch.hpp"

namespace bsq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));

constexpr int GBM = 256, GBN = 256;
constexpr int GTHREADS = 256;
constexpr int ROWB = 64;   // code bytes per row per K slice (both formats)

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

template <int FMT>
struct Fmt {
    static constexpr int BK = FMT == 0 ? 128 : 64;    // K elements per slice
    static constexpr int EPB = FMT == 0 ? 2 : 1;      // elements per code byte
    static constexpr int BLK = FMT == 0 ? 16 : 32;    // elements per scale
    static constexpr int SPR = BK / BLK;              // scale bytes per row per slice (8 or 2)
    // LDS bytes per row for scales: NVFP4 keeps each scale as a packed f16 pair (4 bytes),
    // MXFP8 keeps the raw E8M0 bytes (padded to 4).
    static constexpr int SCB = FMT == 0 ? 4 * SPR : 4;
    static constexpr int STAGE = (GBM + GBN) * (ROWB + SCB);
    static constexpr int LDS = 2 * STAGE;
};

// Byte offset of 16-byte chunk c (0..3) of LDS code row r.
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + ((c ^ ((r >> 1) & 3)) << 4); }

// Staging registers of one K slice: chunks (tid + 256p) of the 256 x 4 chunk grid of A and
// of B, and the scale bytes of two rows of one operand.
struct Stage {
    uint4 a[4], b[4];
    uint32_t s[2][2];   // [row half][word]
};

template <int FMT>
__device__ __forceinline__ void stage_load(const GemmArgs& g, int64_t m0, int64_t n0, int64_t k0, Stage& st) {
    using F = Fmt<FMT>;
    const int tid = threadIdx.x;
    const int64_t rowbytes = g.K / F::EPB;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int idx = tid + GTHREADS * p;
        const int r = idx >> 2, c = idx & 3;
        const int64_t kc = k0 + (int64_t)c * 16 * F::EPB;   // first element of the chunk
        const bool kok = kc < g.K;
        const int64_t ar = m0 + r, br = n0 + r;
        st.a[p] = (kok && ar < g.M) ? *(const uint4*)(g.a_codes + ar * rowbytes + kc / F::EPB) : make_uint4(0, 0, 0, 0);
        st.b[p] = (kok && br < g.N) ? *(const uint4*)(g.b_codes + br * rowbytes + kc / F::EPB) : make_uint4(0, 0, 0, 0);
    }
    // scales: threads 0..127 own A rows t and t + 128; threads 128..255 the same B rows
    const int op = tid >> 7, rr = tid & 127;
    const int64_t nrows = op ? g.N : g.M;
    const int64_t base = op ? n0 : m0;
    const uint8_t* sp = op ? g.b_scales : g.a_scales;
    const int64_t sstride = g.K / F::BLK;
    const bool full = (k0 + F::BK <= g.K) && (sstride % F::SPR == 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t row = base + rr + 128 * h;
        uint32_t w0 = 0, w1 = 0;
        if (row < nrows) {
            const uint8_t* q = sp + row * sstride + k0 / F::BLK;
            if (full) {
                if (F::SPR == 8) {
                    const uint2 v = *(const uint2*)q;
                    w0 = v.x;
                    w1 = v.y;
                } else {
                    w0 = *(const uint16_t*)q;
                }
            } else {
#pragma unroll
                for (int i = 0; i < F::SPR; ++i) {
                    const uint32_t b = (k0 + (int64_t)i * F::BLK < g.K) ? q[i] : 0u;
                    if (i < 4) w0 |= b << (8 * i); else w1 |= b << (8 * (i - 4));
                }
            }
        }
        st.s[h][0] = w0;
        st.s[h][1] = w1;
    }
}

// f16 pair {s, s} of an E4M3 scale byte b, times 2^-8: bit pattern b << 7 in each half.
__device__ __forceinline__ uint32_t scale_pair(uint32_t b) {
    const uint32_t v = (b & 0x7Fu) << 7;
    return v | (v << 16);
}

template <int FMT>
__device__ __forceinline__ void stage_store(uint8_t* buf, const Stage& st) {
    using F = Fmt<FMT>;
    const int tid = threadIdx.x;
    uint8_t* sA = buf;
    uint8_t* sB = buf + GBM * ROWB;
    uint8_t* sAs = buf + (GBM + GBN) * ROWB;
    uint8_t* sBs = sAs + GBM * F::SCB;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int idx = tid + GTHREADS * p;
        const int r = idx >> 2, c = idx & 3;
        *(uint4*)(sA + swz(r, c)) = st.a[p];
        *(uint4*)(sB + swz(r, c)) = st.b[p];
    }
    const int op = tid >> 7, rr = tid & 127;
    uint8_t* ss = op ? sBs : sAs;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = rr + 128 * h;
        if (FMT == 0) {
            // 8 scales -> 8 packed f16 pairs (32 bytes); the two 16-byte halves (blocks 0-3 and
            // 4-7) are swapped on rows with bit 2 set so that 8 consecutive rows read distinct banks
            const uint32_t w0 = st.s[h][0], w1 = st.s[h][1];
            const uint4 lo = make_uint4(scale_pair(w0), scale_pair(w0 >> 8), scale_pair(w0 >> 16), scale_pair(w0 >> 24));
            const uint4 hi = make_uint4(scale_pair(w1), scale_pair(w1 >> 8), scale_pair(w1 >> 16), scale_pair(w1 >> 24));
            const int sw = (r >> 2) & 1;
            *(uint4*)(ss + r * F::SCB + (sw << 4)) = lo;
            *(uint4*)(ss + r * F::SCB + ((sw ^ 1) << 4)) = hi;
        } else {
            *(uint32_t*)(ss + r * F::SCB) = st.s[h][0];
        }
    }
}

template <int FMT>
__device__ __forceinline__ void compute_slice(const uint8_t* buf, floatx16 (&acc)[4][4], int wm, int wn, int lane) {
    using F = Fmt<FMT>;
    const uint8_t* sA = buf;
    const uint8_t* sB = buf + GBM * ROWB;
    const uint8_t* sAs = buf + (GBM + GBN) * ROWB;
    const uint8_t* sBs = sAs + GBM * F::SCB;
    const int frow = lane & 31, kh = lane >> 5;
    if constexpr (FMT == 0) {
        // lane (row, kh) owns code bytes [32kh, 32kh + 32) of the slice: step s uses its dword s
        // (K elements 64kh + 8s .. +8, block 4kh + s/2)
        uint4 ca[4][2], cb[4][2], sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm + 32 * i + frow;
            ca[i][0] = *(const uint4*)(sA + swz(r, 2 * kh));
            ca[i][1] = *(const uint4*)(sA + swz(r, 2 * kh + 1));
            sa[i] = *(const uint4*)(sAs + r * F::SCB + ((kh ^ ((r >> 2) & 1)) << 4));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn + 32 * j + frow;
            cb[j][0] = *(const uint4*)(sB + swz(r, 2 * kh));
            cb[j][1] = *(const uint4*)(sB + swz(r, 2 * kh + 1));
            sb[j] = *(const uint4*)(sBs + r * F::SCB + ((kh ^ ((r >> 2) & 1)) << 4));
        }
        auto dword = [](const uint4 (&c)[2], int s) -> uint32_t {
            const uint4& q = c[s >> 2];
            const int d = s & 3;
            return d == 0 ? q.x : (d == 1 ? q.y : (d == 2 ? q.z : q.w));
        };
        auto sword = [](const uint4& q, int b) -> uint32_t {
            return b == 0 ? q.x : (b == 1 ? q.y : (b == 2 ? q.z : q.w));
        };
        auto dq = [](uint32_t w, uint32_t sc2) -> half8_t {
            const half2_t s = __builtin_bit_cast(half2_t, sc2);
            const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s;
            const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s;
            const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s;
            const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s;
            return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
        };
        static_for<0, 8>([&](auto s_c) {
            constexpr int s = decltype(s_c)::value;
            half8_t a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = dq(dword(ca[i], s), sword(sa[i], s >> 1));
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = dq(dword(cb[j], s), sword(sb[j], s >> 1));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
            // keep each step's dequantized operands live only for that step
            __builtin_amdgcn_sched_barrier(0);
        });
    } else {
        intx8 a[4], b[4];
        int as[4], bs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm + 32 * i + frow;
            const uint4 lo = *(const uint4*)(sA + swz(r, kh));
            const uint4 hi = *(const uint4*)(sA + swz(r, 2 + kh));
            a[i] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            as[i] = sAs[r * F::SCB + kh];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn + 32 * j + frow;
            const uint4 lo = *(const uint4*)(sB + swz(r, kh));
            const uint4 hi = *(const uint4*)(sB + swz(r, 2 + kh));
            b[j] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            bs[j] = sBs[r * F::SCB + kh];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, as[i], 0,
                                                                             bs[j]);
    }
}

// Output tile of this workgroup.  Workgroup ids are dealt to the 8 XCDs round-robin; the
// id is remapped so that XCD x receives the contiguous tile range [x*T/8, (x+1)*T/8),
// walked in bands of GROUP tile-rows (column-major inside a band) for L2 reuse.
__device__ __forceinline__ void tile_of(int64_t nbm, int64_t nbn, int64_t& tm, int64_t& tn) {
    const int64_t T = nbm * nbn;
    int64_t id = blockIdx.x;
    const int64_t T8 = (T / 8) * 8;
    if (id < T8) id = (id % 8) * (T8 / 8) + id / 8;
    constexpr int64_t GROUP = 8;
    const int64_t band = id / (GROUP * nbn);
    const int64_t first = band * GROUP;
    const int64_t rows = (nbm - first) < GROUP ? (nbm - first) : GROUP;
    const int64_t in = id - band * GROUP * nbn;
    tm = first + in % rows;
    tn = in / rows;
}

template <int FMT, int OUT_F32>
__global__ __launch_bounds__(GTHREADS, 1) void gemm_kernel(GemmArgs g) {
    using F = Fmt<FMT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t tm, tn;
    tile_of((g.M + GBM - 1) / GBM, (g.N + GBN - 1) / GBN, tm, tn);
    const int64_t m0 = tm * GBM, n0 = tn * GBN;
    const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (g.K + F::BK - 1) / F::BK;
    Stage st;
    if (nk > 0) {
        stage_load<FMT>(g, m0, n0, 0, st);
        stage_store<FMT>(lds, st);
        __syncthreads();
        if (nk > 1) stage_load<FMT>(g, m0, n0, F::BK, st);
    }
    for (int64_t kt = 0; kt < nk; ++kt) {
        compute_slice<FMT>(lds + (kt & 1) * F::STAGE, acc, wm, wn, lane);
        if (kt + 1 < nk) stage_store<FMT>(lds + ((kt + 1) & 1) * F::STAGE, st);
        if (kt + 2 < nk) stage_load<FMT>(g, m0, n0, (kt + 2) * F::BK, st);
        __syncthreads();
    }

    float alpha = 1.0f;
    if (FMT == 0) alpha = (float)(1.0 / ((double)g.a_s_enc[0] * (double)g.b_s_enc[0]));
    const int frow = lane & 31, kh = lane >> 5;
    static_for<0, 16>([&](auto t_c) {
        constexpr int i = decltype(t_c)::value >> 2, j = decltype(t_c)::value & 3;
        const int64_t col = n0 + wn + 32 * j + frow;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * kh + (r & 3);
            if (row < g.M && col < g.N) {
                const float v = acc[i][j][r] * alpha;
                if (OUT_F32) ((float*)g.c)[row * g.N + col] = v;
                else ((uint16_t*)g.c)[row * g.N + col] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

template <int FMT, int OUT>
static int launch_one(const GemmArgs& g, hipStream_t s) {
    using F = Fmt<FMT>;
    static bool configured = false;   // raising the dynamic-LDS limit is a per-process, per-kernel setting
    if (!configured) {
        const hipError_t e = hipFuncSetAttribute((const void*)gemm_kernel<FMT, OUT>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, F::LDS);
        if (e != hipSuccess) return (int)e;
        configured = true;
    }
    const int64_t tiles = ((g.M + GBM - 1) / GBM) * ((g.N + GBN - 1) / GBN);
    hipLaunchKernelGGL((gemm_kernel<FMT, OUT>), dim3((unsigned)tiles), dim3(GTHREADS), F::LDS, s, g);
    return (int)hipGetLastError();
}

int launch_blockscaled_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const uint8_t* a_scales, const float* a_s_enc, const uint8_t* b_codes,
                            const uint8_t* b_scales, const float* b_s_enc, void* c, int c_dtype, void* hip_stream) {
    if (M == 0 || N == 0) return 0;
    hipStream_t s = (hipStream_t)hip_stream;
    GemmArgs g{M, N, K, a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc, c};
    if (fmt == 0) return c_dtype == 1 ? launch_one<0, 1>(g, s) : launch_one<0, 0>(g, s);
    return c_dtype == 1 ? launch_one<1, 1>(g, s) : launch_one<1, 0>(g, s);
}

}  // namespace bsq
