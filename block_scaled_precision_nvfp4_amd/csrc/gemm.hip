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
// Tiling: a workgroup computes a 256 x 256 tile of C.  NVFP4 runs 8 waves (two per SIMD),
// each a 128 x 64 block of 4 x 2 MFMA tiles of 32 x 32 (128 fp32 accumulators per lane), so
// that one wave's dequantization overlaps the other's MFMAs; MXFP8 runs 4 waves of 128 x
// 128 (4 x 4 tiles, 256 accumulators).  Each K slice (128 elements for NVFP4, 64 for MXFP8)
// of both operands is 64 bytes of codes per row, loaded with buffer loads (the hardware
// range check zero-fills rows beyond M or N, an out-of-range offset the K tail) into
// registers and stored to a ring of 3 LDS buffers, two slices ahead of its use, with one
// barrier per slice.  16-byte chunks are XOR-swizzled by row for conflict-free fragment
// reads.  Inside a slice the operands of the next MFMA step are read from LDS (and, for
// NVFP4, dequantized) while the current step's MFMAs issue.  Workgroups are renumbered so
// that each of the 8 XCDs (which take workgroups round-robin) works on a contiguous band of
// output tiles and reuses operand rows from its own L2.
#include "device_common.hpp"
#include "launch.hpp"

namespace bsq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));

constexpr int GBM = 256, GBN = 256;
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
    static constexpr int SCB = FMT == 0 ? 8 : 4;      // LDS bytes per row for scales (raw bytes)
    static constexpr int STAGE = (GBM + GBN) * (ROWB + SCB);
    static constexpr int NSTAGE = 3;
    static constexpr int LDS = NSTAGE * STAGE;
    // waves per workgroup and MFMA tiles per wave: NVFP4 runs 8 waves (two per SIMD) of
    // 128 x 64 so that one wave's dequantization overlaps the other's MFMAs; MXFP8 (no
    // dequantization) runs 4 waves of 128 x 128.
#ifndef BSQ_MX_WAVES
#define BSQ_MX_WAVES 4
#endif
    static constexpr int NW = FMT == 0 ? 8 : BSQ_MX_WAVES;
    static constexpr int THREADS = 64 * NW;
    static constexpr int TM = 4;                             // 32-row A fragments per wave
    static constexpr int TN = FMT == 0 ? 2 : (NW == 8 ? 2 : 4);   // 32-row B fragments per wave
    static constexpr int WAVES_N = GBN / (32 * TN);
};

// Byte offset of 16-byte chunk c (0..3) of LDS code row r.  The XOR with bits 3..4 of the
// row was the fastest placement measured for the fragment reads (32 consecutive rows, one
// chunk per lane half): about 110 B/clk/CU against 90 for bits 1..2 and 55 unswizzled.
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + ((c ^ ((r >> 3) & 3)) << 4); }

// MXFP8 LDS scale byte of row r (0..255), K-block kb (0..1) of the slice:
// [half r/128][block][row mod 32][fragment (r/32) mod 4].
__device__ __forceinline__ int mx_sidx(int r, int kb) {
    return (((r >> 7) * 2 + kb) << 7) + ((r & 31) << 2) + ((r >> 5) & 3);
}

// Byte offset of scale dword w (0..1) of LDS scale row r (NVFP4: 8 raw E4M3 bytes per row,
// the two dwords swapped on rows with bit 4 set so that 32 consecutive rows reading the
// same dword hit 32 distinct banks).
__device__ __forceinline__ int sswz(int r, int w) { return r * 8 + ((w ^ ((r >> 4) & 1)) << 2); }

// Staging registers of one K slice: chunks (tid + 256p) of the 256 x 4 chunk grid of A and
// of B, and the scale bytes of two rows of one operand.
struct Stage {
    uint4 a[4], b[4];
    uint32_t s[2][2];   // [row half][word]
};

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

// Buffer resources of this workgroup's operand rows.  Each resource starts at the tile's
// first row and covers the rows that exist, so a load from a row beyond M or N returns zero
// (hardware range check); a chunk beyond K gets an offset past the range.  Loads are issued
// unconditionally (a branch around a load makes the compiler wait for it before the next
// one), each with one 32-bit lane offset and the slice's byte offset as a scalar.
struct Operands {
    __amdgpu_buffer_rsrc_t a, b, as, bs;
};

constexpr int RSRC_FLAGS = 0x00020000;   // raw 32-bit data, no format conversion
constexpr uint32_t OOB = 0x80000000u;    // an offset beyond every resource's range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, RSRC_FLAGS);
}

template <int FMT>
__device__ __forceinline__ Operands make_operands(const GemmArgs& g, int64_t m0, int64_t n0) {
    using F = Fmt<FMT>;
    const int64_t rowbytes = g.K / F::EPB, sstride = g.K / F::BLK;
    Operands o;
    o.a = make_rsrc(g.a_codes + m0 * rowbytes, (g.M - m0) * rowbytes);
    o.b = make_rsrc(g.b_codes + n0 * rowbytes, (g.N - n0) * rowbytes);
    o.as = make_rsrc(g.a_scales + m0 * sstride, (g.M - m0) * sstride);
    o.bs = make_rsrc(g.b_scales + n0 * sstride, (g.N - n0) * sstride);
    return o;
}

template <int FMT>
__device__ __forceinline__ void stage_load(const GemmArgs& g, const Operands& o, int64_t k0, Stage& st) {
    using F = Fmt<FMT>;
    const int tid = threadIdx.x;
    const uint32_t rowbytes = (uint32_t)(g.K / F::EPB);
    const int soff = (int)(k0 / F::EPB);
    const bool tail = k0 + F::BK > g.K;   // uniform
#pragma unroll
    for (int p = 0; p < GBM * 4 / F::THREADS; ++p) {
        const int idx = tid + F::THREADS * p;
        const int r = idx >> 2, c = idx & 3;
        uint32_t off = (uint32_t)r * rowbytes + 16u * c;
        if (tail && k0 + (int64_t)c * 16 * F::EPB >= g.K) off = OOB;
        st.a[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(o.a, off, soff, 0));
        st.b[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(o.b, off, soff, 0));
    }
    // scales: the first half of the threads own A rows (two rows each with 256 threads, one
    // with 512), the second half the same B rows.  The operand choice is wave-uniform;
    // reading it through readfirstlane lets the resource stay in scalar registers.
    constexpr int HT = F::THREADS / 2, RPT = GBM / HT;
    const int op = __builtin_amdgcn_readfirstlane(tid / HT), rr = tid % HT;
    const uint32_t sstride = (uint32_t)(g.K / F::BLK);
    const int ssoff = (int)(k0 / F::BLK);
    const bool aligned = (sstride % F::SPR) == 0 && !tail;   // uniform
#pragma unroll
    for (int h = 0; h < RPT; ++h) {
        const uint32_t off = (uint32_t)(rr + HT * h) * sstride;
        const __amdgpu_buffer_rsrc_t rs = op ? o.bs : o.as;
        uint32_t w0 = 0, w1 = 0;
        if (aligned) {
            if (F::SPR == 8) {
                const u32x2v v = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(rs, off, ssoff, 0));
                w0 = v.x;
                w1 = v.y;
            } else {
                w0 = __builtin_amdgcn_raw_buffer_load_b16(rs, off, ssoff, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < F::SPR; ++i) {
                const uint32_t o_i = (k0 + (int64_t)i * F::BLK < g.K) ? off + i : OOB;
                const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(rs, o_i, ssoff, 0);
                if (i < 4) w0 |= b << (8 * i); else w1 |= b << (8 * (i - 4));
            }
        }
        st.s[h][0] = w0;
        st.s[h][1] = w1;
    }
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
    for (int p = 0; p < GBM * 4 / F::THREADS; ++p) {
        const int idx = tid + F::THREADS * p;
        const int r = idx >> 2, c = idx & 3;
        *(uint4*)(sA + swz(r, c)) = st.a[p];
        *(uint4*)(sB + swz(r, c)) = st.b[p];
    }
    constexpr int HT = F::THREADS / 2, RPT = GBM / HT;
    const int op = tid / HT, rr = tid % HT;
    uint8_t* ss = op ? sBs : sAs;
#pragma unroll
    for (int h = 0; h < RPT; ++h) {
        const int r = rr + HT * h;
        const uint32_t w0 = st.s[h][0], w1 = st.s[h][1];
        if (FMT == 0) {
            const bool sw = ((r >> 4) & 1) != 0;
            *(uint2*)(ss + r * 8) = sw ? make_uint2(w1, w0) : make_uint2(w0, w1);
        } else {
            // MXFP8: the 4 scale bytes a lane needs for its 4 fragments (rows r, r+32, r+64,
            // r+96 of a 128-row half, one K-block) are adjacent, so one dword read fetches them
            ss[mx_sidx(r, 0)] = (uint8_t)(w0 & 0xFF);
            ss[mx_sidx(r, 1)] = (uint8_t)((w0 >> 8) & 0xFF);
        }
    }
}

// ---------------------------------------------------------------- NVFP4 fragments

// Code words of one MFMA step for the wave's 4 A and 4 B fragments: lane (row, kh) of step
// s (0..7) holds the 8 codes of K elements 64kh + 8s .. +8 of the slice, i.e. dword s%4 of
// chunk 2kh + s/4 of its row; they belong to block 4kh + s/2 of the slice.
constexpr int NVTN = Fmt<0>::TN;   // B fragments per NVFP4 wave

struct NvWords {
    uint32_t a[4], b[NVTN];
};

template <int S>
__device__ __forceinline__ void nv_read_words(const uint8_t* buf, int wm, int wn, int frow, int kh, NvWords& w) {
    const uint8_t* sA = buf;
    const uint8_t* sB = buf + GBM * ROWB;
#pragma unroll
    for (int i = 0; i < 4; ++i) w.a[i] = *(const uint32_t*)(sA + swz(wm + 32 * i + frow, 2 * kh + (S >> 2)) + 4 * (S & 3));
#pragma unroll
    for (int j = 0; j < NVTN; ++j) w.b[j] = *(const uint32_t*)(sB + swz(wn + 32 * j + frow, 2 * kh + (S >> 2)) + 4 * (S & 3));
}

__device__ __forceinline__ void nv_read_scales(const uint8_t* buf, int wm, int wn, int frow, int kh, uint32_t (&sa)[4],
                                               uint32_t (&sb)[NVTN]) {
    const uint8_t* sAs = buf + (GBM + GBN) * ROWB;
    const uint8_t* sBs = sAs + GBM * Fmt<0>::SCB;
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = *(const uint32_t*)(sAs + sswz(wm + 32 * i + frow, kh));
#pragma unroll
    for (int j = 0; j < NVTN; ++j) sb[j] = *(const uint32_t*)(sBs + sswz(wn + 32 * j + frow, kh));
}

// E2M1 x 2^8 from the hardware conversion (byte `sel` of w, two codes), times the f16 scale
// s * 2^-8; exact.
template <int SEL>
__device__ __forceinline__ half2_t nv_cvt(uint32_t w, half2_t s) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, SEL) * s;
}

__device__ __forceinline__ half8_t nv_dequant(uint32_t w, half2_t s) {
    const half2_t h0 = nv_cvt<0>(w, s), h1 = nv_cvt<1>(w, s), h2 = nv_cvt<2>(w, s), h3 = nv_cvt<3>(w, s);
    return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// f16 scale (times 2^-8) of block b (0..3) of a lane's raw scale dword w: the f16 with bit
// pattern (E4M3 byte << 7).  Bytes 0 and 2 come from (w << 7), bytes 1 and 3 from (w >> 1),
// each masked to the two f16 halves; the half is then broadcast.
__device__ __forceinline__ half2_t nv_scale(uint32_t w, int b) {
    const uint32_t t = ((b & 1) ? (w >> 1) : (w << 7)) & 0x7F807F80u;
    const half2_t p = __builtin_bit_cast(half2_t, t);
    return (b >> 1) ? half2_t{p[1], p[1]} : half2_t{p[0], p[0]};
}

// Dequantized operands of one MFMA step for the wave's 4 A and 4 B fragments.
struct NvOps {
    half8_t a[4], b[NVTN];
};

template <int S>
__device__ __forceinline__ void nv_ops(const NvWords& w, const uint32_t (&sa)[4], const uint32_t (&sb)[NVTN], NvOps& o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o.a[i] = nv_dequant(w.a[i], nv_scale(sa[i], S >> 1));
#pragma unroll
    for (int j = 0; j < NVTN; ++j) o.b[j] = nv_dequant(w.b[j], nv_scale(sb[j], S >> 1));
}

__device__ __forceinline__ void nv_mfma16(const NvOps& o, floatx16 (&acc)[4][NVTN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NVTN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.a[i], o.b[j], acc[i][j], 0, 0, 0);
}

// Scheduling hint for one pipelined step: the LDS reads of the next step's code words first,
// then 2 MFMAs alone while they land, then the remaining MFMAs each followed by an equal share
// of the next step's dequantization instructions (8 per fragment).
__device__ __forceinline__ void nv_interleave() {
    constexpr int NM = 4 * NVTN;                           // MFMAs per step
    __builtin_amdgcn_sched_group_barrier(0x100, 4 + NVTN + 4, 0);  // DS reads of the next step
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);     // MFMAs while the reads land
#pragma unroll
    for (int i = 0; i < NM - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, (8 * (4 + NVTN) + NM - 3) / (NM - 2), 0);  // VALU
    }
}

// ---------------------------------------------------------------- MXFP8 slice

constexpr int MXTN = Fmt<1>::TN;   // B fragments per MXFP8 wave

struct MxFrag {
    intx8 a[4], b[MXTN];
    uint32_t as, bs;   // byte i: scale of fragment i (K-block of the lane half)
};

// Lane (row, g) of fragment i: K elements 16g..16g+15 (chunk g) and 32+16g.. (chunk 2+g) of the
// slice, and the E8M0 byte of K-block g.
__device__ __forceinline__ void mx_read(const uint8_t* buf, int wm, int wn, int lane, MxFrag& f) {
    using F = Fmt<1>;
    const uint8_t* sA = buf;
    const uint8_t* sB = buf + GBM * ROWB;
    const uint8_t* sAs = buf + (GBM + GBN) * ROWB;
    const uint8_t* sBs = sAs + GBM * F::SCB;
    const int frow = lane & 31, kh = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm + 32 * i + frow;
        const uint4 lo = *(const uint4*)(sA + swz(r, kh));
        const uint4 hi = *(const uint4*)(sA + swz(r, 2 + kh));
        f.a[i] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    f.as = *(const uint32_t*)(sAs + mx_sidx(wm + frow, kh));
#pragma unroll
    for (int j = 0; j < MXTN; ++j) {
        const int r = wn + 32 * j + frow;
        const uint4 lo = *(const uint4*)(sB + swz(r, kh));
        const uint4 hi = *(const uint4*)(sB + swz(r, 2 + kh));
        f.b[j] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    f.bs = *(const uint32_t*)(sBs + mx_sidx(wn + frow, kh));
}

__device__ __forceinline__ void mx_mfma16(const MxFrag& f, floatx16 (&acc)[4][MXTN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < MXTN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, 0,
                                                                         (int)((f.as >> (8 * i)) & 0xFF), 0,
                                                                         (int)((f.bs >> (8 * j)) & 0xFF));
}

// Scheduling hint for one MXFP8 slice: 2 MFMAs on the current operands first (so the wait for
// them does not also wait for the new reads), then the next slice's 18 LDS reads spread
// between the remaining MFMAs.
__device__ __forceinline__ void mx_interleave() {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
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
__global__ __launch_bounds__(Fmt<FMT>::THREADS, 1) void gemm_kernel(GemmArgs g) {
    using F = Fmt<FMT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t tm, tn;
    tile_of((g.M + GBM - 1) / GBM, (g.N + GBN - 1) / GBN, tm, tn);
    const int64_t m0 = tm * GBM, n0 = tn * GBN;
    constexpr int TN = F::TN;
    const int wm = (wave / F::WAVES_N) * 128, wn = (wave % F::WAVES_N) * 32 * TN;

    floatx16 acc[4][TN];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nk = (g.K + F::BK - 1) / F::BK;
    const int frow = lane & 31, kh = lane >> 5;
    // Pipeline over K slices with NSTAGE = 3 LDS buffers.  At the top of iteration kt a
    // barrier makes slice kt+1 (stored during iteration kt-1) visible and guarantees that
    // every wave is done with slice kt-1; the staged registers of slice kt+2 then go to
    // slice kt-1's buffer and the global loads of slice kt+3 are issued, two iterations
    // ahead of their use.
    const Operands ops = make_operands<FMT>(g, m0, n0);
    Stage st;
    if (nk > 0) {
        stage_load<FMT>(g, ops, 0, st);
        stage_store<FMT>(lds, st);
        if (nk > 1) {
            stage_load<FMT>(g, ops, F::BK, st);
            stage_store<FMT>(lds + F::STAGE, st);
        }
        if (nk > 2) stage_load<FMT>(g, ops, 2 * F::BK, st);
        __syncthreads();
    }
    if constexpr (FMT == 0) {
        // NVFP4 software pipeline, one MFMA step (16 MFMAs of K = 16) at a time: while step s
        // issues its MFMAs, the code words of step s+1 are read from LDS and dequantized into
        // the next operand set.  The last step of a slice reads and dequantizes step 0 of the
        // next slice, whose buffer is complete since the barrier at the top of this slice; the
        // next slice's scale dwords are read at step 6.
        NvWords w;
        NvOps cur, nxt;
        uint32_t sa[4], sb[NVTN], san[4] = {0, 0, 0, 0}, sbn[NVTN] = {};
        auto bufp = [&](int64_t k) { return lds + (int)(k % F::NSTAGE) * F::STAGE; };
        if (nk > 0) {
            nv_read_scales(bufp(0), wm, wn, frow, kh, sa, sb);
            nv_read_words<0>(bufp(0), wm, wn, frow, kh, w);
            nv_ops<0>(w, sa, sb, cur);
        }
        for (int64_t kt = 0; kt < nk; ++kt) {
            const uint8_t* cb = bufp(kt);
            const bool more = kt + 1 < nk;
            if (kt > 0) __syncthreads();
            if (kt + 2 < nk) stage_store<FMT>(bufp(kt + 2), st);
            if (kt + 3 < nk) stage_load<FMT>(g, ops, (kt + 3) * F::BK, st);
            static_for<0, 8>([&](auto s_c) {
                constexpr int S = decltype(s_c)::value;
                if constexpr (S < 7) {
                    nv_read_words<S + 1>(cb, wm, wn, frow, kh, w);
                    if constexpr (S == 6) {
                        if (more) nv_read_scales(bufp(kt + 1), wm, wn, frow, kh, san, sbn);
                    }
                    nv_ops<S + 1>(w, sa, sb, nxt);
                } else {
                    if (more) {
                        nv_read_words<0>(bufp(kt + 1), wm, wn, frow, kh, w);
                        nv_ops<0>(w, san, sbn, nxt);
                    }
                }
                nv_mfma16(cur, acc);
                nv_interleave();
                cur = nxt;
            });
#pragma unroll
            for (int i = 0; i < 4; ++i) sa[i] = san[i];
#pragma unroll
            for (int j = 0; j < NVTN; ++j) sb[j] = sbn[j];
        }
    } else {
        // MXFP8: the fragments of slice kt+1 (visible since the barrier at the top of slice kt)
        // are read into the second register set while slice kt's 16 MFMAs issue; the loop is
        // unrolled by two so that the sets alternate without copies.
        MxFrag f0, f1;
        if (nk > 0) mx_read(lds, wm, wn, lane, f0);
        auto iter = [&](int64_t kt, const MxFrag& fc, MxFrag& fn) {
            if (kt > 0) __syncthreads();
            if (kt + 2 < nk) stage_store<FMT>(lds + (int)((kt + 2) % F::NSTAGE) * F::STAGE, st);
            if (kt + 3 < nk) stage_load<FMT>(g, ops, (kt + 3) * F::BK, st);
            // unconditional so the reads share a scheduling region with the MFMAs; after the
            // last slice they read a stale (but in-bounds) buffer whose values go unused
            mx_mfma16(fc, acc);
            mx_read(lds + (int)((kt + 1) % F::NSTAGE) * F::STAGE, wm, wn, lane, fn);
            mx_interleave();
        };
        for (int64_t kt = 0; kt < nk; kt += 2) {
            iter(kt, f0, f1);
            if (kt + 1 < nk) iter(kt + 1, f1, f0);
        }
    }

    float alpha = 1.0f;
    if (FMT == 0) alpha = (float)(1.0 / ((double)g.a_s_enc[0] * (double)g.b_s_enc[0]));
    static_for<0, 4 * TN>([&](auto t_c) {
        constexpr int i = decltype(t_c)::value / TN, j = decltype(t_c)::value % TN;
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
    hipLaunchKernelGGL((gemm_kernel<FMT, OUT>), dim3((unsigned)tiles), dim3(F::THREADS), F::LDS, s, g);
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
