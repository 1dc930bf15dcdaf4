// quantize.hip -- NVFP4 / MXFP8 quantization, NVFP4 dequantization and the standalone
// 16-point Hadamard transform for gfx950.
//
// Work decomposition (all quantize kernels).  A workgroup of 256 threads owns a tile of
// 256 rows x 128 columns of the bf16 input.  Thread t = 16*rb + cc loads the 16 x 8
// sub-tile rows [16rb, 16rb+16) x columns [8cc, 8cc+8) with sixteen 16-byte loads; one
// wave therefore reads four 256-byte row segments per load instruction (coalesced).
//   * Rowwise 16-blocks span a lane pair (cc, cc^1); their amax and the stride-8
//     Hadamard stage use one cross-lane exchange.  Rowwise 32-blocks (MXFP8) span four
//     lanes.
//   * Columnwise 16-blocks are entirely inside one thread (its 16 rows of one column);
//     columnwise 32-blocks span the lanes t and t^16.  Columnwise codes are transposed
//     through LDS so that every output row (= input column) receives a full 128-byte
//     (NVFP4) or 256-byte (MXFP8) segment from one wave.
// The NVFP4 path runs an amax pass before the encode pass, because every block scale
// depends on the per-tensor scale.  The amax pass runs at most AMAX_PARTS workgroups, each
// walking its share of the tensor; workgroup w stores its maximum to slot w of the caller's
// workspace (a plain store, one per direction it serves).  Every encode workgroup reduces the
// stored maxima itself, and workgroup 0 publishes amax and S.  Nothing accumulates from one
// call to the next: the workspace needs no initial contents, each call writes every slot it
// reads before reading it, and a replayed graph or a failed launch leaves nothing that a later
// call could read.
#include <mutex>
#include <type_traits>
#include <utility>

#include "../../include/bsq.h"
#include "device_common.hpp"
#include "launch.hpp"

namespace bsq {

constexpr int TILE_R = 256;
constexpr int TILE_C = 128;
constexpr int NTHREADS = 256;

struct TileCoord {
    int64_t r0, c0;   // origin of this thread's 16 x 8 sub-tile
    int rb, cc;       // sub-tile coordinates inside the workgroup tile
};

// The thread's sub-tile in tile (ty, tx) of the TR x TC tile grid (TC / 8 threads per row of
// sub-tiles; 256 x 128 unless a kernel says otherwise).
template <int TR = TILE_R, int TC = TILE_C>
__device__ __forceinline__ TileCoord tile_coord_at(int64_t ty, int64_t tx) {
    TileCoord t;
    t.rb = threadIdx.x / (TC / 8);
    t.cc = threadIdx.x % (TC / 8);
    t.r0 = ty * TR + 16 * t.rb;
    t.c0 = tx * TC + 8 * t.cc;
    return t;
}

// The thread's sub-tile in the workgroup's own tile (one workgroup per tile).
__device__ __forceinline__ TileCoord tile_coord() { return tile_coord_at(blockIdx.y, blockIdx.x); }

// Load the thread's 16 x 8 bf16 sub-tile; rows >= R or a column chunk >= C read as zero
// (C % 8 == 0, so a chunk is either entirely inside or entirely outside).
// The sub-tile lives in registers as q[row][word], word w holding columns 2w and 2w+1;
// every loop that indexes it is fully unrolled so that all indices are constants.
// The loads go through a buffer resource over the tile's rows that exist (rows past R read
// as zero through its range check, a column chunk past C through an offset beyond it), so a
// row costs one 32-bit offset add instead of 64-bit address arithmetic and a branch; tensors
// whose TR-row tile spans 2^31 bytes or more (C TR >= 2^30) take 64-bit addresses instead.
typedef uint32_t SubTile[16][4];

template <int TR = TILE_R>
__device__ __forceinline__ void load_subtile(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                             const TileCoord& t, SubTile q) {
    const bool colok = t.c0 < C;
    if (C * TR < ((int64_t)1 << 30)) {   // uniform
        const int64_t row0 = t.r0 - 16 * t.rb;   // the tile's first row
        const int64_t rows = (R - row0) < TR ? (R - row0) : TR;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(x + row0 * C), (short)0, (int)(rows * C * 2), 0x00020000);
        const uint32_t stride = (uint32_t)C * 2u;
        const uint32_t off0 = colok ? (uint32_t)(16 * t.rb) * stride + (uint32_t)t.c0 * 2u : 0x80000000u;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            // aux 2: non-temporal (the data is read once)
            const u32v4 v = __builtin_bit_cast(u32v4, __builtin_amdgcn_raw_buffer_load_b128(rs, off0 + j * stride, 0, 2));
            q[j][0] = v.x; q[j][1] = v.y; q[j][2] = v.z; q[j][3] = v.w;
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int64_t r = t.r0 + j;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (colok && r < R) v = load16_stream(x + r * C + t.c0);
        q[j][0] = v.x; q[j][1] = v.y; q[j][2] = v.z; q[j][3] = v.w;
    }
}

// Sign flips of the 16-point transform applied to the packed sub-tile.  Columnwise blocks run
// down the sub-tile's 16 rows, so row j takes sign d_j in both halves of each word; rowwise
// blocks run along a lane pair's 16 columns, so word w takes the signs of its two columns.
__device__ __forceinline__ uint32_t col_sign_word(uint32_t negmask, int j) {
    return ((negmask >> j) & 1u) ? 0x80008000u : 0u;
}

// Row j of the sub-tile as 8 floats.
__device__ __forceinline__ void row_of(const SubTile q, int j, float v[8]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        v[2 * w] = bf16_lo(q[j][w]);
        v[2 * w + 1] = bf16_hi(q[j][w]);
    }
}

// Column k of the sub-tile as 16 floats.
__device__ __forceinline__ void col_of(const SubTile q, int k, float v[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = (k & 1) ? bf16_hi(q[j][k >> 1]) : bf16_lo(q[j][k >> 1]);
}

__device__ __forceinline__ uint32_t sign_mask16(const int8_t* __restrict__ signs) {
    if (!signs) return 0u;
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) m |= (signs[i] < 0 ? 1u : 0u) << i;
    return m;
}

// Maximum of m over aligned groups of 2^lg lanes (1 <= lg <= 6, uniform), returned to every lane
// of the group, without LDS traffic: DPP quad moves (lane ^ 1, lane ^ 2), the half-row and row
// mirrors (which, once quads agree, pair each quad with the other quad of its 8 and each 8 with
// the other 8 of its row of 16), then v_permlane16_swap and v_permlane32_swap across rows.
// Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_max_step(float m) {
    const int b = __builtin_bit_cast(int, m);
    return __builtin_fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, 0xF, 0xF, false)));
}

__device__ __forceinline__ float group_max_dpp(float m, int lg) {
    m = dpp_max_step<0xB1>(m);                 // quad_perm [1, 0, 3, 2]
    if (lg >= 2) m = dpp_max_step<0x4E>(m);    // quad_perm [2, 3, 0, 1]
    if (lg >= 3) m = dpp_max_step<0x141>(m);   // row_half_mirror
    if (lg >= 4) m = dpp_max_step<0x140>(m);   // row_mirror
    if (lg >= 5) {
        const uint32_t b = __builtin_bit_cast(uint32_t, m);
        const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
        m = __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
    }
    if (lg >= 6) {
        const uint32_t b = __builtin_bit_cast(uint32_t, m);
        const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
        m = __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
    }
    return m;
}

// Maximum of v over the wave, returned to every lane (DPP and lane swaps: no LDS round trips).
__device__ __forceinline__ float wave_max(float v) { return group_max_dpp(v, 6); }

// ------------------------------------------------------------------ per-tensor amax

// Largest number of amax-pass workgroups; the workspace holds AMAX_PARTS partial maxima per
// direction (rowwise at [0, AMAX_PARTS), columnwise at [AMAX_PARTS, 2 AMAX_PARTS)).
constexpr int AMAX_PARTS = 1024;
static_assert(2 * AMAX_PARTS * sizeof(float) == BSQ_NVFP4_QUANTIZE_WORKSPACE_BYTES, "workspace size");

// Maximum of a workgroup (NT threads) of per-thread values a and b, returned to thread 0.
template <int NT>
__device__ __forceinline__ void block_max2(float& a, float& b) {
    __shared__ float red[2][NT / 64];
    a = wave_max(a);
    b = wave_max(b);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red[0][wave] = a;
        red[1][wave] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
#pragma unroll
        for (int w = 1; w < NT / 64; ++w) {
            a = __builtin_fmaxf(a, red[0][w]);
            b = __builtin_fmaxf(b, red[1][w]);
        }
    }
}

// Amax pass epilogue: the workgroup's maxima of the rowwise (a) and columnwise (b) values go to
// its slots of the directions in DIRS.
template <int NT, int DIRS>
__device__ __forceinline__ void store_parts(float a, float b, float* __restrict__ parts) {
    block_max2<NT>(a, b);
    if (threadIdx.x == 0) {
        if (DIRS & 1) parts[blockIdx.x] = a;
        if (DIRS & 2) parts[AMAX_PARTS + blockIdx.x] = b;
    }
}

// Encode pass prologue: the tensor amax of the directions in DIRS, reduced by the whole
// workgroup (NT threads) from the nparts partial maxima the amax pass stored, returned to
// every thread.  parts_load issues a thread's share of the loads (slots threadIdx.x + NT k)
// and returns them unreduced, so that a kernel can issue its own loads behind them before
// parts_reduce waits; parts_reduce contains barriers: every thread must call it.  The slots
// are read through buffer resources whose range ends at slot nparts: a slot past it reads as
// 0, neutral for a maximum of non-negative values, so every load is unconditional and all of
// them are in flight together (with a branch per slot each load waited for the previous one).
template <int NT>
struct PartsShare {
    uint32_t a[(AMAX_PARTS + NT - 1) / NT], b[(AMAX_PARTS + NT - 1) / NT];
};

template <int NT, int DIRS>
__device__ __forceinline__ PartsShare<NT> parts_load(const float* __restrict__ parts, int nparts) {
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)parts, (short)0, nparts * 4, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)(parts + AMAX_PARTS), (short)0, nparts * 4, 0x00020000);
    PartsShare<NT> sh;
#pragma unroll
    for (int k = 0; k < (AMAX_PARTS + NT - 1) / NT; ++k) {
        const int off = 4 * ((int)threadIdx.x + NT * k);
        sh.a[k] = (DIRS & 1) ? __builtin_amdgcn_raw_buffer_load_b32(ra, off, 0, 0) : 0u;
        sh.b[k] = (DIRS & 2) ? __builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0) : 0u;
    }
    return sh;
}

template <int NT, int DIRS>
__device__ __forceinline__ float2 parts_reduce(const PartsShare<NT>& sh) {
    __shared__ float red[2][NT / 64];
    float a = 0.0f, b = 0.0f;
#pragma unroll
    for (int k = 0; k < (AMAX_PARTS + NT - 1) / NT; ++k) {
        a = __builtin_fmaxf(a, __builtin_bit_cast(float, sh.a[k]));
        b = __builtin_fmaxf(b, __builtin_bit_cast(float, sh.b[k]));
    }
    a = wave_max(a);
    b = wave_max(b);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red[0][wave] = a;
        red[1][wave] = b;
    }
    __syncthreads();
    a = red[0][0];
    b = red[1][0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
        a = __builtin_fmaxf(a, red[0][w]);
        b = __builtin_fmaxf(b, red[1][w]);
    }
    return make_float2(a, b);
}

// max(m, m of lane ^ 1), the other half of a 16-block, by a DPP quad move (a lane whose
// partner is inactive keeps its own m).
__device__ __forceinline__ float pair_max(float m) {
    const int b = __builtin_bit_cast(int, m);
    return __builtin_fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false)));
}

// Workgroup 0 of an encode pass publishes amax and S of the directions in DIRS.
template <int DIRS>
__device__ __forceinline__ void publish_scales(float2 am, float* amax_out, float* s_enc_out) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        if (DIRS & 1) {
            amax_out[0] = am.x;
            s_enc_out[0] = nvfp4_tensor_scale(am.x);
        }
        if (DIRS & 2) {
            amax_out[1] = am.y;
            s_enc_out[1] = nvfp4_tensor_scale(am.y);
        }
    }
}

// Amax of the transformed values per direction (DIRS: bit 0 rowwise, bit 1 columnwise; with
// RHT each direction takes the amax of its own transformed values), over 256 x 128 tiles: a
// grid of at most AMAX_PARTS workgroups, workgroup w taking tiles w, w + grid, ...  The
// butterfly's outputs h are four times the transform's values, exactly, so the maxima of |h|
// are taken and quartered once at the end.
// ROWPLAIN (DIRS 3): the rowwise maximum over the untransformed values (a rowwise direction
// cast without the transform, beside a transformed columnwise one).
template <int DIRS, bool ROWPLAIN = false>
__global__ __launch_bounds__(NTHREADS) void nvfp4_amax_rht_kernel(const uint16_t* __restrict__ x, int64_t R,
                                                                  int64_t C, const int8_t* __restrict__ signs,
                                                                  float* __restrict__ parts) {
    const int64_t ntc = (C + TILE_C - 1) / TILE_C, nt = ntc * ((R + TILE_R - 1) / TILE_R);
    const uint32_t neg = sign_mask16(signs);
    const bool upper = (threadIdx.x & 1) != 0;   // the lane's half of its rowwise blocks (cc & 1)
    float mrow = 0.0f, mcol = 0.0f;
    for (int64_t tix = blockIdx.x; tix < nt; tix += gridDim.x) {
        const TileCoord t = tile_coord_at(tix / ntc, tix % ntc);
        SubTile q;
        load_subtile(x, R, C, t, q);
        if (DIRS & 1) {
            static_for<0, 16>([&](auto j_c) {
                constexpr int j = decltype(j_c)::value;
                float v[8];
                if constexpr (ROWPLAIN) {
                    row_of(q, j, v);
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t word = q[j][w] ^ row_sign_word(neg, upper, w);
                        v[2 * w] = bf16_lo(word);
                        v[2 * w + 1] = bf16_hi(word);
                    }
                    rht16_pair_core(v, upper);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) mrow = __builtin_fmaxf(mrow, __builtin_fabsf(v[k]));
            });
        }
        if (DIRS & 2) {
            static_for<0, 8>([&](auto k_c) {
                constexpr int k = decltype(k_c)::value;
                float v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t word = q[j][k >> 1] ^ col_sign_word(neg, j);
                    v[j] = (k & 1) ? bf16_hi(word) : bf16_lo(word);
                }
                rht16_core(v);
#pragma unroll
                for (int j = 0; j < 16; ++j) mcol = __builtin_fmaxf(mcol, __builtin_fabsf(v[j]));
            });
        }
    }
    store_parts<NTHREADS, DIRS>(ROWPLAIN ? mrow : mrow * 0.25f, mcol * 0.25f, parts);
}

// ------------------------------------------------------------------ NVFP4 encode

// Scale byte of a 32-block with amax m: X = floor(log2 m) - 8 clamped at -127, byte X+127;
// for a normal binary32 m that is max(exponent_field - 8, 0), and 0 for subnormal or zero m.
__device__ __forceinline__ uint32_t mx_scale_byte(float m) {
    const int e = (int)(__float_as_uint(m) >> 23);
    return (uint32_t)(e > 8 ? e - 8 : 0);
}

// 2^-X for scale byte b (X = b - 127): binary32 with exponent field 254 - b (b <= 246).
__device__ __forceinline__ float mx_inv_scale(uint32_t b) { return __uint_as_float((254u - b) << 23); }

// Two 16-bit lanes of a 32-bit word, unsigned or signed: packed minima and maxima
// (v_pk_max_u16, v_pk_min_u16, v_pk_min_i16).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}
__device__ __forceinline__ uint32_t pk_min_i16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(i16x2_t, a), __builtin_bit_cast(i16x2_t, b)));
}

// Four E4M3 codes (bytes 0..3: a.lo, a.hi, b.lo, b.hi) of bf16 pairs a and b divided by the
// binary32 power of two s, rounded to nearest even (v_cvt_scalef32_pk_fp8_bf16: exact for a
// normal s and quotients below 464 in magnitude; larger ones give the NaN code, so callers clamp).
__device__ __forceinline__ uint32_t fp8x4_scaled(uint32_t a, uint32_t b, float s) {
    typedef short s16x2_t __attribute__((ext_vector_type(2)));
    // the first conversion replaces the low word of a's own register; the second the high one
    s16x2_t o = __builtin_bit_cast(s16x2_t, a);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, __builtin_bit_cast(bf16x2_t, a), s, false);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(o, __builtin_bit_cast(bf16x2_t, b), s, true);
    return __builtin_bit_cast(uint32_t, o);
}

// Packed MXFP8 rowwise encode of an 8-element unit w[0..3] (bf16 pairs of one row) whose 32-block
// spans the 4 lanes of an aligned quad: the same codes and scale byte as the binary32 form.  The
// block amax is a 16-bit unsigned maximum over magnitude bits (within the unit, across its two
// halves, then across the quad by DPP); the clamp to 448 * 2^X and the scaled conversion are the
// columnwise encoder's.  Returns false, for every lane of the wave, when some block of the wave
// has scale byte 0 (amax exponent field <= 8, all-zero blocks included): the caller then takes the
// binary32 form.  The lanes of a quad are all active or all inactive (an inactive lane adds
// nothing: DPP reads from it return 0 and the ballot skips it).
__device__ __forceinline__ bool mx_row_unit_packed(const uint32_t w[4], uint32_t& lo, uint32_t& hi, uint32_t& sb) {
    uint32_t M = pk_max_u16(pk_max_u16(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu),
                            pk_max_u16(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu));
    M = pk_max_u16(M, __builtin_amdgcn_alignbit(M, M, 16));   // both halves: the unit's amax
    M = pk_max_u16(M, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)M, 0xB1, 0xF, 0xF, false));   // lane ^ 1
    M = pk_max_u16(M, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)M, 0x4E, 0xF, 0xF, false));   // lane ^ 2
    if (__builtin_amdgcn_ballot_w64((M & 0xFFFFu) < 0x480u) != 0) return false;   // wave-uniform
    const uint32_t T = (M & 0x7F807F80u) | 0x00600060u, T2 = T | 0x80008000u;
    sb = ((M >> 7) & 0xFFu) - 8u;
    const float s = __uint_as_float(sb << 23);
    uint32_t z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = pk_min_u16(pk_min_i16(w[i], T), T2);
    lo = fp8x4_scaled(z[0], z[1], s);
    hi = fp8x4_scaled(z[2], z[3], s);
    return true;
}

// Byte offset of code (r, k) of a [rows][K] code matrix in the slab layout: rows in bands of
// 256 (the last band holds the rest), band b at byte 256 b K, holding its n rows as K/64
// consecutive slabs of n x 64 bytes (K a multiple of 64).  A GEMM tile's rows are one band,
// and each 64-element K slice of them one contiguous block.
__device__ __forceinline__ int64_t slab_offset(int64_t r, int64_t k, int64_t rows, int64_t K) {
    const int64_t b = r >> 8, left = rows - (b << 8), n = left < 256 ? left : 256;
    return (b << 8) * K + (k >> 6) * n * 64 + (r & 255) * 64 + (k & 63);
}

// MXFP8 rowwise cast of a thread's 16 x 8 sub-tile of a TR-row tile: 32-blocks along the row
// span the 4 lanes cc .. cc+3; codes (8 bytes per row) go to the row-major or slab-layout code
// matrix and each block's scale byte to its row of the scale matrix.  The tile's rows of either
// matrix are one contiguous range (slab bands are 256 rows and tiles start on a band), so the
// stores go through buffer resources over it: a thread steps a 32-bit offset by the row pitch,
// and rows past R fall outside the range and are dropped -- except slab rows in a partial last
// band, whose offsets would land in the band's next slab and are dropped explicitly.  Tensors
// whose tile spans 2^31 bytes or more (C TR >= 2^31) take 64-bit addresses instead.
template <int TR>
__device__ __forceinline__ void mx_row_tile(const SubTile& q, const TileCoord& t, int64_t R, int64_t C,
                                            uint8_t* row_codes, uint8_t* row_scales, int slab) {
    const bool colok = t.c0 < C;
    auto encode_row = [&](int j, uint32_t& lo, uint32_t& hi, uint32_t& sb) {
        if (mx_row_unit_packed(q[j], lo, hi, sb)) return;
        float v[8];
        row_of(q, j, v);
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(v[k]));
        m = __builtin_fmaxf(m, __shfl_xor(m, 1));
        m = __builtin_fmaxf(m, __shfl_xor(m, 2));
        lo = hi = sb = 0;
        if (m != 0.0f) {
            sb = mx_scale_byte(m);
            const float inv = mx_inv_scale(sb);
            lo = e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
            hi = e4m3_pack4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
        }
    };
    // the sub-tile's 16 rows lie in one 256-row band (r0 is a multiple of 16), so in either
    // layout row r0 + j's codes sit j row pitches (64 bytes in a slab, C row-major) after row r0's
    const int64_t code_at = slab ? slab_offset(t.r0, t.c0, R, C) : t.r0 * C + t.c0;
    if (C * TR < ((int64_t)1 << 31)) {   // uniform
        typedef unsigned int u32v2_t __attribute__((ext_vector_type(2)));
        const int64_t row0 = t.r0 - 16 * t.rb;   // the tile's first row
        const int64_t rows = (R - row0) < TR ? (R - row0) : TR;
        const __amdgpu_buffer_rsrc_t rc =
            __builtin_amdgcn_make_buffer_rsrc((void*)(row_codes + row0 * C), (short)0, (int)(rows * C), 0x00020000);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(row_scales + row0 * (C / 32)), (short)0, (int)(rows * (C / 32)), 0x00020000);
        const uint32_t oc = colok ? (uint32_t)(code_at - row0 * C) : 0x80000000u;
        const uint32_t os = (colok && (t.cc & 3) == 0) ? (uint32_t)((t.r0 - row0) * (C / 32) + t.c0 / 32) : 0x80000000u;
        const uint32_t pc = slab ? 64u : (uint32_t)C, ps = (uint32_t)(C / 32);
        const bool cut = slab && rows < TR;   // uniform
        static_for<0, 16>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            uint32_t lo, hi, sb;
            encode_row(j, lo, hi, sb);
            uint32_t ocj = oc + (uint32_t)j * pc;
            if (cut && t.r0 + j >= R) ocj = 0x80000000u;
            __builtin_amdgcn_raw_buffer_store_b64(u32v2_t{lo, hi}, rc, (int)ocj, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((unsigned char)sb, rs, (int)(os + (uint32_t)j * ps), 0, 0);
        });
        return;
    }
    uint8_t* code0 = row_codes + code_at;
    const int64_t pitch = slab ? 64 : C;
    uint8_t* scale0 = row_scales + t.r0 * (C / 32) + t.c0 / 32;
    static_for<0, 16>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        const int64_t r = t.r0 + j;
        uint32_t lo, hi, sb;
        encode_row(j, lo, hi, sb);
        if (colok && r < R) {
            *(uint2*)(code0 + j * pitch) = make_uint2(lo, hi);
            if ((t.cc & 3) == 0) scale0[j * (C / 32)] = (uint8_t)sb;
        }
    });
}

struct NvEncodeArgs {
    const uint16_t* x;
    int64_t R, C;
    const int8_t* signs;
    uint8_t* row_codes;
    uint8_t* row_scales;
    uint8_t* col_codes;
    uint8_t* col_scales;
    const float* parts;  // the amax pass's partial maxima (AMAX_PARTS per direction)
    int nparts;          // how many the amax pass stored per direction
    float* amax_out;
    float* s_enc_out;
    uint64_t seed;
    uint32_t stream;
    uint8_t* mx_codes;    // MXFP8 rowwise output of the same input (hybrid calls; else unused)
    uint8_t* mx_scales;
    int mx_slab;
};

// The encode multiplier S / fp32(s_b) of every nonzero scale code s_b (codes 1..126) for tensor
// scale S, built by the workgroup in LDS (threads [base, base + 128) of it), so that a block
// reads its multiplier instead of dividing.  The caller synchronises before use.
__device__ __forceinline__ void build_enc_table(float S, float* tab, int base) {
    const int c = (int)threadIdx.x - base;
    if (c >= 0 && c < 128) tab[c] = (c >= 1 && c <= 126) ? S / e4m3_decode_nonneg((uint32_t)c) : 0.0f;
}

// Encode one 16-block's worth of values held by this thread (N = 8 or 16 values) whose
// largest magnitude vmax (over the block) is known.  Writes the packed codes (N/2 bytes as
// N/8 words) into w[] and returns the scale code.  first_index: output-layout index of v[0];
// consecutive values are consecutive indices.  enc_tab: the workgroup's multiplier table for
// S, or null (then the multiplier is divided out here).  QUARTER: v holds the butterfly's
// outputs h, four times the transform's values (exactly); the block is then encoded from
// h * fl(enc / 4), which equals fl((h / 4) * enc) whenever enc / 4 is exact (one rounding of
// the same product), and otherwise from (h / 4) * enc.
template <int N, bool SR, bool QUARTER>
__device__ __forceinline__ uint32_t encode_block(float* v, float vmax, float S, const float* enc_tab,
                                                 uint64_t first_index, uint64_t seed, uint32_t stream, uint32_t dir,
                                                 uint32_t* w) {
    const uint32_t sb = block_scale_code(QUARTER ? vmax * 0.25f : vmax, S);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) w[i] = 0u;
    if (sb != 0u) {
        float enc = enc_tab ? enc_tab[sb] : S / e4m3_decode_nonneg(sb);
        if (QUARTER) {
            const float e4 = enc * 0.25f;
            if (e4 * 4.0f == enc) {
                enc = e4;
            } else {
#pragma unroll
                for (int j = 0; j < N; ++j) v[j] *= 0.25f;
            }
        }
        if (SR) {
#pragma unroll
            for (int g = 0; g < N / 4; ++g) {
                const u32x4 rw = sr_words((first_index >> 2) + g, seed, stream, dir);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 4 * g + e;
                    const uint32_t c = e2m1_encode_sr(v[j] * enc, word_of(rw, e));
                    w[j >> 3] |= c << (4 * (j & 7));
                }
            }
        } else {
            static_for<0, N / 8>([&](auto g_c) {
                constexpr int g = decltype(g_c)::value;
                uint32_t x = 0;
                x = e2m1_pack2_rne<0>(x, v[8 * g + 0] * enc, v[8 * g + 1] * enc);
                x = e2m1_pack2_rne<1>(x, v[8 * g + 2] * enc, v[8 * g + 3] * enc);
                x = e2m1_pack2_rne<2>(x, v[8 * g + 4] * enc, v[8 * g + 5] * enc);
                x = e2m1_pack2_rne<3>(x, v[8 * g + 6] * enc, v[8 * g + 7] * enc);
                w[g] = x;
            });
        }
    }
    return sb;
}

// The columnwise scales of a TR x TC tile: column col's BN = TR / BLK scale bytes sit in LDS at
// sc[col][b ^ x(col)] (the placement the encode writes them in: x = (col >> 3) mod BN) and
// are contiguous in the output row of column tc0 + col.  One thread per column gathers them
// and, where the tile's rows are all inside R and the output row's bytes are aligned for it,
// writes them with one BN-byte store (16 for NVFP4 and the 512-row MXFP8 tile, 8 for the
// 256-row MXFP8 tile) instead of BN byte stores spread over the workgroup.
template <int BLK, int TR = TILE_R, int TC = TILE_C>
__device__ __forceinline__ void store_col_scales(const uint8_t* sc, uint8_t* out, int64_t R, int64_t C, int64_t tr0,
                                                 int64_t tc0) {
    constexpr int BN = TR / BLK;
    const int col = threadIdx.x;
    if (col >= TC) return;
    const int64_t c = tc0 + col;
    if (c >= C) return;
    const int x = (col >> 3) & (BN - 1);
    uint8_t* dst = out + c * (R / BLK) + tr0 / BLK;
    if (tr0 + TR <= R && ((uintptr_t)dst % BN) == 0) {
        uint32_t w[BN / 4];
#pragma unroll
        for (int i = 0; i < BN / 4; ++i) {
            uint32_t v = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) v |= (uint32_t)sc[col * BN + ((4 * i + k) ^ x)] << (8 * k);
            w[i] = v;
        }
        if constexpr (BN == 16) *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
        else *(uint2*)dst = make_uint2(w[0], w[1]);
    } else {
        for (int b = 0; b < BN && tr0 + (int64_t)b * BLK < R; ++b) dst[b] = sc[col * BN + (b ^ x)];
    }
}

// MXROW: also the MXFP8 rowwise cast of the same tile (from the untransformed values), so that
// the per-direction recipe's backward operand (MXFP8 rowwise, NVFP4 columnwise) reads its
// input once.  ROWPLAIN (DIRS 3): the rowwise direction without the transform and with RNE
// (the forward operand), the columnwise one with RHT and SR as given (the wgrad operand).
template <int DIRS, bool RHT, bool SR, bool MXROW = false, bool ROWPLAIN = false>
__global__ __launch_bounds__(NTHREADS) void nvfp4_encode_kernel(NvEncodeArgs a) {
    constexpr bool RHT_ROW = RHT && !ROWPLAIN, SR_ROW = SR && !ROWPLAIN;
    const TileCoord t = tile_coord();
    const int64_t R = a.R, C = a.C;
    // the tile's loads, then the partial maxima's, all in flight together before the first wait
    SubTile q;
    load_subtile(a.x, R, C, t, q);
    const PartsShare<NTHREADS> parts = parts_load<NTHREADS, DIRS>(a.parts, a.nparts);
    if constexpr (MXROW) mx_row_tile<TILE_R>(q, t, R, C, a.mx_codes, a.mx_scales, a.mx_slab);
    const uint32_t neg = RHT ? sign_mask16(a.signs) : 0u;
    const float2 am = parts_reduce<NTHREADS, DIRS>(parts);
    const float Srow = nvfp4_tensor_scale(am.x);
    const float Scol = nvfp4_tensor_scale(am.y);
    publish_scales<DIRS>(am, a.amax_out, a.s_enc_out);
    __shared__ float enc_tab[2][128];
    if (DIRS & 1) build_enc_table(Srow, enc_tab[0], 0);
    if (DIRS & 2) build_enc_table(Scol, enc_tab[1], DIRS == 3 ? 128 : 0);
    __syncthreads();
    const bool colok = t.c0 < C;

    if (DIRS & 1) {
        const bool upper = (t.cc & 1) != 0;
        // row r0 + j's code word and scale byte, j row pitches after row r0's.  Where the tile's
        // rows of codes span less than 2^31 bytes they are stored through buffer resources over
        // those rows: a 32-bit offset per row, rows past R dropped by the range check.
        uint8_t* code0 = a.row_codes + t.r0 * (C / 2) + t.c0 / 2;
        uint8_t* scale0 = a.row_scales + t.r0 * (C / 16) + t.c0 / 16;
        const bool rsrc_ok = C * TILE_R < ((int64_t)1 << 32);   // uniform
        const int64_t row0 = t.r0 - 16 * t.rb;                  // the tile's first row
        const int64_t rows = (R - row0) < TILE_R ? (R - row0) : TILE_R;
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.row_codes + row0 * (C / 2)), (short)0, rsrc_ok ? (int)(rows * (C / 2)) : 0, 0x00020000);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.row_scales + row0 * (C / 16)), (short)0, rsrc_ok ? (int)(rows * (C / 16)) : 0, 0x00020000);
        const uint32_t oc = colok ? (uint32_t)(16 * t.rb * (C / 2) + t.c0 / 2) : 0x80000000u;
        const uint32_t os = (colok && !upper) ? (uint32_t)(16 * t.rb * (C / 16) + t.c0 / 16) : 0x80000000u;
        static_for<0, 16>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            const int64_t r = t.r0 + j;
            float v[8];
            if (RHT_ROW) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t word = q[j][w] ^ row_sign_word(neg, upper, w);
                    v[2 * w] = bf16_lo(word);
                    v[2 * w + 1] = bf16_hi(word);
                }
                rht16_pair_core(v, upper);
            } else {
                row_of(q, j, v);
            }
            float m = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(v[k]));
            m = pair_max(m);
            uint32_t w;
            const uint32_t sb = encode_block<8, SR_ROW, RHT_ROW>(v, m, Srow, enc_tab[0],
                                                         (uint64_t)r * (uint64_t)C + (uint64_t)t.c0, a.seed, a.stream,
                                                         0u, &w);
            if (rsrc_ok) {
                __builtin_amdgcn_raw_buffer_store_b32(w, rc, (int)(oc + (uint32_t)j * (uint32_t)(C / 2)), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)sb, rs, (int)(os + (uint32_t)j * (uint32_t)(C / 16)), 0, 0);
            } else if (colok && r < R) {
                *(uint32_t*)(code0 + j * (C / 2)) = w;
                if (!upper) scale0[j * (C / 16)] = (uint8_t)sb;
            }
        });
    }

    if (DIRS & 2) {
        // codes of column (8cc + k), row block rb -> lds_codes[8cc + k][rb ^ cc]: the XOR spreads
        // the 16 column groups of a wave's writes over all banks (a column's 16 blocks stay in
        // its own 128-byte row, so the read-back of a column is still one contiguous row)
        __shared__ uint2 lds_codes[TILE_C][TILE_R / 16];
        __shared__ uint8_t lds_sc[TILE_C][TILE_R / 16];
        if (RHT) {
            // column blocks run down the rows: flip row j's sign once for both columns of a word
#pragma unroll
            for (int j = 0; j < 16; ++j)
#pragma unroll
                for (int w = 0; w < 4; ++w) q[j][w] ^= col_sign_word(neg, j);
        }
        static_for<0, 8>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            float v[16];
            col_of(q, k, v);
            if (RHT) rht16_core(v);
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
            uint32_t w[2];
            const uint64_t c = (uint64_t)(t.c0 + k);
            const uint32_t sb = encode_block<16, SR, RHT>(v, m, Scol, enc_tab[1],
                                                          c * (uint64_t)R + (uint64_t)t.r0, a.seed, a.stream, 1u, w);
            lds_codes[8 * t.cc + k][t.rb ^ t.cc] = make_uint2(w[0], w[1]);
            lds_sc[8 * t.cc + k][t.rb ^ t.cc] = (uint8_t)sb;
        });
        __syncthreads();
        const int64_t tr0 = (int64_t)blockIdx.y * TILE_R;
        const int64_t tc0 = (int64_t)blockIdx.x * TILE_C;
        if (R * TILE_C < ((int64_t)1 << 32)) {   // uniform
            // the tile's output rows tc0 .. tc0 + 127 of the codes [C][R/2] through a buffer
            // resource over them: a thread's 8 pieces lie 16 output rows apart (one 32-bit add
            // each), output rows past C fall outside the range, and a thread whose input rows
            // lie past R (the same for all 8) stores nothing
            const int64_t ncols = (C - tc0) < TILE_C ? (C - tc0) : TILE_C;
            const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(a.col_codes + tc0 * (R / 2)), (short)0, (int)(ncols * (R / 2)), 0x00020000);
            const int col0 = threadIdx.x >> 4, rbk = threadIdx.x & 15;
            const int64_t r = tr0 + 16 * rbk;
            const uint32_t off0 = r < R ? (uint32_t)(col0 * (R / 2) + r / 2) : 0x80000000u;
            const uint32_t step = (uint32_t)(16 * (R / 2));
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int col = col0 + 16 * p;
                const uint2 v = lds_codes[col][rbk ^ (col >> 3)];
                typedef unsigned int u32v2_t __attribute__((ext_vector_type(2)));
                __builtin_amdgcn_raw_buffer_store_b64(u32v2_t{v.x, v.y}, rc, (int)(off0 + (uint32_t)p * step), 0, 0);
            }
        } else {
#pragma unroll
            for (int p = 0; p < (TILE_C * TILE_R / 16) / NTHREADS; ++p) {
                const int idx = threadIdx.x + NTHREADS * p;
                const int col = idx >> 4, rbk = idx & 15;
                const int64_t c = tc0 + col, r = tr0 + 16 * rbk;
                if (c < C && r < R) *(uint2*)(a.col_codes + c * (R / 2) + r / 2) = lds_codes[col][rbk ^ (col >> 3)];
            }
        }
        store_col_scales<16>(&lds_sc[0][0], a.col_scales, R, C, tr0, tc0);
    }
}

// ------------------------------------------------------------------ MXFP8 cast


// bf16 bits of the dequantized NVFP4 element with code c (4 bits) in a block with scale value
// sc: bf16_RNE((E2M1(c) * sc) / S).  The product is exact; one rounded division, then RNE.
__device__ __forceinline__ uint32_t nvfp4_dequant_bf16(uint32_t c, float sc, float S) {
    const uint32_t m = c & 7u;
    const float mag = m <= 4u ? 0.5f * (float)m : (m == 5u ? 3.0f : (m == 6u ? 4.0f : 6.0f));
    const float e = (c & 8u) ? -mag : mag;
    return f32_to_bf16_rne((e * sc) / S);
}

// Sub-tile of the bf16 tensor bf16(dequant(NVFP4 rowwise)) -- the same values the dequantize
// kernel writes -- computed from the codes and scales: row j of the thread's 16 x 8 sub-tile
// is code word c0/8 of the row and scale byte c0/16.
//
// The seven nonzero E2M1 magnitudes are 0.5 * 2^k (k = 0..3) and 1.5 * 2^k (k = 0..2), so per
// row two quotients suffice: with qa = fl32(0.5 sc / S) and qb = fl32(1.5 sc / S) both normal
// and far enough from overflow (exponent field 1..250), fl32(2^k x) = 2^k fl32(x) and
// bf16(2^k q) = 2^k bf16(q), so the bf16 result of magnitude m is bf16(qa or qb) with k added
// to its exponent field -- bit-identical to rounding each product separately.  Rows outside
// that range (zero or tiny scales, extreme tensor scales) take the per-element path.
__device__ __forceinline__ void load_subtile_nvfp4(const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales, float S, int64_t R,
                                                   int64_t C, const TileCoord& t, SubTile q) {
    const bool colok = t.c0 < C;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int64_t r = t.r0 + j;
        uint32_t cw = 0u, sbyte = 0u;
        if (colok && r < R) {
            cw = *(const uint32_t*)(codes + r * (C / 2) + t.c0 / 2);
            sbyte = scales[r * (C / 16) + t.c0 / 16];
        }
        const float sc = e4m3_decode_nonneg(sbyte & 0x7Fu);
        const float qa = (0.5f * sc) / S, qb = (1.5f * sc) / S;
        const uint32_t ea = __float_as_uint(qa) >> 23, eb = __float_as_uint(qb) >> 23;
        if (ea - 1u < 250u && eb - 1u < 250u) {
            const uint32_t ba = f32_to_bf16_rne(qa), bb = f32_to_bf16_rne(qb);
            auto deq = [&](uint32_t c) {
                const uint32_t m = c & 7u;
                const uint32_t k = (0x23120100u >> (4u * m)) & 0xFu;       // exponent step of magnitude m
                const uint32_t base = ((0xA8u >> m) & 1u) ? bb : ba;       // m = 3, 5, 7: the 1.5 family
                const uint32_t mag = m ? base + (k << 7) : 0u;
                return mag | ((c & 8u) << 12);
            };
#pragma unroll
            for (int w = 0; w < 4; ++w) q[j][w] = deq((cw >> (8 * w)) & 0xFu) | (deq((cw >> (8 * w + 4)) & 0xFu) << 16);
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t lo = nvfp4_dequant_bf16((cw >> (8 * w)) & 0xFu, sc, S);
                const uint32_t hi = nvfp4_dequant_bf16((cw >> (8 * w + 4)) & 0xFu, sc, S);
                q[j][w] = lo | (hi << 16);
            }
        }
    }
}

// The workgroup's 256 x 128 tile of an NVFP4 rowwise tensor staged in LDS: codes (64 bytes a
// row; row r at LDS row r ^ ((r >> 4) & 3), so that the four rows a wave reads together, 16
// apart, fall on different banks), scale bytes (8 a row), and for every scale byte s the bf16
// bits of the eight non-negative codes' dequantized values, nvfp4_dequant_bf16(m, fp32(s), S)
// for m = 0..7, as byte tables (lut[s] = low bytes of m = 0..3, of m = 4..7, high bytes of
// m = 0..3, of m = 4..7), built once per workgroup.  A negative code's value is the same bits
// with the sign set (the rounding is symmetric; code 8 gives -0).
struct NvTileLds {
    uint4 codes[TILE_R][4];
    uint2 scales[TILE_R];
    uint4 lut[128];   // scale byte s (bit 7 ignored)
};

// Stage the tile (tr0, tc0) of codes [R][C/2] and scales [R][C/16] (C % 32 == 0, so each
// 16-byte code chunk lies inside or outside the tensor and rows are 16-byte aligned); rows and
// chunks outside read as zero.  Ends with a barrier.
__device__ __forceinline__ void stage_nvfp4_tile(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales, float S, int64_t R,
                                                 int64_t C, int64_t tr0, int64_t tc0, NvTileLds& L) {
    const int tid = threadIdx.x;
    // every load of the tile first (four 16-byte code chunks and a row of scale bytes per
    // thread), so that their latencies overlap; the lookup table is computed while the code
    // chunks are in flight, and the LDS stores come last
    uint4 v[4];
    if (C < ((int64_t)1 << 24)) {   // uniform: the tile's rows of codes span less than 2^31 bytes
        // through a buffer resource over those rows, with no branch: rows past R lie past its
        // range and a chunk past C gets an offset beyond it, and both read as zero
        const int64_t rows = (R - tr0) < TILE_R ? (R - tr0) : TILE_R;
        const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(codes + tr0 * (C / 2)), (short)0, (int)(rows * (C / 2)), 0x00020000);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int id = tid + NTHREADS * p, row = id >> 2, part = id & 3;
            const uint32_t off = tc0 + 32 * part + 32 <= C ? (uint32_t)(row * (C / 2) + tc0 / 2 + 16 * part)
                                                           : 0x80000000u;
            v[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, (int)off, 0, 0));
        }
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int id = tid + NTHREADS * p, row = id >> 2, part = id & 3;
            const int64_t r = tr0 + row;
            v[p] = make_uint4(0u, 0u, 0u, 0u);
            if (r < R && tc0 + 32 * part + 32 <= C) v[p] = *(const uint4*)(codes + r * (C / 2) + tc0 / 2 + 16 * part);
        }
    }
    // thread (s, half): codes 4 half .. 4 half + 3 of scale byte s
    static_assert(NTHREADS == 256, "two threads per scale byte");
    const int sbyte = tid >> 1, half = tid & 1;
    uint32_t llo = 0u, lhi = 0u;
    {
        const float sc = e4m3_decode_nonneg((uint32_t)sbyte);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t x = nvfp4_dequant_bf16((uint32_t)(4 * half + i), sc, S);
            llo |= (x & 0xFFu) << (8 * i);
            lhi |= (x >> 8) << (8 * i);
        }
    }
    uint32_t slo = 0u, shi = 0u;
    {
        const int64_t r = tr0 + tid;
        if (r < R) {
            const uint8_t* src = scales + r * (C / 16) + tc0 / 16;
            const int64_t nb = (C - tc0) / 16;   // scale bytes of the row inside the tile
            if (nb >= 8 && ((uintptr_t)src & 7u) == 0) {
                const uint2 w = *(const uint2*)src;
                slo = w.x;
                shi = w.y;
            } else {
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const uint32_t x = b < nb ? (uint32_t)src[b] : 0u;
                    if (b < 4) slo |= x << (8 * b); else shi |= x << (8 * (b - 4));
                }
            }
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int id = tid + NTHREADS * p, row = id >> 2, part = id & 3;
        L.codes[row ^ ((row >> 4) & 3)][part] = v[p];
    }
    L.scales[tid] = make_uint2(slo, shi);
    uint32_t* w = (uint32_t*)&L.lut[sbyte];
    w[half] = llo;
    w[2 + half] = lhi;
    __syncthreads();
}

// load_subtile_nvfp4 from the staged tile: the same values, bit for bit.  Per row, the code word
// is split into its even and odd codes; per bf16 pair, v_perm_b32 gathers the pair's codes into
// the two halves, two more look up the low and high bytes of their magnitudes in the row's
// scale table, a fourth interleaves them, and the code's sign bit is moved to bit 15.
__device__ __forceinline__ void load_subtile_nvfp4_lds(const NvTileLds& L, const TileCoord& t, SubTile q) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int lr = 16 * t.rb + j;
        const uint32_t cw = ((const uint32_t*)&L.codes[lr ^ ((lr >> 4) & 3)][0])[t.cc];
        const uint32_t sbyte = (((t.cc >> 1) < 4 ? L.scales[lr].x : L.scales[lr].y) >> (8 * ((t.cc >> 1) & 3))) & 0x7Fu;
        const uint4 T = L.lut[sbyte];
        const uint32_t even = cw & 0x0F0F0F0Fu, odd = (cw >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            // halves: code 2w (byte w of even), code 2w + 1 (byte w of odd); selector 12 gives 0
            const uint32_t c = __builtin_amdgcn_perm(odd, even, 0x0C000C00u | ((4u + w) << 16) | (uint32_t)w);
            const uint32_t sel = c & 0x00070007u;
            const uint32_t lo = __builtin_amdgcn_perm(T.y, T.x, sel), hi = __builtin_amdgcn_perm(T.w, T.z, sel);
            q[j][w] = __builtin_amdgcn_perm(hi, lo, 0x06020400u) | ((c << 12) & 0x80008000u);
        }
    }
}

struct MxArgs {
    const uint16_t* x;         // bf16 source, or
    const uint8_t* nv_codes;   // NVFP4 rowwise source (codes, scales, tensor scale)
    const uint8_t* nv_scales;
    const float* nv_s_enc;
    int64_t R, C;
    uint8_t* row_codes;
    uint8_t* row_scales;
    uint8_t* col_codes;
    uint8_t* col_scales;
    int slab;   // codes in the slab layout (see slab_offset)
};


// Tile of workgroup id among G tiles in an XCD-aware order: workgroups are dispatched to the
// chip's 8 XCDs in turn (id mod 8), so XCD x is given the x-th contiguous run of tiles in row-major
// tile order and streams one band of the tensor through its own L2 instead of every eighth tile.
__device__ __forceinline__ int64_t xcd_tile(int64_t id, int64_t G) {
    const int64_t q = G / 8, rmd = G % 8, x = id % 8;
    return x * q + (x < rmd ? x : rmd) + id / 8;
}

// Maximum of the packed 16-bit lanes of m and of lane t ^ CCS's m (the other half of a 32-row
// block, CCS = 16 or 32 sub-tiles per tile row): v_permlane16_swap / v_permlane32_swap leave a
// lane's own value and its partner's in the two results.
template <int CCS>
__device__ __forceinline__ uint32_t pk_max_u16_block_pair(uint32_t m) {
    static_assert(CCS == 16 || CCS == 32, "partner lane within the wave");
    if constexpr (CCS == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(m, m, false, false);
        return pk_max_u16(r[0], r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(m, m, false, false);
        return pk_max_u16(r[0], r[1]);
    }
}

// MXFP8 cast of TR x TC tiles (TR TC / 128 threads of 16 x 8 sub-tiles; a 1-D grid of tiles in
// XCD-aware order).  SRC 0: bf16 input, 512 x 256 tiles (16 waves; a wave reads two 512-byte row
// segments per load and the columnwise transpose leaves as 512-byte pieces of each output row).
// SRC 1: the rowwise-dequantized value of an NVFP4 tensor, 256 x 128 tiles staged through LDS.
template <int DIRS, int SRC, int TR, int TC>
__global__ __launch_bounds__(TR * TC / 128) void mxfp8_kernel(MxArgs a) {
    constexpr int CCS = TC / 8, RBS = TR / 16, BN = TR / 32;
    static_assert(SRC == 0 || (TR == TILE_R && TC == TILE_C), "the NVFP4 staging is 256 x 128");
    const int64_t R = a.R, C = a.C;
    const int64_t ntx = (C + TC - 1) / TC, ntile = ntx * ((R + TR - 1) / TR);
    const int64_t tile = xcd_tile(blockIdx.x, ntile);
    const int64_t tr0 = tile / ntx * TR, tc0 = tile % ntx * TC;
    const TileCoord t = tile_coord_at<TR, TC>(tile / ntx, tile % ntx);
    SubTile q;
    if constexpr (SRC == 0) {
        load_subtile<TR>(a.x, R, C, t, q);
    } else {
        const float S = a.nv_s_enc[0];
        if (C % 32 == 0) {   // uniform: 16-byte code chunks, staged through LDS
            __shared__ NvTileLds stage;
            stage_nvfp4_tile(a.nv_codes, a.nv_scales, S, R, C, tr0, tc0, stage);
            load_subtile_nvfp4_lds(stage, t, q);
        } else {
            load_subtile_nvfp4(a.nv_codes, a.nv_scales, S, R, C, t, q);
        }
    }

    if (DIRS & 1) mx_row_tile<TR>(q, t, R, C, a.row_codes, a.row_scales, a.slab);

    if (DIRS & 2) {
        // the NVFP4 columnwise transpose's placement: block rb of column 8cc + k at
        // [8cc + k][rb ^ cc] (scales at [8cc + k][(rb >> 1) ^ (cc mod BN)])
        __shared__ uint4 lds_codes[TC][RBS];
        __shared__ uint8_t lds_sc[TC][BN];
        static_assert(CCS <= RBS, "swizzle stays inside a column's slots");
        const bool upper = (t.rb & 1) != 0;
        const int slot = t.rb ^ t.cc, sslot = (t.rb >> 1) ^ (t.cc & (BN - 1));
        // binary32 form of column k: amax, scale byte, x * 2^-X clamped to +-448, E4M3 codes
        auto col_f32 = [&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            float v[16];
            col_of(q, k, v);
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(v[j]));
            m = __builtin_fmaxf(m, __shfl_xor(m, CCS));
            uint32_t w[4] = {0, 0, 0, 0}, sb = 0;
            if (m != 0.0f) {
                sb = mx_scale_byte(m);
                const float inv = mx_inv_scale(sb);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = e4m3_pack4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
            }
            lds_codes[8 * t.cc + k][slot] = make_uint4(w[0], w[1], w[2], w[3]);
            if (!upper) lds_sc[8 * t.cc + k][sslot] = (uint8_t)sb;
        };
        // Packed form of the column pair (2w, 2w + 1) held in word w of every row: the same codes
        // and scale bytes.  For finite bf16 the magnitude bits order like the values, so one
        // 16-bit unsigned maximum per row gives both columns' amax; the amax exponent field E
        // gives the scale byte E - 8 (X = E - 135).  Each element is clamped to 448 * 2^X (bf16
        // exponent E, mantissa 1.75), the largest value whose code is finite, by a signed and an
        // unsigned 16-bit minimum; v_cvt_scalef32_pk_fp8_bf16 then divides two elements of one
        // column by 2^X (exact) and rounds them to nearest even E4M3.  The conversion neither
        // saturates nor takes a zero scale operand, so a wave in which some block has E <= 8
        // (all zero, or amax below 2^-118: scale byte 0) takes the binary32 form.
        static_for<0, 4>([&](auto w_c) {
            constexpr int w = decltype(w_c)::value;
            uint32_t M = 0u;
#pragma unroll
            for (int j = 0; j < 16; ++j) M = pk_max_u16(M, q[j][w] & 0x7FFF7FFFu);
            M = pk_max_u16_block_pair<CCS>(M);
            const bool fast = (M & 0xFFFFu) >= 0x480u && M >= 0x04800000u;   // both E >= 9
            if (__builtin_amdgcn_ballot_w64(!fast) == 0) {   // wave-uniform
                const uint32_t T = (M & 0x7F807F80u) | 0x00600060u;
                const uint32_t sb = ((M >> 7) & 0x00FF00FFu) - 0x00080008u;
                const float s_lo = __uint_as_float((sb & 0xFFu) << 23), s_hi = __uint_as_float((sb >> 16) << 23);
                uint32_t z[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) z[j] = pk_min_u16(pk_min_i16(q[j][w], T), T | 0x80008000u);
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    lo[d] = fp8x4_scaled(__builtin_amdgcn_perm(z[4 * d + 1], z[4 * d], 0x05040100u),
                                         __builtin_amdgcn_perm(z[4 * d + 3], z[4 * d + 2], 0x05040100u), s_lo);
                    hi[d] = fp8x4_scaled(__builtin_amdgcn_perm(z[4 * d + 1], z[4 * d], 0x07060302u),
                                         __builtin_amdgcn_perm(z[4 * d + 3], z[4 * d + 2], 0x07060302u), s_hi);
                }
                lds_codes[8 * t.cc + 2 * w][slot] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
                lds_codes[8 * t.cc + 2 * w + 1][slot] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
                if (!upper) {
                    lds_sc[8 * t.cc + 2 * w][sslot] = (uint8_t)(sb & 0xFFu);
                    lds_sc[8 * t.cc + 2 * w + 1][sslot] = (uint8_t)(sb >> 16);
                }
            } else {
                col_f32(std::integral_constant<int, 2 * w>{});
                col_f32(std::integral_constant<int, 2 * w + 1>{});
            }
        });
        __syncthreads();
        // TC x RBS 16-byte pieces, 8 per thread: piece p of thread t is output row (= input
        // column) col0 + p NT/RBS, input rows r .. r + 15 (the same r for all 8).  Non-temporal:
        // the codes are not read again by this pass (21.9 against 22.4 us).
        constexpr int NT = TR * TC / 128;
        const int col0 = threadIdx.x / RBS, rbk = threadIdx.x % RBS;
        const int64_t r = tr0 + 16 * rbk;
        const int64_t ncols = (C - tc0) < TC ? (C - tc0) : TC;
        if (R * 256 < ((int64_t)1 << 31)) {   // uniform
            // Through a buffer resource over the output rows the tile writes: row-major, rows
            // tc0 .. tc0 + TC - 1 (rows past C fall outside the range); slab layout, the whole
            // 256-row band of tc0 (a tile's TC <= 256 rows lie in one band), in which output row
            // c's piece of input rows r.. sits at (r / 64) n 64 + (c mod 256) 64 + r mod 64 for
            // the band's n rows -- rows past C would land in the next slab and are dropped here.
            // Each piece is one 32-bit offset add from the thread's first.
            int64_t base, nbytes;
            uint32_t off0, step;
            if (a.slab) {
                const int64_t band = tc0 >> 8, left = C - (band << 8), n = left < 256 ? left : 256;
                base = (band << 8) * R;
                nbytes = n * R;
                off0 = (uint32_t)((r >> 6) * n * 64 + ((tc0 & 255) + col0) * 64 + (r & 63));
                step = (uint32_t)(NT / RBS) * 64u;
            } else {
                base = tc0 * R;
                nbytes = ncols * R;
                off0 = (uint32_t)(col0 * R + r);
                step = (uint32_t)((NT / RBS) * R);
            }
            const __amdgpu_buffer_rsrc_t rc =
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.col_codes + base), (short)0, (int)nbytes, 0x00020000);
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int col = col0 + (NT / RBS) * p;
                const bool ok = r < R && col < ncols;
                const uint4 cv = lds_codes[col][rbk ^ (col >> 3)];
                __builtin_amdgcn_raw_buffer_store_b128(u32v4{cv.x, cv.y, cv.z, cv.w}, rc,
                                                       (int)(ok ? off0 + (uint32_t)p * step : 0x80000000u), 0, 2);
            }
        } else {
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int col = col0 + (NT / RBS) * p;
                const int64_t c = tc0 + col;
                if (c < C && r < R) {
                    const uint4 cv = lds_codes[col][rbk ^ (col >> 3)];
                    __builtin_nontemporal_store(u32v4{cv.x, cv.y, cv.z, cv.w},
                                                (u32v4*)(a.col_codes + (a.slab ? slab_offset(c, r, C, R) : c * R + r)));
                }
            }
        }
        store_col_scales<32, TR, TC>(&lds_sc[0][0], a.col_scales, R, C, tr0, tc0);
    }
}

// ------------------------------------------------------------------ NVFP4 dequantize

// One thread per 16-element block: out = bf16((E2M1 * fp32(s_b)) / S).
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const float* __restrict__ s_enc, int64_t nblocks,
                                                            uint16_t* __restrict__ out) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const float S = s_enc[0];
    const float sc = e4m3_decode_nonneg(scales[b] & 0x7Fu);
    const uint2 cw = *(const uint2*)(codes + 8 * b);
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const uint32_t c = ((j < 8 ? cw.x : cw.y) >> (4 * (j & 7))) & 0xFu;
        const uint32_t h = nvfp4_dequant_bf16(c, sc, S);
        if (j & 1) o[j >> 1] |= h << 16; else o[j >> 1] = h;
    }
    uint4* dst = (uint4*)(out + 16 * b);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// ------------------------------------------------------------------ standalone RHT

template <int AXIS>
__global__ __launch_bounds__(NTHREADS) void rht_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                       const int8_t* __restrict__ signs, float* __restrict__ out) {
    const TileCoord t = tile_coord();
    SubTile q;
    load_subtile(x, R, C, t, q);
    const uint32_t neg = sign_mask16(signs);
    const bool colok = t.c0 < C;
    if (AXIS == 1) {
        const bool upper = (t.cc & 1) != 0;
        static_for<0, 16>([&](auto j_c) {
            constexpr int j = decltype(j_c)::value;
            float v[8];
            row_of(q, j, v);
            rht16_pair(v, neg, upper);
            const int64_t r = t.r0 + j;
            if (colok && r < R) {
                float4* d = (float4*)(out + r * C + t.c0);
                d[0] = make_float4(v[0], v[1], v[2], v[3]);
                d[1] = make_float4(v[4], v[5], v[6], v[7]);
            }
        });
    } else {
        float y[16][8];
        static_for<0, 8>([&](auto k_c) {
            constexpr int k = decltype(k_c)::value;
            float v[16];
            col_of(q, k, v);
            rht16(v, neg);
#pragma unroll
            for (int j = 0; j < 16; ++j) y[j][k] = v[j];
        });
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int64_t r = t.r0 + j;
            if (colok && r < R) {
                float4* d = (float4*)(out + r * C + t.c0);
                d[0] = make_float4(y[j][0], y[j][1], y[j][2], y[j][3]);
                d[1] = make_float4(y[j][4], y[j][5], y[j][6], y[j][7]);
            }
        }
    }
}

// ------------------------------------------------------------------ linear (rowwise) kernels
//
// Rowwise quantization never crosses a row (cols is a multiple of the block size), so the
// tensor is a flat array of blocks: block b covers elements [16b, 16b + 16) (NVFP4) or
// [32b, 32b + 32) (MXFP8), its codes and scale sit at linear offsets in the row-major
// outputs, and the SR index of an element is its linear index.  These kernels stream the
// tensor with grid-stride loops: lane u of a sweep owns the 16-byte unit u (8 values),
// every wave-wide load is 1 KB contiguous, and UNITS independent loads per lane are in
// flight.  They reach the HBM streaming rate where the 256 x 128 tile kernels (needed for
// columnwise blocks) do not.

// Launch shape swept on MI355X over 2-16 units per lane, 128-512 threads and 512-8192
// workgroups on [8192, 4096] and [16384, 4096]: 4 units, 256 threads, up to 4096 workgroups
// gave the MXFP8 rowwise cast 17.9 us (was 19.1 with 8 units and 2048 workgroups) and the
// two-pass NVFP4 rowwise cast 29.0 us (29.1).
constexpr int LIN_UNITS = 4;                 // 16-byte units per lane per sweep
constexpr int LIN_THREADS = 256;
constexpr int LIN_MAX_BLOCKS = 256 * 16;     // a few workgroups per CU

__device__ __forceinline__ void lin_range(int64_t n16, int64_t& first, int64_t& stride) {
    first = (int64_t)blockIdx.x * LIN_THREADS * LIN_UNITS + threadIdx.x;
    stride = (int64_t)gridDim.x * LIN_THREADS * LIN_UNITS;
    (void)n16;
}

// Plain tensor amax: max |x| over n16 16-byte units, stored to the slots of the directions in
// DIRS (without RHT both directions share it).
template <int DIRS>
__global__ __launch_bounds__(LIN_THREADS) void amax_linear_kernel(const uint4* __restrict__ x, int64_t n16,
                                                                  float* __restrict__ parts) {
    int64_t first, stride;
    lin_range(n16, first, stride);
    float m = 0.0f;
    for (int64_t base = first; base < n16; base += stride) {
        uint4 q[LIN_UNITS];
#pragma unroll
        for (int k = 0; k < LIN_UNITS; ++k) {
            const int64_t u = base + (int64_t)k * LIN_THREADS;
            // Before a columnwise (tile) encode the loads are temporal, so that the tensor can
            // stay in the memory-side cache for the encode's second read (measured: that encode
            // 13-15 % faster on 64-134 MB tensors, this pass ~4 % slower); before the streaming
            // rowwise encode, which gained nothing from it, they stay non-temporal.
            q[k] = u < n16 ? (DIRS == 1 ? load16_stream(x + u) : x[u]) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < LIN_UNITS; ++k) {
            float v[8];
            unpack_bf16x8(q[k], v);
#pragma unroll
            for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
        }
    }
    store_parts<LIN_THREADS, DIRS>(m, m, parts);
}

// Row-RHT amax: the 16-point transform of each block, the block held by a lane pair (the
// maximum of the butterfly's |h|, quartered at the end: exact).
__global__ __launch_bounds__(LIN_THREADS) void amax_rht_row_linear_kernel(const uint4* __restrict__ x, int64_t n16,
                                                                          const int8_t* __restrict__ signs,
                                                                          float* __restrict__ parts) {
    int64_t first, stride;
    lin_range(n16, first, stride);
    const uint32_t neg = sign_mask16(signs);
    const bool upper = (threadIdx.x & 1) != 0;
    uint32_t sw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) sw[w] = row_sign_word(neg, upper, w);
    float m = 0.0f;
    for (int64_t base = first; base < n16; base += stride) {
        uint4 q[LIN_UNITS];
#pragma unroll
        for (int k = 0; k < LIN_UNITS; ++k) {
            const int64_t u = base + (int64_t)k * LIN_THREADS;
            q[k] = u < n16 ? load16_stream(x + u) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < LIN_UNITS; ++k) {
            float v[8];
            unpack_bf16x8(make_uint4(q[k].x ^ sw[0], q[k].y ^ sw[1], q[k].z ^ sw[2], q[k].w ^ sw[3]), v);
            rht16_pair_core(v, upper);
#pragma unroll
            for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
        }
    }
    store_parts<LIN_THREADS, 1>(m * 0.25f, 0.0f, parts);
}

// Rowwise NVFP4 encode: unit u = half u%2 of block u/2.
template <bool RHT, bool SR>
__global__ __launch_bounds__(LIN_THREADS) void nvfp4_row_linear_kernel(const uint4* __restrict__ x, int64_t n16,
                                                                       const int8_t* __restrict__ signs,
                                                                       uint32_t* __restrict__ codes,
                                                                       uint8_t* __restrict__ scales,
                                                                       const float* __restrict__ parts, int nparts,
                                                                       float* __restrict__ amax_out,
                                                                       float* __restrict__ s_enc_out, uint64_t seed,
                                                                       uint32_t stream) {
    int64_t first, stride;
    lin_range(n16, first, stride);
    uint4 q[LIN_UNITS];
    auto load_sweep = [&](int64_t base) {
#pragma unroll
        for (int k = 0; k < LIN_UNITS; ++k) {
            const int64_t u = base + (int64_t)k * LIN_THREADS;
            q[k] = u < n16 ? load16_stream(x + u) : make_uint4(0, 0, 0, 0);
        }
    };
    // the partial maxima, then the first sweep's units: the prologue's reduction and table
    // build run while the units are in flight
    const PartsShare<LIN_THREADS> mine = parts_load<LIN_THREADS, 1>(parts, nparts);
    load_sweep(first);
    const float2 am = parts_reduce<LIN_THREADS, 1>(mine);
    const float S = nvfp4_tensor_scale(am.x);
    publish_scales<1>(am, amax_out, s_enc_out);
    __shared__ float enc_tab[128];
    build_enc_table(S, enc_tab, 0);
    __syncthreads();
    const uint32_t neg = RHT ? sign_mask16(signs) : 0u;
    const bool upper = (threadIdx.x & 1) != 0;
    uint32_t sw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) sw[w] = RHT ? row_sign_word(neg, upper, w) : 0u;
    for (int64_t base = first; base < n16; base += stride) {
        if (base != first) load_sweep(base);
#pragma unroll
        for (int k = 0; k < LIN_UNITS; ++k) {
            const int64_t u = base + (int64_t)k * LIN_THREADS;
            float v[8];
            if (RHT) {
                unpack_bf16x8(make_uint4(q[k].x ^ sw[0], q[k].y ^ sw[1], q[k].z ^ sw[2], q[k].w ^ sw[3]), v);
                rht16_pair_core(v, upper);
            } else {
                unpack_bf16x8(q[k], v);
            }
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
            m = pair_max(m);
            uint32_t w;
            const uint32_t sb = encode_block<8, SR, RHT>(v, m, S, enc_tab, (uint64_t)u * 8u, seed, stream, 0u, &w);
            if (u < n16) {
                codes[u] = w;
                if (!upper) scales[u >> 1] = (uint8_t)sb;
            }
        }
    }
}

// ------------------------------------------------------------------ row-scaled NVFP4
//
// Per-row outer scale: row r is quantized with S_r = 2688 / amax(row r) (the rowwise
// quantizer of the Composer-style recipe on the page "[Pytorch][Common] Hybrid
// quantization"; the "outer scale rowwise, inner scale 1x16" recipe of the review on "Add an
// NVFP4 quantization converter").  A group of T = 2^lgt threads (2 <= T <= 256) owns a row:
// thread `sub` of the group holds the 16-byte units sub + T*k (k < RS_UNITS) of each chunk
// of T * RS_UNITS units, so adjacent lanes read adjacent units and the two halves of a
// 16-block sit on a lane pair.  A row of at most one chunk (cols <= 8192 at T = 256) is
// read once and kept in registers (as bf16; the transform is recomputed) between its amax
// reduction and its encode; a longer row is
// walked twice, the second walk re-reading it (normal loads, so the first walk leaves it
// in L2).  The SR index of an element is its linear index, as in the per-tensor rowwise
// quantization.
constexpr int RS_UNITS = 4;
constexpr int RS_THREADS = 256;
constexpr int RS_MAX_BLOCKS = 256 * 32;

template <bool RHT, bool SR>
__global__ __launch_bounds__(RS_THREADS) void nvfp4_rowscaled_kernel(const uint4* __restrict__ x, int64_t R,
                                                                     int64_t upr, int lgt,
                                                                     const int8_t* __restrict__ signs,
                                                                     uint32_t* __restrict__ codes,
                                                                     uint8_t* __restrict__ scales,
                                                                     float* __restrict__ amax_rows,
                                                                     float* __restrict__ s_enc_rows, uint64_t seed,
                                                                     uint32_t stream) {
    const int T = 1 << lgt;
    const int sub = threadIdx.x & (T - 1);
    const int grp = threadIdx.x >> lgt;
    const int rpw = RS_THREADS >> lgt;                 // rows per workgroup pass
    const int64_t chunk = (int64_t)T * RS_UNITS;
    const bool one = upr <= chunk;                     // uniform
    const uint32_t neg = RHT ? sign_mask16(signs) : 0u;
    const bool upper = (threadIdx.x & 1) != 0;
    __shared__ float red[RS_THREADS / 64];

    // The loop bounds are the same for every thread of the workgroup (the barrier below
    // needs that); rows past R are computed on zeros and not stored.
    for (int64_t rb = (int64_t)blockIdx.x * rpw; rb < R; rb += (int64_t)gridDim.x * rpw) {
        const int64_t r = rb + grp;
        const bool live = r < R;
        const int64_t base = (live ? r : 0) * upr;
        uint4 q[RS_UNITS];   // the raw bf16 units of the current chunk
        auto load_chunk = [&](int64_t c0, auto streaming) {
#pragma unroll
            for (int k = 0; k < RS_UNITS; ++k) {
                const int64_t u = c0 + sub + (int64_t)T * k;
                if (live && u < upr) q[k] = decltype(streaming)::value ? load16_stream(x + base + u) : x[base + u];
                else q[k] = make_uint4(0, 0, 0, 0);
            }
        };
        // values of unit k (transformed when RHT is on) and their largest magnitude
        auto values = [&](int k, float v[8]) {
            unpack_bf16x8(q[k], v);
            if (RHT) rht16_pair(v, neg, upper);
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
            return m;
        };
        float m = 0.0f;
        if (one) {
            load_chunk(0, std::true_type{});
#pragma unroll
            for (int k = 0; k < RS_UNITS; ++k) {
                float v[8];
                m = __builtin_fmaxf(m, values(k, v));
            }
        } else {
            for (int64_t c0 = 0; c0 < upr; c0 += chunk) {
                load_chunk(c0, std::false_type{});
#pragma unroll
                for (int k = 0; k < RS_UNITS; ++k) {
                    float v[8];
                    m = __builtin_fmaxf(m, values(k, v));
                }
            }
        }
        // row amax: across the group's lanes, then across its waves
        m = group_max_dpp(m, lgt < 6 ? lgt : 6);
        if (T > 64) {
            if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
            __syncthreads();
            const int w0 = (grp * T) >> 6;
            m = red[w0];
            for (int w = 1; w < (T >> 6); ++w) m = __builtin_fmaxf(m, red[w0 + w]);
            __syncthreads();
        }
        const float S = nvfp4_tensor_scale(m);
        if (live && sub == 0) {
            amax_rows[r] = m;
            s_enc_rows[r] = S;
        }
        // the empty asm makes the units opaque, so the encode recomputes each unit's values from
        // its 4 registers instead of the compiler keeping the amax pass's 8 floats per unit alive
#pragma unroll
        for (int k = 0; k < RS_UNITS; ++k) asm volatile("" : "+v"(q[k].x), "+v"(q[k].y), "+v"(q[k].z), "+v"(q[k].w));
        for (int64_t c0 = 0; c0 < upr; c0 += chunk) {
            if (!one) load_chunk(c0, std::false_type{});
#pragma unroll
            for (int k = 0; k < RS_UNITS; ++k) {
                const int64_t u = c0 + sub + (int64_t)T * k;
                float v[8];
                float bm = values(k, v);
                bm = pair_max(bm);
                uint32_t w;
                const uint32_t sb = encode_block<8, SR, false>(v, bm, S, nullptr, (uint64_t)(base + u) * 8u, seed, stream,
                                                               0u, &w);
                if (live && u < upr) {
                    codes[base + u] = w;
                    if (!upper) scales[(base + u) >> 1] = (uint8_t)sb;
                }
            }
        }
    }
}

// Rowwise MXFP8 cast: unit u = quarter u%4 of block u/4 (elements 8u..8u+7 in row-major
// order).  SLAB writes the codes in the slab layout of a [R][C] matrix: the unit's row is
// u / (C/8), from a binary64 estimate (exact to within one for u < 2^52) corrected exactly.
template <bool SLAB>
__global__ __launch_bounds__(LIN_THREADS) void mxfp8_row_linear_kernel(const uint4* __restrict__ x, int64_t n16,
                                                                       uint2* __restrict__ codes,
                                                                       uint8_t* __restrict__ scales, int64_t R,
                                                                       int64_t C, double inv_c8) {
    int64_t first, stride;
    lin_range(n16, first, stride);
    for (int64_t base = first; base < n16; base += stride) {
        uint4 q[LIN_UNITS];
#pragma unroll
        for (int k = 0; k < LIN_UNITS; ++k) {
            const int64_t u = base + (int64_t)k * LIN_THREADS;
            q[k] = u < n16 ? load16_stream(x + u) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < LIN_UNITS; ++k) {
            const int64_t u = base + (int64_t)k * LIN_THREADS;
            uint32_t lo = 0, hi = 0, sb = 0;
            const uint32_t wk[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
            if (!mx_row_unit_packed(wk, lo, hi, sb)) {
                float v[8];
                unpack_bf16x8(q[k], v);
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
                m = __builtin_fmaxf(m, __shfl_xor(m, 1));
                m = __builtin_fmaxf(m, __shfl_xor(m, 2));
                lo = hi = sb = 0;
                if (m != 0.0f) {
                    sb = mx_scale_byte(m);
                    const float inv = mx_inv_scale(sb);
                    lo = e4m3_pack4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
                    hi = e4m3_pack4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
                }
            }
            if (u < n16) {
                int64_t at = u;
                if constexpr (SLAB) {
                    const int64_t c8 = C >> 3;
                    int64_t r = (int64_t)((double)u * inv_c8);
                    if (r * c8 > u) --r;
                    else if ((r + 1) * c8 <= u) ++r;
                    at = slab_offset(r, (u - r * c8) << 3, R, C) >> 3;
                }
                codes[at] = make_uint2(lo, hi);
                if ((u & 3) == 0) scales[u >> 2] = (uint8_t)sb;
            }
        }
    }
}

static inline unsigned lin_grid(int64_t n16) {
    const int64_t per = (int64_t)LIN_THREADS * LIN_UNITS;
    int64_t g = (n16 + per - 1) / per;
    if (g > LIN_MAX_BLOCKS) g = LIN_MAX_BLOCKS;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// ------------------------------------------------------------------ launchers

// MXFP8 cast tiles from bf16: columnwise alone 512 x 256 (1024 threads), rowwise + columnwise
// MX_TR3 x MX_TC3; a 1-D grid of one workgroup per tile.
constexpr int MX_TR = 512, MX_TC = 256, MX_TR3 = 512, MX_TC3 = 256;
template <int TR, int TC>
static inline unsigned mx_tiles(int64_t R, int64_t C) {
    return (unsigned)(((C + TC - 1) / TC) * ((R + TR - 1) / TR));
}

static inline dim3 tile_grid(int64_t R, int64_t C) {
    return dim3((unsigned)((C + TILE_C - 1) / TILE_C), (unsigned)((R + TILE_R - 1) / TILE_R), 1);
}

__global__ void empty_tensor_scales_kernel(float* amax, float* s_enc) {
    if (threadIdx.x < 2) {
        amax[threadIdx.x] = 0.0f;
        s_enc[threadIdx.x] = 1.0f;
    }
}

static inline unsigned amax_grid(int64_t units, int64_t per) {
    int64_t g = (units + per - 1) / per;
    if (g > AMAX_PARTS) g = AMAX_PARTS;
    if (g < 1) g = 1;
    return (unsigned)g;
}

// The error of the launch just made (0 if it was accepted).
static inline int launch_status() { return (int)hipGetLastError(); }

template <int DIRS, bool RHT, bool SR>
static int launch_encode_tiles(const NvEncodeArgs& a, hipStream_t s) {
    if (DIRS == 2 && a.mx_codes != nullptr)
        hipLaunchKernelGGL((nvfp4_encode_kernel<DIRS, RHT, SR, true>), tile_grid(a.R, a.C), dim3(NTHREADS), 0, s, a);
    else hipLaunchKernelGGL((nvfp4_encode_kernel<DIRS, RHT, SR>), tile_grid(a.R, a.C), dim3(NTHREADS), 0, s, a);
    return launch_status();
}

template <int DIRS, bool RHT>
static int launch_encode_tiles(const NvEncodeArgs& a, bool sr, hipStream_t s) {
    return sr ? launch_encode_tiles<DIRS, RHT, true>(a, s) : launch_encode_tiles<DIRS, RHT, false>(a, s);
}

int launch_nvfp4_quantize(const void* x, int64_t R, int64_t C, int direction, int rounding, uint64_t seed,
                          uint32_t stream, const int8_t* signs, uint8_t* row_codes, uint8_t* row_scales,
                          uint8_t* col_codes, uint8_t* col_scales, float* amax, float* s_enc, float* parts,
                          void* hip_stream, uint8_t* mx_codes, uint8_t* mx_scales, int mx_slab) {
    hipStream_t s = (hipStream_t)hip_stream;
    if (R == 0 || C == 0) {
        hipLaunchKernelGGL(empty_tensor_scales_kernel, dim3(1), dim3(64), 0, s, amax, s_enc);
        return launch_status();
    }
    const bool rht = signs != nullptr, sr = rounding == 1;
    const int64_t n16 = R * C / 8;
    const uint4* xv = (const uint4*)x;
    // amax pass: the streaming kernels, except for a columnwise transform (along rows)
    unsigned np;
    if (rht && (direction & 2)) {
        np = amax_grid(((R + TILE_R - 1) / TILE_R) * ((C + TILE_C - 1) / TILE_C), 1);
        if (direction == 2)
            hipLaunchKernelGGL(nvfp4_amax_rht_kernel<2>, dim3(np), dim3(NTHREADS), 0, s, (const uint16_t*)x, R, C, signs, parts);
        else
            hipLaunchKernelGGL(nvfp4_amax_rht_kernel<3>, dim3(np), dim3(NTHREADS), 0, s, (const uint16_t*)x, R, C, signs, parts);
    } else {
        np = amax_grid(n16, (int64_t)LIN_THREADS * LIN_UNITS);
        if (rht) hipLaunchKernelGGL(amax_rht_row_linear_kernel, dim3(np), dim3(LIN_THREADS), 0, s, xv, n16, signs, parts);
        else if (direction == 1) hipLaunchKernelGGL(amax_linear_kernel<1>, dim3(np), dim3(LIN_THREADS), 0, s, xv, n16, parts);
        else if (direction == 2) hipLaunchKernelGGL(amax_linear_kernel<2>, dim3(np), dim3(LIN_THREADS), 0, s, xv, n16, parts);
        else hipLaunchKernelGGL(amax_linear_kernel<3>, dim3(np), dim3(LIN_THREADS), 0, s, xv, n16, parts);
    }
    if (const int e = launch_status()) return e;
    const int nparts = (int)np;
    if (direction == 1) {
        // rowwise only: the streaming encode
        const dim3 lg(lin_grid(n16));
        uint32_t* rc = (uint32_t*)row_codes;
        if (rht && sr) hipLaunchKernelGGL((nvfp4_row_linear_kernel<true, true>), lg, dim3(LIN_THREADS), 0, s, xv, n16, signs, rc, row_scales, parts, nparts, amax, s_enc, seed, stream);
        else if (rht) hipLaunchKernelGGL((nvfp4_row_linear_kernel<true, false>), lg, dim3(LIN_THREADS), 0, s, xv, n16, signs, rc, row_scales, parts, nparts, amax, s_enc, seed, stream);
        else if (sr) hipLaunchKernelGGL((nvfp4_row_linear_kernel<false, true>), lg, dim3(LIN_THREADS), 0, s, xv, n16, signs, rc, row_scales, parts, nparts, amax, s_enc, seed, stream);
        else hipLaunchKernelGGL((nvfp4_row_linear_kernel<false, false>), lg, dim3(LIN_THREADS), 0, s, xv, n16, signs, rc, row_scales, parts, nparts, amax, s_enc, seed, stream);
        return launch_status();
    }
    // columnwise, alone or with rowwise: the 256 x 128 tile kernels
    const NvEncodeArgs a{(const uint16_t*)x, R, C, signs, row_codes, row_scales, col_codes, col_scales,
                         parts, nparts, amax, s_enc, seed, stream, mx_codes, mx_scales, mx_slab};
    if (direction == 2) return rht ? launch_encode_tiles<2, true>(a, sr, s) : launch_encode_tiles<2, false>(a, sr, s);
    return rht ? launch_encode_tiles<3, true>(a, sr, s) : launch_encode_tiles<3, false>(a, sr, s);
}

// The rowwise forward operand (RNE, no transform) and the columnwise wgrad operand (RHT and SR
// as given) of one tensor from one amax pass and one encode pass.  Without RHT and SR both
// directions are the plain cast, which nvfp4_quantize already does in one pass.
int launch_nvfp4_quantize_fprop_wgrad(const void* x, int64_t R, int64_t C, int rounding, uint64_t seed,
                                      uint32_t stream, const int8_t* signs, uint8_t* row_codes, uint8_t* row_scales,
                                      uint8_t* col_codes, uint8_t* col_scales, float* amax, float* s_enc,
                                      float* parts, void* hip_stream) {
    const bool rht = signs != nullptr, sr = rounding == 1;
    if (!rht && !sr)
        return launch_nvfp4_quantize(x, R, C, 3, 0, seed, stream, nullptr, row_codes, row_scales, col_codes,
                                     col_scales, amax, s_enc, parts, hip_stream);
    hipStream_t s = (hipStream_t)hip_stream;
    if (R == 0 || C == 0) {
        hipLaunchKernelGGL(empty_tensor_scales_kernel, dim3(1), dim3(64), 0, s, amax, s_enc);
        return launch_status();
    }
    unsigned np;
    if (rht) {
        np = amax_grid(((R + TILE_R - 1) / TILE_R) * ((C + TILE_C - 1) / TILE_C), 1);
        hipLaunchKernelGGL((nvfp4_amax_rht_kernel<3, true>), dim3(np), dim3(NTHREADS), 0, s, (const uint16_t*)x, R, C,
                           signs, parts);
    } else {
        const int64_t n16 = R * C / 8;
        np = amax_grid(n16, (int64_t)LIN_THREADS * LIN_UNITS);
        hipLaunchKernelGGL(amax_linear_kernel<3>, dim3(np), dim3(LIN_THREADS), 0, s, (const uint4*)x, n16, parts);
    }
    if (const int e = launch_status()) return e;
    const NvEncodeArgs a{(const uint16_t*)x, R, C, signs, row_codes, row_scales, col_codes, col_scales,
                         parts, (int)np, amax, s_enc, seed, stream, nullptr, nullptr, 0};
    const dim3 g = tile_grid(R, C);
    if (rht && sr) hipLaunchKernelGGL((nvfp4_encode_kernel<3, true, true, false, true>), g, dim3(NTHREADS), 0, s, a);
    else if (rht) hipLaunchKernelGGL((nvfp4_encode_kernel<3, true, false, false, true>), g, dim3(NTHREADS), 0, s, a);
    else hipLaunchKernelGGL((nvfp4_encode_kernel<3, false, true, false, true>), g, dim3(NTHREADS), 0, s, a);
    return launch_status();
}

// ------------------------------------------------------------------ allocation-free variant
//
// nvfp4_quantize_noalloc keeps the amax pass's partial maxima in this file-scope device array
// instead of a caller workspace: one copy per GPU, BSQ_NVFP4_QUANTIZE_WORKSPACE_BYTES, held
// until the process ends.  Host code never passes the array's name to a kernel (on the host
// it is a stand-in, not a device address): the device address comes from hipGetSymbolAddress,
// taken once per device with that device current and kept in scratch_addr.  No initial
// contents are needed (each call stores every slot it reads), so nothing is cleared; calls
// that overlap on one GPU share the array and race.
static __device__ __align__(256) float scratch[2 * AMAX_PARTS];

constexpr int SCRATCH_DEVICES = 64;

// Device address of this device's `scratch` (looked up on the first call on the device).
static int scratch_addr(float** out) {
    static std::mutex mu;
    static float* addr[SCRATCH_DEVICES] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= SCRATCH_DEVICES) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        addr[dev] = static_cast<float*>(p);
    }
    *out = addr[dev];
    return 0;
}

int launch_nvfp4_quantize_noalloc(const void* x, int64_t R, int64_t C, int direction, int rounding, uint64_t seed,
                                  uint32_t stream, const int8_t* signs, uint8_t* row_codes, uint8_t* row_scales,
                                  uint8_t* col_codes, uint8_t* col_scales, float* amax, float* s_enc,
                                  void* hip_stream) {
    float* parts = nullptr;
    if (const int e = scratch_addr(&parts)) return e;
    return launch_nvfp4_quantize(x, R, C, direction, rounding, seed, stream, signs, row_codes, row_scales, col_codes,
                                 col_scales, amax, s_enc, parts, hip_stream);
}

int launch_nvfp4_quantize_rowscaled(const void* x, int64_t R, int64_t C, int rounding, uint64_t seed,
                                    uint32_t stream, const int8_t* signs, uint8_t* codes, uint8_t* scales,
                                    float* amax_rows, float* s_enc_rows, void* hip_stream) {
    if (R == 0) return 0;
    hipStream_t s = (hipStream_t)hip_stream;
    const int64_t upr = C / 8;
    // threads per row: the power of two that holds the row in at most RS_UNITS units per lane
    int lgt = 1;
    while (lgt < 8 && ((int64_t)RS_UNITS << lgt) < upr) ++lgt;
    const int64_t rpw = RS_THREADS >> lgt;
    int64_t g = (R + rpw - 1) / rpw;
    if (g > RS_MAX_BLOCKS) g = RS_MAX_BLOCKS;
    const uint4* xv = (const uint4*)x;
    uint32_t* cw = (uint32_t*)codes;
    const bool rht = signs != nullptr, sr = rounding == 1;
    const dim3 grid((unsigned)g), block(RS_THREADS);
    if (rht && sr) hipLaunchKernelGGL((nvfp4_rowscaled_kernel<true, true>), grid, block, 0, s, xv, R, upr, lgt, signs, cw, scales, amax_rows, s_enc_rows, seed, stream);
    else if (rht) hipLaunchKernelGGL((nvfp4_rowscaled_kernel<true, false>), grid, block, 0, s, xv, R, upr, lgt, signs, cw, scales, amax_rows, s_enc_rows, seed, stream);
    else if (sr) hipLaunchKernelGGL((nvfp4_rowscaled_kernel<false, true>), grid, block, 0, s, xv, R, upr, lgt, signs, cw, scales, amax_rows, s_enc_rows, seed, stream);
    else hipLaunchKernelGGL((nvfp4_rowscaled_kernel<false, false>), grid, block, 0, s, xv, R, upr, lgt, signs, cw, scales, amax_rows, s_enc_rows, seed, stream);
    return (int)hipGetLastError();
}

int launch_mxfp8_quantize(const void* x, int64_t R, int64_t C, int direction, uint8_t* row_codes,
                          uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales, void* hip_stream) {
    if (R == 0 || C == 0) return 0;
    hipStream_t s = (hipStream_t)hip_stream;
    const int slab = (direction & 4) != 0;
    direction &= 3;
    MxArgs a{(const uint16_t*)x, nullptr, nullptr, nullptr, R, C, row_codes, row_scales, col_codes, col_scales, slab};
    if (direction == 1) {
        const int64_t n16 = R * C / 8;
        const double inv_c8 = 8.0 / (double)C;
        if (slab)
            hipLaunchKernelGGL(mxfp8_row_linear_kernel<true>, dim3(lin_grid(n16)), dim3(LIN_THREADS), 0, s,
                               (const uint4*)x, n16, (uint2*)row_codes, row_scales, R, C, inv_c8);
        else
            hipLaunchKernelGGL(mxfp8_row_linear_kernel<false>, dim3(lin_grid(n16)), dim3(LIN_THREADS), 0, s,
                               (const uint4*)x, n16, (uint2*)row_codes, row_scales, R, C, inv_c8);
    } else {
        const dim3 g(mx_tiles<MX_TR, MX_TC>(R, C));
        if (direction == 2) hipLaunchKernelGGL((mxfp8_kernel<2, 0, MX_TR, MX_TC>), g, dim3(MX_TR * MX_TC / 128), 0, s, a);
        else hipLaunchKernelGGL((mxfp8_kernel<3, 0, MX_TR3, MX_TC3>), dim3(mx_tiles<MX_TR3, MX_TC3>(R, C)),
                                dim3(MX_TR3 * MX_TC3 / 128), 0, s, a);
    }
    return (int)hipGetLastError();
}

int launch_mxfp8_requantize_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* s_enc, int64_t R,
                                  int64_t C, int direction, uint8_t* row_codes, uint8_t* row_scales,
                                  uint8_t* col_codes, uint8_t* col_scales, void* hip_stream) {
    if (R == 0 || C == 0) return 0;
    hipStream_t s = (hipStream_t)hip_stream;
    const int slab = (direction & 4) != 0;
    direction &= 3;
    MxArgs a{nullptr, codes, scales, s_enc, R, C, row_codes, row_scales, col_codes, col_scales, slab};
    const dim3 g(mx_tiles<TILE_R, TILE_C>(R, C));
    if (direction == 1) hipLaunchKernelGGL((mxfp8_kernel<1, 1, TILE_R, TILE_C>), g, dim3(NTHREADS), 0, s, a);
    else if (direction == 2) hipLaunchKernelGGL((mxfp8_kernel<2, 1, TILE_R, TILE_C>), g, dim3(NTHREADS), 0, s, a);
    else hipLaunchKernelGGL((mxfp8_kernel<3, 1, TILE_R, TILE_C>), g, dim3(NTHREADS), 0, s, a);
    return (int)hipGetLastError();
}

int launch_nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* s_enc, int64_t rows,
                            int64_t cols, void* out, void* hip_stream) {
    const int64_t nb = rows * (cols / 16);
    if (nb == 0) return 0;
    hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0,
                       (hipStream_t)hip_stream, codes, scales, s_enc, nb, (uint16_t*)out);
    return (int)hipGetLastError();
}

int launch_rht_apply(const void* x, int64_t R, int64_t C, int axis, const int8_t* signs, float* out,
                     void* hip_stream) {
    if (R == 0 || C == 0) return 0;
    const dim3 g = tile_grid(R, C);
    if (axis == 1)
        hipLaunchKernelGGL(rht_kernel<1>, g, dim3(NTHREADS), 0, (hipStream_t)hip_stream, (const uint16_t*)x, R, C,
                           signs, out);
    else
        hipLaunchKernelGGL(rht_kernel<0>, g, dim3(NTHREADS), 0, (hipStream_t)hip_stream, (const uint16_t*)x, R, C,
                           signs, out);
    return (int)hipGetLastError();
}

const char* hip_error_string(int e) { return hipGetErrorString((hipError_t)e); }

}  // namespace bsq
