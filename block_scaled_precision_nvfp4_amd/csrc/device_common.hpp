// device_common.hpp -- gfx950 device helpers shared by the quantization and GEMM kernels:
// bf16 widening, E4M3 / E2M1 encoders, Philox4x32-10, the 16-point Hadamard butterfly.
//
// Every floating-point step is a single binary32 operation in round-to-nearest-even
// (the library is built with -ffp-contract=off and correctly rounded division), so the
// results are bit-identical to any implementation performing the same operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bsq {

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).  Used where a loop
// body indexes a register array and must see constant indices even when it is too large
// for the unroller's heuristics.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

typedef unsigned int u32v4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal: the data is read once).
__device__ __forceinline__ uint4 load16_stream(const void* p) {
    const u32v4 v = __builtin_nontemporal_load((const u32v4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight bf16 values packed in a uint4 -> eight floats (exact).
__device__ __forceinline__ void unpack_bf16x8(const uint4 q, float v[8]) {
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}

// binary32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two binary32 values -> packed bf16 (lo = a, hi = b), round to nearest even: the hardware
// conversion v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    const bf16x2_t p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, p);
}

// ---------------------------------------------------------------- E4M3 (OCP "fn")
// Non-negative t -> E4M3 code, nearest-even, saturating at 448 (code 0x7E).
// Subnormal range [0, 2^-6): code = rint(t * 2^9) (0..8; 8 is the first normal).
// Normal range: round the binary32 mantissa to 3 bits (ties to even) and rebias the
// exponent from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float t) {
    if (!(t < 448.0f)) return 0x7Eu;
    if (t < 0x1p-6f) return (uint32_t)__builtin_rintf(t * 512.0f);
    uint32_t u = __float_as_uint(t);
    u += 0x7FFFFu + ((u >> 20) & 1u);
    return (u >> 20) - (120u << 3);
}

// Signed value -> E4M3 code (sign bit copied, including -0).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    return e4m3_encode_nonneg(__builtin_fabsf(v)) | ((__float_as_uint(v) >> 24) & 0x80u);
}

// Four values -> four E4M3 codes (nearest-even, saturating at 448, sign kept), value i in
// byte i.  The hardware conversion v_cvt_pk_fp8_f32 rounds to nearest-even but returns NaN
// above 464 instead of saturating, so each value is first clamped to [-448, 448] (one
// v_med3).  Checked on MI355X against e4m3_encode on 1.6 million values (every code, every
// midpoint and its neighbours, the subnormal range, +-0, values up to 3e38): identical codes.
__device__ __forceinline__ uint32_t e4m3_pack4(float v0, float v1, float v2, float v3) {
    const float lo = -448.0f, hi = 448.0f;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(v0, lo, hi), __builtin_amdgcn_fmed3f(v1, lo, hi),
                                            0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(v2, lo, hi), __builtin_amdgcn_fmed3f(v3, lo, hi), w,
                                        true);
    return (uint32_t)w;
}

// Non-negative E4M3 code (<= 0x7E) -> float.
__device__ __forceinline__ float e4m3_decode_nonneg(uint32_t c) {
    if (c < 8u) return (float)c * 0x1p-9f;
    return __uint_as_float((((c >> 3) + 120u) << 23) | ((c & 7u) << 20));
}

// ---------------------------------------------------------------- E2M1
// Round-to-nearest-even onto {0, .5, 1, 1.5, 2, 3, 4, 6} with saturation: the code is
// the number of decision boundaries below |v|; a boundary that is a tie rounds toward
// the even code, hence '>' where the lower neighbour has an even code and '>=' where
// it is odd.
__device__ __forceinline__ uint32_t e2m1_encode_rne(float v) {
    float a = __builtin_fabsf(v);
    uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                 (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                 (uint32_t)(a > 5.0f);
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// Two values -> two E2M1 codes (RNE, saturating, sign kept) written into byte SEL of w, the
// first value in the low nibble.  v_cvt_scalef32_pk_fp4_f32 with scale 1 was checked on
// MI355X against the nearest-even definition on 165 592 inputs (every tie, +-0, values far
// above 6): identical codes.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2_rne(uint32_t w, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, SEL);
}

// Stochastic rounding onto the E2M1 grid: with lo the grid value at or below |v| and p =
// (|v| - lo) / spacing (exact), round up iff (u >> 8) * 2^-24 < p; |v| >= 6 saturates.
// Branch-free integer form of that comparison:
//   |v| in [1, 6): p = (low 22 mantissa bits) / 2^22 and lo's code is 2 + 2e + (mantissa
//     bit 22) = (|v| bits >> 22) - 252; (u >> 8) < 4 * low22 <=> u < low22 << 10, and
//     (v bits << 10) is low22 << 10 (sign, exponent and bit 22 shifted out);
//   |v| in [0.5, 1): grid {0.5, 1}, p = (23 mantissa bits) / 2^23, up iff u < (v bits << 9);
//     the code below is 1, which max((|v| bits >> 22) - 252, 1) also gives;
//   |v| < 0.5: grid {0, 0.5}, p = 2|v|, up iff (u >> 8) * 2^-25 < |v| (both sides exact);
//   codes above 7 (|v| >= 6) are clamped to 7.  The sign bit is copied (-0 gives code 0x8).
__device__ __forceinline__ uint32_t e2m1_encode_sr(float v, uint32_t u) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t ab = b & 0x7FFFFFFFu;
    const uint32_t thr = b << (ab >= 0x3F800000u ? 10 : 9);
    const int lo = max((int)(ab >> 22) - 252, 1);
    const uint32_t big = min((uint32_t)lo + (u < thr ? 1u : 0u), 7u);
    const uint32_t small = (float)(u >> 8) * 0x1p-25f < __uint_as_float(ab) ? 1u : 0u;
    return (ab < 0x3F000000u ? small : big) | ((b >> 28) & 8u);
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon et al., "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        // one 32 x 32 -> 64-bit multiply per product (v_mad_u64_u32) instead of mul_lo + mul_hi
        const uint64_t p0 = (uint64_t)M0 * c.x, p1 = (uint64_t)M1 * c.z;
        u32x4 n;
        // three-input XOR in one v_bitop3_b32 (truth table 0x96)
        n.x = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96);
        n.y = (uint32_t)p1;
        n.z = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96);
        n.w = (uint32_t)p0;
        c = n;
        k0 += W0;
        k1 += W1;
    }
    return c;
}

// The four SR words of output elements 4q .. 4q+3 of direction dir.
__device__ __forceinline__ u32x4 sr_words(uint64_t q, uint64_t seed, uint32_t stream, uint32_t dir) {
    u32x4 c{(uint32_t)q, (uint32_t)(q >> 32), stream, dir};
    return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t word_of(const u32x4& w, int i) {
    return i == 0 ? w.x : (i == 1 ? w.y : (i == 2 ? w.z : w.w));
}

// ---------------------------------------------------------------- Hadamard
// y = v diag(d) H16 / 4 per 16-block: sign flip, butterfly strides 1, 2, 4, 8 with (a, b) ->
// (a + b, a - b), then the exact scaling by 1/4.  d is a bitmask: bit i set means d_i = -1.
// The quantize kernels flip the signs on the packed bf16 words before unpacking and fold the
// 1/4 into the encode multiplier, so they call the butterfly alone (rht16_core /
// rht16_pair_core); every butterfly output is a multiple of 2^-133 (a sum of bf16 values,
// rounded to fp32), which makes its quarter exact.

// The butterfly on 16 registers (no sign, no scaling).
__device__ __forceinline__ void rht16_core(float v[16]) {
#pragma unroll
    for (int h = 1; h < 16; h *= 2) {
#pragma unroll
        for (int i = 0; i < 16; i += 2 * h) {
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
}

__device__ __forceinline__ void rht16(float v[16], uint32_t negmask) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = ((negmask >> i) & 1u) ? -v[i] : v[i];
    rht16_core(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= 0.25f;
}

// The butterfly of a 16-block held by a lane pair: this lane holds elements 8*upper ..
// 8*upper+7 and its partner (lane ^ 1) the other half.  Strides 1, 2, 4 are local; stride 8
// pairs element j of the lower half with element j of the upper half.
__device__ __forceinline__ void rht16_pair_core(float v[8], bool upper) {
#pragma unroll
    for (int h = 1; h < 8; h *= 2) {
#pragma unroll
        for (int i = 0; i < 8; i += 2 * h) {
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float other = __shfl_xor(v[j], 1);
        // lower lane: a + b with a = own; upper lane: a - b with a = partner's
        v[j] = upper ? (other - v[j]) : (v[j] + other);
    }
}

__device__ __forceinline__ void rht16_pair(float v[8], uint32_t negmask, bool upper) {
    const int off = upper ? 8 : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ((negmask >> (i + off)) & 1u) ? -v[i] : v[i];
    rht16_pair_core(v, upper);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] *= 0.25f;
}

// XOR masks that flip the signs of a lane's packed bf16 words (two values per word) for the
// transform along a row: word w of the lane's 8 values holds block elements 8*upper + 2w and
// 8*upper + 2w + 1.
__device__ __forceinline__ uint32_t row_sign_word(uint32_t negmask, bool upper, int w) {
    const uint32_t n = negmask >> ((upper ? 8 : 0) + 2 * w);
    return ((n & 1u) << 15) | ((n & 2u) << 30);
}

// Block-scale code of a block with largest magnitude bmax under tensor scale S: the E4M3 code
// of (bmax * S) / 6, the quotient formed with two fused multiply-adds from RN(1/6):
// q0 = t RN(1/6), q = q0 + (t - 6 q0) RN(1/6).  For every binary32 t in [0, 2688 (1 + 2^-21)]
// (t never exceeds 2688 (1 + 2^-23)) q equals the correctly rounded t / 6 except where t is
// below 10^-30, where both encode to code 0 -- checked exhaustively over all 1.16 * 10^9 values.
__device__ __forceinline__ uint32_t block_scale_code(float bmax, float S) {
    const float t = bmax * S;
    const float r6 = 0x1.555556p-3f;
    const float q0 = t * r6;
    return e4m3_encode_nonneg(__builtin_fmaf(__builtin_fmaf(-q0, 6.0f, t), r6, q0));
}

// NVFP4 per-tensor scale from the amax: 2688 / A, A = 0 -> 1, overflow -> FLT_MAX.
__device__ __forceinline__ float nvfp4_tensor_scale(float amax) {
    if (amax == 0.0f) return 1.0f;
    float s = 2688.0f / amax;
    if (__builtin_isinf(s)) s = 3.40282347e38f;
    return s;
}

}  // namespace bsq
