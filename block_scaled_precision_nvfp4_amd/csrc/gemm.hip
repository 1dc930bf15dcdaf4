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
// tensor scales enter once, in the epilogue: alpha = 1 / (S_a * S_b).  An operand may
// instead carry one outer scale per row (row-scaled NVFP4); the epilogue then takes
// alpha(m, n) from a per-tile table of row and column factors (see tile_factors).
//
// MXFP8 operands (E4M3 codes, one E8M0 scale per 32 K-elements) map one-to-one onto the
// scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4.  Its K layout: in lane (row, g), bytes
// 0-15 of the 32-byte operand are K-elements 16g..16g+15 of the step and bytes 16-31 are
// K-elements 32+16g..32+16g+15; the scale of K-block 0 (elements 0-31) comes from lanes
// 0-31, that of K-block 1 from lanes 32-63.
//
// Tiling: a workgroup computes a 256 x 256 tile of C with 4 waves of 128 x 128 (4 x 4 MFMA
// tiles of 32 x 32, 256 fp32 accumulators per lane).  Each K slice (128 elements for NVFP4, 64
// for MXFP8) of both operands is 64 bytes of codes per row, moved from memory straight into a
// ring of 4 LDS stages by LDS DMA, three slices ahead of its use, with one barrier per slice.
// Scales: 16-byte records of a row's scale bytes where scale rows lie 16 bytes apart (NVFP4 K a
// multiple of 256; MXFP8 also at an offset inside the record, or per-slice bytes otherwise),
// and for NVFP4 with any other K (or K-grouped) per-slice records of 3 aligned dwords per row.
// MXFP8 codes may come in the slab layout, where each slice of a tile's rows is one contiguous
// block.  Plain NVFP4 launches with per-tensor scales run persistently (gemm_nvp_kernel),
// carrying the LDS ring from one tile to the next.  The buffer loads' range check zero-fills
// rows beyond M or N, and an out-of-range offset the K tail.  16-byte chunks are XOR-swizzled
// by row.  Inside a slice the operands of the next MFMA step are read from LDS (and, for
// NVFP4, dequantized) while the current step's MFMAs issue.  Workgroups are renumbered so that
// each of the 8 XCDs (which take workgroups round-robin) works on a contiguous band of output
// tiles and reuses operand rows from its own L2.
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
    int a_rows, b_rows;   // the operand's tensor scale is per row (float[M] / float[N])
    int64_t ld;           // elements between consecutive rows of A and of B (K unless grouped along K)
    int slab;             // MXFP8 codes in the slab layout (K a multiple of 512): bit 0 A, bit 1 B
    int64_t k0;           // K-grouped: the group's first element along the rows of a slab operand
};

// FMT 1: MXFP8; FMT 2: NVFP4 with grouped scale records (K a multiple of 256); FMT 3: NVFP4
// with per-slice scale records (K a multiple of 32).  All three: 4 waves of 128 x 128, 4 LDS
// stages filled by LDS DMA.
template <int FMT>
struct Fmt {
    static constexpr bool NV = FMT != 1;
    static constexpr int BK = NV ? 128 : 64;          // K elements per slice
    static constexpr int EPB = NV ? 2 : 1;            // elements per code byte
    static constexpr int BLK = NV ? 16 : 32;          // elements per scale
    // static LDS per workgroup: MXFP8 4 x 36 KiB stages + an 8 KiB scale-record buffer; NVFP4
    // with records 4 x 32 KiB code stages + 2 x 8 KiB record groups; NVFP4 per slice 4 x 38 KiB
    static constexpr int LDS = FMT == 3 ? 4 * (2 * GBM * ROWB + 2 * GBM * 12)
                                        : 4 * (GBM + GBN) * (ROWB + 8) + (FMT == 1 ? 8192 : 0);
    static constexpr int THREADS = 256;               // 4 waves
    static constexpr int TN = 4;                      // 32-row B fragments per wave (128 x 128)
    static constexpr int WAVES_N = GBN / (32 * TN);
};

// Byte offset of 16-byte chunk c (0..3) of LDS code row r (64-byte rows, so 4 rows fill the 64
// banks): the chunk index is XORed with bits 2..3 of the row (the DMAs apply the same
// permutation on the global side, swzd_chunk), so that the 16 lanes of a 16-byte read that takes
// one chunk of 16 consecutive rows cover all 64 banks once (bits 3..4 would leave rows r and
// r + 4 on the same banks).
__device__ __forceinline__ int swzd_chunk(int r, int c) { return c ^ ((r >> 2) & 3); }
__device__ __forceinline__ int swzd(int r, int c) { return r * ROWB + (swzd_chunk(r, c) << 4); }


constexpr int RSRC_FLAGS = 0x00020000;   // raw 32-bit data, no format conversion
constexpr uint32_t OOB = 0x80000000u;    // an offset beyond every resource's range

// Rows of an operand that a tile's resource covers: the tile's own rows that exist.  (Covering
// only the tile keeps the byte range far below the resource's 2^31 limit for any K the C ABI
// accepts, and rows past M or N still read as zero.)
__device__ __forceinline__ int64_t tile_rows(int64_t left, int64_t tile) { return left < tile ? left : tile; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)n, RSRC_FLAGS);
}

// ---------------------------------------------------------------- NVFP4 fragments

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

// ---------------------------------------------------------------- MXFP8 slice

constexpr int MXTN = Fmt<1>::TN;   // B fragments per MXFP8 wave
static_assert(MXTN == 4 && Fmt<1>::THREADS == 256, "the MXFP8 slice is written for 4 waves of 4 x 4 tiles");

struct MxFrag {
    intx8 a[4], b[MXTN];
    uint32_t as[4], bs[MXTN];   // low byte: E8M0 scale of the fragment row's K-block (lane half)
};

// MXFP8 LDS layout.  A code stage (one K slice) is A codes [256][64 B] then B codes
// [256][64 B], the 16-byte chunks swizzled by swzd().  Scales use one of three layouts:
//  - grouped (MX_RECS; K a multiple of 512, 16-byte aligned rows): the scale bytes of 8
//    consecutive slices (16 K-blocks) of a row form one aligned 16-byte global record,
//    fetched with one DMA lane per row every 8 slices into a double-buffered region
//    [group parity][operand][256 rows][16 B] after the 4 code stages;
//  - offset records (MX_OFFRECS; rows a multiple of 16 scale bytes apart, any K and base):
//    the aligned 16-byte records that hold a row's scale bytes, which start delta bytes into
//    the first one (the same delta for every row of an operand).  Slice group G reads bytes
//    of records G and G+1, so the records rotate through three buffers of the grouped
//    region's shape, record j in buffer j mod 3;
//  - per slice (MX_SLOTS; any other row pitch): one dword slot per (row, K-block) after the
//    codes of each stage, [operand][256 rows][2 slots], holding the byte in its low 8 bits
//    (a byte DMA fills one dword slot per lane).
// MX_SLAB is MX_RECS with the codes of one or both operands in the slab layout: a 256-row
// band of an operand (one tile's rows) stored slice by slice, [K/64][n rows][64 B], so that
// each slice of the band is one contiguous block that the DMAs read whole (row-major codes
// come as 64-byte pieces of rows 2 KiB and more apart, which fill LDS at about 60 % of the
// rate).  The API admits slab operands only where K % 512 == 0, so they always meet the
// aligned-record conditions.  MX_GSLAB is the K-grouped launch with slab operands: a group's
// K range starts at any multiple of 32, so its scales take offset records and its codes are
// addressed from the whole band (mx_gslab_codes).
constexpr int MX_SLOTS = 0, MX_RECS = 1, MX_OFFRECS = 2, MX_SLAB = 3, MX_GSLAB = 4;
constexpr int MX_CODES = 2 * GBM * ROWB;                  // 32 KiB
constexpr int MX_STAGE_SLOTS = MX_CODES + 2 * GBM * 2 * 4;  // 36 KiB
constexpr int MX_GROUP = 8;                                // slices per grouped scale record
constexpr int MX_SREC = 2 * GBM * 16;                      // 8 KiB per scale group
static_assert(4 * MX_STAGE_SLOTS <= Fmt<1>::LDS && 4 * MX_CODES + 3 * MX_SREC <= Fmt<1>::LDS, "MXFP8 LDS");

// LDS DMA: a buffer load whose data goes straight to LDS.  A wave-wide DMA writes 64
// consecutive LDS slots starting at the wave-uniform address in M0 -- 16 bytes per lane for
// dwordx4, one dword slot per lane for a byte (the byte in its low 8 bits).  The loads are
// issued as inline assembly so that the compiler does not track them: the loop waits for them
// itself with s_waitcnt vmcnt (which only ever makes the compiler's own waits stricter), and
// the compiler does not serialise every LDS read behind every DMA in flight.
typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));

struct RsrcWords {
    u32x4s a, b, as, bs;
};

__device__ __forceinline__ u32x4s rsrc_words(const uint8_t* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
    const uint64_t a = (uint64_t)base;
    return u32x4s{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, (uint32_t)n, (uint32_t)RSRC_FLAGS};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void dma_b128(const u32x4s& rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "m0");
}

__device__ __forceinline__ void dma_u8(const u32x4s& rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ubyte %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "m0");
}

// Waits until at most N of this wave's vector-memory operations are in flight, then joins the
// workgroup barrier.  The memory clobber keeps the compiler from moving LDS accesses across.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" :: "n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Per-wave DMA plan of one MXFP8 K slice, in four parts that the main loop spreads between its
// MFMAs.  Part P (0..3) moves rows 64P + 16w .. +16 (w = wave) of both operands' codes; the
// chunk swizzle is applied on the global side (the lane that fills LDS chunk slot cs of row r
// fetches global chunk swzd_chunk(r, cs)).  In the per-slice scale layout parts 0 and 1
// also move scale slots 256P + 64w .. +64 of both operands.  A slice past the end of K is
// issued with out-of-range offsets (no memory traffic; the zeros they write land in a free
// buffer) so that every slice issues the same number of DMAs.
struct MxDma {
    RsrcWords o;
    uint32_t rowbytes, sstride;   // code and scale bytes between consecutive rows
    uint32_t kbytes, kblocks;     // code and scale bytes of a row's K elements
    uint32_t slab_a, slab_b;      // slab layout: bytes of one slice of the tile's A / B rows
    uint32_t gslab, gchunk;       // K-grouped slab operands: slab and chunk of the group's first element
    int wave, lane;
};

// Codes of the slice whose first code byte in each row is b0 (64 bytes per row).
template <int P, int NW = 4>
__device__ __forceinline__ void mx_dma_codes(const MxDma& d, int64_t b0, bool live, uint8_t* buf) {
    const int r0 = 16 * NW * P + 16 * d.wave;
    const int r = r0 + (d.lane >> 2), c = swzd_chunk(r, d.lane & 3);
    uint32_t off = (uint32_t)r * d.rowbytes + 16u * c;
    if (!live || b0 + 16 * c >= (int64_t)d.kbytes) off = OOB;
    const uint32_t soff = live ? (uint32_t)b0 : 0u;
    dma_b128(d.o.a, lds_addr(buf + r0 * ROWB), off, soff);
    dma_b128(d.o.b, lds_addr(buf + GBM * ROWB + r0 * ROWB), off, soff);
}

// MXFP8 per-slice scale slots of the slice starting at element k0.
template <int P>
__device__ __forceinline__ void mx_dma_slots(const MxDma& d, int64_t k0, bool live, uint8_t* buf) {
    const int s0 = 256 * P + 64 * d.wave;
    const int sl = s0 + d.lane, r = sl >> 1, kb = sl & 1;
    const int64_t kb0 = k0 / 32;
    const uint32_t off = (live && kb0 + kb < (int64_t)d.kblocks) ? (uint32_t)r * d.sstride + kb : OOB;
    const uint32_t soff = live ? (uint32_t)kb0 : 0u;
    dma_u8(d.o.as, lds_addr(buf + MX_CODES + 4 * s0), off, soff);
    dma_u8(d.o.bs, lds_addr(buf + MX_CODES + 8 * GBM + 4 * s0), off, soff);
}

// The same DMAs where K is a multiple of the slice group (the NVFP4 kernel: K % 256 == 0; the
// MXFP8 kernel with grouped scale records: K % 512 == 0): a slice inside K never reaches past
// K in any lane, so the one decision per slice is uniform -- a slice (or scale group) past the
// end of K is issued with resources of zero size, which put every lane out of range (no memory
// traffic; the zeros land in a free buffer).  The lane offsets are fixed for the tile, and the
// whole per-slice selection is scalar work.
__device__ __forceinline__ u32x4s sized(u32x4s rsrc, bool live) {
    rsrc[2] = live ? rsrc[2] : 0u;
    return rsrc;
}

template <int P, int NW>
__device__ __forceinline__ void nv4_dma_codes(const MxDma& d, uint32_t b0, bool live, uint8_t* buf) {
    const int r0 = 16 * NW * P + 16 * d.wave;
    const int r = r0 + (d.lane >> 2), c = swzd_chunk(r, d.lane & 3);
    const uint32_t off = (uint32_t)r * d.rowbytes + 16u * c;
    const uint32_t soff = live ? b0 : 0u;
    dma_b128(sized(d.o.a, live), lds_addr(buf + r0 * ROWB), off, soff);
    dma_b128(sized(d.o.b, live), lds_addr(buf + GBM * ROWB + r0 * ROWB), off, soff);
}

// Grouped scales: the 16-byte record grp (scale bytes 16grp..16grp+15) of every row of both
// operands, one lane per row: lane l of wave w takes row 64w + l of A and of B.
template <int NW>
__device__ __forceinline__ void nv4_dma_group(const MxDma& d, uint32_t grp, bool live, uint8_t* sbuf) {
    static_assert(NW == 4, "one lane per row of each operand");
    const uint32_t soff = live ? 16u * grp : 0u;
    const uint32_t off = (uint32_t)(64 * d.wave + d.lane) * d.sstride;
    dma_b128(sized(d.o.as, live), lds_addr(sbuf + 64 * d.wave * 16), off, soff);
    dma_b128(sized(d.o.bs, live), lds_addr(sbuf + GBM * 16 + 64 * d.wave * 16), off, soff);
}

// Offset records: record j (16 aligned bytes) of every row of both operands, one lane per row
// as in nv4_dma_group; offa / offb hold the lane's row offset from the resource base (an
// out-of-range offset for a row past the tile).  The record offset goes into the vector offset
// so that the resource's range check covers the whole address.
__device__ __forceinline__ void mx_dma_offrec(const MxDma& d, uint32_t offa, uint32_t offb, uint32_t j, bool live,
                                              uint8_t* sbuf) {
    dma_b128(sized(d.o.as, live), lds_addr(sbuf + 64 * d.wave * 16), offa + 16u * j, 0u);
    dma_b128(sized(d.o.bs, live), lds_addr(sbuf + GBM * 16 + 64 * d.wave * 16), offb + 16u * j, 0u);
}

// Slab layout: the resource of slice k's block (`bytes` long, none when not live), whose rows
// sit 64 bytes apart; rows past the tile's fall outside it.
__device__ __forceinline__ u32x4s slab_rsrc(u32x4s r, uint32_t k, uint32_t bytes, bool live) {
    const uint64_t base = (((uint64_t)(r[1] & 0xFFFFu) << 32) | r[0]) + (uint64_t)k * bytes;
    r[0] = (uint32_t)base;
    r[1] = (r[1] & 0xFFFF0000u) | ((uint32_t)(base >> 32) & 0xFFFFu);
    r[2] = live ? bytes : 0u;
    return r;
}

// Slice k's codes where at least one operand is in the slab layout (SL bit 0: A is, bit 1: B
// is); the other operand is read row-major as in nv4_dma_codes.  The layouts are template
// parameters: chosen at run time, the two resources of an operand cost the main loop its
// scalar DMA setup.
template <int P, int SL>
__device__ __forceinline__ void mx_slab_codes(const MxDma& d, uint32_t k, bool live, uint8_t* buf) {
    const int r0 = 64 * P + 16 * d.wave;
    const int r = r0 + (d.lane >> 2), c = swzd_chunk(r, d.lane & 3);
    const uint32_t off_s = (uint32_t)r * 64u + 16u * c;
    const uint32_t off_r = (uint32_t)r * d.rowbytes + 16u * c;
    const uint32_t soff = live ? 64u * k : 0u;
    if constexpr (SL & 1) dma_b128(slab_rsrc(d.o.a, k, d.slab_a, live), lds_addr(buf + r0 * ROWB), off_s, 0u);
    else dma_b128(sized(d.o.a, live), lds_addr(buf + r0 * ROWB), off_r, soff);
    if constexpr (SL & 2) dma_b128(slab_rsrc(d.o.b, k, d.slab_b, live), lds_addr(buf + GBM * ROWB + r0 * ROWB), off_s, 0u);
    else dma_b128(sized(d.o.b, live), lds_addr(buf + GBM * ROWB + r0 * ROWB), off_r, soff);
}

// Slice k's codes in a K-grouped launch with at least one operand in the slab layout (SL as in
// mx_slab_codes).  The group starts gchunk 16-byte chunks into slab gslab (gchunk 0 or 2: group
// boundaries are multiples of 32), so the lane's local chunk c of slice k is chunk
// (gchunk + c) % 4 of slab gslab + k + (gchunk + c) / 4.  The resource spans the tile's band
// (n rows, slabs of n x 64 bytes); rows past n and chunks past the group's K are sent out of
// range, and the whole offset is in the vector offset, which the range check covers.
template <int P, int SL>
__device__ __forceinline__ void mx_gslab_codes(const MxDma& d, uint32_t k, bool live, uint8_t* buf) {
    const int r0 = 64 * P + 16 * d.wave;
    const int r = r0 + (d.lane >> 2), c = swzd_chunk(r, d.lane & 3);
    const bool in = live && 64u * k + 16u * (uint32_t)c < d.kbytes;
    const uint32_t gc = d.gchunk + (uint32_t)c;
    const uint32_t sl = d.gslab + k + (gc >> 2), within = (uint32_t)r * 64u + 16u * (gc & 3u);
    const uint32_t off_r = in ? (uint32_t)r * d.rowbytes + 16u * c + 64u * k : OOB;
    if constexpr (SL & 1) {
        const uint32_t off = (in && within < d.slab_a) ? sl * d.slab_a + within : OOB;
        dma_b128(d.o.a, lds_addr(buf + r0 * ROWB), off, 0u);
    } else {
        dma_b128(d.o.a, lds_addr(buf + r0 * ROWB), off_r, 0u);
    }
    if constexpr (SL & 2) {
        const uint32_t off = (in && within < d.slab_b) ? sl * d.slab_b + within : OOB;
        dma_b128(d.o.b, lds_addr(buf + GBM * ROWB + r0 * ROWB), off, 0u);
    } else {
        dma_b128(d.o.b, lds_addr(buf + GBM * ROWB + r0 * ROWB), off_r, 0u);
    }
}

// DMA plan of the tile at (m0, n0); its B rows are the first `brows` (GBN, or 128 for the
// persistent kernel's half tiles) -- the DMAs of B rows past them read nothing and write zeros.
template <int EPB, int BLK>
__device__ __forceinline__ MxDma make_dma(const GemmArgs& g, int64_t m0, int64_t n0, int lane, int64_t brows = GBN) {
    MxDma d;
    const int64_t rb = g.ld / EPB, sb = g.ld / BLK;
    const int64_t ra = tile_rows(g.M - m0, GBM), rbn = tile_rows(g.N - n0, brows);
    d.o.a = rsrc_words(g.a_codes + m0 * rb, ra * rb);
    d.o.b = rsrc_words(g.b_codes + n0 * rb, rbn * rb);
    d.o.as = rsrc_words(g.a_scales + m0 * sb, ra * sb);
    d.o.bs = rsrc_words(g.b_scales + n0 * sb, rbn * sb);
    d.rowbytes = (uint32_t)rb;
    d.sstride = (uint32_t)sb;
    d.kbytes = (uint32_t)(g.K / EPB);
    d.kblocks = (uint32_t)(g.K / BLK);
    d.slab_a = (uint32_t)ra * 64u;
    d.slab_b = (uint32_t)rbn * 64u;
    d.gslab = (uint32_t)(g.k0 / 64);
    d.gchunk = (uint32_t)((g.k0 / 16) & 3);
    d.wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    d.lane = lane;
    return d;
}

// The lane's scale bytes of a slice in the offset-record layout: a at A fragment row 0's byte,
// b at B fragment row 0's (fragment P's rows are 512P bytes further).
struct MxSPtr {
    const uint8_t* a;
    const uint8_t* b;
};

// Fragment reads of part P of a slice: A fragment P and B fragment P (lane (row, g): K elements
// 16g..16g+15 (chunk g) and 32+16g.. (chunk 2+g) of the slice) and their scales (K-block g).
// Grouped scales: byte 2q + g of the row's record, q = slice index within its group.
template <int P, int MODE>
__device__ __forceinline__ void mx_read_part(const uint8_t* buf, const uint8_t* sbuf, int q, MxSPtr sp, int wm,
                                             int wn, int lane, MxFrag& f) {
    const int frow = lane & 31, kh = lane >> 5;
    const int ra = wm + 32 * P + frow, rb = wn + 32 * P + frow;
    const uint8_t* sA = buf;
    const uint8_t* sB = buf + GBM * ROWB;
    uint4 lo = *(const uint4*)(sA + swzd(ra, kh));
    uint4 hi = *(const uint4*)(sA + swzd(ra, 2 + kh));
    f.a[P] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    lo = *(const uint4*)(sB + swzd(rb, kh));
    hi = *(const uint4*)(sB + swzd(rb, 2 + kh));
    f.b[P] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    if constexpr (MODE == MX_RECS || MODE == MX_SLAB) {
        f.as[P] = sbuf[ra * 16 + 2 * q + kh];
        f.bs[P] = sbuf[GBM * 16 + rb * 16 + 2 * q + kh];
    } else if constexpr (MODE == MX_OFFRECS || MODE == MX_GSLAB) {
        f.as[P] = sp.a[512 * P];
        f.bs[P] = sp.b[512 * P];
    } else {
        const uint32_t* slots = (const uint32_t*)(buf + MX_CODES);
        f.as[P] = slots[2 * ra + kh];
        f.bs[P] = slots[2 * GBM + 2 * rb + kh];
    }
}

template <int MODE>
__device__ __forceinline__ void mx_read(const uint8_t* buf, const uint8_t* sbuf, int q, MxSPtr sp, int wm, int wn,
                                        int lane, MxFrag& f) {
    mx_read_part<0, MODE>(buf, sbuf, q, sp, wm, wn, lane, f);
    mx_read_part<1, MODE>(buf, sbuf, q, sp, wm, wn, lane, f);
    mx_read_part<2, MODE>(buf, sbuf, q, sp, wm, wn, lane, f);
    mx_read_part<3, MODE>(buf, sbuf, q, sp, wm, wn, lane, f);
}

// The 4 MFMAs of A fragment P against the 4 B fragments.  As in the NVFP4 LDS-DMA kernel the B
// fragment (with its scales) is the first operand, so the accumulators hold C^T tiles (see
// nvw_mfma).
template <int P>
__device__ __forceinline__ void mx_mfma_row(const MxFrag& f, floatx16 (&acc)[4][MXTN]) {
#pragma unroll
    for (int j = 0; j < MXTN; ++j)
        acc[P][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[P], acc[P][j], 0, 0, 0, (int)f.bs[j], 0,
                                                                     (int)f.as[P]);
}

// MXFP8 main loop over K slices with 4 LDS code stages.  At the top of slice kt each wave
// waits for its own DMAs of slice kt+1 (issued two slices earlier; only those issued during
// slice kt-1 may still be in flight), then a barrier publishes slice kt+1 to the workgroup
// and confirms that every wave has consumed slice kt-1, whose buffer then receives the DMA of
// slice kt+3.  The slice's 16 MFMAs run in four parts; each part also issues a quarter of the
// DMAs of slice kt+3 (so that the vector-memory queue never stalls the wave) and reads one A
// and one B fragment of slice kt+1 into the other register set.  In the grouped layout the
// scale record of group G+1 is fetched during slice 8G+1 (its buffer held group G-1, whose
// last slice was consumed by then) and is complete, being older than the codes waited for,
// when slice 8G+7 reads the fragments of slice 8G+8.  Offset records follow the same
// schedule one record later: records 0 and 1 come with the first slices, record G+2 is
// fetched during slice 8G+1 into the buffer of record G-1 (last read for slice 8G-1) and is
// first read for slice 8G+8.
template <int MODE>
struct MxLds {
    static constexpr bool REC = MODE != MX_SLOTS;
    static constexpr int STRIDE = REC ? MX_CODES : MX_STAGE_SLOTS;
    static __device__ __forceinline__ uint8_t* buf(uint8_t* lds, int64_t k) { return lds + (int)(k & 3) * STRIDE; }
    static __device__ __forceinline__ uint8_t* sbuf(uint8_t* lds, int64_t grp) {
        return lds + 4 * MX_CODES + (int)(grp & 1) * MX_SREC;
    }
    // offset record j, j3 = j mod 3
    static __device__ __forceinline__ uint8_t* rbuf(uint8_t* lds, int j3) { return lds + 4 * MX_CODES + j3 * MX_SREC; }
};

// A tile's DMA plan and, for offset records, where its scale bytes sit in their records.
struct MxPlan {
    MxDma d;
    int dla, dlb;         // offset records: bytes into its first record where every A / B row starts
    uint32_t offa, offb;  // offset records: the lane's row offset from the resource base
    int nk32, kbl;        // slices; K-blocks (scale bytes) per row
};

template <int MODE>
__device__ __forceinline__ MxPlan mx_plan(const GemmArgs& g, int64_t m0, int64_t n0, int64_t nk, int lane) {
    MxPlan p;
    p.d = make_dma<1, 32>(g, m0, n0, lane);
    p.nk32 = (int)nk;   // nk <= 2^17 (K <= 2^23)
    p.kbl = (int)p.d.kblocks;
    p.dla = p.dlb = 0;
    p.offa = p.offb = OOB;
    // Offset records: the resources span the aligned records that hold the tile's scale bytes,
    // from the one holding its first byte through the one holding its last (whole records:
    // the range check drops a dword that reaches past the range; the bytes past the tensor's
    // end share the last byte's 16 aligned bytes, so its page).  Every row of an operand
    // starts dl bytes into its first record.
    if constexpr (MODE == MX_OFFRECS || MODE == MX_GSLAB) {
        const int64_t sb = g.ld / 32;
        const int64_t ra = tile_rows(g.M - m0, GBM), rbn = tile_rows(g.N - n0, GBN);
        const uint8_t* pa = g.a_scales + m0 * sb;
        const uint8_t* pb = g.b_scales + n0 * sb;
        p.dla = (int)((uintptr_t)pa & 15);
        p.dlb = (int)((uintptr_t)pb & 15);
        p.d.o.as = rsrc_words(pa - p.dla, (p.dla + (ra - 1) * sb + p.kbl + 15) & ~(int64_t)15);
        p.d.o.bs = rsrc_words(pb - p.dlb, (p.dlb + (rbn - 1) * sb + p.kbl + 15) & ~(int64_t)15);
        const int row = 64 * p.d.wave + lane;
        p.offa = row < ra ? (uint32_t)(row * sb) : OOB;
        p.offb = row < rbn ? (uint32_t)(row * sb) : OOB;
    }
    return p;
}

// Slice k's code DMAs, part P (K a multiple of 512 with grouped records: the scalar form).
template <int MODE, int SL, int P>
__device__ __forceinline__ void mx_dma_part(const MxDma& d, int64_t k, bool live, uint8_t* b) {
    if constexpr (MODE == MX_RECS) nv4_dma_codes<P, 4>(d, 64u * (uint32_t)k, live, b);
    else if constexpr (MODE == MX_SLAB) mx_slab_codes<P, SL>(d, (uint32_t)k, live, b);
    else if constexpr (MODE == MX_GSLAB) mx_gslab_codes<P, SL>(d, (uint32_t)k, live, b);
    else mx_dma_codes<P>(d, k * 64, live, b);
}

// All DMAs of slice k (codes, and per-slice scales in the slot layout).
template <int MODE, int SL>
__device__ __forceinline__ void mx_dma_slice(const MxPlan& p, int64_t k, uint8_t* lds) {
    const bool live = (int)k < p.nk32;
    uint8_t* b = MxLds<MODE>::buf(lds, k);
    static_for<0, 4>([&](auto p_c) { mx_dma_part<MODE, SL, decltype(p_c)::value>(p.d, k, live, b); });
    if constexpr (MODE == MX_SLOTS) {
        mx_dma_slots<0>(p.d, k * 64, live, b);
        mx_dma_slots<1>(p.d, k * 64, live, b);
    }
}

// The DMAs that precede a tile's first slice: its first scale record(s) and slices 0-2.  Per
// lane: 2 + 24 (grouped records), 4 + 24 (offset records) or 32 (slots) operations, of which
// slices 1 and 2 (16 or 24) come last.
template <int MODE, int SL>
__device__ __forceinline__ void mx_prologue(const MxPlan& p, uint8_t* lds) {
    if constexpr (MODE == MX_RECS || MODE == MX_SLAB) nv4_dma_group<4>(p.d, 0, true, MxLds<MODE>::sbuf(lds, 0));
    if constexpr (MODE == MX_OFFRECS || MODE == MX_GSLAB) {
        mx_dma_offrec(p.d, p.offa, p.offb, 0, true, MxLds<MODE>::rbuf(lds, 0));
        mx_dma_offrec(p.d, p.offa, p.offb, 1, 16 < 15 + p.kbl, MxLds<MODE>::rbuf(lds, 1));
    }
    mx_dma_slice<MODE, SL>(p, 0, lds);
    mx_dma_slice<MODE, SL>(p, 1, lds);
    mx_dma_slice<MODE, SL>(p, 2, lds);
}

template <int MODE, int SL = 0>
__device__ __forceinline__ void mx_main_loop(const GemmArgs& g, int64_t m0, int64_t n0, int64_t nk, uint8_t* lds,
                                             int wm, int wn, int lane, floatx16 (&acc)[4][MXTN]) {
    using L = MxLds<MODE>;
    constexpr bool REC = L::REC;
    constexpr bool ALIGNED = MODE == MX_RECS || MODE == MX_SLAB;   // aligned records, nk % MX_GROUP == 0
    constexpr bool OFFR = MODE == MX_OFFRECS || MODE == MX_GSLAB;  // offset records
    constexpr int DC = 8;                    // code DMAs per slice per lane
    constexpr int DS = REC ? 0 : 4;          // per-slice scale DMAs
    constexpr int DG = 2;                    // scale-record DMAs (every MX_GROUP slices)
    if (nk <= 0) return;
    const MxPlan pl = mx_plan<MODE>(g, m0, n0, nk, lane);
    const MxDma& d = pl.d;
    const int nk32 = pl.nk32, kbl = pl.kbl;
    // The lane's scale bytes of slice q of a group whose first record is in buffer c3: byte
    // dl + 2q + kh of the group's two records (below 32).  Where K ends inside a slice (an odd
    // number of K-blocks) the last slice's second K-block has zero codes but its scale bytes
    // belong to other data, where a NaN would leak into the sums: that K-block takes the
    // first one's scale (1 = 0 there), so its products stay zero unless the row's own last
    // scale is NaN.
    const bool hi = lane >= 32;
    const int lrow_a = (wm + (lane & 31)) * 16, lrow_b = GBM * 16 + (wn + (lane & 31)) * 16;
    const int last_odd = (OFFR && (kbl & 1)) ? nk32 - 1 : -1;
    auto rec_ptrs = [&](int c3, int q, int64_t k) {
        const uint8_t* cur = L::rbuf(lds, c3);
        const uint8_t* nxt = L::rbuf(lds, c3 == 2 ? 0 : c3 + 1);
        auto at = [&](int t) { return t < 16 ? cur + t : nxt + (t - 16); };
        const int ta = pl.dla + 2 * q, tb = pl.dlb + 2 * q, up = (int)k == last_odd ? 0 : 1;
        MxSPtr sp;
        sp.a = (hi ? at(ta + up) : at(ta)) + lrow_a;
        sp.b = (hi ? at(tb + up) : at(tb)) + lrow_b;
        return sp;
    };
    int g3 = 0;   // offset records: the current group's index mod 3

    mx_prologue<MODE, SL>(pl, lds);
    wait_vm_barrier<2 * (DC + DS)>();
    MxFrag f0, f1;
    MxSPtr sp0{nullptr, nullptr};
    if constexpr (OFFR) sp0 = rec_ptrs(0, 0, 0);
    mx_read<MODE>(L::buf(lds, 0), L::sbuf(lds, 0), 0, sp0, wm, wn, lane, f0);

    // One slice.  Grouped records: Q = kt mod MX_GROUP (the loop is unrolled by MX_GROUP).
    // Offset records: the slice's place in its group is a run-time value, so that one loop
    // takes any number of slices; only scalar work depends on it.
    auto slice = [&](int64_t kt, auto q_c, const MxFrag& fc, MxFrag& fn) {
        constexpr int Q = decltype(q_c)::value;
        [[maybe_unused]] const int qr = (int)(kt & (MX_GROUP - 1));   // offset records
        [[maybe_unused]] const int g3n = g3 == 2 ? 0 : g3 + 1;
        if constexpr (OFFR) {
            if (qr == 2) wait_vm_barrier<DC + DG>();   // slice kt-1 also issued a record
            else wait_vm_barrier<DC>();
        } else if constexpr (REC && Q == 2) {
            wait_vm_barrier<DC + DG>();
        } else {
            wait_vm_barrier<DC + DS>();
        }
        const int64_t kd = kt + 3;
        const bool live = (int)kd < nk32;
        uint8_t* db = L::buf(lds, kd);
        const int64_t kn = kt + 1;                   // fragments read for the next slice
        const uint8_t* nb = L::buf(lds, kn);
        const uint8_t* ns = L::sbuf(lds, kn / MX_GROUP);
        const int qn = REC ? (Q + 1) % MX_GROUP : 0;
        MxSPtr spn{nullptr, nullptr};
        if constexpr (OFFR) spn = rec_ptrs(qr == MX_GROUP - 1 ? g3n : g3, (qr + 1) & (MX_GROUP - 1), kn);
        static_for<0, 4>([&](auto p_c) {
            constexpr int P = decltype(p_c)::value;
            mx_dma_part<MODE, SL, P>(d, kd, live, db);
            if constexpr (!REC && P < 2) mx_dma_slots<P>(d, kd * 64, live, db);
            if constexpr (ALIGNED && Q == 1 && P == 0) {
                const int grp = (int)(kt / MX_GROUP) + 1;
                nv4_dma_group<4>(d, (uint32_t)grp, grp * MX_GROUP < nk32, L::sbuf(lds, grp));
            }
            if constexpr (OFFR && P == 0) {
                if (qr == 1) {
                    const int j = (int)(kt / MX_GROUP) + 2;
                    mx_dma_offrec(d, pl.offa, pl.offb, (uint32_t)j, 16 * j < 15 + kbl, L::rbuf(lds, g3 == 0 ? 2 : g3 - 1));
                }
            }
            mx_mfma_row<P>(fc, acc);
            // the reads after the last slice touch a stale (in-bounds) buffer and go unused
            mx_read_part<P, MODE>(nb, ns, qn, spn, wm, wn, lane, fn);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (OFFR) g3 = qr == MX_GROUP - 1 ? g3n : g3;
    };
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    using Q3 = std::integral_constant<int, 3>;
    using Q4 = std::integral_constant<int, 4>;
    using Q5 = std::integral_constant<int, 5>;
    using Q6 = std::integral_constant<int, 6>;
    using Q7 = std::integral_constant<int, 7>;
    if constexpr (ALIGNED) {
        // nk is a multiple of MX_GROUP
        for (int64_t kt = 0; kt < nk; kt += MX_GROUP) {
            slice(kt + 0, Q0{}, f0, f1);
            slice(kt + 1, Q1{}, f1, f0);
            slice(kt + 2, Q2{}, f0, f1);
            slice(kt + 3, Q3{}, f1, f0);
            slice(kt + 4, Q4{}, f0, f1);
            slice(kt + 5, Q5{}, f1, f0);
            slice(kt + 6, Q6{}, f0, f1);
            slice(kt + 7, Q7{}, f1, f0);
        }
    } else {
        for (int64_t kt = 0; kt < nk; kt += 2) {
            slice(kt, Q0{}, f0, f1);
            if (kt + 1 < nk) slice(kt + 1, Q0{}, f1, f0);
        }
    }
    wait_vm<0>();   // no DMA may still write this workgroup's LDS when the wave ends
}

// ---------------------------------------------------------------- NVFP4 with LDS DMA

// K a multiple of 256.  Same LDS organisation as the grouped MXFP8 path: 4 code stages of 64
// bytes per row (128 elements), filled by DMA three slices ahead, and double-buffered 16-byte
// scale records, each holding the 16 E4M3 scales of two slices of a row.  4 waves of 128 x 128
// (TN = 4: 4 x 4 MFMA tiles, so each dequantized word feeds 4 MFMAs).  Each wave dequantizes,
// between the MFMAs of step s, the operands of step s+1.  The loop is bound by VALU issue:
// each VALU instruction between two 32-clock MFMAs of a wave adds about one clock (measured),
// and dequantization costs 4 per MFMA (2 conversions, 2 scale multiplies) plus scales.  An
// 8-wave layout of 128 x 64 per wave (TN = 2, two waves per SIMD) needs 6 per MFMA and
// measured slower; the DMA helpers here serve the 4-wave layout only.
constexpr int NV4_CODES = 2 * GBM * ROWB;   // 32 KiB per stage
constexpr int NV4_SREC = 2 * GBM * 16;      // 8 KiB per scale group (2 slices)
static_assert(4 * NV4_CODES + 2 * NV4_SREC <= Fmt<2>::LDS, "NVFP4 DMA LDS");

template <int TN>
struct NvWordsT {
    uint32_t a[4], b[TN];
};
template <int TN>
struct NvOpsT {
    half8_t a[4], b[TN];
};

// Step S (0..7) of a slice: lane (row, kh) holds the 8 codes of K elements 64kh + 8S .. +8,
// dword S % 4 of chunk 2kh + S / 4 of its row (block 4kh + S / 2 of the slice).
// Half H (0/1) of a slice: lane (row, kh) reads chunk 2kh + H of its row with one 16-byte LDS
// read -- the code words of steps 4H .. 4H+3 (dword S % 4 for step S).
template <int TN>
struct NvQuadT {
    uint4 a[4], b[TN];
};

template <int H, int TN>
__device__ __forceinline__ void nvw_read_quad(const uint8_t* buf, int wm, int wn, int frow, int kh, NvQuadT<TN>& q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q.a[i] = *(const uint4*)(buf + swzd(wm + 32 * i + frow, 2 * kh + H));
#pragma unroll
    for (int j = 0; j < TN; ++j) q.b[j] = *(const uint4*)(buf + GBM * ROWB + swzd(wn + 32 * j + frow, 2 * kh + H));
}

template <int D>
__device__ __forceinline__ uint32_t dword_of(const uint4& v) {
    if constexpr (D == 0) return v.x;
    else if constexpr (D == 1) return v.y;
    else if constexpr (D == 2) return v.z;
    else return v.w;
}

template <int S, int TN>
__device__ __forceinline__ void nvw_words_of(const NvQuadT<TN>& q, NvWordsT<TN>& w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w.a[i] = dword_of<S & 3>(q.a[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) w.b[j] = dword_of<S & 3>(q.b[j]);
}

// The 16-byte scale records (two slices' bytes) of the wave's fragment rows of a group, one
// 16-byte read per fragment: 16 lanes read 256 consecutive bytes, which no two of them share
// a bank in (4-byte reads of one dword of 32 consecutive records put rows r and r + 16 on the
// same bank: those reads made up nearly all of the kernel's LDS bank-conflict cycles).
template <int TN>
struct NvRecT {
    uint4 a[4], b[TN];
};

template <int TN>
__device__ __forceinline__ void nvw_read_recs(const uint8_t* sbuf, int wm, int wn, int frow, NvRecT<TN>& r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a[i] = *(const uint4*)(sbuf + (wm + 32 * i + frow) * 16);
#pragma unroll
    for (int j = 0; j < TN; ++j) r.b[j] = *(const uint4*)(sbuf + GBM * 16 + (wn + 32 * j + frow) * 16);
}

// The lane's 4 scale bytes (blocks 4kh .. 4kh+3) of slice Q (0/1) of the records: dword 2Q + kh.
template <int Q, int TN>
__device__ __forceinline__ void nvw_pick_scales(const NvRecT<TN>& r, int kh, uint32_t (&sa)[4], uint32_t (&sb)[TN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = kh ? dword_of<2 * Q + 1>(r.a[i]) : dword_of<2 * Q>(r.a[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] = kh ? dword_of<2 * Q + 1>(r.b[j]) : dword_of<2 * Q>(r.b[j]);
}

template <int S, int TN>
__device__ __forceinline__ void nvw_ops(const NvWordsT<TN>& w, const uint32_t (&sa)[4], const uint32_t (&sb)[TN],
                                        NvOpsT<TN>& o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o.a[i] = nv_dequant(w.a[i], nv_scale(sa[i], S >> 1));
#pragma unroll
    for (int j = 0; j < TN; ++j) o.b[j] = nv_dequant(w.b[j], nv_scale(sb[j], S >> 1));
}

// The B fragment is the MFMA's first operand and the A fragment its second, so each 32 x 32
// accumulator tile holds C^T: lane (frow, kh) has, in acc[i][j][r], row 32i + frow and column
// 32j + 8(r >> 2) + 4kh + (r & 3) of the wave's block -- four consecutive columns of one row
// per group of 4 registers, which the epilogue packs into one 8-byte (bf16) or 16-byte (fp32)
// LDS store instead of transposing single elements.
template <int TN>
__device__ __forceinline__ void nvw_mfma(const NvOpsT<TN>& o, floatx16 (&acc)[4][TN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.b[j], o.a[i], acc[i][j], 0, 0, 0);
}

// The first step of a tile: the accumulators start from zero (no separate clearing, so that a
// tile's accumulators are not live across the previous tile's epilogue).
template <int TN>
__device__ __forceinline__ void nvw_mfma_first(const NvOpsT<TN>& o, floatx16 (&acc)[4][TN]) {
    const floatx16 z = {};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.b[j], o.a[i], z, 0, 0, 0);
}

// One step (after its LDS reads, which a scheduling barrier keeps at the top of the step):
// each MFMA followed by an equal share of the dequantization of the next step, whose words
// were read a step earlier.
template <int TN>
__device__ __forceinline__ void nvw_interleave() {
    constexpr int NM = 4 * TN;                                  // MFMAs per step
    constexpr int NV = ((4 + TN) * 8 + 2 * (4 + TN) + NM - 2) / (NM - 1);   // VALU per MFMA gap
#pragma unroll
    for (int i = 0; i < NM - 1; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// Main loop.  Slice kt: wait for this wave's DMAs of slice kt+1 (everything issued before the
// DMAs of slice kt-1), barrier, then 8 MFMA steps; the code DMAs of slice kt+3 are spread over
// the steps and, in odd slices, the scale group (kt+3)/2 (slices kt+3, kt+4) is fetched at
// step 1 -- its buffer held group (kt-1)/2, whose last scales were read during slice kt-1.
// Operand pipeline: each fragment's code words come in two 16-byte halves per slice (steps
// 0-3 and 4-7): the second half of slice kt is read at step 2, the first half of slice kt+1 at
// step 6 (slice kt+1 is complete since the barrier at the top of slice kt), and its scales at
// step 5; during step s the operands of step s+1 are dequantized.  An odd slice issues DG more DMAs than an even one, so the wait
// at the top of an even slice allows DC + DG in flight; the prologue ends with an out-of-range
// group DMA so that slice 0 fits the rule.  An out-of-range DMA lane still writes (zeros) to
// LDS: every such DMA here targets a buffer whose contents are no longer, or not yet, needed.
// NW waves share the DMAs of a 256 x 256 tile (NW = 16 / TN: the waves cover it); with NW = 4
// and TN = 2 the 4 waves cover 256 x 128 (a half tile, brows = 128).
template <int TN, int NW = 16 / TN>
__device__ __forceinline__ void nvw_main_loop(const GemmArgs& g, int64_t m0, int64_t n0, int64_t nk, uint8_t* lds,
                                              int wm, int wn, int lane, floatx16 (&acc)[4][TN], int64_t brows = GBN) {
    constexpr int PARTS = 16 / NW;        // code DMA parts per slice (4 or 2)
    constexpr int DC = 2 * PARTS;         // code DMAs per lane per slice
    constexpr int DG = NW == 4 ? 2 : 1;   // group DMAs per lane
    constexpr int PSTEP = 8 / PARTS;      // steps between code DMA parts
    if (nk <= 0) return;
    const MxDma d = make_dma<2, 16>(g, m0, n0, lane, brows);
    const int frow = lane & 31, kh = lane >> 5;
    auto buf = [&](int64_t k) { return lds + (int)(k & 3) * NV4_CODES; };
    auto sbuf = [&](int64_t grp) { return lds + 4 * NV4_CODES + (int)(grp & 1) * NV4_SREC; };
    const int nk32 = (int)nk;   // nk <= 2^17 (K <= 2^24)
    auto dma_slice = [&](int k) {
        const bool live = k < nk32;
        static_for<0, PARTS>([&](auto p_c) { nv4_dma_codes<decltype(p_c)::value, NW>(d, 64u * k, live, buf(k)); });
    };
    nv4_dma_group<NW>(d, 0, true, sbuf(0));
    nv4_dma_group<NW>(d, 1, 2 < nk32, sbuf(1));
    dma_slice(0);
    dma_slice(1);
    dma_slice(2);
    // out of range: no memory traffic, but the DMA still writes its zeros -- into code stage 3,
    // which is free until slice 3's DMA (issued after it) refills it
    nv4_dma_group<NW>(d, 0, false, buf(3));
    wait_vm_barrier<2 * DC + DG>();

    // q0: code words of steps 0-3 of the current slice (from step 6 on: of the next slice);
    // q1: steps 4-7 of the current slice, read at step 2
    NvQuadT<TN> q0, q1;
    NvWordsT<TN> w;
    NvOpsT<TN> cur, nxt;
    NvRecT<TN> rec;
    uint32_t sa[4], sb[TN], san[4], sbn[TN];
    nvw_read_recs<TN>(sbuf(0), wm, wn, frow, rec);
    nvw_pick_scales<0, TN>(rec, kh, sa, sb);
    nvw_read_quad<0, TN>(buf(0), wm, wn, frow, kh, q0);
    nvw_words_of<0, TN>(q0, w);
    nvw_ops<0, TN>(w, sa, sb, cur);

    auto slice = [&](int kt, auto odd_c) {
        constexpr bool ODD = decltype(odd_c)::value;
        if constexpr (ODD) wait_vm_barrier<DC>();
        else wait_vm_barrier<DC + DG>();
        const int kd = kt + 3;
        const bool live = kd < nk32;
        uint8_t* db = buf(kd);
        const uint8_t* cb = buf(kt);
        const uint8_t* nb = buf(kt + 1);
        static_for<0, 8>([&](auto s_c) {
            constexpr int S = decltype(s_c)::value;
            if constexpr (S % PSTEP == 0) nv4_dma_codes<S / PSTEP, NW>(d, 64u * kd, live, db);
            if constexpr (ODD && S == 1) {
                const int grp = (kt + 3) / 2;
                nv4_dma_group<NW>(d, grp, 2 * grp < nk32, sbuf(grp));
            }
            // second half of this slice at step 2 (q1 was last read at step 6 of the previous
            // slice), first half of the next slice at step 6 (q0 was last read at step 2; the
            // read after the last slice touches a stale, in-bounds buffer)
            if constexpr (S == 2) nvw_read_quad<1, TN>(cb, wm, wn, frow, kh, q1);
            if constexpr (S == 6) nvw_read_quad<0, TN>(nb, wm, wn, frow, kh, q0);
            // an odd slice reads the records of the next group (its own slice's scales are picked)
            if constexpr (ODD && S == 5) nvw_read_recs<TN>(sbuf((kt + 1) / 2), wm, wn, frow, rec);
            __builtin_amdgcn_sched_barrier(0);
            // dequantize step S+1
            if constexpr (S + 1 < 4) nvw_words_of<S + 1, TN>(q0, w);
            else if constexpr (S + 1 < 8) nvw_words_of<S + 1, TN>(q1, w);
            else nvw_words_of<0, TN>(q0, w);
            if constexpr (S + 1 < 8) nvw_ops<S + 1, TN>(w, sa, sb, nxt);
            else {
                nvw_pick_scales<ODD ? 0 : 1, TN>(rec, kh, san, sbn);
                nvw_ops<0, TN>(w, san, sbn, nxt);
            }
            nvw_mfma<TN>(cur, acc);
            nvw_interleave<TN>();
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
        });
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = san[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) sb[j] = sbn[j];
    };
    // nk is even
    for (int kt = 0; kt < nk32; kt += 2) {
        slice(kt, std::false_type{});
        slice(kt + 1, std::true_type{});
    }
    wait_vm<0>();   // no DMA may still write this workgroup's LDS when the wave ends
}

// ---------------------------------------------------------------- NVFP4 with per-slice scale DMAs

// Any K that is a multiple of 32 (the C ABI's rule), and K-grouped operands whose groups start
// at any multiple of 32: the LDS organisation and operand pipeline of nvw_main_loop, with the
// scales fetched per slice instead of as 16-byte records (which need scale rows 16 bytes
// apart).  A row's 8 scale bytes of a slice start 0 or 2 bytes into an aligned dword (scale
// rows lie an even number of bytes apart), so each comes as the 3 aligned dwords that cover
// it, by dword LDS DMA, into a 12-byte record in the slice's stage; the lane that needs 4 of
// the bytes (blocks 4kh .. 4kh+3) reads two dwords of the record and shifts.  Stage: A codes
// [256][64 B], B codes [256][64 B] (as in nvw_main_loop), A records [256][12 B], B records
// [256][12 B] = 38 KiB.  Per slice each lane issues 8 code DMAs and 6 record DMAs, the same in
// every slice, so every wait allows the previous slice's 14 in flight.  The records' offsets
// go into the vector offset (the scalar offset escapes the buffer range check), so a dword
// past a tile's last scale byte reads as zero.  In a slice that K ends inside (K % 128 != 0)
// the code DMAs check each 16-byte chunk (K % 32 == 0: a chunk lies entirely inside or
// outside K) and the scale bytes past K are cleared, so that nothing beyond the operands' K
// reaches the sums.
constexpr int NVS_REC = 12;
constexpr int NVS_STAGE = NV4_CODES + 2 * GBM * NVS_REC;   // 38 KiB
constexpr int NVS_DS = 6;                                  // record DMAs per lane per slice
static_assert(4 * NVS_STAGE <= Fmt<3>::LDS, "NVFP4 per-slice scale LDS");
static_assert(NVS_DS * 64 * 4 == 2 * GBM * 3, "the records of a slice: 4 waves x 6 DMAs of 64 dwords");

__device__ __forceinline__ void dma_b32(const u32x4s& rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "m0");
}

// Code DMAs of part P of the slice whose first code byte per row is b0; in the slice that K
// ends inside (tail, uniform) every lane checks its chunk and carries the whole offset in the
// vector offset, so that the range check sees it.
template <int P>
__device__ __forceinline__ void nvs_dma_codes(const MxDma& d, uint32_t b0, bool live, bool tail, uint8_t* buf) {
    const int r0 = 64 * P + 16 * d.wave;
    const int r = r0 + (d.lane >> 2), c = swzd_chunk(r, d.lane & 3);
    uint32_t off = (uint32_t)r * d.rowbytes + 16u * c;
    uint32_t soff = live ? b0 : 0u;
    if (tail) {
        off = b0 + 16u * c < d.kbytes ? off + b0 : OOB;
        soff = 0u;
    }
    dma_b128(sized(d.o.a, live), lds_addr(buf + r0 * ROWB), off, soff);
    dma_b128(sized(d.o.b, live), lds_addr(buf + GBM * ROWB + r0 * ROWB), off, soff);
}

// Record DMAs I0 .. I1-1 (of 6) of the slice whose scale bytes start 8k into each row: DMA i
// of wave w fills dword slots 64 (w + 4i) .. +64 of the slice's records (A's 768, then B's).
template <int I0, int I1>
__device__ __forceinline__ void nvs_dma_recs(const u32x4s& rsa, const u32x4s& rsb, const uint32_t (&so)[NVS_DS],
                                             uint32_t k8, bool live, uint8_t* rec, int wave) {
#pragma unroll
    for (int i = I0; i < I1; ++i) {
        const u32x4s& rs = i >= 3 ? rsb : rsa;   // slot groups w + 4i >= 12 belong to B
        dma_b32(sized(rs, live), lds_addr(rec + 256 * (wave + 4 * i)), so[i] + k8, 0u);
    }
}

// The lane's 4 scale bytes (blocks 4kh .. 4kh+3) of each of its fragments from a slice's
// records: two dwords at the record's dword oq (0 or 1), shifted right by sh bits (0 or 16,
// or 8 / 24 for a scale tensor that is not even-aligned), then masked (the bytes past K).
template <int TN>
__device__ __forceinline__ void nvs_read_scales(const uint8_t* rec, int wm, int wn, int frow, uint32_t oqa,
                                                uint32_t sha, uint32_t oqb, uint32_t shb, uint32_t mask,
                                                uint32_t (&sa)[4], uint32_t (&sb)[TN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t* p = (const uint32_t*)(rec + (wm + 32 * i + frow) * NVS_REC) + oqa;
        sa[i] = __builtin_amdgcn_alignbit(p[1], p[0], sha) & mask;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const uint32_t* p = (const uint32_t*)(rec + GBM * NVS_REC + (wn + 32 * j + frow) * NVS_REC) + oqb;
        sb[j] = __builtin_amdgcn_alignbit(p[1], p[0], shb) & mask;
    }
}

template <int TN>
__device__ __forceinline__ void nvs_main_loop(const GemmArgs& g, int64_t m0, int64_t n0, int64_t nk, uint8_t* lds,
                                              int wm, int wn, int lane, floatx16 (&acc)[4][TN]) {
    constexpr int NW = 4, DC = 8, PSTEP = 2;
    static_assert(16 / TN == NW, "4 waves of 128 x 128");
    if (nk <= 0) return;
    const MxDma d = make_dma<2, 16>(g, m0, n0, lane);
    const int frow = lane & 31, kh = lane >> 5;
    auto buf = [&](int k) { return lds + (k & 3) * NVS_STAGE; };
    auto rec = [&](int k) { return buf(k) + NV4_CODES; };
    const int nk32 = (int)nk;   // nk <= 2^20 (host check)
    const uint32_t kscale = d.kblocks;                           // scale bytes of a row's K
    const bool ktail = (d.kbytes & 63u) != 0;                    // K % 128 != 0
    const uint32_t tail_blocks = (kscale & 7u) ? (kscale & 7u) : 8u;   // valid blocks of the last slice
    // Record resources: from the aligned dword at or below the tile's first scale byte to its
    // last row's K scale bytes, rounded up to whole dwords (rows past the tile read as zero).
    const int64_t sbs = g.ld / 16;
    const int64_t ra = tile_rows(g.M - m0, GBM), rbn = tile_rows(g.N - n0, GBN);
    const uint8_t* pa = g.a_scales + m0 * sbs;
    const uint8_t* pb = g.b_scales + n0 * sbs;
    const uint32_t dla = (uint32_t)((uintptr_t)pa & 3), dlb = (uint32_t)((uintptr_t)pb & 3);
    const u32x4s rsa = rsrc_words(pa - dla, (dla + (ra - 1) * sbs + kscale + 3) & ~(int64_t)3);
    const u32x4s rsb = rsrc_words(pb - dlb, (dlb + (rbn - 1) * sbs + kscale + 3) & ~(int64_t)3);
    uint32_t so[NVS_DS];   // the lane's record DMA offsets for slice 0
#pragma unroll
    for (int i = 0; i < NVS_DS; ++i) {
        const bool opb = i >= 3;
        const int s = 64 * (d.wave + 4 * i - (opb ? 12 : 0)) + lane, r = s / 3, dw = s - 3 * r;
        const int64_t rows = opb ? rbn : ra;
        const uint32_t dl = opb ? dlb : dla;
        so[i] = r < rows ? (uint32_t)((dl + (uint64_t)r * (uint64_t)sbs) & ~(uint64_t)3) + 4u * dw : OOB;
    }
    // where the lane's 4 bytes start in a record: row R's bytes start ((dl + R sbs) mod 4) into
    // it, and R sbs mod 4 depends only on R's parity (sbs is even), which is frow's
    const uint32_t par = (uint32_t)(frow & 1) * ((uint32_t)sbs & 2u);
    const uint32_t oa = ((dla + par) & 3u) + 4u * kh, ob = ((dlb + par) & 3u) + 4u * kh;
    const uint32_t oqa = oa >> 2, sha = 8u * (oa & 3u), oqb = ob >> 2, shb = 8u * (ob & 3u);
    // scale bytes of the last slice past K read as zero blocks
    const int vb = (int)tail_blocks - 4 * kh;   // valid bytes of the lane's 4 in the last slice
    const uint32_t tmask = vb >= 4 ? ~0u : (vb <= 0 ? 0u : (1u << (8 * vb)) - 1u);
    auto mask_of = [&](int k) { return k == nk32 - 1 ? tmask : ~0u; };

    auto dma_slice = [&](int k) {
        const bool live = k < nk32, tail = ktail && k == nk32 - 1;
        static_for<0, 4>([&](auto p_c) { nvs_dma_codes<decltype(p_c)::value>(d, 64u * k, live, tail, buf(k)); });
        nvs_dma_recs<0, NVS_DS>(rsa, rsb, so, 8u * k, live, rec(k), d.wave);
    };
    dma_slice(0);
    dma_slice(1);
    dma_slice(2);
    wait_vm_barrier<2 * (DC + NVS_DS)>();

    NvQuadT<TN> q0, q1;
    NvWordsT<TN> w;
    NvOpsT<TN> cur, nxt;
    uint32_t sa[4], sb[TN], san[4], sbn[TN];
    nvs_read_scales<TN>(rec(0), wm, wn, frow, oqa, sha, oqb, shb, mask_of(0), sa, sb);
    nvw_read_quad<0, TN>(buf(0), wm, wn, frow, kh, q0);
    nvw_words_of<0, TN>(q0, w);
    nvw_ops<0, TN>(w, sa, sb, cur);

    // Slice kt: the DMAs of slice kt+3 spread over the steps (codes at steps 0, 2, 4, 6,
    // records at steps 1 and 3), the operand reads as in nvw_main_loop (second half of this
    // slice at step 2, the next slice's scales at step 5 and first half at step 6).
    for (int kt = 0; kt < nk32; ++kt) {
        wait_vm_barrier<DC + NVS_DS>();
        const int kd = kt + 3;
        const bool live = kd < nk32, tail = ktail && kd == nk32 - 1;
        uint8_t* db = buf(kd);
        uint8_t* dr = rec(kd);
        const uint8_t* cb = buf(kt);
        const uint8_t* nb = buf(kt + 1);
        const uint8_t* nr = rec(kt + 1);
        const uint32_t nmask = mask_of(kt + 1);
        static_for<0, 8>([&](auto s_c) {
            constexpr int S = decltype(s_c)::value;
            if constexpr (S % PSTEP == 0) nvs_dma_codes<S / PSTEP>(d, 64u * kd, live, tail, db);
            if constexpr (S == 1) nvs_dma_recs<0, 3>(rsa, rsb, so, 8u * kd, live, dr, d.wave);
            if constexpr (S == 3) nvs_dma_recs<3, 6>(rsa, rsb, so, 8u * kd, live, dr, d.wave);
            if constexpr (S == 2) nvw_read_quad<1, TN>(cb, wm, wn, frow, kh, q1);
            if constexpr (S == 6) nvw_read_quad<0, TN>(nb, wm, wn, frow, kh, q0);
            if constexpr (S == 5) nvs_read_scales<TN>(nr, wm, wn, frow, oqa, sha, oqb, shb, nmask, san, sbn);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (S + 1 < 4) nvw_words_of<S + 1, TN>(q0, w);
            else if constexpr (S + 1 < 8) nvw_words_of<S + 1, TN>(q1, w);
            else nvw_words_of<0, TN>(q0, w);
            if constexpr (S + 1 < 8) nvw_ops<S + 1, TN>(w, sa, sb, nxt);
            else nvw_ops<0, TN>(w, san, sbn, nxt);
            nvw_mfma<TN>(cur, acc);
            nvw_interleave<TN>();
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
        });
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = san[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) sb[j] = sbn[j];
    }
    wait_vm<0>();   // no DMA may still write this workgroup's LDS when the wave ends
}

// ---------------------------------------------------------------- epilogue

// Epilogue of a tile whose columns lie inside C (4 waves of 128 x 128); rows from m_end on
// (the tile's last rows past M, e.g. the end of an M-group) are not stored.  The accumulators
// hold C^T tiles (see nvw_mfma and mx_mfma_row), so each group of 4 registers is 4 consecutive
// columns of one row.  Each wave stages its block in its own LDS region, row-major with rows
// padded by 16 bytes, one 8-byte (bf16, two packed conversions) or 16-byte (fp32) store per
// group, and reads it back as 16-byte row chunks for fully coalesced 16-byte global stores.
// bf16 output takes all 128 rows in one pass (34 KiB per wave); fp32 output two passes of 64
// rows.  A wave reads back only what it wrote, and the LDS executes one wave's instructions in
// order, so no barrier is needed between the two.  SCALED (NVFP4) with fa == nullptr: every
// output is scaled by the uniform alpha (per-tensor scales on both operands); otherwise the
// lane reads its row and column factors from the tables once, before staging.
template <bool OUT_F32, bool SCALED>
__device__ __forceinline__ void store_tile_lds(const GemmArgs& g, uint8_t* lds, int64_t m0, int64_t n0, int wm,
                                               int wn, int wave, int lane, const float* fa, const float* fb,
                                               float alpha, int64_t m_end, floatx16 (&acc)[4][4]) {
    constexpr int ES = OUT_F32 ? 4 : 2;          // bytes per element
    constexpr int ROWS = OUT_F32 ? 64 : 128;     // rows per pass
    constexpr int RS = 128 * ES + 16;            // LDS row stride
    constexpr int CPR = 128 * ES / 16;           // 16-byte chunks per row
    static_assert(4 * ROWS * RS <= Fmt<2>::LDS && Fmt<2>::LDS <= Fmt<1>::LDS, "epilogue staging");
    uint8_t* reg = lds + wave * ROWS * RS;
    const int frow = lane & 31, kh = lane >> 5;
    uint8_t* cbase = (uint8_t*)g.c + ((m0 + wm) * g.N + n0 + wn) * ES;
    const bool tables = SCALED && fa != nullptr;   // uniform
    float frv[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    float4 fcv[4][4];
    if constexpr (SCALED) {
        if (tables) {
#pragma unroll
            for (int i = 0; i < 4; ++i) frv[i] = fa[wm + 32 * i + frow];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) fcv[j][q] = *(const float4*)(fb + wn + 32 * j + 8 * q + 4 * kh);
        }
    }
    static_for<0, 128 / ROWS>([&](auto h_c) {
        constexpr int H = decltype(h_c)::value;
        constexpr int I0 = H * ROWS / 32;
        static_for<0, ROWS / 32>([&](auto i_c) {
            constexpr int IL = decltype(i_c)::value;
            constexpr int I = I0 + IL;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float4 v = make_float4(acc[I][j][4 * q], acc[I][j][4 * q + 1], acc[I][j][4 * q + 2],
                                           acc[I][j][4 * q + 3]);
                    if constexpr (SCALED) {
                        if (tables) {
                            const float fr = frv[I];
                            const float4 fc = fcv[j][q];
                            v.x *= fr * fc.x; v.y *= fr * fc.y; v.z *= fr * fc.z; v.w *= fr * fc.w;
                        } else {
                            v.x *= alpha; v.y *= alpha; v.z *= alpha; v.w *= alpha;
                        }
                    }
                    // row 32 IL + frow of this pass, columns col .. col + 3 of the block
                    const int row = 32 * IL + frow, col = 32 * j + 8 * q + 4 * kh;
                    if constexpr (OUT_F32) *(float4*)(reg + row * RS + col * 4) = v;
                    else *(uint2*)(reg + row * RS + col * 2) = make_uint2(bf16x2_rne(v.x, v.y), bf16x2_rne(v.z, v.w));
                }
            }
        });
        asm volatile("" ::: "memory");
#pragma unroll
        for (int p = 0; p < ROWS * CPR / 64; ++p) {
            const int q = 64 * p + lane, row = q / CPR, c16 = q % CPR;
            const uint4 v = *(const uint4*)(reg + row * RS + c16 * 16);
            if (wm + H * ROWS + row < m_end) *(uint4*)(cbase + (int64_t)(H * ROWS + row) * g.N * ES + c16 * 16) = v;
        }
        asm volatile("" ::: "memory");
    });
}

// Per-tile output factors, alpha(m, n) = fa[m - m0] * fb[n - n0], written to LDS (two
// float[256] tables after the epilogue's staging regions) by the whole workgroup.
//   per-tensor scales:         fa = 1 / (S_a S_b), fb = 1
//   A per row, B per tensor:   fa[m] = 1 / (S_a[m] S_b), fb = 1
//   A per tensor, B per row:   fa = 1, fb[n] = 1 / (S_a S_b[n])
//   both per row:              fa[m] = 1 / S_a[m], fb[n] = 1 / S_b[n]
// Each factor is the binary64 quotient rounded once to fp32, so with at most one row-scaled
// operand alpha is exactly what the per-tensor formula gives; with two it is the fp32 product
// of two such reciprocals.  MXFP8: fa = fb = 1.  Rows and columns past M and N are not
// read (their factors are never used).
constexpr int FACT_BYTES = 2 * 256 * 4;

template <int FMT>
__device__ __forceinline__ void tile_factors(const GemmArgs& g, int64_t m0, int64_t n0, float* fa, float* fb) {
    using F = Fmt<FMT>;
    for (int i = threadIdx.x; i < 512; i += F::THREADS) {
        float f = 1.0f;
        if constexpr (F::NV) {
            const int t = i & 255;
            if (i < 256) {
                const int64_t m = m0 + t;
                if (m < g.M) {
                    const double sa = g.a_rows ? (double)g.a_s_enc[m] : (double)g.a_s_enc[0];
                    if (g.a_rows) f = (float)(1.0 / (g.b_rows ? sa : sa * (double)g.b_s_enc[0]));
                    else if (!g.b_rows) f = (float)(1.0 / (sa * (double)g.b_s_enc[0]));
                }
            } else {
                const int64_t n = n0 + t;
                if (n < g.N && g.b_rows) {
                    const double sb = (double)g.b_s_enc[n];
                    f = (float)(1.0 / (g.a_rows ? sb : sb * (double)g.a_s_enc[0]));
                }
            }
        }
        (i < 256 ? fa : fb)[i & 255] = f;
    }
}

// Output tile of this workgroup.  Workgroup ids are dealt to the 8 XCDs round-robin; the
// id is remapped so that XCD x receives the contiguous tile range [x*T/8, (x+1)*T/8),
// walked in bands of GROUP tile-rows (column-major inside a band) for L2 reuse.
__device__ __forceinline__ void tile_of(int64_t nbm, int64_t nbn, int64_t id, int64_t& tm, int64_t& tn) {
    const int64_t T = nbm * nbn;
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

// tile_of in 32-bit arithmetic, for launches with fewer than 2^31 tiles (the persistent kernel
// computes an origin per tile; the 64-bit divisions took ~0.8 us of each tile there).
__device__ __forceinline__ void tile_of32(uint32_t nbm, uint32_t nbn, uint32_t id, uint32_t& tm, uint32_t& tn) {
    const uint32_t T = nbm * nbn;
    const uint32_t T8 = T & ~7u;
    if (id < T8) id = (id & 7u) * (T8 >> 3) + (id >> 3);
    constexpr uint32_t GROUP = 8;
    const uint32_t band = id / (GROUP * nbn);
    const uint32_t first = band * GROUP;
    const uint32_t rows = (nbm - first) < GROUP ? (nbm - first) : GROUP;
    const uint32_t in = id - band * GROUP * nbn;
    tm = first + in % rows;
    tn = in / rows;
}

// ---------------------------------------------------------------- grouped launches
//
// A grouped launch runs one GEMM per group g, the groups given by boundaries offs[g] ..
// offs[g+1] on the device (clamped to [0, extent]):
//   M-grouped (the per-expert GEMMs of a mixture-of-experts layer, fprop and dgrad): the
//     group's rows of A [extent][K] and of C [extent][N], against B_g [N][K], the g-th of
//     the stacked B [groups][N][K];
//   K-grouped (wgrad): C_g [M][N], the g-th of the stacked C [groups][M][N], contracts
//     columns offs[g] .. offs[g+1] of A [M][extent] and B [N][extent] (rows of length
//     extent); the boundaries must be multiples of 32 (a group whose are not is computed as
//     empty, C_g = 0).
// Workgroups are dealt to the groups in order, each group taking a multiple of 8 of them so
// that its tiles see the same XCD phase as a plain launch; a workgroup past its group's tiles
// exits at once.  Everything a group needs -- its operand and output bases, its tensor scales
// and its extent -- is folded into the GemmArgs, and the tile code runs unchanged.
struct GroupArgs {
    const int64_t* offs;   // groups + 1 boundaries (device)
    int64_t groups;
    int64_t extent;        // rows of A and C (M-grouped) or K (K-grouped)
};

__device__ __forceinline__ void group_bounds(const GroupArgs& q, int64_t grp, int64_t& o0, int64_t& o1) {
    int64_t a = q.offs[grp], b = q.offs[grp + 1];
    a = a < 0 ? 0 : (a > q.extent ? q.extent : a);
    b = b < a ? a : (b > q.extent ? q.extent : b);
    o0 = a;
    o1 = b;
}

__device__ __forceinline__ int64_t shfl64(int64_t v, int src) {
    const int lo = __shfl((int)(uint32_t)v, src), hi = __shfl((int)(uint32_t)((uint64_t)v >> 32), src);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// A wave-uniform 64-bit value moved to scalar registers (buffer resources built from it must
// be scalar).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// M-grouped: the group of workgroup bid and its index within the group's share (each wave
// scans the boundaries itself, 64 groups at a time, with a wave prefix sum of the shares).
// The loop runs to the end with a uniform trip count and the results pass through
// readfirstlane, so that they stay in scalar registers.
__device__ __forceinline__ bool group_of_m(const GroupArgs& q, int64_t nbn, int64_t bid, int64_t& grp,
                                           int64_t& local) {
    const int lane = threadIdx.x & 63;
    int64_t before = 0, found = -1, loc = 0;
    for (int64_t c0 = 0; c0 < q.groups; c0 += 64) {
        const int64_t gi = c0 + lane;
        int64_t t = 0;
        if (gi < q.groups) {
            int64_t o0, o1;
            group_bounds(q, gi, o0, o1);
            t = (((o1 - o0 + GBM - 1) / GBM) * nbn + 7) & ~(int64_t)7;
        }
        int64_t incl = t;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t v = shfl64(incl, lane >= o ? lane - o : lane);
            if (lane >= o) incl += v;
        }
        const int64_t start = before + incl - t;
        const uint64_t hit = __ballot(t > 0 && bid >= start && bid < start + t);
        if (found < 0 && hit != 0) {
            const int l = __builtin_ctzll(hit);
            found = uniform64(c0 + l);
            loc = uniform64(bid - shfl64(start, l));
        }
        before = uniform64(before + shfl64(incl, 63));
    }
    grp = found;
    local = loc;
    return found >= 0;
}

// The GEMM of K-group grp folded into g: its K range, operand and output bases and tensor
// scales.
template <int FMT, int OUT_F32>
__device__ __forceinline__ void k_group_args(GemmArgs& g, const GroupArgs& q, int64_t grp) {
    using F = Fmt<FMT>;
    constexpr int ES = OUT_F32 ? 4 : 2;
    int64_t o0, o1;
    group_bounds(q, grp, o0, o1);
    if (o0 % 32 != 0 || (o1 - o0) % 32 != 0) o1 = o0 = 0;
    g.K = o1 - o0;
    // a slab operand's group is addressed from its band (mx_gslab_codes); a row-major one
    // from the group's first code byte of each row
    if (!(g.slab & 1)) g.a_codes += o0 / F::EPB;
    if (!(g.slab & 2)) g.b_codes += o0 / F::EPB;
    g.k0 = o0;
    g.a_scales += o0 / F::BLK;
    g.b_scales += o0 / F::BLK;
    g.c = (uint8_t*)g.c + grp * g.M * g.N * ES;
    if constexpr (F::NV) {
        g.a_s_enc += grp;
        g.b_s_enc += grp;
    }
}

// Fold group bookkeeping into g; bid becomes the workgroup's index within its group's tiles.
// Returns false for a workgroup with no tile.
template <int FMT, int OUT_F32, int GM>
__device__ __forceinline__ bool enter_group(GemmArgs& g, const GroupArgs& q, int64_t& bid) {
    using F = Fmt<FMT>;
    constexpr int ES = OUT_F32 ? 4 : 2;
    const int64_t rb = g.ld / F::EPB, sb = g.ld / F::BLK;
    const int64_t nbn = (g.N + GBN - 1) / GBN;
    int64_t grp, local, o0, o1;
    if constexpr (GM == 1) {
        if (!group_of_m(q, nbn, bid, grp, local)) return false;
        group_bounds(q, grp, o0, o1);
        g.M = o1 - o0;
        g.a_codes += o0 * rb;
        g.a_scales += o0 * sb;
        g.b_codes += grp * g.N * rb;
        g.b_scales += grp * g.N * sb;
        g.c = (uint8_t*)g.c + o0 * g.N * ES;
        if constexpr (F::NV) {
            g.a_s_enc += g.a_rows ? o0 : grp;
            g.b_s_enc += g.b_rows ? grp * g.N : grp;
        }
    } else {
        const int64_t nbm = (g.M + GBM - 1) / GBM;
        const int64_t share = (nbm * nbn + 7) & ~(int64_t)7;
        grp = bid / share;
        local = bid - grp * share;
        if (grp >= q.groups) return false;
        k_group_args<FMT, OUT_F32>(g, q, grp);
    }
    bid = local;
    return bid < ((g.M + GBM - 1) / GBM) * nbn;
}

// One output tile per workgroup.  GM 0: a plain launch; 1: M-grouped; 2: K-grouped; 3:
// K-grouped MXFP8 with slab-layout operands.
template <int FMT, int OUT_F32, int GM>
__global__ __launch_bounds__(Fmt<FMT>::THREADS, 1) void gemm_kernel(GemmArgs g, GroupArgs q) {
    using F = Fmt<FMT>;
    // static LDS (up to 152 KiB of gfx950's 160 KiB): no per-kernel attribute to raise at run time
    __shared__ __attribute__((aligned(16))) uint8_t lds[F::LDS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t bid = blockIdx.x;
    if constexpr (GM != 0) {
        if (!enter_group<FMT, OUT_F32, GM>(g, q, bid)) return;   // uniform
    }
    int64_t tm, tn;
    tile_of((g.M + GBM - 1) / GBM, (g.N + GBN - 1) / GBN, bid, tm, tn);
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
    // Uniform output factor of the LDS-DMA NVFP4 kernel with per-tensor scales on both
    // operands, alpha = fp32(1 / (S_a S_b)) with the product and quotient in binary64 (as in
    // tile_factors); computed before the main loop so that the epilogue does not wait for the
    // scale loads.
    float alpha_pt = 1.0f;
    if constexpr (FMT == 2 || FMT == 3) {
        if (!g.a_rows && !g.b_rows) alpha_pt = (float)(1.0 / ((double)g.a_s_enc[0] * (double)g.b_s_enc[0]));
#if __HIP_DEVICE_COMPILE__
        asm volatile("" : "+v"(alpha_pt));
#endif
    }
    const int frow = lane & 31, kh = lane >> 5;
    if constexpr (FMT == 1) {
        // scale records need rows 16 bytes apart; aligned ones also K a multiple of 512 and
        // 16-byte aligned scale tensors
        const bool rows16 = (g.ld / 32) % 16 == 0;
        const bool recs = rows16 && g.K % (MX_GROUP * 64) == 0 &&
                          (((uintptr_t)g.a_scales | (uintptr_t)g.b_scales) % 16) == 0;
        if constexpr (GM == 3) {
            // K-grouped slab operands (a kernel of its own: with the other main loops in one
            // function the register allocation spills): group starts are multiples of 32, not
            // of a slice, so offset records for the scales (their rows are 16 bytes apart: the
            // API asks for K % 512 == 0 here) and band-wide addressing for the codes
            if (g.slab == 3) mx_main_loop<MX_GSLAB, 3>(g, m0, n0, nk, lds, wm, wn, lane, acc);
            else if (g.slab == 2) mx_main_loop<MX_GSLAB, 2>(g, m0, n0, nk, lds, wm, wn, lane, acc);
            else mx_main_loop<MX_GSLAB, 1>(g, m0, n0, nk, lds, wm, wn, lane, acc);
        } else if (recs && g.slab == 3) mx_main_loop<MX_SLAB, 3>(g, m0, n0, nk, lds, wm, wn, lane, acc);
        else if (recs && g.slab == 2) mx_main_loop<MX_SLAB, 2>(g, m0, n0, nk, lds, wm, wn, lane, acc);
        else if (recs && g.slab == 1) mx_main_loop<MX_SLAB, 1>(g, m0, n0, nk, lds, wm, wn, lane, acc);
        else if (recs) mx_main_loop<MX_RECS>(g, m0, n0, nk, lds, wm, wn, lane, acc);
        else if (rows16) mx_main_loop<MX_OFFRECS>(g, m0, n0, nk, lds, wm, wn, lane, acc);
        else mx_main_loop<MX_SLOTS>(g, m0, n0, nk, lds, wm, wn, lane, acc);
    } else if constexpr (FMT == 2) {
        nvw_main_loop<TN>(g, m0, n0, nk, lds, wm, wn, lane, acc);
    } else {
        nvs_main_loop<TN>(g, m0, n0, nk, lds, wm, wn, lane, acc);
    }
    (void)alpha_pt;

    static_assert(F::LDS - FACT_BYTES >= 4 * 128 * (128 * 2 + 16) && F::LDS - FACT_BYTES >= 4 * 64 * (128 * 4 + 16),
                  "factor tables overlap the epilogue staging");
    // NVFP4 output factors (MXFP8 needs none: its scales are inside the MFMA)
    float* fa = (float*)(lds + F::LDS - FACT_BYTES);
    float* fb = fa + 256;
    __syncthreads();   // every wave is done with the operand buffers (and its DMAs)
    constexpr int ES = OUT_F32 ? 4 : 2;
    // staged epilogue: every column of the tile inside C (rows past M are skipped there)
    const bool staged = n0 + GBN <= g.N && (g.N * ES) % 16 == 0;   // uniform
    const int64_t m_end = g.M - m0;
    if constexpr (FMT == 2 || FMT == 3) {
        // per-tensor scales on both operands: one uniform factor, no tables
        if (staged && !g.a_rows && !g.b_rows) {
            store_tile_lds<OUT_F32, true>(g, lds, m0, n0, wm, wn, wave, lane, nullptr, nullptr, alpha_pt, m_end, acc);
            return;
        }
    }
    if constexpr (F::NV) {
        tile_factors<FMT>(g, m0, n0, fa, fb);
        __syncthreads();
    }
    if (staged) {
        store_tile_lds<OUT_F32, F::NV>(g, lds, m0, n0, wm, wn, wave, lane, fa, fb, 1.0f, m_end, acc);
        return;
    }
    // the accumulators hold C^T tiles (see nvw_mfma): lane (frow, kh), register r of tile (i, j)
    // is row 32i + frow, column 32j + within
    static_for<0, 4 * TN>([&](auto t_c) {
        constexpr int i = decltype(t_c)::value / TN, j = decltype(t_c)::value % TN;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int within = 8 * (r >> 2) + 4 * kh + (r & 3);
            const int lrow = wm + 32 * i + frow;
            const int lcol = wn + 32 * j + within;
            const int64_t row = m0 + lrow, col = n0 + lcol;
            if (row < g.M && col < g.N) {
                const float v = F::NV ? acc[i][j][r] * (fa[lrow] * fb[lcol]) : acc[i][j][r];
                if (OUT_F32) {
                    // two 16-bit halves: one 32-bit store per accumulator here changes the
                    // MXFP8 kernel's register allocation so that its main loop spills ~220
                    // registers per lane
                    const uint32_t b = __float_as_uint(v);
                    uint16_t* p = (uint16_t*)((float*)g.c + row * g.N + col);
                    p[0] = (uint16_t)(b & 0xFFFFu);
                    p[1] = (uint16_t)(b >> 16);
                }
                else ((uint16_t*)g.c)[row * g.N + col] = (uint16_t)f32_to_bf16_rne(v);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    });
}

// ---------------------------------------------------------------- persistent NVFP4 kernel
//
// Plain NVFP4 launches with a per-tensor scale on B and on A (or, with bf16 output, one per
// row of A) and K a multiple of 256 (at least 512).  At most one workgroup per CU: workgroup b computes the output tiles b, b + P,
// b + 2P, ... (P = gridDim.x, a multiple of 8 whenever it is below the tile count, so that all
// tiles of a workgroup have the XCD phase tile_of assumes).  The LDS ring and the operand
// pipeline of nvw_main_loop run on from one tile to the next: the next tile's slices 0-2 and
// its first two scale groups are fetched during the current tile's last three slices, and its
// first MFMA step is read and dequantized during the current tile's last step.  In between,
// each lane stores its accumulators straight to C (the ring already holds the next tile, so
// the epilogue cannot stage through LDS) and the next tile starts at once.  With one tile per
// workgroup, every workgroup of the chip stores its tile at the same moment and then waits for
// its successor's first slices: at M = 16384, N = 14336 that launch spends about 9 us per tile
// outside the K loop (a K sweep), 5.7 us of them on the stores (the same kernel with the
// stores dropped).
//
// Between two tiles the output goes out through the one LDS stage that is free at that point,
// the stage of the tile's last slice (the next tile's slice 3 lands there only after the DMA
// issued in its slice 0): each wave stages its 128 x 32 TN block in passes through its own
// 8 KiB of that stage and stores whole 16-byte chunks of rows, so that a store instruction
// covers whole 128-byte lines of C (storing 4 accumulators per lane straight from registers
// touches 32 lines per instruction and measured slower).  The stores are buffer stores through
// a resource over the tile's rows of C, issued by every lane (a chunk outside C gets an offset
// past the range and is dropped), so a wave issues exactly nvp_stores<OUT_F32>() of them per
// tile.  The vector-memory counter retires operations in issue order, and the DMAs that the
// tops of the next tile's slices 0 and 1 wait for were issued before the stores: those two
// waits allow the stores and the DMAs issued after them in flight, and the stores drain while
// the two slices run.  Every other wait is the one of nvw_main_loop.
template <bool OUT_F32>
constexpr int nvp_stores() { return OUT_F32 ? 64 : 32; }   // 128 rows x 256 or 512 bytes / (64 x 16)

__device__ __forceinline__ RsrcWords nvp_rsrc(const GemmArgs& g, int64_t m0, int64_t n0) {
    const int64_t rb = g.ld / 2, sb = g.ld / 16;
    const int64_t ra = tile_rows(g.M - m0, GBM), rbn = tile_rows(g.N - n0, GBN);
    return RsrcWords{rsrc_words(g.a_codes + m0 * rb, ra * rb), rsrc_words(g.b_codes + n0 * rb, rbn * rb),
                     rsrc_words(g.a_scales + m0 * sb, ra * sb), rsrc_words(g.b_scales + n0 * sb, rbn * sb)};
}

// An accumulator read where it is used.  The "a" constraint keeps the value in its AGPR up to
// this point; with plain reads the register allocator copies all 256 accumulators of a tile
// to VGPRs right after their last MFMAs, and the persistent kernel then spills.
__device__ __forceinline__ float acc_read(float a) {
    float v;
    asm("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One tile's accumulators (C^T layout, see nvw_mfma) times alpha, to C.  The tile at (m0, n0)
// is 256 x 64 TN (2 x 2 waves of 128 x 32 TN); `stage` is 32 KiB of LDS no other wave touches
// until the next barrier.  A pass stages 32 rows (one accumulator row group i) by JS x 32
// columns of the wave's block in the wave's 8 KiB, row-major with the 16-byte chunk index
// XORed with the row, then each lane stores CPL chunks.  Every lane takes part in every pass.
// With rowf, row r of the tile takes the factor rowf[r] instead of alpha (a row-scaled A).
template <bool OUT_F32, int TN>
__device__ __forceinline__ void nvp_store(const GemmArgs& g, int64_t m0, int64_t n0, int wm, int wn, int wave,
                                          int lane, float alpha, const floatx16 (&acc)[4][TN], uint8_t* stage,
                                          const float* rowf = nullptr) {
    constexpr int ES = OUT_F32 ? 4 : 2;
    constexpr int JS = 8 / ES < TN ? 8 / ES : TN;   // 32-column groups per pass (8 KiB / 32 rows / 32 / ES)
    constexpr int RB = 32 * JS * ES;                // staged bytes per row
    constexpr int CPR = RB / 16;                    // 16-byte chunks per row (a power of 2)
    constexpr int CPL = 32 * CPR / 64;              // chunks per lane per pass
    static_assert(32 * RB <= 8192 && (CPR & (CPR - 1)) == 0 && CPL * 64 == 32 * CPR, "pass shape");
    uint8_t* reg = stage + wave * 8192;
    const int frow = lane & 31, kh = lane >> 5;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc((const uint8_t*)g.c + m0 * g.N * ES, tile_rows(g.M - m0, GBM) * g.N * ES);
    const uint32_t pitch = (uint32_t)(g.N * ES);
    const int64_t cleft = g.N - n0 - wn;   // columns of C from the block's first one on
    const uint32_t cbase = (uint32_t)(n0 + wn) * ES;
    static_for<0, 4 * (TN / JS)>([&](auto p_c) {
        constexpr int I = decltype(p_c)::value / (TN / JS), J0 = (decltype(p_c)::value % (TN / JS)) * JS;
        const float f = rowf ? rowf[wm + 32 * I + frow] : alpha;   // the lane's row in this pass
#pragma unroll
        for (int jj = 0; jj < JS; ++jj)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = J0 + jj;
                const float x = acc_read(acc[I][j][4 * q]) * f, y = acc_read(acc[I][j][4 * q + 1]) * f;
                const float z = acc_read(acc[I][j][4 * q + 2]) * f, w = acc_read(acc[I][j][4 * q + 3]) * f;
                const int col = 32 * jj + 8 * q + 4 * kh;   // first of the 4 columns, within the pass
                uint8_t* dst = reg + frow * RB + (((col * ES / 16) ^ (frow & (CPR - 1))) << 4) + (col * ES) % 16;
                if constexpr (OUT_F32) *(float4*)dst = make_float4(x, y, z, w);
                else *(uint2*)dst = make_uint2(bf16x2_rne(x, y), bf16x2_rne(z, w));
            }
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            const int t = 64 * k + lane, r = t / CPR, c = t % CPR;
            const uint4 v = *(const uint4*)(reg + r * RB + ((c ^ (r & (CPR - 1))) << 4));
            const int col = 32 * J0 + c * (16 / ES);   // first column of the chunk in the block
            const uint32_t off = col < cleft ? (uint32_t)(wm + 32 * I + r) * pitch + cbase + (uint32_t)(col * ES) : OOB;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4s{v.x, v.y, v.z, v.w}, rs, (int)off, 0, 0);
        }
    });
}

// AROWS: A is row-scaled (one tensor scale per row of A, B per-tensor): each tile's rows take
// fp32(1 / (S_a[m] S_b)) (product and quotient in binary64, as tile_factors), the row's scale
// loaded at the top of the tile and the factors put in LDS between the last slice and the
// stores.
template <bool OUT_F32, bool AROWS = false>
__global__ __launch_bounds__(256, 1) void gemm_nvp_kernel(GemmArgs g, int64_t t_full, int64_t halves) {
    constexpr int TN = 4, NW = 4, DC = 8, DG = 2, PSTEP = 2;
    __shared__ __attribute__((aligned(16))) uint8_t lds[Fmt<2>::LDS];
    __shared__ float rowf[AROWS ? GBM : 1];   // a row-scaled A's factors of the tile being stored
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int frow = lane & 31, kh = lane >> 5;
    const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;
    const int64_t nbm = (g.M + GBM - 1) / GBM, nbn = (g.N + GBN - 1) / GBN;
    const int64_t P = gridDim.x;
    const int items = (int)((t_full - 1 - (int64_t)blockIdx.x) / P) + 1;   // t_full >= P
    const int nk = (int)(g.K / 128);   // even, >= 4
    // alpha = fp32(1 / (S_a S_b)), product and quotient in binary64 (as in tile_factors)
    const double sbd = (double)g.b_s_enc[0];
    float alpha = AROWS ? 1.0f : (float)(1.0 / ((double)g.a_s_enc[0] * sbd));
#if __HIP_DEVICE_COMPILE__
    asm volatile("" : "+v"(alpha));
#endif
    // thread t's row of the tile (t < 256 = GBM): its A tensor scale and output factor
    auto row_scale = [&](int64_t tm0) { return g.a_s_enc[tm0 + threadIdx.x < g.M ? tm0 + threadIdx.x : g.M - 1]; };
    auto put_factors = [&](int64_t tm0, float sa) {
        rowf[threadIdx.x] = tm0 + threadIdx.x < g.M ? (float)(1.0 / ((double)sa * sbd)) : 1.0f;
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    auto origin = [&](int it, int64_t& m0, int64_t& n0) {   // tiles < 2^31 (host check)
        uint32_t tm, tn;
        tile_of32((uint32_t)nbm, (uint32_t)nbn, blockIdx.x + (uint32_t)it * (uint32_t)P, tm, tn);
        m0 = (int64_t)tm * GBM;
        n0 = (int64_t)tn * GBN;
    };
    int64_t m0, n0, m1 = 0, n1 = 0;
    origin(0, m0, n0);
    MxDma d = make_dma<2, 16>(g, m0, n0, lane);
    RsrcWords rc = d.o, rn = d.o;   // resources of the current and of the next tile
    bool has_next = items > 1;
    if (has_next) {
        origin(1, m1, n1);
        rn = nvp_rsrc(g, m1, n1);
    }
    // ring positions by global slice / scale-group index (a tile's slice 0 is slice it * nk)
    auto buf = [&](int k) { return lds + (k & 3) * NV4_CODES; };
    auto sbuf = [&](int grp) { return lds + 4 * NV4_CODES + (grp & 1) * NV4_SREC; };

    floatx16 acc[4][TN];   // each tile's first step writes them (nvw_mfma_first)

    // prologue of the first tile, as in nvw_main_loop (nk >= 4: groups 0 and 1 both exist)
    nv4_dma_group<NW>(d, 0, true, sbuf(0));
    nv4_dma_group<NW>(d, 1, true, sbuf(1));
    static_for<0, 3>([&](auto k_c) {
        constexpr int K0 = decltype(k_c)::value;
        static_for<0, 4>([&](auto p_c) { nv4_dma_codes<decltype(p_c)::value, NW>(d, 64u * K0, true, buf(K0)); });
    });
    nv4_dma_group<NW>(d, 0, false, buf(3));   // no traffic; keeps the wait counts uniform
    wait_vm_barrier<2 * DC + DG>();

    NvQuadT<TN> q0, q1;
    NvWordsT<TN> w;
    NvOpsT<TN> cur, nxt;
    NvRecT<TN> rec;
    uint32_t sa[4], sb[TN], san[4], sbn[TN];
    nvw_read_recs<TN>(sbuf(0), wm, wn, frow, rec);
    nvw_pick_scales<0, TN>(rec, kh, sa, sb);
    nvw_read_quad<0, TN>(buf(0), wm, wn, frow, kh, q0);
    nvw_words_of<0, TN>(q0, w);
    nvw_ops<0, TN>(w, sa, sb, cur);

    for (int it = 0; it < items; ++it) {
        const int gs0 = it * nk;
        [[maybe_unused]] float sa_row = 0.0f;
        if constexpr (AROWS) sa_row = row_scale(m0);   // used by the stores at the tile's end
        // slice kt of this tile; in the tile's last slice (LAST) the last step neither reads nor
        // dequantizes the next tile's first step: that happens after the stores, so that those
        // operands are not live across the epilogue
        auto slice = [&](int kt, auto odd_c, auto last_c, auto first_c) {
            constexpr bool ODD = decltype(odd_c)::value, LAST = decltype(last_c)::value;
            constexpr bool FIRST = decltype(first_c)::value;
            // the previous tile's stores may be in flight at the tops of slices 0 and 1
            constexpr int NST = nvp_stores<OUT_F32>();
            constexpr int W0 = DC + DG + NST < 63 ? DC + DG + NST : 63, W1 = DC + NST < 63 ? DC + NST : 63;
            if (kt < 2 && it > 0) {
                if constexpr (ODD) wait_vm_barrier<W1>();
                else wait_vm_barrier<W0>();
            } else if constexpr (ODD) wait_vm_barrier<DC>();
            else wait_vm_barrier<DC + DG>();
            const int kd = kt + 3;
            const bool nx = kd >= nk;              // the slice fetched now belongs to the next tile
            const bool live = !nx || has_next;
            MxDma dd = d;
            dd.o = nx ? rn : rc;
            const uint32_t kloc = (uint32_t)(nx ? kd - nk : kd);
            uint8_t* db = buf(gs0 + kd);
            const uint8_t* cb = buf(gs0 + kt);
            const uint8_t* nb = buf(gs0 + kt + 1);
            static_for<0, 8>([&](auto s_c) {
                constexpr int S = decltype(s_c)::value;
                if constexpr (S % PSTEP == 0) nv4_dma_codes<S / PSTEP, NW>(dd, 64u * kloc, live, db);
                if constexpr (ODD && S == 1) nv4_dma_group<NW>(dd, kloc / 2, live, sbuf((gs0 + kd) / 2));
                if constexpr (S == 2) nvw_read_quad<1, TN>(cb, wm, wn, frow, kh, q1);
                if constexpr (S == 6 && !LAST) nvw_read_quad<0, TN>(nb, wm, wn, frow, kh, q0);
                if constexpr (ODD && S == 5) nvw_read_recs<TN>(sbuf((gs0 + kt + 1) / 2), wm, wn, frow, rec);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (S + 1 < 8) {
                    if constexpr (S + 1 < 4) nvw_words_of<S + 1, TN>(q0, w);
                    else nvw_words_of<S + 1, TN>(q1, w);
                    nvw_ops<S + 1, TN>(w, sa, sb, nxt);
                } else if constexpr (!LAST) {
                    nvw_words_of<0, TN>(q0, w);
                    nvw_pick_scales<ODD ? 0 : 1, TN>(rec, kh, san, sbn);
                    nvw_ops<0, TN>(w, san, sbn, nxt);
                }
                if constexpr (FIRST && S == 0) nvw_mfma_first<TN>(cur, acc);
                else nvw_mfma<TN>(cur, acc);
                if constexpr (S + 1 < 8 || !LAST) nvw_interleave<TN>();
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (S + 1 < 8 || !LAST) cur = nxt;
            });
            if constexpr (!LAST) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sa[i] = san[i];
#pragma unroll
                for (int j = 0; j < TN; ++j) sb[j] = sbn[j];
            }
        };
        using F_ = std::false_type;
        using T_ = std::true_type;
        slice(0, F_{}, F_{}, T_{});
        slice(1, T_{}, F_{}, F_{});
        for (int kt = 2; kt < nk - 2; kt += 2) {
            slice(kt, F_{}, F_{}, F_{});
            slice(kt + 1, T_{}, F_{}, F_{});
        }
        slice(nk - 2, F_{}, F_{}, F_{});
        slice(nk - 1, T_{}, T_{}, F_{});
        lds_barrier();   // every wave is done with the stage of the last slice
        if constexpr (AROWS) {
            put_factors(m0, sa_row);
            nvp_store<OUT_F32, TN>(g, m0, n0, wm, wn, wave, lane, alpha, acc, buf(gs0 + nk - 1), rowf);
        } else {
            nvp_store<OUT_F32, TN>(g, m0, n0, wm, wn, wave, lane, alpha, acc, buf(gs0 + nk - 1));
        }
        // the next tile's first step (its slice 0 landed before the top of this tile's last
        // slice, whose step 5 read its first scale records)
        nvw_read_quad<0, TN>(buf(gs0 + nk), wm, wn, frow, kh, q0);
        nvw_words_of<0, TN>(q0, w);
        nvw_pick_scales<0, TN>(rec, kh, sa, sb);
        nvw_ops<0, TN>(w, sa, sb, cur);
        m0 = m1;
        n0 = n1;
        rc = rn;
        has_next = it + 2 < items;
        if (has_next) {
            origin(it + 2, m1, n1);
            rn = nvp_rsrc(g, m1, n1);
        }
    }
    wait_vm<0>();   // no DMA may still write this workgroup's LDS when the wave ends

    // The last, partial round of tiles (t_full .. t_full + halves / 2), each split into two
    // 256 x 128 halves, one per workgroup: 4 waves of 128 x 64 (TN = 2) with the full tile's
    // DMA plan (the B rows past 128 read nothing).  A half costs a little more than half a tile
    // (6 dequantization VALU per MFMA against 4.4), against a whole tile for the workgroups of
    // a partial round that is left whole.
    if ((int64_t)blockIdx.x < halves) {
        __syncthreads();   // every wave is done with the ring
        uint32_t tm, tn;
        tile_of32((uint32_t)nbm, (uint32_t)nbn, (uint32_t)t_full + blockIdx.x / 2, tm, tn);
        const int64_t hm0 = (int64_t)tm * GBM, hn0 = (int64_t)tn * GBN + 128 * (blockIdx.x & 1);
        if (hn0 < g.N) {   // uniform
            const int hwm = (wave >> 1) * 128, hwn = (wave & 1) * 64;
            floatx16 hacc[4][2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) hacc[i][j][r] = 0.0f;
            nvw_main_loop<2, 4>(g, hm0, hn0, nk, lds, hwm, hwn, lane, hacc, 128);
            lds_barrier();   // every wave is done with the ring
            if constexpr (AROWS) {
                put_factors(hm0, row_scale(hm0));
                nvp_store<OUT_F32, 2>(g, hm0, hn0, hwm, hwn, wave, lane, alpha, hacc, lds, rowf);
            } else {
                nvp_store<OUT_F32, 2>(g, hm0, hn0, hwm, hwn, wave, lane, alpha, hacc, lds);
            }
        }
    }
}

template <int FMT, int OUT, int GM>
static int launch_one(const GemmArgs& g, const GroupArgs& q, int64_t tiles, hipStream_t s) {
    if (tiles <= 0) return 0;
    hipLaunchKernelGGL((gemm_kernel<FMT, OUT, GM>), dim3((unsigned)tiles), dim3(Fmt<FMT>::THREADS), 0, s, g, q);
    return (int)hipGetLastError();
}

// Slab-layout MXFP8 codes are read only by the aligned-record main loop and, in K-grouped
// launches, by the offset-record loop with band-wide code addressing; any other path would
// address them as row-major.  The C ABI admits slab operands only where those loops apply;
// this check keeps every launch path to the same rule.
static bool slab_ok(const GemmArgs& g, int fmt, int mode) {
    if (g.slab == 0) return true;
    if (fmt != 1 || g.K % (MX_GROUP * 64) != 0) return false;
    if ((((uintptr_t)g.a_scales | (uintptr_t)g.b_scales) % 16) != 0) return false;
    if (mode == 2) return (int64_t)GBM * g.K <= 0x7FFFFFFF;   // K-grouped: a band within one resource
    if (mode == 1 && (g.slab & 1)) return false;    // M-grouped: group bands cut the token operand
    return true;
}

// Workgroups of a persistent NVFP4 launch over `tiles` output tiles, or 0 where that kernel does
// not apply: a per-tensor scale on B and on A (or one per row of A, bf16 output only: with fp32
// output that variant spills), K a multiple of 256 and at least 512, N a
// multiple of 8 (every 16-byte chunk of a row of C lies inside C or outside it), C 16-byte aligned, a
// tile's rows of C within a 2^31-byte resource, and the global slice count of a workgroup
// within int range.
static int64_t persistent_workgroups(const GemmArgs& g, int c_dtype, int64_t tiles) {
    if (tiles >= ((int64_t)1 << 31) || g.N >= ((int64_t)1 << 34)) return 0;   // 32-bit tile arithmetic
    const int64_t es = c_dtype == 1 ? 4 : 2;
    if (g.b_rows || (g.a_rows && c_dtype == 1) || g.K % 256 != 0 || g.K < 512 || g.N % 8 != 0) return 0;
    if ((uintptr_t)g.c % 16 != 0 || (int64_t)GBM * g.N * es > 0x7FFFFFFF) return 0;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
        return 0;
    const int64_t p = tiles <= cus ? tiles : (int64_t)(cus / 8) * 8;
    if (((tiles + p - 1) / p) * (g.K / 128) >= ((int64_t)1 << 30)) return 0;
    return p;
}

template <int GM>
static int launch_fmt(int fmt, int c_dtype, const GemmArgs& g, const GroupArgs& q, int64_t tiles, hipStream_t s) {
    if constexpr (GM == 0) {
        if (fmt == 0) {
            const int64_t p = persistent_workgroups(g, c_dtype, tiles);
            if (p > 0) {
                // a last round that would leave at least half the workgroups idle is split into
                // half tiles, one per workgroup
                const int64_t r = tiles % p;
                const int64_t t_full = (r != 0 && 2 * r <= p) ? tiles - r : tiles;
                const int64_t halves = t_full < tiles ? 2 * r : 0;
                const dim3 grid((unsigned)p), block(256);
                if (g.a_rows) {   // bf16 output (persistent_workgroups)
                    hipLaunchKernelGGL((gemm_nvp_kernel<false, true>), grid, block, 0, s, g, t_full, halves);
                } else if (c_dtype == 1) {
                    hipLaunchKernelGGL((gemm_nvp_kernel<true>), grid, block, 0, s, g, t_full, halves);
                } else {
                    hipLaunchKernelGGL((gemm_nvp_kernel<false>), grid, block, 0, s, g, t_full, halves);
                }
                return (int)hipGetLastError();
            }
        }
    }
    // NVFP4: the LDS DMA kernel with scale records when every K handled is a multiple of 256
    // (known on the host unless K varies per group), with per-slice scale records otherwise
    if constexpr (GM != 2) {
        if (fmt == 0 && g.K % 256 == 0)
            return c_dtype == 1 ? launch_one<2, 1, GM>(g, q, tiles, s) : launch_one<2, 0, GM>(g, q, tiles, s);
    }
    if (fmt == 0) return c_dtype == 1 ? launch_one<3, 1, GM>(g, q, tiles, s) : launch_one<3, 0, GM>(g, q, tiles, s);
    return c_dtype == 1 ? launch_one<1, 1, GM>(g, q, tiles, s) : launch_one<1, 0, GM>(g, q, tiles, s);
}

int launch_blockscaled_gemm(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const uint8_t* a_scales, const float* a_s_enc, const uint8_t* b_codes,
                            const uint8_t* b_scales, const float* b_s_enc, int a_rows, int b_rows, void* c,
                            int c_dtype, void* hip_stream, int slab) {
    if (M == 0 || N == 0) return 0;
    GemmArgs g{M, N, K, a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc, c, a_rows, b_rows, K, slab};
    if (!slab_ok(g, fmt, 0)) return (int)hipErrorInvalidValue;
    const int64_t tiles = ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
    return launch_fmt<0>(fmt, c_dtype, g, GroupArgs{nullptr, 0, 0}, tiles, (hipStream_t)hip_stream);
}

int64_t grouped_gemm_workgroups(int mode, int64_t groups, int64_t M, int64_t N) {
    const int64_t nbm = (M + GBM - 1) / GBM, nbn = (N + GBN - 1) / GBN;
    if (mode == 1) return nbn * (nbm + groups) + 7 * groups;   // >= the sum of the groups' shares
    return groups * ((nbm * nbn + 7) & ~(int64_t)7);
}

int launch_blockscaled_grouped_gemm(int fmt, int mode, int64_t groups, const int64_t* offsets, int64_t M, int64_t N,
                                    int64_t K, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_s_enc,
                                    const uint8_t* b_codes, const uint8_t* b_scales, const float* b_s_enc,
                                    int a_rows, int b_rows, void* c, int c_dtype, void* hip_stream, int slab) {
    if (groups == 0 || M == 0 || N == 0) return 0;
    GemmArgs g{M, N, K, a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc, c, a_rows, b_rows, K, slab};
    const GroupArgs q{offsets, groups, mode == 1 ? M : K};
    if (!slab_ok(g, fmt, mode)) return (int)hipErrorInvalidValue;
    const int64_t tiles = grouped_gemm_workgroups(mode, groups, M, N);
    hipStream_t s = (hipStream_t)hip_stream;
    if (mode == 1) return launch_fmt<1>(fmt, c_dtype, g, q, tiles, s);
    if (g.slab != 0)   // MXFP8 (slab_ok): the K-grouped kernel for slab-layout operands
        return c_dtype == 1 ? launch_one<1, 1, 3>(g, q, tiles, s) : launch_one<1, 0, 3>(g, q, tiles, s);
    return launch_fmt<2>(fmt, c_dtype, g, q, tiles, s);
}

}  // namespace bsq
