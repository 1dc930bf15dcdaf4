"""GPU parity of the block-scaled GEMM against the CPU oracle (binary64 over the same
quantized operands).  The bar: relative Frobenius error <= 2e-3 against the oracle
output rounded as the GPU stores it (bf16 RNE for Y and dX, none for the fp32 dW).
Every compared element must also lie within the rounding-error bound of fp32
accumulation (assert_gemm_elements).  Small shapes are compared in full (several tiles,
ragged M/N, a K tail shorter than the K slice); the workload shapes are compared on rows
x columns of C that include the first and last row and column of every 256-wide band
(so every output tile is checked), with the GEMM launched exactly as the bench
launches it."""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsq
from synthetic import (SEED_DY, SEED_SIGNS, SEED_SR_KEY, SEED_W, SEED_X, STD_DY, STD_W, gaussian_bf16,
                       outlier_bf16, rht_signs)
from tests.gpu_common import (GEMM_TOL, assert_bytes_equal, assert_f32_equal, assert_gemm_elements, bf16_round,
                              from_slab, note, rel_fro, stratified)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def sampled_output(y: torch.Tensor, rows=None, cols=None) -> np.ndarray:
    """C (or rows x cols of it) as float64 on the host, indexed on the device first."""
    if rows is not None:
        y = y[torch.from_numpy(np.asarray(rows, np.int64)).to(y.device)][:, torch.from_numpy(
            np.asarray(cols, np.int64)).to(y.device)]
    return y.float().cpu().numpy().astype(np.float64)


def nv_gemm_check(a_cpu, b_cpu, out_dtype=torch.bfloat16, rows=None, cols=None, label="",
                  a_dir=1, b_dir=1, rounding=0, signs=None):
    """Quantize both operands on the GPU and run the GEMM; quantize the same bf16 inputs with
    the oracle (codes, scales and tensor scales must agree bit for bit) and compare the GEMM
    against the oracle GEMM of the oracle's own operands."""
    import oracle
    note("nvfp4 gemm %s A%s B%s out=%s" % (label, tuple(a_cpu.shape), tuple(b_cpu.shape), out_dtype))
    qa = bsq.nvfp4_quantize(a_cpu.to(DEV), direction=a_dir, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=0,
                            rht_signs=signs)
    qb = bsq.nvfp4_quantize(b_cpu.to(DEV), direction=b_dir, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=1,
                            rht_signs=signs)
    ka, kb = ("row" if a_dir == 1 else "col"), ("row" if b_dir == 1 else "col")
    ia, ib = (0 if a_dir == 1 else 1), (0 if b_dir == 1 else 1)
    y = bsq.blockscaled_gemm(bsq.FMT_NVFP4, qa[ka + "_codes"], qa[ka + "_scales"], qa["s_enc"][ia:ia + 1],
                             qb[kb + "_codes"], qb[kb + "_scales"], qb["s_enc"][ib:ib + 1], out_dtype=out_dtype)
    torch.cuda.synchronize()
    sg = None if signs is None else signs.numpy()
    ra = oracle.nvfp4_quantize(a_cpu, direction=a_dir, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=0, signs=sg)
    rb = oracle.nvfp4_quantize(b_cpu, direction=b_dir, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=1, signs=sg)
    for q, r, nm in ((qa, ra, "A"), (qb, rb, "B")):
        k = ka if nm == "A" else kb
        i = ia if nm == "A" else ib
        assert_bytes_equal(q[k + "_codes"], r[k + "_codes"], nm + " codes")
        assert_bytes_equal(q[k + "_scales"], r[k + "_scales"], nm + " scales")
        assert_f32_equal(q["s_enc"][i:i + 1], np.asarray(r["s_enc"][i:i + 1], dtype=np.float32), nm + " s_enc")
    ref, sabs = oracle.blockscaled_gemm(oracle.FMT_NVFP4, ra[ka + "_codes"], ra[ka + "_scales"],
                                        float(ra["s_enc"][ia]), rb[kb + "_codes"], rb[kb + "_scales"],
                                        float(rb["s_enc"][ib]), rows=rows, cols=cols, with_abs=True)
    yc = sampled_output(y, rows, cols)
    want = bf16_round(ref) if out_dtype == torch.bfloat16 else ref
    err = rel_fro(yc, want)
    note("  rel_fro vs rounded oracle = %.3e, vs exact oracle = %.3e" % (err, rel_fro(yc, ref)))
    assert err <= GEMM_TOL, err
    K = a_cpu.shape[1] if a_dir == 1 else a_cpu.shape[0]
    assert_gemm_elements(yc, ref, sabs, K, out_dtype == torch.bfloat16, "nvfp4 " + label)
    return err


def mx_gemm_check(a_cpu, b_cpu, a_dir, b_dir, out_dtype=torch.bfloat16, rows=None, cols=None, label=""):
    """As nv_gemm_check for MXFP8 operands (no tensor scale)."""
    import oracle
    note("mxfp8 gemm %s A%s B%s out=%s" % (label, tuple(a_cpu.shape), tuple(b_cpu.shape), out_dtype))
    qa = bsq.mxfp8_quantize(a_cpu.to(DEV), direction=a_dir)
    qb = bsq.mxfp8_quantize(b_cpu.to(DEV), direction=b_dir)
    ka, kb = ("row" if a_dir == 1 else "col"), ("row" if b_dir == 1 else "col")
    y = bsq.blockscaled_gemm(bsq.FMT_MXFP8, qa[ka + "_codes"], qa[ka + "_scales"], None,
                             qb[kb + "_codes"], qb[kb + "_scales"], None, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ra = oracle.mxfp8_quantize(a_cpu, direction=a_dir)
    rb = oracle.mxfp8_quantize(b_cpu, direction=b_dir)
    for q, r, k, nm in ((qa, ra, ka, "A"), (qb, rb, kb, "B")):
        assert_bytes_equal(q[k + "_codes"], r[k + "_codes"], nm + " codes")
        assert_bytes_equal(q[k + "_scales"], r[k + "_scales"], nm + " scales")
    ref, sabs = oracle.blockscaled_gemm(oracle.FMT_MXFP8, ra[ka + "_codes"], ra[ka + "_scales"], 1.0,
                                        rb[kb + "_codes"], rb[kb + "_scales"], 1.0, rows=rows, cols=cols,
                                        with_abs=True)
    yc = sampled_output(y, rows, cols)
    want = bf16_round(ref) if out_dtype == torch.bfloat16 else ref
    err = rel_fro(yc, want)
    note("  rel_fro vs rounded oracle = %.3e" % err)
    assert err <= GEMM_TOL, err
    K = a_cpu.shape[1] if a_dir == 1 else a_cpu.shape[0]
    assert_gemm_elements(yc, ref, sabs, K, out_dtype == torch.bfloat16, "mxfp8 " + label,
                         mx=(ra[ka + "_codes"], ra[ka + "_scales"], rb[kb + "_codes"], rb[kb + "_scales"], rows, cols))
    return err


def test_tiny_config_full():
    """X[128,256], W[256,256] ~ N(0,1); both NVFP4 rowwise RNE; Y = X W^T bf16."""
    nv_gemm_check(gaussian_bf16((128, 256), 1.0, SEED_X), gaussian_bf16((256, 256), 1.0, SEED_W), label="tiny")


# K a multiple of 256 runs the 4-wave kernel with grouped scale records, any other K the 8-wave one;
# (300, 520, 2048) and (40, 512, 512) have tiles with every column inside C but rows past M
# (staged through LDS with those rows skipped)
@pytest.mark.parametrize("M,N,K", [(200, 72, 96), (128, 128, 32), (1, 1, 64), (384, 260, 320), (64, 512, 1056),
                                   (200, 72, 256), (1, 1, 256), (384, 260, 768), (300, 520, 2048), (40, 512, 512)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_nvfp4_ragged_full(M, N, K, out_dtype):
    nv_gemm_check(outlier_bf16((M, K), seed=M, mask_seed=K), gaussian_bf16((N, K), 0.02, N + 7), out_dtype=out_dtype,
                  label="ragged")


@pytest.mark.parametrize("fa,fb", [(2.0 ** -60, 2.0 ** 40), (2.0 ** 50, 2.0 ** -50), (3.0e-20, 7.0e15)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_nvfp4_full_tiles_extreme_tensor_scales(fa, fb, out_dtype):
    """Full 256 x 256 tiles with K a multiple of 256 (the LDS-DMA kernel, whose per-tensor
    epilogue multiplies by one alpha = 1 / (S_a S_b) computed per lane before the main loop)
    with operands scaled far apart, so that S_a and S_b sit near the ends of the fp32 range
    while their product does not."""
    a = (gaussian_bf16((512, 512), 1.0, 93).float() * fa).to(torch.bfloat16)
    b = (outlier_bf16((256, 512), seed=94, mask_seed=95).float() * fb).to(torch.bfloat16)
    assert torch.isfinite(a.float()).all() and torch.isfinite(b.float()).all()
    nv_gemm_check(a, b, out_dtype=out_dtype, label="extreme scales %g %g" % (fa, fb))


# K = 96, 256, 1056: scales fetched per K slice; K = 512, 1536: grouped 16-block scale records.
# (300, 512, *): tiles whose columns all lie inside C but whose last rows do not -- staged
# through LDS with the rows past M skipped.
@pytest.mark.parametrize("M,N,K", [(200, 72, 96), (256, 256, 256), (96, 160, 1056), (200, 72, 512), (300, 260, 1536),
                                   (300, 512, 512), (300, 512, 1056)])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mxfp8_ragged_full(M, N, K, out_dtype):
    mx_gemm_check(outlier_bf16((M, K), seed=M + 1, mask_seed=K + 1), gaussian_bf16((N, K), 0.02, N + 9), 1, 1,
                  out_dtype=out_dtype, label="ragged")


@pytest.mark.parametrize("fmt", [0, 1])
def test_largest_k(fmt):
    """The largest K the C ABI accepts (2^24 - 256 NVFP4, 2^23 - 512 MXFP8, both on the
    LDS-DMA kernels): a 256-row operand tile then spans just under 2^31 bytes, the largest
    range of a buffer resource, and the lane offsets reach their top bits.  Seeded random codes
    and scales (no quantization at this size); sampled rows x columns against the oracle."""
    import oracle
    K = (1 << 24) - 256 if fmt == 0 else (1 << 23) - 512
    M = N = 256
    rng = np.random.default_rng(97 + fmt)
    if fmt == 0:
        ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
        bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        asc = rng.integers(0x30, 0x48, (M, K // 16), dtype=np.uint8)
        bsc = rng.integers(0x30, 0x48, (N, K // 16), dtype=np.uint8)
    else:
        ac = rng.integers(0, 256, (M, K), dtype=np.uint8) & 0x77   # finite E4M3 codes
        bc = rng.integers(0, 256, (N, K), dtype=np.uint8) & 0x77
        asc = rng.integers(120, 134, (M, K // 32), dtype=np.uint8)
        bsc = rng.integers(120, 134, (N, K // 32), dtype=np.uint8)
    note("largest K: fmt=%d K=%d" % (fmt, K))
    t = lambda x: torch.from_numpy(x).to(DEV)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    sa, sb = (one, one) if fmt == 0 else (None, None)
    y = bsq.blockscaled_gemm(fmt, t(ac), t(asc), sa, t(bc), t(bsc), sb)
    torch.cuda.synchronize()
    rows, cols = np.array([0, 77, 128, 255]), np.array([0, 31, 200, 255])
    ref, sabs = oracle.blockscaled_gemm(fmt, ac, asc, 1.0, bc, bsc, 1.0, rows=rows, cols=cols, with_abs=True)
    yc = y.float().cpu().numpy().astype(np.float64)[rows][:, cols]
    err = rel_fro(yc, bf16_round(ref))
    note("  rel_fro vs rounded oracle = %.3e" % err)
    assert err <= GEMM_TOL, err
    assert_gemm_elements(yc, ref, sabs, K, True, "largest K fmt %d" % fmt,
                         mx=None if fmt == 0 else (ac, asc, bc, bsc, rows, cols))


def test_largest_k_slab():
    """Slab-layout MXFP8 operands at the largest K the C ABI accepts (2^23 - 512): slice k's
    block starts k * n * 64 bytes into a band, just under 2^31 for the last slice of a full
    band, and A has a ragged second band (300 rows).  Codes +1, -1 or 0 with A's scales 2^0
    and B's 2^0 or 2^-1 keep every partial sum a multiple of 1/2 below 2^23, exact in fp32
    whatever the summation order, so the fp32 output must equal the oracle exactly: a code
    or scale read from the wrong place would show.  Sampled outputs."""
    import oracle
    K, M, N = (1 << 23) - 512, 300, 256
    rng = np.random.default_rng(131)
    lut = np.array([0x38, 0xB8, 0x00], np.uint8)   # E4M3 +1, -1, 0
    ac = lut[rng.integers(0, 3, (M, K), dtype=np.uint8)]
    bc = lut[rng.integers(0, 3, (N, K), dtype=np.uint8)]
    asc = np.full((M, K // 32), 127, np.uint8)
    bsc = rng.integers(126, 128, (N, K // 32), dtype=np.uint8)
    note("largest K slab: K=%d M=%d N=%d" % (K, M, N))

    def to_slab(c):
        rows = c.shape[0]
        out = np.empty(rows * K, np.uint8)
        for b0 in range(0, rows, 256):
            n = min(256, rows - b0)
            out[b0 * K:(b0 + n) * K] = c[b0:b0 + n].reshape(n, K // 64, 64).transpose(1, 0, 2).reshape(-1)
        return out.reshape(rows, K)

    sa, sb = to_slab(ac), to_slab(bc)
    assert np.array_equal(from_slab(torch.from_numpy(sa), M, K), ac)
    t = lambda x: torch.from_numpy(x).to(DEV)
    y = bsq.blockscaled_gemm(bsq.FMT_MXFP8 | bsq.FMT_MX_SLAB, t(sa), t(asc), None, t(sb), t(bsc), None,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    del sa, sb
    rows, cols = np.array([0, 77, 255, 256, 299]), np.array([0, 31, 200, 255])
    ref = oracle.blockscaled_gemm(1, ac, asc, 1.0, bc, bsc, 1.0, rows=rows, cols=cols)
    yc = y.cpu().numpy().astype(np.float64)[rows][:, cols]
    note("  max |diff| = %g over %d outputs (|C| up to %g)" % (np.abs(yc - ref).max(), yc.size, np.abs(ref).max()))
    assert np.array_equal(yc, ref)


@pytest.mark.parametrize("fmt", [0, 1])
def test_output_beyond_2g_elements(fmt):
    """C of [65792, 32768] (2^31 + 2^24 elements, bf16 output offsets past 2^32 bytes) with a
    short K: both operands quantized on the GPU and by the oracle (bit for bit), C compared on
    sampled rows x columns, the last rows and columns among them."""
    import oracle
    M, N, K = 65536 + 256, 32768, 512
    note("gemm output beyond 2^31 elements: fmt=%d M=%d N=%d K=%d" % (fmt, M, N, K))
    a = gaussian_bf16((M, K), 1.0, 201)
    b = gaussian_bf16((N, K), 0.05, 202)
    if fmt == 0:
        qa, qb = bsq.nvfp4_quantize(a.to(DEV), direction=1), bsq.nvfp4_quantize(b.to(DEV), direction=1)
        ra, rb = oracle.nvfp4_quantize(a, direction=1), oracle.nvfp4_quantize(b, direction=1)
        y = bsq.blockscaled_gemm(fmt, qa["row_codes"], qa["row_scales"], qa["s_enc"][0:1], qb["row_codes"],
                                 qb["row_scales"], qb["s_enc"][0:1])
        sa, sb = float(ra["s_enc"][0]), float(rb["s_enc"][0])
    else:
        qa, qb = bsq.mxfp8_quantize(a.to(DEV), direction=1), bsq.mxfp8_quantize(b.to(DEV), direction=1)
        ra, rb = oracle.mxfp8_quantize(a, direction=1), oracle.mxfp8_quantize(b, direction=1)
        y = bsq.blockscaled_gemm(fmt, qa["row_codes"], qa["row_scales"], None, qb["row_codes"], qb["row_scales"], None)
        sa = sb = 1.0
    torch.cuda.synchronize()
    for q, r, nm in ((qa, ra, "A"), (qb, rb, "B")):
        assert_bytes_equal(q["row_codes"], r["row_codes"], nm + " codes")
        assert_bytes_equal(q["row_scales"], r["row_scales"], nm + " scales")
    rng = np.random.default_rng(203 + fmt)
    rows = np.unique(np.concatenate([[0, M // 2, M - 1], rng.choice(M, 13, replace=False)]))
    cols = np.unique(np.concatenate([[0, N // 2, N - 1], rng.choice(N, 13, replace=False)]))
    yc = y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy().astype(np.float64)
    del y
    ref, sabs = oracle.blockscaled_gemm(fmt, ra["row_codes"], ra["row_scales"], sa, rb["row_codes"], rb["row_scales"],
                                        sb, rows=rows, cols=cols, with_abs=True)
    err = rel_fro(yc, bf16_round(ref))
    note("  rel_fro vs rounded oracle = %.3e" % err)
    assert err <= GEMM_TOL, err
    assert_gemm_elements(yc, ref, sabs, K, True, "output beyond 2^31 fmt %d" % fmt,
                         mx=None if fmt == 0 else (ra["row_codes"], ra["row_scales"], rb["row_codes"],
                                                   rb["row_scales"], rows, cols))


def test_constant_operands_closed_form():
    """All elements 1.0 in A and 0.5 in B: every output is K * 1.0 * 0.5 exactly."""
    M, N, K = 160, 96, 512
    a = torch.ones((M, K), dtype=torch.bfloat16)
    b = torch.full((N, K), 0.5, dtype=torch.bfloat16)
    qa = bsq.nvfp4_quantize(a.to(DEV))
    qb = bsq.nvfp4_quantize(b.to(DEV))
    y = bsq.blockscaled_gemm(0, qa["row_codes"], qa["row_scales"], qa["s_enc"][0:1], qb["row_codes"],
                             qb["row_scales"], qb["s_enc"][0:1], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(y.cpu() == K * 0.5)


def test_k_zero_writes_zeros():
    a = torch.empty((64, 0), dtype=torch.uint8, device=DEV)
    s = torch.empty((64, 0), dtype=torch.uint8, device=DEV)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    y = torch.full((64, 64), 7.0, dtype=torch.float32, device=DEV)
    bsq.blockscaled_gemm(0, a, s, one, a, s, one, out_dtype=torch.float32, out=y)
    torch.cuda.synchronize()
    assert torch.all(y.cpu() == 0)


def test_wgrad_small_rht_sr_full():
    """wgrad pairing at a small shape: dW = dY^T X, both columnwise with RHT + SR, fp32 out."""
    nv_gemm_check(gaussian_bf16((512, 192), STD_DY, SEED_DY), gaussian_bf16((512, 160), 1.0, SEED_X),
                  out_dtype=torch.float32, a_dir=2, b_dir=2, rounding=1, signs=rht_signs(SEED_SIGNS), label="wgrad-small")


def test_fwd_llama3_8b_sampled():
    """Y[16384, 14336] = X W^T at the Llama-3-8B FFN up-proj shape; every 256 x 256 output tile
    sampled (192 x 168 outputs)."""
    nv_gemm_check(gaussian_bf16((16384, 4096), 1.0, SEED_X), gaussian_bf16((14336, 4096), STD_W, SEED_W),
                  rows=stratified(16384, 1), cols=stratified(14336, 2), label="fwd")


def test_wgrad_llama3_8b_sampled():
    """dW[14336, 4096] = dY^T X with RHT + SR columnwise operands (K = 16384 tokens), fp32;
    every output tile sampled, and both 128-column halves of each (on a 256-CU device the 896
    tiles leave a last round of 128, which the persistent kernel splits into halves)."""
    nv_gemm_check(gaussian_bf16((16384, 14336), STD_DY, SEED_DY), gaussian_bf16((16384, 4096), 1.0, SEED_X),
                  out_dtype=torch.float32, rows=stratified(14336, 3), cols=stratified(4096, 4, band=128),
                  a_dir=2, b_dir=2, rounding=1, signs=rht_signs(SEED_SIGNS), label="wgrad")


@pytest.mark.parametrize("M,N,K,out_dtype", [
    (1100, 700, 4032, torch.bfloat16),    # K % 256 = 192: a last slice of 64 elements
    (700, 1100, 4064, torch.float32),     # K % 64 = 32: scale rows 254 bytes apart (alternating alignment)
    (520, 300, 544, torch.bfloat16),      # 5 slices, the last one of 32 elements
])
def test_nvfp4_per_slice_scales(M, N, K, out_dtype):
    """NVFP4 GEMMs whose K is not a multiple of 256 (the per-slice scale-record kernel): scale
    rows at any even byte alignment, a last K slice that K ends inside.  Every 256-row and
    256-column band is sampled."""
    nv_gemm_check(gaussian_bf16((M, K), 1.0, SEED_X + 20), gaussian_bf16((N, K), STD_W, SEED_W + 20),
                  out_dtype=out_dtype, rows=stratified(M, 7), cols=stratified(N, 8),
                  label="per-slice scales %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K,out_dtype", [
    (4352, 4096, 768, torch.bfloat16),    # 272 tiles: last round split into halves; K / 128 = 6 slices
    (4352, 4160, 512, torch.float32),     # 289 tiles, the last column band 64 wide
    (6144, 4864, 1024, torch.bfloat16),   # 456 tiles: a last round too large to split
    (8192, 8192, 512, torch.float32),     # 1024 tiles: 4 whole tiles per workgroup
])
def test_persistent_tiles(M, N, K, out_dtype):
    """Launches that take the persistent NVFP4 kernel (per-tensor scales, K a multiple of 256,
    more tiles than a 256-CU device has CUs): several tiles per workgroup with the LDS ring and
    the operand pipeline carried from tile to tile (also when a tile's slice count is not a
    multiple of the ring's 4 stages), and a last round either whole or split into 256 x 128
    halves.  Every 256-row band and every 128-column band is sampled."""
    nv_gemm_check(gaussian_bf16((M, K), 1.0, SEED_X + 10), gaussian_bf16((N, K), STD_W, SEED_W + 10),
                  out_dtype=out_dtype, rows=stratified(M, 5), cols=stratified(N, 6, band=128),
                  label="persistent %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K,out_dtype", [
    (4352, 4104, 512, torch.bfloat16),   # 289 tiles, the last column band 8 wide
    (4100, 4160, 1024, torch.float32),   # 17 x 17 tiles, a ragged last row band
])
def test_mxfp8_ragged_bands_sampled(M, N, K, out_dtype):
    """MXFP8 launches of more tiles than a 256-CU device has CUs with narrow or ragged last
    bands (aligned scale records: K a multiple of 512).  Every 256-row and 128-column band is
    sampled."""
    mx_gemm_check(gaussian_bf16((M, K), 1.0, SEED_X + 30), gaussian_bf16((N, K), STD_W, SEED_W + 30), 1, 1,
                  out_dtype=out_dtype, rows=stratified(M, 13), cols=stratified(N, 14, band=128),
                  label="ragged bands %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mxfp8_slab_ragged_bands_sampled(out_dtype):
    """Slab-layout MXFP8 codes for a 4352 x 4160 output (289 tiles, ragged last column band),
    K = 1024."""
    slab_dgrad_check(4352, 1024, 4160, out_dtype, rows=stratified(4352, 15), cols=stratified(4160, 16, band=128),
                     label="slab ragged bands")


def test_hybrid_qwen3_8b_sampled():
    """Per-direction recipe at the Qwen3-8B FFN shape: NVFP4 rowwise forward GEMM; MXFP8
    dgrad dX = dY W (dY rowwise, W columnwise) and wgrad dW = dY^T X (both columnwise);
    plus the columnwise operand built from the rowwise-dequantized NVFP4 forward value."""
    X = gaussian_bf16((65536, 4096), 1.0, SEED_X)
    W = gaussian_bf16((12288, 4096), STD_W, SEED_W)
    nv_gemm_check(X, W, rows=stratified(65536, 5, extra=0), cols=stratified(12288, 6), label="hybrid fwd")
    dY = gaussian_bf16((65536, 12288), STD_DY, SEED_DY)
    mx_gemm_check(dY, W, 1, 2, rows=stratified(65536, 7, extra=0), cols=stratified(4096, 8), label="hybrid dgrad")
    mx_gemm_check(dY, X, 2, 2, out_dtype=torch.float32, rows=stratified(12288, 9), cols=stratified(4096, 10),
                  label="hybrid wgrad")


@pytest.mark.parametrize("shape,direction", [((4096, 1024), 2), ((256, 512), 3), ((96, 160), 1), ((200, 64), 1),
                                             ((320, 448), 1 | 4), ((320, 448), 3 | 4), ((1088, 128), 1 | 4),
                                             ((64, 144), 2), ((288, 416), 3)])
def test_fused_requantize_matches_chain(shape, direction):
    """mxfp8_requantize_nvfp4 = mxfp8_quantize(nvfp4_dequantize(.)) bit for bit, against the
    oracle's chain and the library's own two-call chain (ragged row counts for rowwise); with
    MX_SLAB (direction | 4) the codes are compared in the slab layout (ragged last bands).
    Column counts that are multiples of 32 stage the NVFP4 tile through LDS (416: a last tile
    with one of its four 16-byte code chunks per row inside), 144 takes the per-thread loads."""
    import oracle
    X = outlier_bf16(shape, seed=shape[0] + 3, mask_seed=shape[1] + 5)
    note("fused requantize %s dir=%d" % (shape, direction))
    q = bsq.nvfp4_quantize(X.to(DEV), direction=1)
    f = bsq.mxfp8_requantize_nvfp4(q["row_codes"], q["row_scales"], q["s_enc"][0:1], direction=direction)
    d = bsq.nvfp4_dequantize(q["row_codes"], q["row_scales"], q["s_enc"][0:1])
    m = bsq.mxfp8_quantize(d, direction=direction)
    torch.cuda.synchronize()
    rq = oracle.nvfp4_quantize(X, direction=1)
    rd = oracle.nvfp4_dequantize(rq["row_codes"], rq["row_scales"], float(rq["s_enc"][0]))
    rm = oracle.mxfp8_quantize(rd, direction=direction & 3)
    R, C = shape
    for key in (("row",) if direction & 1 else ()) + (("col",) if direction & 2 else ()):
        for part in ("_codes", "_scales"):
            got = f[key + part]
            if direction & 4 and part == "_codes":
                got = torch.from_numpy(from_slab(got, R, C) if key == "row" else from_slab(got, C, R))
            assert_bytes_equal(got, rm[key + part], "fused vs oracle " + key + part)
            assert torch.equal(f[key + part], m[key + part]), "fused vs two-call chain " + key + part


def slab_dgrad_check(T, N_out, N_in, out_dtype, rows=None, cols=None, label="", which=3):
    """dX[T, N_in] = dY W as the MXFP8 dgrad with slab-layout codes: dY rowwise (MX_SLAB) and
    W columnwise from its NVFP4 rowwise codes (fused requantize, MX_SLAB).  The slab buffers
    must hold exactly the oracle's codes, and the GEMM must match the oracle's GEMM.  which:
    1 only dY, 2 only W in the slab layout (the other row-major), 3 both."""
    import oracle
    note("mxfp8 slab dgrad %s T=%d out=%d in=%d %s" % (label, T, N_out, N_in, out_dtype))
    dy = gaussian_bf16((T, N_out), STD_DY, SEED_DY)
    W = gaussian_bf16((N_out, N_in), STD_W, SEED_W)
    qa = bsq.mxfp8_quantize(dy.to(DEV), direction=bsq.ROW | (bsq.MX_SLAB if which & 1 else 0))
    qw = bsq.nvfp4_quantize(W.to(DEV), direction=bsq.ROW)
    qb = bsq.mxfp8_requantize_nvfp4(qw["row_codes"], qw["row_scales"], qw["s_enc"][0:1],
                                    direction=bsq.COL | (bsq.MX_SLAB if which & 2 else 0))
    flags = (bsq.FMT_MX_SLAB_A if which & 1 else 0) | (bsq.FMT_MX_SLAB_B if which & 2 else 0)
    y = bsq.blockscaled_gemm(bsq.FMT_MXFP8 | flags, qa["row_codes"], qa["row_scales"], None,
                             qb["col_codes"], qb["col_scales"], None, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ra = oracle.mxfp8_quantize(dy, direction=oracle.ROW)
    rw = oracle.nvfp4_quantize(W, direction=oracle.ROW)
    rb = oracle.mxfp8_quantize(oracle.nvfp4_dequantize(rw["row_codes"], rw["row_scales"], float(rw["s_enc"][0])),
                               direction=oracle.COL)
    ga = from_slab(qa["row_codes"], T, N_out) if which & 1 else qa["row_codes"].cpu().numpy()
    gb = from_slab(qb["col_codes"], N_in, N_out) if which & 2 else qb["col_codes"].cpu().numpy()
    assert np.array_equal(ga, ra["row_codes"]), "dY slab codes"
    assert np.array_equal(gb, rb["col_codes"]), "W slab codes"
    assert_bytes_equal(qa["row_scales"], ra["row_scales"], "dY scales")
    assert_bytes_equal(qb["col_scales"], rb["col_scales"], "W scales")
    ref, sabs = oracle.blockscaled_gemm(oracle.FMT_MXFP8, ra["row_codes"], ra["row_scales"], 1.0,
                                        rb["col_codes"], rb["col_scales"], 1.0, rows=rows, cols=cols, with_abs=True)
    yc = sampled_output(y, rows, cols)
    want = bf16_round(ref) if out_dtype == torch.bfloat16 else ref
    err = rel_fro(yc, want)
    note("  rel_fro = %.3e" % err)
    assert err <= GEMM_TOL, err
    assert_gemm_elements(yc, ref, sabs, N_out, out_dtype == torch.bfloat16, "slab dgrad " + label,
                         mx=(ra["row_codes"], ra["row_scales"], rb["col_codes"], rb["col_scales"], rows, cols))


@pytest.mark.parametrize("shape", [(320, 448), (64, 64), (1088, 128)])
def test_mxfp8_cast_slab_layout(shape):
    """mxfp8_quantize with MX_SLAB in both directions and rowwise alone: the slab buffers hold
    exactly the oracle's row-major codes (ragged last bands, a single short band), scales
    unchanged."""
    import oracle
    R, C = shape
    note("mxfp8 slab cast shape=%s" % (shape,))
    x = outlier_bf16(shape, seed=R + 7, mask_seed=C + 9)
    q = bsq.mxfp8_quantize(x.to(DEV), direction=bsq.ROW | bsq.COL | bsq.MX_SLAB)
    torch.cuda.synchronize()
    r = oracle.mxfp8_quantize(x, direction=oracle.ROW | oracle.COL)
    assert np.array_equal(from_slab(q["row_codes"], R, C), r["row_codes"]), "row codes"
    assert np.array_equal(from_slab(q["col_codes"], C, R), r["col_codes"]), "col codes"
    assert_bytes_equal(q["row_scales"], r["row_scales"], "row scales")
    assert_bytes_equal(q["col_scales"], r["col_scales"], "col scales")
    # rowwise alone takes the streaming kernel
    q1 = bsq.mxfp8_quantize(x.to(DEV), direction=bsq.ROW | bsq.MX_SLAB)
    torch.cuda.synchronize()
    assert np.array_equal(from_slab(q1["row_codes"], R, C), r["row_codes"]), "row codes (rowwise only)"
    assert_bytes_equal(q1["row_scales"], r["row_scales"], "row scales (rowwise only)")


@pytest.mark.parametrize("which", [3, 1, 2])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mxfp8_slab_operands_ragged(out_dtype, which):
    """Slab-layout MXFP8 dgrad with a ragged last band in both operands (300 tokens, 320
    input features) and K = 1536 (three 8-slice scale groups): both operands in the slab
    layout, or one of them with the other row-major."""
    slab_dgrad_check(300, 1536, 320, out_dtype, label="ragged which=%d" % which, which=which)


def test_mxfp8_slab_dgrad_llama3_8b_sampled():
    """The slab-layout MXFP8 dgrad at the Llama-3-8B FFN shape, dX[16384, 4096] = dY W with
    K = 14336, as the bench launches it; every output tile sampled."""
    slab_dgrad_check(16384, 14336, 4096, torch.bfloat16, rows=stratified(16384, 11), cols=stratified(4096, 12),
                     label="llama3-8b")


@pytest.mark.parametrize("factor", [1e-34, 1e-25, 1e30, 5e35])
def test_fused_requantize_extreme_tensor_scales(factor):
    """Inputs scaled so that the per-block quotients leave the normal range (tiny tensor amax
    with small block scales) or approach overflow (huge amax): the fused kernel's two-quotient
    shortcut must hand those rows to its per-element path and stay bit-identical."""
    import oracle
    X = (outlier_bf16((256, 512), seed=91, mask_seed=92).float() * factor).to(torch.bfloat16)
    assert torch.isfinite(X.float()).all()
    note("fused requantize extreme factor=%g" % factor)
    q = bsq.nvfp4_quantize(X.to(DEV), direction=1)
    f = bsq.mxfp8_requantize_nvfp4(q["row_codes"], q["row_scales"], q["s_enc"][0:1], direction=3)
    torch.cuda.synchronize()
    rq = oracle.nvfp4_quantize(X, direction=1)
    rd = oracle.nvfp4_dequantize(rq["row_codes"], rq["row_scales"], float(rq["s_enc"][0]))
    rm = oracle.mxfp8_quantize(rd, direction=3)
    for key in ("row", "col"):
        for part in ("_codes", "_scales"):
            assert_bytes_equal(f[key + part], rm[key + part], "fused vs oracle " + key + part)


def test_hybrid_rowwise_dequantized_source():
    """columnwise_source = rowwise_dequantized: MXFP8 columnwise of bf16(dequant(NVFP4 rowwise X));
    compared bit for bit with the oracle's chain on a [4096, 1024] slice of the workload."""
    import oracle
    from tests.gpu_common import assert_bytes_equal
    X = gaussian_bf16((4096, 1024), 1.0, SEED_X)
    note("hybrid rowwise_dequantized chain [4096,1024]")
    q = bsq.nvfp4_quantize(X.to(DEV), direction=1)
    d = bsq.nvfp4_dequantize(q["row_codes"], q["row_scales"], q["s_enc"][0:1])
    m = bsq.mxfp8_quantize(d, direction=2)
    torch.cuda.synchronize()
    rq = oracle.nvfp4_quantize(X, direction=1)
    rd = oracle.nvfp4_dequantize(rq["row_codes"], rq["row_scales"], float(rq["s_enc"][0]))
    rm = oracle.mxfp8_quantize(rd, direction=2)
    assert_bytes_equal(m["col_codes"], rm["col_codes"], "col codes")
    assert_bytes_equal(m["col_scales"], rm["col_scales"], "col scales")
