"""GPU parity of row-scaled NVFP4 (one outer scale per row) against the CPU oracle, through
the C ABI: bit-exact codes, scales, per-row amax and per-row tensor scales; and the GEMM
with per-row tensor scales on either or both operands, to the GEMM bar (relative Frobenius
error <= 2e-3 against the oracle output rounded as the GPU stores it).

The quantizer splits a row over 2..256 threads depending on its length (at most four
16-byte units per thread and chunk), so the shapes cover every split: cols 16 and 64 (2
threads), 400 (16), 4096 (128, two waves), 8192 (256, one register-resident chunk) and
rows longer than one chunk (cols 14336, 16400, 40000: read twice); row counts that leave
a partial workgroup, and enough rows that the grid-stride loop runs more than once.  The GEMM cases cover full 256 x 256
tiles (staged epilogue), ragged edge tiles and K not a multiple of 256 (the register-staged
NVFP4 kernel)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsq
from synthetic import SEED_SIGNS, SEED_SR_KEY, SEED_X, STD_W, gaussian_bf16, outlier_bf16, rht_signs
from tests.gpu_common import (GEMM_TOL, assert_bytes_equal, assert_f32_equal, assert_gemm_elements, bf16_round, note,
                              rel_fro, stratified)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def check_rowscaled(x_cpu, rounding=0, seed=0, stream=0, signs=None, label=""):
    import oracle
    note("nvfp4 rowscaled %s shape=%s rnd=%d rht=%s" % (label, tuple(x_cpu.shape), rounding, signs is not None))
    got = bsq.nvfp4_quantize_rowscaled(x_cpu.to(DEV), rounding=rounding, sr_seed=seed, sr_stream=stream,
                                       rht_signs=signs)
    torch.cuda.synchronize()
    ref = oracle.nvfp4_quantize_rowscaled(x_cpu, rounding=rounding, sr_seed=seed, sr_stream=stream,
                                          signs=None if signs is None else signs.numpy())
    assert_f32_equal(got["amax"], ref["amax"], label + " amax")
    assert_f32_equal(got["s_enc"], ref["s_enc"], label + " s_enc")
    assert_bytes_equal(got["scales"], ref["scales"], label + " scales")
    assert_bytes_equal(got["codes"], ref["codes"], label + " codes")
    return got, ref


@pytest.mark.parametrize("shape", [(64, 16), (37, 64), (300, 400), (5, 4096), (129, 4096), (3, 8192),
                                   (17, 14336), (4, 16400), (3, 40000)])
def test_rowscaled_rne_every_row_split(shape):
    check_rowscaled(outlier_bf16(shape, seed=shape[1], mask_seed=shape[0]), label="rne")


@pytest.mark.parametrize("shape", [(33, 64), (70, 4096), (3, 8192), (2, 20000)])
def test_rowscaled_rht_sr(shape):
    check_rowscaled(gaussian_bf16(shape, 1e-2, 61), rounding=1, seed=-987654321, stream=5,
                    signs=rht_signs(SEED_SIGNS), label="rht+sr")


@pytest.mark.parametrize("rounding,use_rht", [(0, True), (1, False)])
def test_rowscaled_rht_or_sr_alone(rounding, use_rht):
    check_rowscaled(gaussian_bf16((96, 1024), 1.0, 62), rounding=rounding, seed=SEED_SR_KEY,
                    signs=rht_signs(SEED_SIGNS) if use_rht else None, label="rht-or-sr")


def test_rowscaled_grid_stride():
    """More row groups than the grid holds (8192 workgroups): 2 threads per row
    (1100000 rows of 16) and 256 threads per row (8300 rows of 14336), so workgroups walk
    several row groups.  Rows are quantized independently under RNE, so the oracle runs on
    sampled rows -- the last ones (reached only on a second pass of the stride loop) and a
    random spread."""
    import oracle
    for rows, cols, seed in ((1100000, 16, 63), (8300, 14336, 64)):
        x = gaussian_bf16((rows, cols), 1.0, seed)
        note("nvfp4 rowscaled stride shape=%s" % ((rows, cols),))
        got = bsq.nvfp4_quantize_rowscaled(x.to(DEV))
        torch.cuda.synchronize()
        rng = np.random.default_rng(seed)
        pick = np.unique(np.concatenate([np.arange(rows - 40, rows), rng.choice(rows, 200, replace=False)]))
        ref = oracle.nvfp4_quantize_rowscaled(x[torch.from_numpy(pick)].contiguous())
        idx = torch.from_numpy(pick).to(DEV)
        assert_f32_equal(got["amax"][idx], ref["amax"], "stride amax")
        assert_f32_equal(got["s_enc"][idx], ref["s_enc"], "stride s_enc")
        assert_bytes_equal(got["scales"][idx], ref["scales"], "stride scales")
        assert_bytes_equal(got["codes"][idx], ref["codes"], "stride codes")


def test_rowscaled_rows_of_very_different_magnitude():
    """Rows whose amax differ by many binades (where the per-row scale matters), zero rows,
    subnormal and huge bf16 values."""
    g = torch.Generator().manual_seed(65)
    x = torch.randn((64, 512), generator=g) * torch.logspace(-30, 30, 64).reshape(64, 1)
    x[5] = 0.0
    x[9, :16] = torch.tensor([1e-40, -1e-39] + [0.0] * 14)
    x[11, 3] = -3.0e38
    check_rowscaled(x.to(torch.bfloat16), label="magnitudes")
    check_rowscaled(x.to(torch.bfloat16), rounding=1, seed=7, label="magnitudes-sr")


def test_rowscaled_empty_and_zero_cols():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    got = bsq.nvfp4_quantize_rowscaled(x)
    torch.cuda.synchronize()
    assert got["amax"].numel() == 0
    note("nvfp4 rowscaled cols=0")
    x = torch.zeros((5, 0), dtype=torch.bfloat16, device=DEV)
    got = bsq.nvfp4_quantize_rowscaled(x)
    torch.cuda.synchronize()
    assert got["amax"].cpu().tolist() == [0.0] * 5 and got["s_enc"].cpu().tolist() == [1.0] * 5


def test_rowscaled_activations_llama3_8b():
    """The Llama-3-8B FFN input activations [16384, 4096], row-scaled RNE."""
    check_rowscaled(gaussian_bf16((16384, 4096), 1.0, SEED_X), label="fwd X")


# ----------------------------------------------------------------- GEMM with per-row scales

def rowscaled_gemm_check(M, N, K, a_rows, b_rows, out_dtype=torch.bfloat16, rows=None, cols=None, label=""):
    import oracle
    note("nvfp4 gemm rowscaled %s M=%d N=%d K=%d a_rows=%d b_rows=%d out=%s"
         % (label, M, N, K, a_rows, b_rows, out_dtype))
    # A rows span many binades so that a per-row scale applied to the wrong row shows
    a_cpu = (gaussian_bf16((M, K), 1.0, 71).float()
             * torch.logspace(-3, 3, M).reshape(M, 1)).to(torch.bfloat16)
    b_cpu = (gaussian_bf16((N, K), STD_W, 72).float()
             * torch.logspace(2, -2, N).reshape(N, 1)).to(torch.bfloat16)
    ops, refs = [], []
    for t, per_row in ((a_cpu, a_rows), (b_cpu, b_rows)):
        if per_row:
            q = bsq.nvfp4_quantize_rowscaled(t.to(DEV))
            r = oracle.nvfp4_quantize_rowscaled(t)
            ops.append((q["codes"], q["scales"], q["s_enc"]))
            refs.append((r["codes"], r["scales"], r["s_enc"]))
        else:
            q = bsq.nvfp4_quantize(t.to(DEV), direction=bsq.ROW)
            r = oracle.nvfp4_quantize(t, direction=oracle.ROW)
            ops.append((q["row_codes"], q["row_scales"], q["s_enc"][0:1]))
            refs.append((r["row_codes"], r["row_scales"], float(r["s_enc"][0])))
    fmt = bsq.FMT_NVFP4 | (bsq.FMT_A_ROWSCALED if a_rows else 0) | (bsq.FMT_B_ROWSCALED if b_rows else 0)
    y = bsq.blockscaled_gemm(fmt, *ops[0], *ops[1], out_dtype=out_dtype)
    torch.cuda.synchronize()
    for (gc, gs, gS), (rc, rs, rS), nm in zip(ops, refs, "AB"):
        assert_bytes_equal(gc, rc, nm + " codes")
        assert_bytes_equal(gs, rs, nm + " scales")
        assert_f32_equal(gS, np.atleast_1d(np.asarray(rS, np.float32)), nm + " s_enc")
    ref, sabs = oracle.blockscaled_gemm(oracle.FMT_NVFP4, *refs[0], *refs[1], rows=rows, cols=cols, with_abs=True)
    yc = y.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        yc = yc[np.asarray(rows)][:, np.asarray(cols)]
    assert_gemm_elements(yc, ref, sabs, K, out_dtype == torch.bfloat16, "row-scaled " + label)
    want = bf16_round(ref) if out_dtype == torch.bfloat16 else ref
    # relative error per output row, so that rows of small magnitude count as much as large
    den = np.maximum(np.linalg.norm(want, axis=1), 1e-300)
    err = float(np.max(np.linalg.norm(yc - want, axis=1) / den))
    note("  max per-row rel_fro = %.3e, total = %.3e" % (err, rel_fro(yc, want)))
    assert err <= GEMM_TOL, err


@pytest.mark.parametrize("a_rows,b_rows", [(1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(512, 512, 1024), (200, 72, 256), (300, 520, 768), (130, 96, 160)])
def test_rowscaled_gemm(M, N, K, a_rows, b_rows):
    rowscaled_gemm_check(M, N, K, a_rows, b_rows, label="small")


@pytest.mark.parametrize("a_rows,b_rows", [(1, 0), (1, 1)])
def test_rowscaled_gemm_f32_out(a_rows, b_rows):
    rowscaled_gemm_check(512, 256, 512, a_rows, b_rows, out_dtype=torch.float32, label="f32")
    rowscaled_gemm_check(260, 100, 288, a_rows, b_rows, out_dtype=torch.float32, label="f32-ragged")


@pytest.mark.parametrize("M,N,K", [(4352, 4160, 512), (8192, 8192, 768)])
def test_rowscaled_gemm_persistent(M, N, K):
    """Row-scaled A with per-tensor B and bf16 out on the persistent kernel: several tiles per
    workgroup, each tile's per-row factors put in LDS before its stores, a last round split
    into halves (289 tiles) or whole (1024 tiles), a ragged last column band.  Every 256-row
    and 128-column band is sampled."""
    from tests.gpu_common import stratified
    rowscaled_gemm_check(M, N, K, 1, 0, rows=stratified(M, 78), cols=stratified(N, 79, band=128),
                         label="persistent")


def test_rowscaled_gemm_equal_scales_is_bitwise_per_tensor():
    """Per-row scales that all equal the tensor scale give the per-tensor GEMM bit for bit
    when one operand is row-scaled (the factor is the same binary64 quotient rounded once)."""
    x = gaussian_bf16((512, 512), 1.0, 73).to(DEV)
    w = gaussian_bf16((256, 512), 1.0, 74).to(DEV)
    qa = bsq.nvfp4_quantize(x, direction=bsq.ROW)
    qb = bsq.nvfp4_quantize(w, direction=bsq.ROW)
    note("nvfp4 gemm rowscaled equal-scales")
    per_t = bsq.blockscaled_gemm(bsq.FMT_NVFP4, qa["row_codes"], qa["row_scales"], qa["s_enc"][0:1],
                                 qb["row_codes"], qb["row_scales"], qb["s_enc"][0:1])
    sa = qa["s_enc"][0:1].repeat(512).contiguous()
    per_r = bsq.blockscaled_gemm(bsq.FMT_NVFP4 | bsq.FMT_A_ROWSCALED, qa["row_codes"], qa["row_scales"], sa,
                                 qb["row_codes"], qb["row_scales"], qb["s_enc"][0:1])
    torch.cuda.synchronize()
    assert torch.equal(per_t.view(torch.int16), per_r.view(torch.int16))


def test_rowscaled_gemm_llama3_8b_fprop_sampled():
    """Forward GEMM of the Llama-3-8B FFN up-projection with row-scaled activations
    [16384, 4096] and per-tensor weights [14336, 4096], compared on rows x cols that touch
    every output tile."""
    import oracle
    M, N, K = 16384, 14336, 4096
    note("nvfp4 gemm rowscaled llama3-8b fprop")
    x = gaussian_bf16((M, K), 1.0, SEED_X)
    w = gaussian_bf16((N, K), STD_W, 75)
    qa = bsq.nvfp4_quantize_rowscaled(x.to(DEV))
    qb = bsq.nvfp4_quantize(w.to(DEV), direction=bsq.ROW)
    y = bsq.blockscaled_gemm(bsq.FMT_NVFP4 | bsq.FMT_A_ROWSCALED, qa["codes"], qa["scales"], qa["s_enc"],
                             qb["row_codes"], qb["row_scales"], qb["s_enc"][0:1])
    torch.cuda.synchronize()
    ra = oracle.nvfp4_quantize_rowscaled(x)
    rb = oracle.nvfp4_quantize(w, direction=oracle.ROW)
    assert_bytes_equal(qa["codes"], ra["codes"], "A codes")
    assert_f32_equal(qa["s_enc"], ra["s_enc"], "A s_enc")
    rows, cols = stratified(M, 76), stratified(N, 77)
    ref, sabs = oracle.blockscaled_gemm(oracle.FMT_NVFP4, ra["codes"], ra["scales"], ra["s_enc"], rb["row_codes"],
                                        rb["row_scales"], float(rb["s_enc"][0]), rows=rows, cols=cols, with_abs=True)
    yc = y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy().astype(np.float64)
    err = rel_fro(yc, bf16_round(ref))
    note("  rel_fro = %.3e" % err)
    assert err <= GEMM_TOL, err
    assert_gemm_elements(yc, ref, sabs, K, True, "row-scaled llama3-8b fprop")
