"""GPU parity of the NVFP4 linear layer (nvfp4_linear_forward / nvfp4_linear_backward)
against the same sequence of oracle steps: forward Y from rowwise RNE operands, the saved
activation X columnwise with RHT + SR (stream 1), backward dY in both directions with RHT +
SR (stream 0), W columnwise with RHT + SR (stream 2), dW over tokens and dX over the output
features.  Every quantized operand is checked bit for bit through the standalone entry
points (which the layer calls), and Y, dX, dW to the GEMM bar (relative Frobenius error
<= 2e-3 against the oracle output rounded as stored, and every element within the
rounding-error bound of fp32 accumulation)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsq
from synthetic import (SEED_DY, SEED_SIGNS, SEED_W, SEED_X, STD_DY, STD_W, gaussian_bf16, rht_signs)
from tests.gpu_common import GEMM_TOL, assert_gemm_elements, bf16_round, note, rel_fro, stratified

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SEED = 42


def oracle_layer(x, w, dy, signs, rows=None, cols=None, wrows=None, wcols=None, xrows=None, xcols=None):
    """The layer's steps on the oracle (each step is a pinned oracle function)."""
    import oracle
    sg = signs.numpy()
    qx = oracle.nvfp4_quantize(x, direction=oracle.ROW)
    qw = oracle.nvfp4_quantize(w, direction=oracle.ROW)
    y = oracle.blockscaled_gemm(oracle.FMT_NVFP4, qx["row_codes"], qx["row_scales"], float(qx["s_enc"][0]),
                                qw["row_codes"], qw["row_scales"], float(qw["s_enc"][0]), rows=rows, cols=cols,
                                with_abs=True)
    xc = oracle.nvfp4_quantize(x, direction=oracle.COL, rounding=oracle.SR, sr_seed=SEED, sr_stream=1, signs=sg)
    qdy = oracle.nvfp4_quantize(dy, direction=oracle.ROW | oracle.COL, rounding=oracle.SR, sr_seed=SEED,
                                sr_stream=0, signs=sg)
    wc = oracle.nvfp4_quantize(w, direction=oracle.COL, rounding=oracle.SR, sr_seed=SEED, sr_stream=2, signs=sg)
    dw = oracle.blockscaled_gemm(oracle.FMT_NVFP4, qdy["col_codes"], qdy["col_scales"], float(qdy["s_enc"][1]),
                                 xc["col_codes"], xc["col_scales"], float(xc["s_enc"][1]), rows=wrows, cols=wcols,
                                 with_abs=True)
    dx = oracle.blockscaled_gemm(oracle.FMT_NVFP4, qdy["row_codes"], qdy["row_scales"], float(qdy["s_enc"][0]),
                                 wc["col_codes"], wc["col_scales"], float(wc["s_enc"][1]), rows=xrows, cols=xcols,
                                 with_abs=True)
    return y, dx, dw   # each (C, sum of absolute products)


def run_layer(T, K, N, sample=None):
    note("nvfp4 linear T=%d K=%d N=%d" % (T, K, N))
    x = gaussian_bf16((T, K), 1.0, SEED_X)
    w = gaussian_bf16((N, K), STD_W, SEED_W)
    dy = gaussian_bf16((T, N), STD_DY, SEED_DY)
    signs = rht_signs(SEED_SIGNS)
    y, saved = bsq.nvfp4_linear_forward(x.to(DEV), w.to(DEV), SEED, signs)
    dx, dw = bsq.nvfp4_linear_backward(dy.to(DEV), w.to(DEV), saved, SEED, signs)
    torch.cuda.synchronize()
    if sample is None:
        ry, rdx, rdw = oracle_layer(x, w, dy, signs)
        gy, gdx, gdw = (t.float().cpu().numpy().astype(np.float64) for t in (y, dx, dw))
    else:
        # every 256 x 256 output tile of each GEMM: first and last index of each band and one more
        r, c, wr, wcl, xr, xcl = (stratified(n, sample + i) for i, n in enumerate((T, N, N, K, T, K)))
        ry, rdx, rdw = oracle_layer(x, w, dy, signs, r, c, wr, wcl, xr, xcl)

        def pick(t, rows, cols):
            return t[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy()
        gy, gdw, gdx = (pick(t, a, b).astype(np.float64) for t, a, b in ((y, r, c), (dw, wr, wcl), (dx, xr, xcl)))
    for got, (ref, sabs), nm, bf, kk in ((gy, ry, "Y", True, K), (gdx, rdx, "dX", True, N), (gdw, rdw, "dW", False, T)):
        err = rel_fro(got, bf16_round(ref) if bf else ref)
        note("  %s rel_fro = %.3e" % (nm, err))
        assert err <= GEMM_TOL, (nm, err)
        assert_gemm_elements(got, ref, sabs, kk, bf, nm)


@pytest.mark.parametrize("T,K,N", [(256, 512, 384), (96, 160, 224), (512, 256, 1024)])
def test_linear_layer_small(T, K, N):
    run_layer(T, K, N)


def test_linear_quantized_operands_match_the_standalone_calls():
    """The layer's saved activation is the columnwise RHT + SR quantization of X (stream 1):
    the saved buffer starts with exactly those codes."""
    import oracle
    T, K, N = 128, 256, 96
    x = gaussian_bf16((T, K), 1.0, 5)
    w = gaussian_bf16((N, K), STD_W, 6)
    signs = rht_signs(SEED_SIGNS)
    note("nvfp4 linear saved operand")
    _, saved = bsq.nvfp4_linear_forward(x.to(DEV), w.to(DEV), SEED, signs)
    torch.cuda.synchronize()
    ref = oracle.nvfp4_quantize(x, direction=oracle.COL, rounding=oracle.SR, sr_seed=SEED, sr_stream=1,
                                signs=signs.numpy())
    n = K * T // 2
    assert np.array_equal(saved[:n].cpu().numpy(), ref["col_codes"].reshape(-1))
    assert saved.numel() * 3 < T * K * 2, "the saved activation must be smaller than bf16 X"


def test_linear_layer_llama3_8b_sampled():
    """The Llama-3-8B FFN up-projection layer (16384 tokens, 4096 -> 14336), outputs compared
    on rows x columns that touch every output tile of each GEMM."""
    run_layer(16384, 4096, 14336, sample=77)
