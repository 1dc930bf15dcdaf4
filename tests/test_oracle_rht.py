"""Pins of the oracle's 16-point random Hadamard transform (RHT).

The recipe applies an RHT with a random +-1 sign vector along the quantized
(contraction) dimension and relies on the transform cancelling in the GEMM when
both operands share the sign vector (torchtitan PR #3914 "Add an NVFP4
quantization converter", Summary / What changed, and the review reply on why the
sign vector must be replicated).  Pins: the closed-form matrix (Sylvester order,
1/4 normalisation, sign vector on the input side), exact orthogonality, exact
inversion on integer inputs, preservation of products within the binary32 error
bound, and the negative case of different sign vectors.
"""
import numpy as np
import pytest


def sylvester16():
    H = np.empty((16, 16))
    for i in range(16):
        for j in range(16):
            H[i, j] = (-1) ** bin(i & j).count("1")
    return H


def rht_matrix(orc, signs):
    """The oracle's transform as a matrix R with y = x R (rows = images of the unit vectors)."""
    return np.stack([orc.rht16(np.eye(16)[i], signs) for i in range(16)]).astype(np.float64)


def test_matrix_closed_form(orc):
    from synthetic import rht_signs
    for seed in [7, 8, 9]:
        d = rht_signs(seed).numpy().astype(np.float64)
        R = rht_matrix(orc, d)
        assert np.array_equal(R, np.diag(d) @ sylvester16() / 4.0)


def test_orthogonal_exactly(orc):
    from synthetic import rht_signs
    d = rht_signs(7).numpy()
    R = rht_matrix(orc, d)
    assert np.array_equal(R @ R.T, np.eye(16))
    assert np.array_equal(sylvester16() @ sylvester16().T, 16 * np.eye(16))


def test_integer_inputs_invert_exactly(orc):
    """With integer inputs |x| <= 2^10 every butterfly sum is exact, so applying the
    transform and then its transpose (H d / 4, H symmetric) returns x bit for bit."""
    from synthetic import rht_signs
    d = rht_signs(7).numpy()
    rng = np.random.default_rng(0)
    for _ in range(200):
        x = rng.integers(-1024, 1025, 16).astype(np.float32)
        y = orc.rht16(x, d)
        back = orc.rht16(y, np.ones(16, np.int8)) * d.astype(np.float32)
        assert np.array_equal(back, x)


def test_one_hot(orc):
    from synthetic import rht_signs
    d = rht_signs(7).numpy()
    for i in range(16):
        y = orc.rht16(np.eye(16, dtype=np.float32)[i], d)
        assert np.all(np.abs(y) == 0.25)
        assert np.all(np.sign(y) == d[i] * sylvester16()[i])


def test_product_preserved_with_shared_signs(orc):
    """(x R)(w R)^T = x w^T: the transform cancels in a GEMM when both operands share d."""
    import torch
    from synthetic import gaussian_bf16, rht_signs
    d = rht_signs(7).numpy()
    x = gaussian_bf16((8, 256), 1.0, 1)
    w = gaussian_bf16((8, 256), 1.0, 2)
    xr = orc.rht_apply(x, 1, d).astype(np.float64)
    wr = orc.rht_apply(w, 1, d).astype(np.float64)
    ref = x.to(torch.float64).numpy() @ w.to(torch.float64).numpy().T
    got = xr @ wr.T
    # binary32 butterfly: each output carries <= 4 roundings of relative size 2^-24
    scale = np.abs(x.to(torch.float64).numpy()) @ np.abs(w.to(torch.float64).numpy()).T
    assert np.all(np.abs(got - ref) <= 1e-5 * scale + 1e-30)


def test_product_not_preserved_with_different_signs(orc):
    import torch
    from synthetic import gaussian_bf16, rht_signs
    x = gaussian_bf16((8, 256), 1.0, 1)
    w = gaussian_bf16((8, 256), 1.0, 2)
    xr = orc.rht_apply(x, 1, rht_signs(7).numpy()).astype(np.float64)
    wr = orc.rht_apply(w, 1, rht_signs(8).numpy()).astype(np.float64)
    ref = x.to(torch.float64).numpy() @ w.to(torch.float64).numpy().T
    rel = np.linalg.norm(xr @ wr.T - ref) / np.linalg.norm(ref)
    assert rel > 0.1


def test_axes_agree_with_transpose(orc):
    import torch
    from synthetic import gaussian_bf16, rht_signs
    d = rht_signs(7).numpy()
    x = gaussian_bf16((48, 32), 1.0, 3)
    a0 = orc.rht_apply(x, 0, d)
    a1t = orc.rht_apply(x.t().contiguous(), 1, d)
    assert np.array_equal(a0, a1t.T)
    # and along a row, rht_apply is rht16 on each 16-block
    xf = x.to(torch.float32).numpy()
    a1 = orc.rht_apply(x, 1, d)
    assert np.array_equal(a1[5, 16:32], orc.rht16(xf[5, 16:32], d))


def test_rht_quantize_uses_transformed_amax(orc):
    """With a sign vector, each direction's tensor amax is the amax of the transformed values."""
    from synthetic import gaussian_bf16, rht_signs
    d = rht_signs(7).numpy()
    x = gaussian_bf16((64, 32), 1.0, 4)
    q = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL, signs=d)
    assert q["amax"][0] == np.abs(orc.rht_apply(x, 1, d)).max()
    assert q["amax"][1] == np.abs(orc.rht_apply(x, 0, d)).max()
    assert q["amax"][0] != q["amax"][1]
