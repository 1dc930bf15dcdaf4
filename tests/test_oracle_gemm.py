"""Pins of the oracle's block-scaled GEMM and of the hybrid (per-direction) pairings.

The GEMM consumes quantized operands with fp32 (here: binary64) accumulation,
C = A B^T with both operands stored along K; the operand direction that each
GEMM of a linear layer uses follows TransformerEngine PR #2817 "Hybrid
quantization" (GEMM dispatch flowchart: rowwise for fprop's operands,
columnwise for the wgrad operands).  Pins: a pure-Python triple loop over
closed-form decoded values on tiny shapes, a constant-operand closed form,
numpy's matmul of independently dequantized operands, and the hybrid-recipe
invariants of that page (a hybrid with the same format in both directions is
the plain recipe; the rowwise-dequantized source of an exactly representable
tensor equals the original).
"""
import numpy as np
import pytest
import torch

E2M1 = [0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6]


def e4m3_py(b: int) -> float:
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    v = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if s else v


def nvfp4_elem(codes, scales, s, r, k):
    byte = int(codes[r, k // 2])
    c = byte & 0xF if k % 2 == 0 else byte >> 4
    return E2M1[c] * e4m3_py(int(scales[r, k // 16])) / s


def test_nvfp4_gemm_bruteforce_tiny(orc):
    from synthetic import gaussian_bf16
    x = gaussian_bf16((6, 32), 1.0, 1)
    w = gaussian_bf16((5, 32), 0.02, 2)
    qa = orc.nvfp4_quantize(x)
    qb = orc.nvfp4_quantize(w)
    sa, sb = float(qa["s_enc"][0]), float(qb["s_enc"][0])
    got = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["row_codes"], qa["row_scales"], sa,
                               qb["row_codes"], qb["row_scales"], sb)
    for m in range(6):
        for n in range(5):
            ref = 0.0
            for k in range(32):
                ref += nvfp4_elem(qa["row_codes"], qa["row_scales"], sa, m, k) * \
                    nvfp4_elem(qb["row_codes"], qb["row_scales"], sb, n, k)
            assert got[m, n] == pytest.approx(ref, rel=1e-14, abs=1e-300)


def test_mxfp8_gemm_bruteforce_tiny(orc):
    from synthetic import gaussian_bf16
    x = gaussian_bf16((4, 64), 1.0, 3)
    w = gaussian_bf16((3, 64), 1.0, 4)
    qa = orc.mxfp8_quantize(x)
    qb = orc.mxfp8_quantize(w)
    got = orc.blockscaled_gemm(orc.FMT_MXFP8, qa["row_codes"], qa["row_scales"], 1.0,
                               qb["row_codes"], qb["row_scales"], 1.0)
    for m in range(4):
        for n in range(3):
            ref = 0.0
            for k in range(64):
                va = e4m3_py(int(qa["row_codes"][m, k])) * 2.0 ** (int(qa["row_scales"][m, k // 32]) - 127)
                vb = e4m3_py(int(qb["row_codes"][n, k])) * 2.0 ** (int(qb["row_scales"][n, k // 32]) - 127)
                ref += va * vb
            assert got[m, n] == pytest.approx(ref, rel=1e-14)


def test_constant_operands_closed_form(orc):
    """All codes c, all scales s: C = K * (E2M1(ca) E4M3(sa) / Sa) * (E2M1(cb) E4M3(sb) / Sb)."""
    M, N, K = 3, 4, 64
    a_codes = np.full((M, K // 2), 0x55, np.uint8)     # code 5 (3.0) in both nibbles
    b_codes = np.full((N, K // 2), 0xEE, np.uint8)     # code 0xE (-4.0)
    a_sc = np.full((M, K // 16), 0x38, np.uint8)       # 1.0
    b_sc = np.full((N, K // 16), 0x4C, np.uint8)       # 1.5 * 2^2 = 6.0
    out = orc.blockscaled_gemm(orc.FMT_NVFP4, a_codes, a_sc, 2.0, b_codes, b_sc, 0.5)
    assert np.all(out == K * (3.0 * 1.0 / 2.0) * (-4.0 * 6.0 / 0.5))


def test_matches_numpy_matmul_of_dequantized(orc):
    from synthetic import gaussian_bf16
    x = gaussian_bf16((40, 96), 1.0, 5)
    w = gaussian_bf16((24, 96), 0.02, 6)
    qa, qb = orc.nvfp4_quantize(x), orc.nvfp4_quantize(w)

    def deq(q):
        c = q["row_codes"]
        codes = np.empty((c.shape[0], c.shape[1] * 2), np.int64)
        codes[:, 0::2], codes[:, 1::2] = c & 0xF, c >> 4
        sc = np.vectorize(e4m3_py)(q["row_scales"].astype(np.int64))
        return np.array(E2M1)[codes] * np.repeat(sc, 16, axis=1) / float(q["s_enc"][0])
    ref = deq(qa) @ deq(qb).T
    got = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["row_codes"], qa["row_scales"], qa["s_enc"][0],
                               qb["row_codes"], qb["row_scales"], qb["s_enc"][0])
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)
    sub = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["row_codes"], qa["row_scales"], qa["s_enc"][0],
                               qb["row_codes"], qb["row_scales"], qb["s_enc"][0],
                               rows=[39, 0, 7], cols=[3, 23])
    assert np.array_equal(sub, got[[39, 0, 7]][:, [3, 23]])
    # the sum of absolute products (the error-bound scale the GPU parity gates use) is the
    # product of the absolute dequantized operands, and at least |C|
    c2, s2 = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["row_codes"], qa["row_scales"], qa["s_enc"][0],
                                  qb["row_codes"], qb["row_scales"], qb["s_enc"][0], rows=[39, 0, 7], cols=[3, 23],
                                  with_abs=True)
    assert np.array_equal(c2, sub)
    np.testing.assert_allclose(s2, (np.abs(deq(qa)) @ np.abs(deq(qb)).T)[[39, 0, 7]][:, [3, 23]], rtol=1e-12)
    assert np.all(s2 >= np.abs(c2))


def test_quantized_gemm_close_to_exact_product(orc):
    """NVFP4 is a ~4-bit format: the quantized product tracks x w^T to within the
    format's error (a few percent), far from a transposed or mis-scaled result."""
    from synthetic import gaussian_bf16
    x = gaussian_bf16((64, 256), 1.0, 7)
    w = gaussian_bf16((48, 256), 0.02, 8)
    qa, qb = orc.nvfp4_quantize(x), orc.nvfp4_quantize(w)
    got = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["row_codes"], qa["row_scales"], qa["s_enc"][0],
                               qb["row_codes"], qb["row_scales"], qb["s_enc"][0])
    ref = x.to(torch.float64).numpy() @ w.to(torch.float64).numpy().T
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 0.02 < rel < 0.2


def test_wgrad_rht_sr_product_tracks_exact(orc):
    """wgrad pairing: both operands columnwise (blocks along the token dim), RHT with a
    shared sign vector and SR; dW = dY^T X is recovered to the format's accuracy."""
    from synthetic import gaussian_bf16, rht_signs
    dy = gaussian_bf16((128, 32), 1e-4, 1)
    x = gaussian_bf16((128, 48), 1.0, 2)
    d = rht_signs(7).numpy()
    qa = orc.nvfp4_quantize(dy, direction=orc.COL, rounding=orc.SR, sr_seed=42, sr_stream=0, signs=d)
    qb = orc.nvfp4_quantize(x, direction=orc.COL, rounding=orc.SR, sr_seed=42, sr_stream=1, signs=d)
    got = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["col_codes"], qa["col_scales"], qa["s_enc"][1],
                               qb["col_codes"], qb["col_scales"], qb["s_enc"][1])
    ref = dy.to(torch.float64).numpy().T @ x.to(torch.float64).numpy()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 0.25
    # with different sign vectors the transform no longer cancels
    qb2 = orc.nvfp4_quantize(x, direction=orc.COL, rounding=orc.SR, sr_seed=42, sr_stream=1,
                             signs=rht_signs(8).numpy())
    bad = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["col_codes"], qa["col_scales"], qa["s_enc"][1],
                               qb2["col_codes"], qb2["col_scales"], qb2["s_enc"][1])
    assert np.linalg.norm(bad - ref) / np.linalg.norm(ref) > 0.5


def test_hybrid_same_format_is_plain_recipe(orc):
    """A per-direction recipe with NVFP4 in both directions gives the plain NVFP4 row+col
    quantization bit for bit (the page's hybrid-vs-base parity check)."""
    from synthetic import gaussian_bf16
    x = gaussian_bf16((64, 96), 1.0, 10)
    both = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL)
    row = orc.nvfp4_quantize(x, direction=orc.ROW)
    col = orc.nvfp4_quantize(x, direction=orc.COL)
    for k in ("row_codes", "row_scales"):
        assert np.array_equal(both[k], row[k])
    for k in ("col_codes", "col_scales"):
        assert np.array_equal(both[k], col[k])
    m_both = orc.mxfp8_quantize(x, direction=orc.ROW | orc.COL)
    m_col = orc.mxfp8_quantize(x, direction=orc.COL)
    assert np.array_equal(m_both["col_codes"], m_col["col_codes"])


def test_rowwise_dequantized_source_of_representable_tensor(orc):
    """columnwise_source = rowwise_dequantized: for a tensor NVFP4 represents exactly,
    the dequantized rowwise value is the tensor itself, so the MXFP8 columnwise operand
    built from it equals the one built from the original."""
    rng = np.random.default_rng(3)
    x = np.zeros((64, 64))
    for r in range(64):
        for b in range(4):
            codes = rng.integers(0, 16, 16)
            codes[0] = 7
            x[r, 16 * b:16 * b + 16] = np.array(E2M1)[codes] * e4m3_py(int(rng.integers(0x30, 0x50)))
    x[0, :16] = 0.0
    x[0, 0] = 2688.0                                   # tensor amax alone in its block
    xt = torch.from_numpy(x).to(torch.bfloat16)
    q = orc.nvfp4_quantize(xt, direction=orc.ROW)
    deq = orc.nvfp4_dequantize(q["row_codes"], q["row_scales"], float(q["s_enc"][0]))
    deq_t = torch.from_numpy(deq.view(np.int16)).view(torch.bfloat16)
    assert torch.equal(deq_t, xt)
    a = orc.mxfp8_quantize(xt, direction=orc.COL)
    b = orc.mxfp8_quantize(deq_t, direction=orc.COL)
    assert np.array_equal(a["col_codes"], b["col_codes"]) and np.array_equal(a["col_scales"], b["col_scales"])


def test_rowwise_dequantized_values_on_grid(orc):
    """dequant(code) * S / s_b lies on the E2M1 grid (before the bf16 rounding)."""
    from synthetic import gaussian_bf16
    x = gaussian_bf16((16, 64), 1.0, 11)
    q = orc.nvfp4_quantize(x, direction=orc.ROW)
    s = float(q["s_enc"][0])
    deq = orc.nvfp4_dequantize(q["row_codes"], q["row_scales"], s)
    d = torch.from_numpy(deq.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    sc = np.repeat(np.vectorize(e4m3_py)(q["row_scales"].astype(np.int64)), 16, axis=1)
    codes = np.empty((16, 64), np.int64)
    codes[:, 0::2], codes[:, 1::2] = q["row_codes"] & 0xF, q["row_codes"] >> 4
    exact = np.array(E2M1)[codes] * sc / s
    want = torch.from_numpy(exact).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(d, want)
