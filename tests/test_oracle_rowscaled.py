"""Pins of the oracle's row-scaled NVFP4 (outer fp32 scale per row, inner E4M3 scale per
16 elements -- the "row_scaled_nvfp4" rowwise quantizer of the Composer-style recipe on the
page "[Pytorch][Common] Hybrid quantization", and the "outer scale rowwise, inner scale 1x16"
recipe asked about in the review of "Add an NVFP4 quantization converter") and of the GEMM
with per-row tensor scales.

Each row is quantized exactly like a one-row tensor under the per-tensor recipe, whose
oracle is pinned separately; these tests tie the two together and check what the per-row
outer scale adds: rows are independent, a power-of-two scaling of a row only rescales its
outer scale, every row's largest element lands on code +-6 in a block with scale 448.
"""
import numpy as np
import pytest
import torch

from synthetic import gaussian_bf16, outlier_bf16, rht_signs

E2M1 = [0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6]


def e4m3_py(b: int) -> float:
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    v = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if s else v


@pytest.mark.parametrize("cols", [16, 64, 1056])
@pytest.mark.parametrize("rounding,rht", [(0, False), (1, False), (0, True), (1, True)])
def test_one_row_equals_per_tensor(orc, cols, rounding, rht):
    x = outlier_bf16((1, cols), seed=cols, mask_seed=cols + 1)
    sg = rht_signs(7).numpy() if rht else None
    r = orc.nvfp4_quantize_rowscaled(x, rounding=rounding, sr_seed=42, sr_stream=3, signs=sg)
    t = orc.nvfp4_quantize(x, direction=orc.ROW, rounding=rounding, sr_seed=42, sr_stream=3, signs=sg)
    assert np.array_equal(r["codes"], t["row_codes"]) and np.array_equal(r["scales"], t["row_scales"])
    assert r["amax"][0] == t["amax"][0] and r["s_enc"][0] == t["s_enc"][0]


@pytest.mark.parametrize("rounding", [0, 1])
def test_rows_sharing_the_amax_equal_per_tensor(orc, rounding):
    """When every row holds the tensor amax, the per-row outer scales all equal the tensor
    scale and the row-scaled result is the per-tensor result (SR words included)."""
    x = gaussian_bf16((48, 256), 1.0, 5).float()
    x[:, 17] = 7.5
    x[::3, 200] = -7.5
    x = x.to(torch.bfloat16)
    r = orc.nvfp4_quantize_rowscaled(x, rounding=rounding, sr_seed=9)
    t = orc.nvfp4_quantize(x, direction=orc.ROW, rounding=rounding, sr_seed=9)
    assert np.all(r["amax"] == 7.5) and np.all(r["s_enc"] == t["s_enc"][0])
    assert np.array_equal(r["codes"], t["row_codes"]) and np.array_equal(r["scales"], t["row_scales"])


def test_power_of_two_row_scaling_only_moves_the_outer_scale(orc):
    x = gaussian_bf16((12, 128), 1.0, 11).float()
    y = x.clone()
    y[3] *= 4.0
    y[7] *= 0.125
    r = orc.nvfp4_quantize_rowscaled(x.to(torch.bfloat16))
    s = orc.nvfp4_quantize_rowscaled(y.to(torch.bfloat16))
    assert np.array_equal(r["codes"], s["codes"]) and np.array_equal(r["scales"], s["scales"])
    assert s["s_enc"][3] == r["s_enc"][3] / 4 and s["s_enc"][7] == r["s_enc"][7] * 8
    assert s["amax"][3] == r["amax"][3] * 4 and s["amax"][7] == r["amax"][7] / 8
    keep = [i for i in range(12) if i not in (3, 7)]
    assert np.array_equal(r["s_enc"][keep], s["s_enc"][keep])


def test_each_row_amax_maps_to_six_with_scale_448(orc):
    x = outlier_bf16((32, 512), seed=21, mask_seed=22)
    r = orc.nvfp4_quantize_rowscaled(x)
    xf = x.float().numpy()
    for row in range(32):
        k = int(np.argmax(np.abs(xf[row])))
        assert r["amax"][row] == abs(xf[row, k])
        assert r["s_enc"][row] == np.float32(2688.0) / np.float32(r["amax"][row])
        assert r["scales"][row, k // 16] == 0x7E
        byte = int(r["codes"][row, k // 2])
        code = byte & 0xF if k % 2 == 0 else byte >> 4
        assert code & 7 == 7 and (code >> 3) == (1 if xf[row, k] < 0 else 0)


def test_zero_row_and_independent_rows(orc):
    x = gaussian_bf16((6, 64), 1.0, 31).float()
    x[2] = 0.0
    r = orc.nvfp4_quantize_rowscaled(x.to(torch.bfloat16))
    assert r["amax"][2] == 0 and r["s_enc"][2] == 1.0
    assert not r["codes"][2].any() and not r["scales"][2].any()
    for row in (0, 1, 3, 4, 5):
        one = orc.nvfp4_quantize_rowscaled(x[row:row + 1].to(torch.bfloat16))
        assert np.array_equal(one["codes"][0], r["codes"][row]) and one["s_enc"][0] == r["s_enc"][row]


def _deq_rows(codes, scales, s_rows):
    """float64 dequantized operand from codes/scales with one outer scale per row, decoded
    with the closed-form tables above (not the oracle's decoders)."""
    R, half = codes.shape
    out = np.zeros((R, 2 * half))
    for r in range(R):
        for k in range(2 * half):
            byte = int(codes[r, k // 2])
            c = byte & 0xF if k % 2 == 0 else byte >> 4
            out[r, k] = E2M1[c] * e4m3_py(int(scales[r, k // 16])) / float(s_rows[r])
    return out


def test_rowscaled_gemm_matches_independent_dequant(orc):
    x = outlier_bf16((10, 96), seed=41, mask_seed=42)
    w = gaussian_bf16((7, 96), 0.02, 43)
    qa = orc.nvfp4_quantize_rowscaled(x)
    qb = orc.nvfp4_quantize(w, direction=orc.ROW)
    got = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["codes"], qa["scales"], qa["s_enc"],
                               qb["row_codes"], qb["row_scales"], float(qb["s_enc"][0]))
    ref = _deq_rows(qa["codes"], qa["scales"], qa["s_enc"]) @ _deq_rows(
        qb["row_codes"], qb["row_scales"], np.full(7, qb["s_enc"][0])).T
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    # both operands row-scaled
    qc = orc.nvfp4_quantize_rowscaled(w)
    got2 = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["codes"], qa["scales"], qa["s_enc"],
                                qc["codes"], qc["scales"], qc["s_enc"])
    ref2 = _deq_rows(qa["codes"], qa["scales"], qa["s_enc"]) @ _deq_rows(qc["codes"], qc["scales"], qc["s_enc"]).T
    assert np.allclose(got2, ref2, rtol=1e-12, atol=0)


def test_rowscaled_gemm_with_equal_row_scales_is_the_per_tensor_gemm(orc):
    x = gaussian_bf16((9, 64), 1.0, 51)
    w = gaussian_bf16((5, 64), 1.0, 52)
    qa = orc.nvfp4_quantize(x, direction=orc.ROW)
    qb = orc.nvfp4_quantize(w, direction=orc.ROW)
    sa, sb = float(qa["s_enc"][0]), float(qb["s_enc"][0])
    per_tensor = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["row_codes"], qa["row_scales"], sa,
                                      qb["row_codes"], qb["row_scales"], sb)
    per_row = orc.blockscaled_gemm(orc.FMT_NVFP4, qa["row_codes"], qa["row_scales"], np.full(9, sa, np.float32),
                                   qb["row_codes"], qb["row_scales"], np.full(5, sb, np.float32))
    assert np.array_equal(per_tensor, per_row)
