"""Pins of the oracle's NVFP4 quantization (tensor scale, block scales, codes, layouts).

NVFP4 = 16-element blocks with an inner (block) scale and an outer per-tensor
scale (torchtitan PR #3914 "Add an NVFP4 quantization converter", review thread
about the recipe's inner 1x16 scale); rowwise and columnwise directions are the
two quantizations of one tensor that a GEMM operand chooses between
(TransformerEngine PR #2817 "Hybrid quantization", Description and the GEMM
dispatch flowchart).  Pins: the hand-derived worked example in
tests/golden/nvfp4_worked_example.txt and closed forms that a wrong scale
formula, a dropped term, a wrong packing order or a transposed layout breaks.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _to_bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)


def unpack(codes: np.ndarray) -> np.ndarray:
    """[rows][cols/2] bytes -> [rows][cols] 4-bit codes (element 2j low nibble)."""
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def e4m3_value(b):
    b = np.asarray(b, np.int64)
    e = (b >> 3) & 15
    m = b & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))
    return np.where(b >> 7, -v, v)


def dequant_f64(q, key="row"):
    codes = unpack(q[key + "_codes"])
    sc = np.repeat(e4m3_value(q[key + "_scales"]), 16, axis=1)
    s = q["s_enc"][0 if key == "row" else 1]
    return E2M1[codes] * sc / float(s)


def test_worked_example(orc):
    rec = {}
    with open(os.path.join(GOLDEN, "nvfp4_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, *v = line.split()
            rec[k] = v
    x = _to_bf16([[float(v) for v in rec["x"]]])
    q = orc.nvfp4_quantize(x, direction=orc.ROW)
    codes = unpack(q["row_codes"])[0]
    assert [int(c) for c in codes] == [int(c, 16) for c in rec["codes"]]
    assert [int(s) for s in q["row_scales"][0]] == [int(s, 16) for s in rec["scales"]]
    assert q["s_enc"][0] == float(rec["s_enc"][0])
    assert q["amax"][0] == float(rec["amax"][0])
    # packing: element 0 in the low nibble of byte 0
    assert q["row_codes"][0, 0] == (0x7 | 0x5 << 4)


def test_tensor_scale_closed_form(orc):
    for a in [1.0, 6.0, 2688.0, 0.5, 1e-3, 3.0e38, 1e-38]:
        with np.errstate(over="ignore"):
            want = np.float32(2688.0) / np.float32(a)
        want = np.float32(np.finfo(np.float32).max) if np.isinf(want) else want
        assert orc.nvfp4_tensor_scale(a) == want
    assert orc.nvfp4_tensor_scale(0.0) == 1.0


def test_block_scale_op_order(orc):
    """t = (block_amax * S) / 6, binary32, in this order; then E4M3 RNE."""
    rng = np.random.default_rng(0)
    for _ in range(3000):
        b = np.float32(rng.uniform(0, 10) * 10.0 ** rng.integers(-3, 3))
        s = np.float32(rng.uniform(1, 3000))
        t = np.float32(np.float32(b * s) / np.float32(6.0))
        assert orc.nvfp4_block_scale(float(b), float(s)) == orc.e4m3_encode(float(t))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_amax_block_maps_to_448_and_6(orc, seed):
    """The block holding the tensor amax gets scale 448 (0x7E) and its amax element code +-6;
    every block whose scale is a normal E4M3 value encodes its amax element to +-6 under RNE."""
    from synthetic import outlier_bf16
    x = outlier_bf16((64, 128), seed=100 + seed, mask_seed=200 + seed)
    q = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL)
    xf = x.to(torch.float32).numpy()
    A = np.abs(xf).max()
    assert q["amax"][0] == q["amax"][1] == A
    for key, v in (("row", xf), ("col", xf.T)):
        codes = unpack(q[key + "_codes"])
        sc = q[key + "_scales"]
        blocks = np.abs(v).reshape(v.shape[0], -1, 16)
        bmax = blocks.max(axis=2)
        arg = blocks.argmax(axis=2)
        r, b = np.unravel_index(np.argmax(bmax), bmax.shape)
        assert sc[r, b] == 0x7E
        amax_codes = codes.reshape(v.shape[0], -1, 16)[np.arange(v.shape[0])[:, None],
                                                        np.arange(bmax.shape[1])[None, :], arg]
        normal = e4m3_value(sc) >= 2.0 ** -6
        assert np.all((amax_codes[normal] & 7) == 7)


def test_columnwise_is_rowwise_of_transpose_layout(orc):
    """Columnwise output [C][R/2] holds the 16-blocks that run down the columns of x."""
    from synthetic import gaussian_bf16
    x = gaussian_bf16((32, 48), 1.0, 7)
    q = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL)
    assert q["col_codes"].shape == (48, 16) and q["col_scales"].shape == (48, 2)
    assert q["row_codes"].shape == (32, 24) and q["row_scales"].shape == (32, 3)
    qt = orc.nvfp4_quantize(x.t().contiguous(), direction=orc.ROW)
    assert np.array_equal(q["col_codes"], qt["row_codes"])
    assert np.array_equal(q["col_scales"], qt["row_scales"])
    # and a column's values really sit in one output row: permuting rows within a
    # 16-row group permutes that column's codes the same way
    perm = np.arange(32); perm[[0, 5]] = perm[[5, 0]]
    qp = orc.nvfp4_quantize(x[torch.from_numpy(perm)].contiguous(), direction=orc.COL)
    cu, pu = unpack(q["col_codes"]), unpack(qp["col_codes"])
    assert np.array_equal(cu[:, perm], pu)


def test_exactly_representable_roundtrip(orc):
    """With A = 2688 * 2^k (S = 2^-k exact) and blocks = E2M1 values times an exact E4M3
    scale whose block max is 6 * scale, dequantization returns the input bit for bit."""
    rng = np.random.default_rng(5)
    for k in [-3, 0, 2]:
        rows, cols = 8, 64
        x = np.zeros((rows, cols))
        for r in range(rows):
            for b in range(cols // 16):
                sbyte = int(rng.integers(0x20, 0x70))       # normal E4M3 block scale
                codes = rng.integers(0, 16, 16)
                codes[int(rng.integers(0, 16))] = 7          # block amax = 6 * scale
                x[r, 16 * b:16 * b + 16] = E2M1[codes] * e4m3_value(sbyte) * 2.0 ** k
        x[0, :16] = 0.0
        x[0, 0] = 2688.0 * 2.0 ** k                          # tensor amax, alone in its block
        xt = torch.from_numpy(x).to(torch.bfloat16)
        assert np.array_equal(xt.to(torch.float64).numpy(), x)  # exact in bf16
        q = orc.nvfp4_quantize(xt, direction=orc.ROW)
        assert q["s_enc"][0] == 2.0 ** -k
        np.testing.assert_array_equal(dequant_f64(q), x)
        deq = orc.nvfp4_dequantize(q["row_codes"], q["row_scales"], float(q["s_enc"][0]))
        assert np.array_equal(deq, xt.view(torch.int16).numpy().view(np.uint16))


def test_rne_error_bound(orc):
    """Each element's dequantized value is the nearest point of its block's scaled E2M1
    grid (up to the binary32 rounding of x * S / s_b), unless it saturates at 6."""
    from synthetic import gaussian_bf16
    x = gaussian_bf16((32, 256), 1.0, 9)
    q = orc.nvfp4_quantize(x, direction=orc.ROW)
    xf = x.to(torch.float64).numpy()
    s = float(q["s_enc"][0])
    sb = np.repeat(e4m3_value(q["row_scales"]), 16, axis=1)
    xs = xf * s / sb                                   # exact-arithmetic scaled value
    deq_s = E2M1[unpack(q["row_codes"])]
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    dist = np.abs(np.abs(xs)[..., None] - grid).min(axis=-1)
    err = np.abs(np.abs(xs) - np.abs(deq_s))
    assert np.all(err <= dist + 1e-6 * np.maximum(1, np.abs(xs)))
    assert np.all(np.sign(deq_s[deq_s != 0]) == np.sign(xs[deq_s != 0]))


def test_zero_tensor_and_zero_blocks(orc):
    x = torch.zeros((16, 32), dtype=torch.bfloat16)
    q = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL)
    assert q["amax"][0] == 0 and q["s_enc"][0] == 1.0
    for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
        assert not q[k].any()
    # a zero block inside a nonzero tensor: scale 0, codes 0 (also for -0)
    y = torch.zeros((1, 32), dtype=torch.float32)
    y[0, :16] = torch.linspace(-3, 3, 16)
    y[0, 16:] = -0.0
    q = orc.nvfp4_quantize(y.to(torch.bfloat16), direction=orc.ROW)
    assert q["row_scales"][0, 1] == 0 and not q["row_codes"][0, 8:].any()


def test_tiny_scale_underflow_gives_zero_block(orc):
    """A block whose amax is far below the tensor amax gets block scale 0 and codes 0."""
    x = torch.zeros((1, 32), dtype=torch.float32)
    x[0, 0] = 1000.0
    x[0, 16:] = 1e-6
    q = orc.nvfp4_quantize(x.to(torch.bfloat16), direction=orc.ROW)
    assert q["row_scales"][0, 1] == 0 and not q["row_codes"][0, 8:].any()


def test_shape_errors(orc):
    with pytest.raises(ValueError):
        orc.nvfp4_quantize(torch.zeros((16, 24), dtype=torch.bfloat16), direction=orc.ROW)
    with pytest.raises(ValueError):
        orc.nvfp4_quantize(torch.zeros((24, 16), dtype=torch.bfloat16), direction=orc.COL)
