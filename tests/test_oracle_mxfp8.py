"""Pins of the oracle's MXFP8 cast (32-element blocks, E8M0 scale, E4M3 codes).

The block size of 32 and one scale per block along the blocked dimension come
from TransformerEngine PR #2817 "Hybrid quantization" (review thread on the
columnwise scale count, MXFP8_BLOCK_SCALING_SIZE); the shared-exponent rule is
the OCP MX one (MX paper, cited in the TorchAO review page's references).
Pins: the closed form byte = floor(log2 amax) + 119 from math.frexp, exact
round trips of blocks of E4M3 values times a power of two, saturation, zero
blocks, and torch's float8_e4m3fn cast of the scaled values.
"""
import math

import numpy as np
import pytest
import torch


def e4m3_value(b):
    b = np.asarray(b, np.int64)
    e = (b >> 3) & 15
    m = b & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * 2.0 ** (e - 7.0))
    return np.where(b >> 7, -v, v)


def test_scale_byte_closed_form(orc):
    rng = np.random.default_rng(0)
    vals = list(np.float32(rng.uniform(0, 1, 3000) * 10.0 ** rng.integers(-30, 30, 3000)))
    for k in range(-120, 120, 7):
        vals += [np.float32(2.0 ** k), np.nextafter(np.float32(2.0 ** k), np.float32(0))]
    for a in vals:
        if a == 0:
            continue
        m, e = math.frexp(float(a))
        want = min(max(e - 1 - 8, -127), 127) + 127
        assert orc.mxfp8_scale_byte(float(a)) == want, a


def test_roundtrip_of_representable_blocks(orc):
    """A block of E4M3 values times 2^X whose largest magnitude lies in [256, 448] quantizes
    to scale byte X + 127 and to exactly those codes."""
    rng = np.random.default_rng(1)
    rows, cols = 4, 128
    x = np.zeros((rows, cols))
    want_codes = np.zeros((rows, cols), np.uint8)
    want_scales = np.zeros((rows, cols // 32), np.uint8)
    for r in range(rows):
        for b in range(cols // 32):
            X = int(rng.integers(-20, 20))
            codes = rng.integers(0, 0x7F, 32).astype(np.uint8)      # finite non-negative
            codes[int(rng.integers(0, 32))] = int(rng.integers(0x78, 0x7F))  # 256..448
            codes |= (rng.integers(0, 2, 32) << 7).astype(np.uint8)
            vals = e4m3_value(codes)
            # keep only values that are exact in bf16 (E4M3 has 3 mantissa bits, bf16 7)
            x[r, 32 * b:32 * b + 32] = vals * 2.0 ** X
            want_codes[r, 32 * b:32 * b + 32] = codes
            want_scales[r, b] = X + 127
    xt = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(xt.to(torch.float64).numpy(), x)
    q = orc.mxfp8_quantize(xt, direction=orc.ROW)
    # -0 codes and +0 codes both decode to 0; compare values, then bits of nonzeros
    assert np.array_equal(q["row_scales"], want_scales)
    nz = x != 0
    assert np.array_equal(q["row_codes"][nz], want_codes[nz])
    assert np.all(e4m3_value(q["row_codes"][~nz]) == 0)


def test_codes_match_torch_cast_and_clip(orc):
    from synthetic import outlier_bf16
    x = outlier_bf16((64, 256), seed=3, mask_seed=4)
    q = orc.mxfp8_quantize(x, direction=orc.ROW | orc.COL)
    for key, v in (("row", x.to(torch.float32).numpy()), ("col", x.to(torch.float32).numpy().T.copy())):
        sc = q[key + "_scales"].astype(np.int64) - 127
        scaled = v * np.repeat(2.0 ** (-sc), 32, axis=1)      # exact power-of-two scaling
        scaled = scaled.astype(np.float32)
        assert np.abs(scaled).max() < 512
        clipped = np.clip(scaled, -448, 448)
        tor = torch.from_numpy(clipped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q[key + "_codes"], tor)
        # each block's largest element lands in [256, 448]
        bm = np.abs(e4m3_value(q[key + "_codes"])).reshape(v.shape[0], -1, 32).max(axis=2)
        assert np.all((bm >= 256) & (bm <= 448))


def test_zero_block(orc):
    x = torch.zeros((2, 64), dtype=torch.float32)
    x[0, :32] = torch.linspace(-1, 1, 32)
    x[1, 32:] = -0.0
    q = orc.mxfp8_quantize(x.to(torch.bfloat16), direction=orc.ROW)
    assert q["row_scales"][0, 1] == 0 and q["row_scales"][1, 0] == 0 and q["row_scales"][1, 1] == 0
    assert not q["row_codes"][0, 32:].any() and not q["row_codes"][1].any()


def test_tiny_block_scale_clamps(orc):
    # the smallest bf16 subnormal 2^-133: floor(log2) - 8 = -141, clamped to -127 -> byte 0
    assert orc.mxfp8_scale_byte(2.0 ** -133) == 0
    assert orc.mxfp8_scale_byte(2.0 ** -118) == 1


def test_scale_count_along_blocked_dim(orc):
    """One scale per 32 elements along the blocked dimension: [R][C/32] and [C][R/32]."""
    x = torch.zeros((96, 64), dtype=torch.bfloat16)
    q = orc.mxfp8_quantize(x, direction=orc.ROW | orc.COL)
    assert q["row_scales"].shape == (96, 2) and q["col_scales"].shape == (64, 3)
    with pytest.raises(ValueError):
        orc.mxfp8_quantize(torch.zeros((48, 64), dtype=torch.bfloat16), direction=orc.COL)
