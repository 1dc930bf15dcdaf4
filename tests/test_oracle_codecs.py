"""Pins of the oracle's element and scale codecs (E2M1, E4M3, E8M0, bf16).

The pages name these formats (NVFP4: E2M1 codes with E4M3 block scales; MXFP8:
E4M3 codes with E8M0 scales) without defining them; the definitions used here
are the public OCP Microscaling (MX) / OCP FP8 ones.  Pins: closed-form decode
of every code, brute-force nearest search on dense sweeps, the hand-derived tie
table in tests/golden/e2m1_ties.txt, and torch's own float8_e4m3fn / bfloat16
casts as independent library routines.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def e2m1_closed_form(code: int) -> float:
    """OCP E2M1: sign bit 3, exponent bits 2:1 (bias 1), mantissa bit 0; exponent 0 is subnormal."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    v = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return -v if s else v


def e4m3_closed_form(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


# ------------------------------------------------------------------ E2M1

def test_e2m1_decode_all_codes(orc):
    for c in range(16):
        got = orc.e2m1_decode(c)
        want = e2m1_closed_form(c)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), c


def test_e2m1_roundtrip_all_codes(orc):
    for c in range(16):
        assert orc.e2m1_encode_rne(e2m1_closed_form(c)) == c


def _load_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b = line.split()
                rows.append((float(a), int(b, 0)))
    return rows


def test_e2m1_ties_golden(orc):
    rows = _load_pairs("e2m1_ties.txt")
    assert len(rows) >= 14
    for v, code in rows:
        assert orc.e2m1_encode_rne(v) == code, (v, code)


def _brute_e2m1(v: float) -> int:
    """Brute force: nearest of the 8 magnitudes by exact (float64) distance, ties to the even code,
    saturation above 6, sign copied."""
    mags = [abs(e2m1_closed_form(c)) for c in range(8)]
    a = abs(v)
    if a >= 6.0:
        best = 7
    else:
        d = [abs(a - m) for m in mags]
        dmin = min(d)
        cands = [i for i in range(8) if d[i] == dmin]
        best = [i for i in cands if i % 2 == 0][0] if len(cands) > 1 else cands[0]
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_encode_dense_sweep(orc):
    grid = np.arange(-8.0, 8.0 + 2 ** -12, 2 ** -12, dtype=np.float64)  # exact in fp32
    rng = np.random.default_rng(5)
    rand = rng.uniform(-10, 10, 20000).astype(np.float32).astype(np.float64)
    for v in np.concatenate([grid, rand, [1e30, -1e30, 6.0000005, -0.0, 0.0]]):
        v = float(np.float32(v))
        assert orc.e2m1_encode_rne(v) == _brute_e2m1(v), v


def test_e2m1_encode_monotone(orc):
    vals = np.float32(np.linspace(0, 7, 4001))
    codes = [orc.e2m1_encode_rne(float(v)) for v in vals]
    assert all(b >= a for a, b in zip(codes, codes[1:]))


# ------------------------------------------------------------------ E4M3

def test_e4m3_decode_closed_form_and_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = orc.e4m3_decode(c)
        want = e4m3_closed_form(c)
        if math.isnan(want):
            assert math.isnan(got) and math.isnan(tv[c])
            continue
        assert got == want == float(tv[c]), c
        assert math.copysign(1, got) == math.copysign(1, want)


def test_e4m3_max_and_min():
    assert e4m3_closed_form(0x7E) == 448.0
    assert e4m3_closed_form(0x01) == 2.0 ** -9
    assert e4m3_closed_form(0x08) == 2.0 ** -6


def test_e4m3_encode_matches_torch_cast(orc):
    """torch's CPU float8_e4m3fn cast is RNE with subnormals and keeps -0; it does not
    saturate, so the comparison stays below 464 (the tie between 448 and 480)."""
    rng = np.random.default_rng(11)
    vals = [rng.uniform(-460, 460, 3000), rng.uniform(-1, 1, 3000) * 2.0 ** rng.integers(-12, 0, 3000),
            np.arange(-463.0, 463.0, 0.25)]
    # all midpoints between adjacent non-negative codes and their neighbours in fp32
    mids = []
    for c in range(0x7E):
        lo, hi = e4m3_closed_form(c), e4m3_closed_form(c + 1)
        m = (lo + hi) / 2
        mids += [m, float(np.nextafter(np.float32(m), np.float32(0))), float(np.nextafter(np.float32(m), np.float32(1e9)))]
    vals.append(np.array(mids))
    vals.append(-np.array(mids))
    v = np.float32(np.concatenate(vals))
    tor = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, t in zip(v, tor):
        assert orc.e4m3_encode(float(x)) == int(t), float(x)
    assert orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(0.0) == 0x00


def test_e4m3_encode_saturates(orc):
    for v in [448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38]:
        assert orc.e4m3_encode(v) == 0x7E
        assert orc.e4m3_encode(-v) == 0xFE


def test_e4m3_roundtrip_all_finite(orc):
    for c in range(256):
        v = e4m3_closed_form(c)
        if math.isnan(v):
            continue
        assert orc.e4m3_encode(v) == c


# ------------------------------------------------------------------ E8M0 / bf16

def test_e8m0_decode(orc):
    for b in range(255):
        assert orc.e8m0_decode(b) == 2.0 ** (b - 127)
    assert math.isnan(orc.e8m0_decode(255))


def test_bf16_rne_matches_torch(orc):
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000),
                        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20])]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, w in zip(v, want):
        assert orc.f32_to_bf16_rne(float(x)) == int(w)
