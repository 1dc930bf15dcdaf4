"""Pins of the oracle's Philox4x32-10 and of stochastic rounding (SR).

The recipe keys SR with a per-rank Philox seed and relies on SR being unbiased
(torchtitan PR #3914 "Add an NVFP4 quantization converter", Summary / What
changed).  The pages give no counter layout; the oracle's reading is documented
in oracle.c.  Pins:
  * Philox against the host-callable Philox4x32-10 of ROCm's rocRAND headers
    (an independent implementation), on random counters and keys;
  * closed-form SR threshold: with p = k 2^-24 the result rounds up exactly for
    the words whose top 24 bits are below k;
  * grid values never move, results are always one of the two neighbours;
  * unbiasedness over 4096 seeds on blocks whose scaling is exact;
  * the same (seed, stream, direction) replays bit-identically, and a different
    stream or direction draws different words.
"""
import ctypes as C
import os
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_philox():
    src = os.path.join(HERE, "philox_ref_shim.cpp")
    inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND headers not installed")
    d = tempfile.mkdtemp(prefix="philox_ref_")
    so = os.path.join(d, "philox_ref.so")
    subprocess.run(["g++", "-O1", "-shared", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I" + inc, src, "-o", so],
                   check=True)
    L = C.CDLL(so)

    def f(ctr, key):
        c = np.ascontiguousarray(np.asarray(ctr, np.uint32))
        k = np.ascontiguousarray(np.asarray(key, np.uint32))
        o = np.zeros(4, np.uint32)
        L.ref_philox(c.ctypes.data_as(C.c_void_p), k.ctypes.data_as(C.c_void_p), o.ctypes.data_as(C.c_void_p))
        return o
    return f


def test_philox_matches_rocrand(orc, rocrand_philox):
    rng = np.random.default_rng(0)
    cases = [([0, 0, 0, 0], [0, 0]), ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2)]
    for _ in range(2000):
        cases.append((rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32),
                      rng.integers(0, 2 ** 32, 2, dtype=np.uint64).astype(np.uint32)))
    for ctr, key in cases:
        assert np.array_equal(orc.philox4x32_10(ctr, key), rocrand_philox(ctr, key)), (ctr, key)


def test_sr_word_counter_layout(orc):
    """Word i of the stream is word i%4 of Philox((i/4 lo, i/4 hi, stream, dir), (seed lo, seed hi))."""
    seed = 0x0123456789ABCDEF
    for i in [0, 1, 2, 3, 4, 7, 2 ** 32 * 4 + 5, 123456789]:
        q = i >> 2
        w = orc.philox4x32_10([q & 0xFFFFFFFF, q >> 32, 3, 1], [seed & 0xFFFFFFFF, seed >> 32])
        assert orc.sr_word(seed, 3, 1, i) == int(w[i & 3])


def test_sr_negative_seed_is_twos_complement(orc):
    # An int64 seed drawn in [-2^63, 2^63) is read as its 64-bit two's complement.
    assert orc.sr_word(-1, 0, 0, 5) == orc.sr_word(2 ** 64 - 1, 0, 0, 5)


def test_sr_threshold_closed_form(orc):
    """For |v| = lo + p (hi - lo) with p = k 2^-24, rounding goes up iff (u >> 8) < k."""
    rng = np.random.default_rng(1)
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for _ in range(400):
        i = int(rng.integers(0, 7))
        lo, hi = grid[i], grid[i + 1]
        k = int(rng.integers(1, 2 ** 24))
        p = k * 2.0 ** -24
        v = lo + p * (hi - lo)
        if float(np.float32(v)) != v:
            continue  # keep only values exact in binary32
        up, down = i + 1, i
        for sgn in (1.0, -1.0):
            sbit = 8 if sgn < 0 else 0
            assert orc.e2m1_encode_sr(sgn * v, (k - 1) << 8 | 0xFF) == (up | sbit)
            assert orc.e2m1_encode_sr(sgn * v, k << 8) == (down | sbit)
            assert orc.e2m1_encode_sr(sgn * v, 0) == (up | sbit)
            assert orc.e2m1_encode_sr(sgn * v, 0xFFFFFFFF) == (down | sbit)


def test_sr_grid_values_fixed_and_saturation(orc):
    rng = np.random.default_rng(2)
    us = [0, 1, 0xFFFFFFFF] + [int(u) for u in rng.integers(0, 2 ** 32, 50, dtype=np.uint64)]
    for c in range(16):
        v = orc.e2m1_decode(c)
        for u in us:
            assert orc.e2m1_encode_sr(v, u) == c
    for v in [6.0, 6.5, 100.0]:
        for u in us:
            assert orc.e2m1_encode_sr(v, u) == 7
            assert orc.e2m1_encode_sr(-v, u) == 15


def test_sr_result_is_a_neighbour(orc):
    rng = np.random.default_rng(4)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    for _ in range(3000):
        v = float(np.float32(rng.uniform(-6, 6)))
        c = orc.e2m1_encode_sr(v, int(rng.integers(0, 2 ** 32, dtype=np.uint64)))
        a = abs(v)
        lo = grid[grid <= a].max()
        hi = grid[grid >= a].min()
        assert abs(orc.e2m1_decode(c)) in (lo, hi)
        assert (c >= 8) == (np.signbit(np.float32(v)))


def _exact_scale_tensor(rng):
    """A [2, 32] bf16 tensor with amax 2688 (so S = 1) whose other 16-blocks have
    amax 6 * 2^j, so their block scale is 2^j and x * S / s_b is exact."""
    import torch
    x = np.zeros((2, 32), np.float32)
    x[0, :16] = rng.uniform(-2688, 2688, 16)
    x[0, 0] = 2688.0
    for (r, b), j in zip([(0, 1), (1, 0), (1, 1)], [-2, 0, 3]):
        blk = rng.uniform(-6, 6, 16) * 2.0 ** j
        blk[int(rng.integers(0, 16))] = 6.0 * 2.0 ** j
        x[r, 16 * b:16 * b + 16] = blk
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t, t.to(torch.float32).numpy()


def test_sr_unbiased_over_seeds(orc):
    rng = np.random.default_rng(9)
    xt, xf = _exact_scale_tensor(rng)
    N = 4096
    acc = np.zeros((2, 32))
    acc2 = np.zeros((2, 32))
    for seed in range(N):
        q = orc.nvfp4_quantize(xt, direction=orc.ROW, rounding=orc.SR, sr_seed=seed * 7919 + 1)
        assert q["s_enc"][0] == 1.0
        deq = orc.nvfp4_dequantize(q["row_codes"], q["row_scales"], float(q["s_enc"][0]))
        import torch
        d = torch.from_numpy(deq.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
        acc += d
        acc2 += d * d
    mean = acc / N
    var = np.maximum(acc2 / N - mean ** 2, 0)
    sel = np.ones_like(xf, bool)
    sel[0, :16] = False  # the block holding the tensor amax has a non power-of-two scale
    err = np.abs(mean - xf)[sel]
    bound = 5 * np.sqrt(var[sel] / N) + 1e-12
    assert np.all(err <= bound), (err.max(), bound.min())
    # and the spread is what SR implies (not collapsed to deterministic rounding)
    assert (var[sel] > 0).sum() > 20


def test_sr_replay_and_streams(orc):
    import torch
    from synthetic import gaussian_bf16
    x = gaussian_bf16((64, 64), 1.0, 5)
    a = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL, rounding=orc.SR, sr_seed=42, sr_stream=0)
    b = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL, rounding=orc.SR, sr_seed=42, sr_stream=0)
    c = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL, rounding=orc.SR, sr_seed=42, sr_stream=1)
    d = orc.nvfp4_quantize(x, direction=orc.ROW | orc.COL, rounding=orc.SR, sr_seed=43, sr_stream=0)
    for k in ("row_codes", "col_codes"):
        assert np.array_equal(a[k], b[k])
        assert not np.array_equal(a[k], c[k])
        assert not np.array_equal(a[k], d[k])
    # scales never depend on the random draw
    for k in ("row_scales", "col_scales"):
        assert np.array_equal(a[k], c[k])
