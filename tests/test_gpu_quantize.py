"""GPU parity of the quantization kernels against the CPU oracle: bit-exact codes, scales,
amax and tensor scales, on the same seeded inputs, through the C ABI.

Shapes: the workloads' own shapes (quantize-only [8192, 4096] with 1 % outliers; the
Llama-3-8B FFN activations and weights; the wgrad output gradient with RHT + SR), small
shapes that span several tiles with ragged tails, and the degenerate cases (empty
tensors, all-zero tensors)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsq
from synthetic import (SEED_DY, SEED_SIGNS, SEED_SR_KEY, SEED_W, SEED_X, STD_DY, STD_W, gaussian_bf16,
                       outlier_bf16, rht_signs)
from tests.gpu_common import assert_bytes_equal, assert_f32_equal, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def check_nvfp4(x_cpu, direction, rounding=0, seed=0, stream=0, signs=None, label=""):
    import oracle
    note("nvfp4 %s shape=%s dir=%d rnd=%d rht=%s" % (label, tuple(x_cpu.shape), direction, rounding,
                                                     signs is not None))
    x = x_cpu.to(DEV)
    got = bsq.nvfp4_quantize(x, direction=direction, rounding=rounding, sr_seed=seed, sr_stream=stream,
                             rht_signs=signs)
    torch.cuda.synchronize()
    ref = oracle.nvfp4_quantize(x_cpu, direction=direction, rounding=rounding, sr_seed=seed, sr_stream=stream,
                                signs=None if signs is None else signs.numpy())
    for d, key in ((1, "row"), (2, "col")):
        if direction & d:
            i = 0 if key == "row" else 1
            assert_f32_equal(got["amax"][i:i + 1], ref["amax"][i:i + 1], label + " amax " + key)
            assert_f32_equal(got["s_enc"][i:i + 1], ref["s_enc"][i:i + 1], label + " s_enc " + key)
            assert_bytes_equal(got[key + "_scales"], ref[key + "_scales"], label + " " + key + "_scales")
            assert_bytes_equal(got[key + "_codes"], ref[key + "_codes"], label + " " + key + "_codes")
    return got, ref


def check_mxfp8(x_cpu, direction, label=""):
    import oracle
    note("mxfp8 %s shape=%s dir=%d" % (label, tuple(x_cpu.shape), direction))
    got = bsq.mxfp8_quantize(x_cpu.to(DEV), direction=direction)
    torch.cuda.synchronize()
    ref = oracle.mxfp8_quantize(x_cpu, direction=direction)
    for d, key in ((1, "row"), (2, "col")):
        if direction & d:
            assert_bytes_equal(got[key + "_scales"], ref[key + "_scales"], label + " " + key + "_scales")
            assert_bytes_equal(got[key + "_codes"], ref[key + "_codes"], label + " " + key + "_codes")


def check_hybrid(x_cpu, rounding=0, seed=0, stream=0, signs=None, slab=False, label=""):
    """One-pass NVFP4 columnwise + MXFP8 rowwise against the oracle's two casts of the same
    input: each half bit-exact to its own format's oracle."""
    import oracle
    from tests.gpu_common import from_slab
    R, Cc = x_cpu.shape
    note("hybrid %s shape=%s rnd=%d rht=%s slab=%s" % (label, (R, Cc), rounding, signs is not None, slab))
    got = bsq.nvfp4_col_mxfp8_row_quantize(x_cpu.to(DEV), rounding=rounding, sr_seed=seed, sr_stream=stream,
                                           rht_signs=signs, mx_slab=slab)
    torch.cuda.synchronize()
    ref = oracle.nvfp4_quantize(x_cpu, direction=2, rounding=rounding, sr_seed=seed, sr_stream=stream,
                                signs=None if signs is None else signs.numpy())
    assert_f32_equal(got["amax"][1:2], ref["amax"][1:2], label + " amax col")
    assert_f32_equal(got["s_enc"][1:2], ref["s_enc"][1:2], label + " s_enc col")
    assert_bytes_equal(got["col_scales"], ref["col_scales"], label + " col_scales")
    assert_bytes_equal(got["col_codes"], ref["col_codes"], label + " col_codes")
    del ref
    mref = oracle.mxfp8_quantize(x_cpu, direction=1)
    codes = got["mx_row_codes"]
    if slab:
        codes = torch.from_numpy(from_slab(codes, R, Cc))
    assert_bytes_equal(got["mx_row_scales"], mref["row_scales"], label + " mxfp8 row_scales")
    assert_bytes_equal(codes, mref["row_codes"], label + " mxfp8 row_codes")


def check_fprop_wgrad(x_cpu, rounding=0, seed=0, stream=0, signs=None, label=""):
    """One-pass rowwise RNE (no transform) + columnwise (given rounding and transform) against
    the oracle's two casts of the same input."""
    import oracle
    note("fprop+wgrad %s shape=%s rnd=%d rht=%s" % (label, tuple(x_cpu.shape), rounding, signs is not None))
    got = bsq.nvfp4_quantize_fprop_wgrad(x_cpu.to(DEV), rounding=rounding, sr_seed=seed, sr_stream=stream,
                                         rht_signs=signs)
    torch.cuda.synchronize()
    rr = oracle.nvfp4_quantize(x_cpu, direction=1)
    assert_f32_equal(got["amax"][0:1], rr["amax"][0:1], label + " amax row")
    assert_f32_equal(got["s_enc"][0:1], rr["s_enc"][0:1], label + " s_enc row")
    assert_bytes_equal(got["row_scales"], rr["row_scales"], label + " row_scales")
    assert_bytes_equal(got["row_codes"], rr["row_codes"], label + " row_codes")
    del rr
    rc = oracle.nvfp4_quantize(x_cpu, direction=2, rounding=rounding, sr_seed=seed, sr_stream=stream,
                               signs=None if signs is None else signs.numpy())
    assert_f32_equal(got["amax"][1:2], rc["amax"][1:2], label + " amax col")
    assert_f32_equal(got["s_enc"][1:2], rc["s_enc"][1:2], label + " s_enc col")
    assert_bytes_equal(got["col_scales"], rc["col_scales"], label + " col_scales")
    assert_bytes_equal(got["col_codes"], rc["col_codes"], label + " col_codes")


# ----------------------------------------------------------------- small and ragged

@pytest.mark.parametrize("shape", [(128, 256), (256, 128), (272, 144), (16, 16), (48, 400), (528, 16)])
@pytest.mark.parametrize("direction", [1, 2, 3])
def test_nvfp4_rne_small(shape, direction):
    check_nvfp4(outlier_bf16(shape, seed=11, mask_seed=12), direction, label="small")


@pytest.mark.parametrize("shape", [(256, 256), (272, 144), (32, 16)])
@pytest.mark.parametrize("direction", [1, 2, 3])
def test_nvfp4_rht_sr_small(shape, direction):
    x = gaussian_bf16(shape, 1e-3, 21)
    check_nvfp4(x, direction, rounding=1, seed=-1234567890123, stream=3, signs=rht_signs(SEED_SIGNS),
                label="rht+sr")


# RHT without SR and SR without RHT, in each direction: rowwise-only runs the streaming
# kernels (amax_rht_row_linear + the rowwise encode), columnwise-only and both directions the
# tile kernels.  Ragged small shapes (rows not a multiple of 16 where rowwise-only allows it,
# cols % 16 == 8 for columnwise-only) and the forward activation shape.
_ALONE_SHAPES = {1: (37, 400), 2: (272, 136), 3: (272, 144)}


@pytest.mark.parametrize("direction", [1, 2, 3])
@pytest.mark.parametrize("rounding,use_rht", [(0, True), (1, False)])
def test_nvfp4_rht_or_sr_alone(rounding, use_rht, direction):
    x = gaussian_bf16(_ALONE_SHAPES[direction], 1.0, 22 + direction)
    check_nvfp4(x, direction, rounding=rounding, seed=SEED_SR_KEY, stream=direction,
                signs=rht_signs(SEED_SIGNS) if use_rht else None, label="rht-or-sr small")


@pytest.mark.parametrize("direction", [1, 2, 3])
@pytest.mark.parametrize("rounding,use_rht", [(0, True), (1, False)])
def test_nvfp4_rht_or_sr_alone_workload(rounding, use_rht, direction):
    """The same variants on the forward activation shape [16384, 4096]."""
    x = gaussian_bf16((16384, 4096), 1.0, SEED_X)
    check_nvfp4(x, direction, rounding=rounding, seed=SEED_SR_KEY, stream=1,
                signs=rht_signs(SEED_SIGNS) if use_rht else None, label="rht-or-sr [16384,4096]")


def test_nvfp4_col_only_cols_multiple_of_8():
    """Columnwise-only quantization allows cols % 16 == 8 (a ragged last 8-column chunk)."""
    check_nvfp4(gaussian_bf16((64, 136), 1.0, 23), 2, label="col-only")


def test_nvfp4_row_only_ragged_rows():
    """Rowwise-only quantization allows any row count (rows beyond a 16-row group)."""
    check_nvfp4(gaussian_bf16((37, 64), 1.0, 24), 1, label="row-ragged")


def test_nvfp4_zero_and_empty():
    check_nvfp4(torch.zeros((64, 64), dtype=torch.bfloat16), 3, label="zeros")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV)
    got = bsq.nvfp4_quantize(x, direction=3)
    torch.cuda.synchronize()
    assert got["amax"].cpu().tolist() == [0.0, 0.0] and got["s_enc"].cpu().tolist() == [1.0, 1.0]


@pytest.mark.parametrize("shape,slab", [((256, 256), False), ((256, 256), True), ((272, 160), False),
                                         ((272, 192), True), ((32, 32), False), ((48, 448), True),
                                         ((528, 64), True)])
@pytest.mark.parametrize("rounding,use_rht", [(0, False), (1, True), (0, True)])
def test_hybrid_small(shape, slab, rounding, use_rht):
    x = outlier_bf16(shape, seed=31, mask_seed=32)
    check_hybrid(x, rounding=rounding, seed=SEED_SR_KEY, stream=3, signs=rht_signs(SEED_SIGNS) if use_rht else None,
                 slab=slab, label="small")


def test_hybrid_zero_and_empty():
    check_hybrid(torch.zeros((64, 64), dtype=torch.bfloat16), label="zeros")
    got = bsq.nvfp4_col_mxfp8_row_quantize(torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV), rounding=1)
    torch.cuda.synchronize()
    assert got["amax"][1].item() == 0.0 and got["s_enc"][1].item() == 1.0
    assert got["mx_row_codes"].shape == (0, 64) and got["col_codes"].shape == (64, 0)


@pytest.mark.parametrize("shape", [(256, 256), (272, 144), (32, 16), (48, 400), (528, 16)])
@pytest.mark.parametrize("rounding,use_rht", [(1, True), (0, True), (1, False), (0, False)])
def test_fprop_wgrad_small(shape, rounding, use_rht):
    x = outlier_bf16(shape, seed=41, mask_seed=42)
    check_fprop_wgrad(x, rounding=rounding, seed=SEED_SR_KEY, stream=5, signs=rht_signs(SEED_SIGNS) if use_rht else None,
                      label="small")


def test_fprop_wgrad_zero_and_empty():
    check_fprop_wgrad(torch.zeros((64, 64), dtype=torch.bfloat16), rounding=1, signs=rht_signs(SEED_SIGNS),
                      label="zeros")
    got = bsq.nvfp4_quantize_fprop_wgrad(torch.zeros((0, 64), dtype=torch.bfloat16, device=DEV), rounding=1,
                                         rht_signs=rht_signs(SEED_SIGNS))
    torch.cuda.synchronize()
    assert got["amax"].cpu().tolist() == [0.0, 0.0] and got["s_enc"].cpu().tolist() == [1.0, 1.0]


def test_calls_share_no_state():
    """Each call reduces only the partial maxima its own amax pass stored: consecutive calls
    with one workspace (a large-amax tensor, then a small one, and back), and calls on two
    streams with a workspace each, never see another call's amax."""
    import oracle
    big = outlier_bf16((256, 512), seed=81, mask_seed=82)        # amax in the hundreds
    small = gaussian_bf16((256, 512), 1e-4, 83)                  # amax ~ 5e-4
    refs = {id(t): oracle.nvfp4_quantize(t, direction=3) for t in (big, small)}
    ws = torch.empty(bsq.NVFP4_QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
    note("one workspace: alternating big/small tensors on one stream")
    for t in (big, small, small, big, small):
        got = bsq.nvfp4_quantize(t.to(DEV), direction=3, workspace=ws)
        torch.cuda.synchronize()
        assert_f32_equal(got["amax"], refs[id(t)]["amax"], "amax")
        assert_bytes_equal(got["row_codes"], refs[id(t)]["row_codes"], "row codes")
        assert_bytes_equal(got["col_codes"], refs[id(t)]["col_codes"], "col codes")
    note("two streams, a workspace each")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    xb, xs = big.to(DEV), small.to(DEV)
    w1 = torch.empty(bsq.NVFP4_QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
    w2 = torch.empty(bsq.NVFP4_QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            g1 = bsq.nvfp4_quantize(xb, direction=1, workspace=w1)
        with torch.cuda.stream(s2):
            g2 = bsq.nvfp4_quantize(xs, direction=1, workspace=w2)
        outs.append((g1, g2))
    torch.cuda.synchronize()
    for g1, g2 in outs:
        assert_f32_equal(g1["amax"][0:1], refs[id(big)]["amax"][0:1], "stream 1 amax")
        assert_f32_equal(g2["amax"][0:1], refs[id(small)]["amax"][0:1], "stream 2 amax")
        assert_bytes_equal(g2["row_codes"], refs[id(small)]["row_codes"], "stream 2 codes")


@pytest.mark.parametrize("direction,rounding,use_rht", [(1, 0, False), (3, 0, False), (2, 1, True)])
def test_graph_replay(direction, rounding, use_rht):
    """nvfp4_quantize captured in a HIP graph (torch.cuda.graph) and replayed on new inputs
    copied into the captured input buffer: a large-amax tensor, then a small-amax one, then
    the large one again, with eager work and synchronisation between replays.  Every replay
    must match the oracle bit for bit (nothing carries over from one replay to the next)."""
    import oracle
    shape = (512, 384)
    inputs = [outlier_bf16(shape, seed=91, mask_seed=92), gaussian_bf16(shape, 1e-4, 93),
              outlier_bf16(shape, seed=91, mask_seed=92), gaussian_bf16(shape, 3.0, 94)]
    signs = rht_signs(SEED_SIGNS) if use_rht else None
    refs = [oracle.nvfp4_quantize(t, direction=direction, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=4,
                                  signs=None if signs is None else signs.numpy()) for t in inputs]
    xin = inputs[3].to(DEV)
    sg = None if signs is None else signs.to(DEV)
    note("graph capture dir=%d rnd=%d rht=%s" % (direction, rounding, use_rht))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture, as torch requires
        bsq.nvfp4_quantize(xin, direction=direction, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=4, rht_signs=sg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = bsq.nvfp4_quantize(xin, direction=direction, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=4,
                                 rht_signs=sg)
    for i, (t, ref) in enumerate(zip(inputs, refs)):
        note("graph replay %d" % i)
        xin.copy_(t.to(DEV))
        eager = bsq.nvfp4_quantize(xin, direction=direction, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=4,
                                   rht_signs=sg)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for d, key in ((1, "row"), (2, "col")):
            if direction & d:
                k = 0 if d == 1 else 1
                assert_f32_equal(out["amax"][k:k + 1], ref["amax"][k:k + 1], "replay %d amax %s" % (i, key))
                assert_f32_equal(out["s_enc"][k:k + 1], ref["s_enc"][k:k + 1], "replay %d s_enc %s" % (i, key))
                assert_bytes_equal(out[key + "_scales"], ref[key + "_scales"], "replay %d %s scales" % (i, key))
                assert_bytes_equal(out[key + "_codes"], ref[key + "_codes"], "replay %d %s codes" % (i, key))
                assert torch.equal(out[key + "_codes"], eager[key + "_codes"]), "replay %d vs eager" % i


def test_graph_replay_one_pass_casts():
    """The two one-pass casts (an activation's rowwise RNE + columnwise RHT + SR; dY's NVFP4
    columnwise RHT + SR + MXFP8 rowwise) captured in one HIP graph and replayed on a large-amax,
    a small-amax and again the large-amax input: every replay matches the oracle bit for bit."""
    import oracle
    shape = (512, 384)
    inputs = [outlier_bf16(shape, seed=95, mask_seed=96), gaussian_bf16(shape, 1e-4, 97),
              outlier_bf16(shape, seed=95, mask_seed=96)]
    signs = rht_signs(SEED_SIGNS)
    sn = signs.numpy()
    refs = [(oracle.nvfp4_quantize(t, direction=1),
             oracle.nvfp4_quantize(t, direction=2, rounding=1, sr_seed=SEED_SR_KEY, sr_stream=1, signs=sn),
             oracle.nvfp4_quantize(t, direction=2, rounding=1, sr_seed=SEED_SR_KEY, sr_stream=0, signs=sn),
             oracle.mxfp8_quantize(t, direction=1)) for t in inputs]
    xin = inputs[2].to(DEV)
    sg = signs.to(DEV)
    note("graph capture of the one-pass casts")
    calls = lambda: (bsq.nvfp4_quantize_fprop_wgrad(xin, rounding=1, sr_seed=SEED_SR_KEY, sr_stream=1, rht_signs=sg),
                     bsq.nvfp4_col_mxfp8_row_quantize(xin, rounding=1, sr_seed=SEED_SR_KEY, sr_stream=0, rht_signs=sg))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fw, hy = calls()
    for i, (t, (rrow, rcol1, rcol0, rmx)) in enumerate(zip(inputs, refs)):
        note("graph replay %d" % i)
        xin.copy_(t.to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_f32_equal(fw["s_enc"][0:1], rrow["s_enc"][0:1], "replay %d fprop s_enc" % i)
        assert_bytes_equal(fw["row_scales"], rrow["row_scales"], "replay %d fprop row_scales" % i)
        assert_bytes_equal(fw["row_codes"], rrow["row_codes"], "replay %d fprop row_codes" % i)
        assert_f32_equal(fw["s_enc"][1:2], rcol1["s_enc"][1:2], "replay %d wgrad s_enc" % i)
        assert_bytes_equal(fw["col_scales"], rcol1["col_scales"], "replay %d wgrad col_scales" % i)
        assert_bytes_equal(fw["col_codes"], rcol1["col_codes"], "replay %d wgrad col_codes" % i)
        assert_f32_equal(hy["s_enc"][1:2], rcol0["s_enc"][1:2], "replay %d dY s_enc" % i)
        assert_bytes_equal(hy["col_scales"], rcol0["col_scales"], "replay %d dY col_scales" % i)
        assert_bytes_equal(hy["col_codes"], rcol0["col_codes"], "replay %d dY col_codes" % i)
        assert_bytes_equal(hy["mx_row_scales"], rmx["row_scales"], "replay %d dY mxfp8 scales" % i)
        assert_bytes_equal(hy["mx_row_codes"], rmx["row_codes"], "replay %d dY mxfp8 codes" % i)


def test_nvfp4_extreme_values():
    """Subnormal bf16, huge values and signed zeros in one tensor."""
    v = torch.tensor([0.0, -0.0, 1e-40, -1e-39, 3.0e38, -2.5e38, 1.0, -6.0] * 64, dtype=torch.float32)
    x = v.reshape(32, 16).to(torch.bfloat16)
    check_nvfp4(x, 3, label="extreme")
    # with RHT the 16-point sums must stay finite (non-finite values are unsupported)
    v2 = torch.tensor([0.0, -0.0, 1e-40, -1e-39, 1.0e37, -2.5e36, 1.0, -6.0] * 64, dtype=torch.float32)
    check_nvfp4(v2.reshape(32, 16).to(torch.bfloat16), 3, rounding=1, seed=5, signs=rht_signs(3),
                label="extreme-sr")


@pytest.mark.parametrize("shape", [(128, 256), (256, 128), (288, 160), (32, 32)])
@pytest.mark.parametrize("direction", [1, 2, 3])
def test_mxfp8_small(shape, direction):
    check_mxfp8(outlier_bf16(shape, seed=31, mask_seed=32), direction, label="small")


def test_mxfp8_extreme_and_zero_blocks():
    v = torch.zeros((64, 64), dtype=torch.float32)
    v[0, :32] = torch.tensor([1e-40, -3e38] + [0.0] * 30)
    v[1, 32:] = -0.0
    v[2:] = torch.randn((62, 64), generator=torch.Generator().manual_seed(1)) * 1e30
    check_mxfp8(v.to(torch.bfloat16), 3, label="extreme")


def block_edge_bf16(R, C, seed):
    """bf16 [R, C] whose columnwise 32-blocks sit on the MXFP8 encoder's edges: each block's amax
    has a random exponent field in 9..254 and a mantissa that is random or one of the saturation
    edges (448, just below / at / above 464, and 511 after scaling); the other elements are bit
    patterns at most the amax (half uniform, so bf16 subnormals and zeros occur, half within 40
    patterns of it), with random signs.  The first 64 rows of columns 128..255 also hold blocks
    whose scale byte is 0 (all zero with -0 entries, or amax exponent 0..8), so that waves with
    and without such blocks meet in one launch."""
    g = np.random.default_rng(seed)
    nb = R // 32
    exp = g.integers(9, 255, size=(nb, C))
    mant = g.integers(0, 128, size=(nb, C))
    pick = g.random((nb, C)) < 0.5
    mant[pick] = g.choice([0x60, 0x67, 0x68, 0x69, 0x7F], size=int(pick.sum()))
    amax = (exp << 7) | mant
    if C > 128:
        amax[0, 130:132] = 0
        amax[1, 140:144] = g.integers(0, 9, size=4) << 7 | g.integers(0, 128, size=4)
    amax3 = amax[:, None, :]
    u = g.random((nb, 32, C))
    near = g.random((nb, 32, C)) < 0.5
    mag = np.where(near, amax3 - np.floor(u * 41), np.floor(u * (amax3 + 1))).astype(np.int64)
    mag = np.clip(mag, 0, amax3)
    at = g.integers(0, 32, size=(nb, C))
    mag[np.arange(nb)[:, None], at, np.arange(C)[None, :]] = amax
    sign = (g.random((nb, 32, C)) < 0.5).astype(np.int64)
    bits = (mag | (sign << 15)).astype(np.uint16).reshape(R, C)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)


@pytest.mark.parametrize("shape", [(512, 256), (288, 160)])
def test_mxfp8_block_edges(shape):
    x = block_edge_bf16(*shape, seed=61)
    for direction in (2, 3):
        check_mxfp8(x, direction, label="block-edges")


@pytest.mark.parametrize("shape", [(576, 64), (832, 128), (1088, 192), (320, 320), (64, 128)])
def test_mxfp8_both_slab_ragged_bands(shape):
    """Rowwise + columnwise MXFP8 with both code matrices in the slab layout, on row counts whose
    512-row tiles end inside a band or span a full band and a partial one (rows past the tensor
    must not land in the band's next slab), against the oracle's row-major codes."""
    import oracle
    from tests.gpu_common import from_slab
    R, Cc = shape
    x = outlier_bf16(shape, seed=71, mask_seed=72)
    note("mxfp8 both slab shape=%s" % (shape,))
    got = bsq.mxfp8_quantize(x.to(DEV), direction=bsq.ROW | bsq.COL | bsq.MX_SLAB)
    torch.cuda.synchronize()
    ref = oracle.mxfp8_quantize(x, direction=3)
    assert_bytes_equal(got["row_scales"], ref["row_scales"], "row_scales")
    assert_bytes_equal(got["col_scales"], ref["col_scales"], "col_scales")
    assert np.array_equal(from_slab(got["row_codes"], R, Cc), ref["row_codes"]), "row codes"
    assert np.array_equal(from_slab(got["col_codes"], Cc, R), ref["col_codes"]), "col codes"


def test_rht_apply_matches_oracle():
    import oracle
    for axis in (0, 1):
        for shape in [(256, 128), (272, 144), (32, 16)]:
            x = gaussian_bf16(shape, 1.0, 41)
            note("rht_apply axis=%d shape=%s" % (axis, shape))
            got = bsq.rht_apply(x.to(DEV), axis, rht_signs(SEED_SIGNS))
            torch.cuda.synchronize()
            assert_f32_equal(got, oracle.rht_apply(x, axis, rht_signs(SEED_SIGNS).numpy()), "rht axis %d" % axis)


def test_dequantize_matches_oracle():
    import oracle
    x = outlier_bf16((256, 512), seed=51, mask_seed=52)
    q = bsq.nvfp4_quantize(x.to(DEV), direction=1)
    note("nvfp4_dequantize [256,512]")
    d = bsq.nvfp4_dequantize(q["row_codes"], q["row_scales"], q["s_enc"][0:1])
    torch.cuda.synchronize()
    r = oracle.nvfp4_quantize(x, direction=1)
    assert_bytes_equal(q["row_codes"], r["row_codes"], "codes")
    assert_bytes_equal(q["row_scales"], r["row_scales"], "scales")
    ref = oracle.nvfp4_dequantize(r["row_codes"], r["row_scales"], float(r["s_enc"][0]))
    assert np.array_equal(d.cpu().view(torch.int16).numpy().view(np.uint16), ref)


# ----------------------------------------------------------------- workload shapes

def test_quant_only_workload():
    """[8192, 4096] N(0,1) with 1 % of entries x100: NVFP4 row + col (RNE) and MXFP8 row + col."""
    x = outlier_bf16((8192, 4096))
    check_nvfp4(x, 3, label="quant-only")
    check_mxfp8(x, 3, label="quant-only")


def test_beyond_2g_elements():
    """A [131088, 16384] tensor (2^31 + 2^18 elements, input byte offsets past 2^32): NVFP4
    rowwise RNE, MXFP8 rowwise, row-scaled NVFP4, NVFP4 columnwise RNE with RHT, the two
    one-pass casts (NVFP4 columnwise + MXFP8 rowwise; NVFP4 rowwise + columnwise), and MXFP8
    columnwise of its first 131072 rows (2^31 elements; MXFP8 columns need rows % 32 == 0).
    The tensor maximum (100, above every N(0,1) draw) is planted at row 0, column 5, so any set of rows containing row 0
    (or of columns containing column 5) has the tensor's scale; rowwise codes depend only on
    their row and that scale, columnwise codes only on their column, so the oracle quantizes
    sampled rows (the first and last, the middle, a random spread) or sampled columns on
    their own."""
    import oracle
    R, C = 131072 + 16, 16384
    note("rowwise beyond 2^31 elements: generating %s on the host (~1 min)" % ((R, C),))
    x = gaussian_bf16((R, C), 1.0, 99)
    x[0, 5] = 100.0
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, 1, R // 2, R - 2, R - 1], rng.choice(R, 12, replace=False)]))
    sub = x[torch.from_numpy(rows)].contiguous()
    note("rowwise beyond 2^31 elements: quantizing on the GPU")
    xd = x.to(DEV)
    del x
    got = bsq.nvfp4_quantize(xd, direction=1)
    idx = torch.from_numpy(rows).to(DEV)
    g_codes, g_scales = got["row_codes"][idx].contiguous(), got["row_scales"][idx].contiguous()
    g_amax, g_senc = got["amax"][0:1].clone(), got["s_enc"][0:1].clone()
    del got
    mx = bsq.mxfp8_quantize(xd, direction=1)
    m_codes, m_scales = mx["row_codes"][idx].contiguous(), mx["row_scales"][idx].contiguous()
    del mx
    rs = bsq.nvfp4_quantize_rowscaled(xd)   # one outer scale per row: rows fully independent
    r_codes, r_scales = rs["codes"][idx].contiguous(), rs["scales"][idx].contiguous()
    r_amax, r_senc = rs["amax"][idx].contiguous(), rs["s_enc"][idx].contiguous()
    del rs
    # columnwise with RHT (blocks and transform run along rows, so columns are independent
    # given the tensor scale; column 5 holds the maximum, about 25 after the transform)
    signs = rht_signs(SEED_SIGNS)
    cols = np.unique(np.concatenate([[0, 5, C // 2, C - 1], rng.choice(C, 8, replace=False)]))
    col = bsq.nvfp4_quantize(xd, direction=2, rht_signs=signs)
    cidx = torch.from_numpy(cols).to(DEV)
    c_codes, c_scales = col["col_codes"][cidx].contiguous(), col["col_scales"][cidx].contiguous()
    c_amax, c_senc = col["amax"][1:2].clone(), col["s_enc"][1:2].clone()
    # the one-pass casts on the same tensor (RNE, so that sampled rows and columns are
    # independent of the element indices SR would draw with): dY's NVFP4 columnwise (RHT) +
    # MXFP8 rowwise, and an activation's rowwise RNE + columnwise RHT
    note("rowwise beyond 2^31 elements: one-pass casts")
    del col
    hy = bsq.nvfp4_col_mxfp8_row_quantize(xd, rht_signs=signs)
    h_codes, h_scales = hy["col_codes"][cidx].contiguous(), hy["col_scales"][cidx].contiguous()
    h_mc, h_ms = hy["mx_row_codes"][idx].contiguous(), hy["mx_row_scales"][idx].contiguous()
    del hy
    fw = bsq.nvfp4_quantize_fprop_wgrad(xd, rht_signs=signs)
    f_rc, f_rs = fw["row_codes"][idx].contiguous(), fw["row_scales"][idx].contiguous()
    f_cc, f_cs = fw["col_codes"][cidx].contiguous(), fw["col_scales"][cidx].contiguous()
    f_senc = fw["s_enc"].clone()
    del fw
    note("rowwise beyond 2^31 elements: MXFP8 columnwise")
    mc = bsq.mxfp8_quantize(xd[:131072], direction=2)
    mc_codes, mc_scales = mc["col_codes"][cidx].contiguous(), mc["col_scales"][cidx].contiguous()
    del mc
    sub_c = xd[:, cidx].cpu().contiguous()
    del xd
    torch.cuda.synchronize()
    ref = oracle.nvfp4_quantize(sub, direction=1)
    assert_f32_equal(g_amax, ref["amax"][0:1], "amax")
    assert_f32_equal(g_senc, ref["s_enc"][0:1], "s_enc")
    assert_bytes_equal(g_scales, ref["row_scales"], "row_scales")
    assert_bytes_equal(g_codes, ref["row_codes"], "row_codes")
    mref = oracle.mxfp8_quantize(sub, direction=1)
    assert_bytes_equal(m_scales, mref["row_scales"], "mxfp8 row_scales")
    assert_bytes_equal(m_codes, mref["row_codes"], "mxfp8 row_codes")
    rref = oracle.nvfp4_quantize_rowscaled(sub)
    assert_f32_equal(r_amax, rref["amax"], "row-scaled amax")
    assert_f32_equal(r_senc, rref["s_enc"], "row-scaled s_enc")
    assert_bytes_equal(r_scales, rref["scales"], "row-scaled scales")
    assert_bytes_equal(r_codes, rref["codes"], "row-scaled codes")
    cref = oracle.nvfp4_quantize(sub_c, direction=2, signs=signs.numpy())
    assert_f32_equal(c_amax, cref["amax"][1:2], "col amax")
    assert_f32_equal(c_senc, cref["s_enc"][1:2], "col s_enc")
    assert_bytes_equal(c_scales, cref["col_scales"], "col_scales")
    assert_bytes_equal(c_codes, cref["col_codes"], "col_codes")
    assert_bytes_equal(h_scales, cref["col_scales"], "one-pass col_scales")
    assert_bytes_equal(h_codes, cref["col_codes"], "one-pass col_codes")
    assert_bytes_equal(h_ms, mref["row_scales"], "one-pass mxfp8 row_scales")
    assert_bytes_equal(h_mc, mref["row_codes"], "one-pass mxfp8 row_codes")
    assert_f32_equal(f_senc[0:1], ref["s_enc"][0:1], "fprop+wgrad s_enc row")
    assert_f32_equal(f_senc[1:2], cref["s_enc"][1:2], "fprop+wgrad s_enc col")
    assert_bytes_equal(f_rs, ref["row_scales"], "fprop+wgrad row_scales")
    assert_bytes_equal(f_rc, ref["row_codes"], "fprop+wgrad row_codes")
    assert_bytes_equal(f_cs, cref["col_scales"], "fprop+wgrad col_scales")
    assert_bytes_equal(f_cc, cref["col_codes"], "fprop+wgrad col_codes")
    mcref = oracle.mxfp8_quantize(sub_c[:131072].contiguous(), direction=2)   # columns are independent
    assert_bytes_equal(mc_scales, mcref["col_scales"], "mxfp8 col_scales")
    assert_bytes_equal(mc_codes, mcref["col_codes"], "mxfp8 col_codes")


def test_fwd_operands_llama3_8b():
    """Forward operands of the Llama-3-8B FFN up-projection, NVFP4 rowwise RNE."""
    check_nvfp4(gaussian_bf16((16384, 4096), 1.0, SEED_X), 1, label="fwd X")
    check_nvfp4(gaussian_bf16((14336, 4096), STD_W, SEED_W), 1, label="fwd W")


def test_x_fprop_wgrad_llama3_8b():
    """The layer input X [16384, 4096] in one pass: rowwise RNE for the forward GEMM and
    columnwise RHT + SR (stream 1) for wgrad."""
    check_fprop_wgrad(gaussian_bf16((16384, 4096), 1.0, SEED_X), rounding=1, seed=SEED_SR_KEY, stream=1,
                      signs=rht_signs(SEED_SIGNS), label="X")


def test_dy_hybrid_llama3_8b():
    """The backward's dY [16384, 14336] in one pass: NVFP4 columnwise with RHT + SR (stream 0)
    for wgrad and MXFP8 rowwise in the slab layout for dgrad."""
    check_hybrid(gaussian_bf16((16384, 14336), STD_DY, SEED_DY), rounding=1, seed=SEED_SR_KEY, stream=0,
                 signs=rht_signs(SEED_SIGNS), slab=True, label="dY")


def test_wgrad_operands_llama3_8b():
    """wgrad operands: 16-point RHT along tokens, columnwise NVFP4, Philox SR (streams 0/1)."""
    signs = rht_signs(SEED_SIGNS)
    check_nvfp4(gaussian_bf16((16384, 14336), STD_DY, SEED_DY), 2, rounding=1, seed=SEED_SR_KEY, stream=0,
                signs=signs, label="wgrad dY")
    check_nvfp4(gaussian_bf16((16384, 4096), 1.0, SEED_X), 2, rounding=1, seed=SEED_SR_KEY, stream=1,
                signs=signs, label="wgrad X")
