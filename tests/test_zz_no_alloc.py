"""GPU check of nvfp4_quantize_noalloc (the variant that keeps its partial maxima in a library
array instead of a caller workspace), through the C ABI: two calls in a row, the second on a
smaller tensor with a smaller amax, each bit for bit equal to nvfp4_quantize with a workspace
on the same input (codes, scales, amax, tensor scales), and to the oracle."""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsq
from synthetic import SEED_SIGNS, SEED_SR_KEY, gaussian_bf16, outlier_bf16, rht_signs
from tests.gpu_common import assert_bytes_equal, assert_f32_equal, note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def outputs(R, C):
    u8 = dict(dtype=torch.uint8, device=DEV)
    return {"row_codes": torch.empty((R, C // 2), **u8), "row_scales": torch.empty((R, C // 16), **u8),
            "col_codes": torch.empty((C, R // 2), **u8), "col_scales": torch.empty((C, R // 16), **u8),
            "amax": torch.empty(2, dtype=torch.float32, device=DEV),
            "s_enc": torch.empty(2, dtype=torch.float32, device=DEV)}


def call_noalloc(x, rounding, seed, stream, signs):
    """nvfp4_quantize_noalloc on x, both directions, outputs allocated here (the caller's)."""
    R, C = x.shape
    o = outputs(R, C)
    st = bsq.lib().nvfp4_quantize_noalloc(
        x.data_ptr(), R, C, 3, rounding, seed, stream, None if signs is None else signs.data_ptr(),
        o["row_codes"].data_ptr(), o["row_scales"].data_ptr(), o["col_codes"].data_ptr(), o["col_scales"].data_ptr(),
        o["amax"].data_ptr(), o["s_enc"].data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, bsq.lib().bsq_last_error().decode()
    return o


def test_noalloc_matches_workspace_entry_point():
    import oracle
    signs = rht_signs(SEED_SIGNS)
    cases = [  # the second input is smaller and has a far smaller amax than the first
        (outlier_bf16((1024, 768), seed=61, mask_seed=62), 0, None),
        (gaussian_bf16((256, 512), 1e-4, 63), 1, signs),
    ]
    for i, (x_cpu, rounding, sg) in enumerate(cases):
        note("noalloc call %d shape=%s rnd=%d rht=%s" % (i, tuple(x_cpu.shape), rounding, sg is not None))
        x = x_cpu.to(DEV)
        sgd = None if sg is None else sg.to(DEV)
        got = call_noalloc(x, rounding, SEED_SR_KEY, 5, sgd)
        want = bsq.nvfp4_quantize(x, direction=3, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=5, rht_signs=sgd)
        torch.cuda.synchronize()
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            assert torch.equal(got[k], want[k]), "call %d %s differs from nvfp4_quantize" % (i, k)
        assert torch.equal(got["amax"].view(torch.int32), want["amax"].view(torch.int32)), "call %d amax" % i
        assert torch.equal(got["s_enc"].view(torch.int32), want["s_enc"].view(torch.int32)), "call %d s_enc" % i
        ref = oracle.nvfp4_quantize(x_cpu, direction=3, rounding=rounding, sr_seed=SEED_SR_KEY, sr_stream=5,
                                    signs=None if sg is None else sg.numpy())
        assert_f32_equal(got["amax"], ref["amax"], "call %d amax vs oracle" % i)
        for k in ("row_codes", "row_scales", "col_codes", "col_scales"):
            assert_bytes_equal(got[k], ref[k], "call %d %s vs oracle" % (i, k))


def test_noalloc_rejects_invalid_arguments():
    """The same validation as nvfp4_quantize (no workspace argument to check)."""
    L = bsq.lib()
    f = L.nvfp4_quantize_noalloc
    assert f(0x10000, 64, 64, 4, 0, 0, 0, None, 0x10000, 0x10000, None, None, 0x10000, 0x10000, None) == 3
    assert f(0x10000, 64, 24, 1, 0, 0, 0, None, 0x10000, 0x10000, None, None, 0x10000, 0x10000, None) == 2
    assert f(0x10000, 64, 64, 1, 0, 0, 0, None, 0x10000, 0x10000, None, None, None, 0x10000, None) == 1
