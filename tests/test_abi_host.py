"""Host-only checks of the C ABI (no GPU needed): the library loads, exports every
entry point include/bsq.h declares, and rejects every invalid argument with the
documented status before any HIP call is made."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsq.h")


@pytest.fixture(scope="module")
def L():
    import block_scaled_precision_nvfp4_amd as bsq
    if not os.path.exists(bsq.LIB_PATH):
        from block_scaled_precision_nvfp4_amd import build
        build.build()
    return bsq.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ["nvfp4_quantize", "nvfp4_quantize_rowscaled", "nvfp4_dequantize", "mxfp8_quantize",
              "mxfp8_requantize_nvfp4", "rht_apply", "blockscaled_gemm", "blockscaled_grouped_gemm",
              "nvfp4_linear_workspace_bytes", "nvfp4_linear_saved_bytes", "nvfp4_linear_forward",
              "nvfp4_linear_backward", "bsq_last_error", "bsq_version", "nvfp4_quantize_noalloc",
              "nvfp4_col_mxfp8_row_quantize", "nvfp4_quantize_fprop_wgrad"]:
        assert f in names


def test_every_declared_symbol_is_exported(L):
    for f in declared_functions():
        assert hasattr(L, f), f


def test_version(L):
    assert L.bsq_version() == 200


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails before any HIP call


def q(L, x=FAKE, rows=256, cols=256, direction=1, rounding=0, signs=None, rc=FAKE, rs=FAKE, cc=FAKE, cs=FAKE,
      amax=FAKE, senc=FAKE, ws=FAKE):
    return L.nvfp4_quantize(x, rows, cols, direction, rounding, 0, 0, signs, rc, rs, cc, cs, amax, senc, ws, None)


def last(L):
    return L.bsq_last_error().decode()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(direction=0), 3, "direction"),
    (dict(direction=4), 3, "direction"),
    (dict(rounding=2), 3, "rounding"),
    (dict(rows=-1), 2, "negative"),
    (dict(cols=12), 2, "multiple of 8"),
    (dict(cols=24, direction=1), 2, "cols % 16"),
    (dict(rows=24, direction=2), 2, "rows % 16"),
    (dict(amax=None), 1, "amax_out"),
    (dict(senc=None), 1, "amax_out"),
    (dict(x=None), 1, "x is NULL"),
    (dict(rc=None, direction=1), 1, "rowwise outputs"),
    (dict(cs=None, direction=3), 1, "columnwise outputs"),
    (dict(x=FAKE + 8), 6, "aligned"),
    (dict(signs=FAKE + 2), 6, "aligned"),
    (dict(ws=None), 1, "workspace"),
    (dict(ws=FAKE + 4), 6, "aligned"),
])
def test_nvfp4_quantize_validation(L, kw, status, needle):
    assert q(L, **kw) == status
    assert needle in last(L)


def test_nvfp4_quantize_workspace_size(L):
    """The header's workspace size matches the binding's constant; an empty tensor needs none."""
    import block_scaled_precision_nvfp4_amd as bsq
    text = open(HEADER).read()
    m = re.search(r"#define BSQ_NVFP4_QUANTIZE_WORKSPACE_BYTES (\d+)", text)
    assert m and int(m.group(1)) == bsq.NVFP4_QUANTIZE_WORKSPACE_BYTES
    # an empty tensor only writes amax = 0 and S = 1 (a launch), so it is not called here; its
    # validation must accept a NULL workspace and NULL outputs: a zero-row columnwise call with
    # misaligned outputs still fails on alignment, proving it got past the NULL checks
    assert q(L, rows=0, rc=None, rs=None, cc=None, cs=None, ws=None, x=FAKE + 8) == 6


def hyb(L, x=FAKE, rows=256, cols=256, rounding=1, signs=None, cc=FAKE, cs=FAKE, amax=FAKE, senc=FAKE, ws=FAKE,
        layout=0, mc=FAKE, ms=FAKE):
    return L.nvfp4_col_mxfp8_row_quantize(x, rows, cols, rounding, 0, 0, signs, cc, cs, amax, senc, ws, layout,
                                          mc, ms, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(layout=1), 3, "mx_layout"),
    (dict(layout=4 | 1), 3, "mx_layout"),
    (dict(rounding=3), 3, "rounding"),
    (dict(rows=24), 2, "rows % 16"),
    (dict(cols=48), 2, "cols % 32"),
    (dict(cols=96, layout=4), 2, "cols % 64"),
    (dict(cc=None), 1, "columnwise outputs"),
    (dict(ws=None), 1, "workspace"),
    (dict(mc=None), 1, "MXFP8 rowwise outputs"),
    (dict(ms=None), 1, "MXFP8 rowwise outputs"),
    (dict(mc=FAKE + 8), 6, "aligned"),
    (dict(x=FAKE + 8), 6, "aligned"),
])
def test_hybrid_quantize_validation(L, kw, status, needle):
    assert hyb(L, **kw) == status
    assert needle in last(L)


def test_hybrid_quantize_empty_needs_no_outputs(L):
    # a zero-row call accepts NULL outputs and workspace: misaligned x still fails on alignment,
    # which proves the call got past the NULL checks without launching anything
    assert hyb(L, rows=0, cc=None, cs=None, ws=None, mc=None, ms=None, x=FAKE + 8) == 6


def fw(L, x=FAKE, rows=256, cols=256, rounding=1, signs=None, rc=FAKE, rs=FAKE, cc=FAKE, cs=FAKE, amax=FAKE,
       senc=FAKE, ws=FAKE):
    return L.nvfp4_quantize_fprop_wgrad(x, rows, cols, rounding, 0, 0, signs, rc, rs, cc, cs, amax, senc, ws, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(rounding=2), 3, "rounding"),
    (dict(rows=24), 2, "rows % 16"),
    (dict(cols=24), 2, "cols % 16"),
    (dict(rows=-16), 2, "negative"),
    (dict(rc=None), 1, "rowwise outputs"),
    (dict(cs=None), 1, "columnwise outputs"),
    (dict(amax=None), 1, "amax_out"),
    (dict(ws=None), 1, "workspace"),
    (dict(x=FAKE + 8), 6, "aligned"),
    (dict(signs=FAKE + 2), 6, "aligned"),
])
def test_fprop_wgrad_quantize_validation(L, kw, status, needle):
    assert fw(L, **kw) == status
    assert needle in last(L)


def test_mxfp8_quantize_validation(L):
    f = L.mxfp8_quantize
    assert f(FAKE, 64, 48, 1, FAKE, FAKE, None, None, None) == 2 and "cols % 32" in last(L)
    assert f(FAKE, 48, 64, 2, None, None, FAKE, FAKE, None) == 2 and "rows % 32" in last(L)
    assert f(FAKE, 64, 64, 8, FAKE, FAKE, None, None, None) == 3 and "direction" in last(L)
    assert f(FAKE, 64, 64, 4, FAKE, FAKE, None, None, None) == 3 and "direction" in last(L)
    # the slab layout needs whole 64-byte slices along the codes' contraction dimension
    assert f(FAKE, 64, 96, 1 | 4, FAKE, FAKE, None, None, None) == 2 and "cols % 64" in last(L)
    assert f(FAKE, 96, 64, 2 | 4, None, None, FAKE, FAKE, None) == 2 and "rows % 64" in last(L)
    # rowwise slab codes leave rows free (this call gets as far as the NULL input)
    assert f(None, 96, 64, 1 | 4, FAKE, FAKE, None, None, None) == 1 and "x is NULL" in last(L)
    assert f(FAKE, 0, 64, 2 | 4, None, None, FAKE, FAKE, None) == 0
    assert f(None, 64, 64, 1, FAKE, FAKE, None, None, None) == 1
    assert f(FAKE, 64, 64, 2, FAKE, FAKE, None, FAKE, None) == 1
    assert f(FAKE + 4, 64, 64, 1, FAKE, FAKE, None, None, None) == 6


def test_mxfp8_requantize_validation(L):
    f = L.mxfp8_requantize_nvfp4
    assert f(FAKE, FAKE, FAKE, 64, 64, 0, FAKE, FAKE, None, None, None) == 3 and "direction" in last(L)
    assert f(FAKE, FAKE, FAKE, 64, 24, 2, None, None, FAKE, FAKE, None) == 2 and "multiple of 16" in last(L)
    assert f(FAKE, FAKE, FAKE, 64, 48, 1, FAKE, FAKE, None, None, None) == 2 and "cols % 32" in last(L)
    assert f(FAKE, FAKE, FAKE, 48, 64, 2, None, None, FAKE, FAKE, None) == 2 and "rows % 32" in last(L)
    assert f(FAKE, None, FAKE, 64, 64, 2, None, None, FAKE, FAKE, None) == 1 and "NVFP4 input" in last(L)
    assert f(FAKE, FAKE, None, 64, 64, 2, None, None, FAKE, FAKE, None) == 1
    assert f(FAKE, FAKE, FAKE, 64, 64, 2, None, None, None, FAKE, None) == 1 and "columnwise outputs" in last(L)
    assert f(FAKE + 4, FAKE, FAKE, 64, 64, 2, None, None, FAKE, FAKE, None) == 6
    assert f(FAKE, FAKE, FAKE, 0, 64, 2, None, None, FAKE, FAKE, None) == 0
    assert f(FAKE, FAKE, FAKE, 64, 96, 1 | 4, FAKE, FAKE, None, None, None) == 2 and "cols % 64" in last(L)
    assert f(FAKE, FAKE, FAKE, 96, 64, 2 | 4, None, None, FAKE, FAKE, None) == 2 and "rows % 64" in last(L)


def test_rht_apply_validation(L):
    f = L.rht_apply
    assert f(FAKE, 64, 64, 2, FAKE, FAKE, None) == 3
    assert f(FAKE, 64, 24, 1, FAKE, FAKE, None) == 2
    assert f(FAKE, 24, 64, 0, FAKE, FAKE, None) == 2
    assert f(FAKE, 64, 64, 1, None, FAKE, None) == 1


def test_gemm_validation(L):
    f = L.blockscaled_gemm
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert f(2, 128, 128, 128, *args, 0, None) == 3 and "fmt" in last(L)
    assert f(0, 128, 128, 128, *args, 2, None) == 3 and "c_dtype" in last(L)
    assert f(0, 128, 128, 48, *args, 0, None) == 2 and "multiple of 32" in last(L)
    assert f(0, -1, 128, 64, *args, 0, None) == 2
    assert f(1, 128, 128, (1 << 23) + 32, *args, 0, None) == 2 and "exceeds" in last(L)
    assert f(0, 128, 128, (1 << 24) + 32, *args, 0, None) == 2 and "exceeds" in last(L)
    # the bound is exclusive: a 256-row tile of 2^24 NVFP4 (2^23 MXFP8) elements per row would
    # span exactly 2^31 bytes, one more than a buffer resource covers
    assert f(0, 128, 128, 1 << 24, *args, 0, None) == 2 and "exceeds" in last(L)
    assert f(1, 128, 128, 1 << 23, *args, 0, None) == 2 and "exceeds" in last(L)
    assert f(0, 128, 128, 64, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == 1 and "tensor scales" in last(L)
    assert f(0, 128, 128, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert f(0, 128, 128, 64, FAKE + 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == 6
    # empty products are valid no-ops that never reach the device
    assert f(0, 0, 128, 64, *args, 0, None) == 0
    assert f(1, 128, 0, 64, *args, 0, None) == 0


def test_gemm_rowscaled_flag_validation(L):
    f = L.blockscaled_gemm
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    # the row-scaled flags are NVFP4-only and must not hide an invalid base format
    assert f(1 | 0x10, 128, 128, 64, *args, 0, None) == 3 and "NVFP4 operands only" in last(L)
    assert f(2 | 0x20, 128, 128, 64, *args, 0, None) == 3 and "fmt" in last(L)
    assert f(0x40, 128, 128, 64, *args, 0, None) == 3
    assert f(0x10 | 0x20, 128, 128, 64, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == 1
    assert f(0x30, 0, 128, 64, *args, 0, None) == 0


def test_gemm_slab_flag_validation(L):
    f = L.blockscaled_gemm
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert f(0 | 0x40, 128, 128, 512, *args, 0, None) == 3 and "MXFP8 operands only" in last(L)
    assert f(1 | 0x40, 128, 128, 1056, *args, 0, None) == 2 and "K % 512" in last(L)
    assert f(1 | 0x40 | 0x10, 128, 128, 512, *args, 0, None) == 3 and "NVFP4 operands only" in last(L)
    assert f(1 | 0x40, 128, 128, 512, FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == 6
    assert f(1 | 0x40, 0, 128, 512, *args, 0, None) == 0
    assert f(1 | 0xC0, 128, 128, 1056, *args, 0, None) == 2 and "K % 512" in last(L)
    assert f(1 | 0x80, 0, 128, 512, *args, 0, None) == 0
    # grouped: B (stacked per-group matrices) may be slab with BSQ_GROUP_M; A and B (whole
    # matrices over the grouped extent) with BSQ_GROUP_K; MXFP8 only, K % 512 == 0
    gg_ = L.blockscaled_grouped_gemm
    assert gg_(1 | 0x40, 1, 4, FAKE, 256, 256, 512, *[FAKE] * 7, 0, None) == 3 and "GROUP_K only" in last(L)
    assert gg_(1 | 0xC0, 1, 4, FAKE, 256, 256, 512, *[FAKE] * 7, 0, None) == 3 and "GROUP_K only" in last(L)
    assert gg_(0 | 0x80, 1, 4, FAKE, 256, 256, 512, *[FAKE] * 7, 0, None) == 3 and "MXFP8 only" in last(L)
    assert gg_(0 | 0x40, 2, 4, FAKE, 256, 256, 512, *[FAKE] * 7, 0, None) == 3 and "MXFP8 only" in last(L)
    assert gg_(1 | 0x80, 1, 4, FAKE, 256, 256, 1056, *[FAKE] * 7, 0, None) == 2 and "K % 512" in last(L)
    assert gg_(1 | 0xC0, 2, 4, FAKE, 256, 256, 1056, *[FAKE] * 7, 0, None) == 2 and "K % 512" in last(L)
    assert gg_(1 | 0x80, 1, 4, None, 256, 256, 512, *[FAKE] * 7, 0, None) == 1
    for fl in (0x40, 0x80, 0xC0):   # accepted: the call gets as far as the NULL offsets
        assert gg_(1 | fl, 2, 4, None, 256, 256, 512, *[FAKE] * 7, 0, None) == 1 and "offsets" in last(L)


def gg(L, fmt=0, mode=1, groups=4, offs=FAKE, M=256, N=256, K=256, ac=FAKE, as_=FAKE, sa=FAKE, bc=FAKE, bs=FAKE,
       sb=FAKE, c=FAKE, c_dtype=0):
    return L.blockscaled_grouped_gemm(fmt, mode, groups, offs, M, N, K, ac, as_, sa, bc, bs, sb, c, c_dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(fmt=2), 3, "fmt"),
    (dict(fmt=1 | 0x10), 3, "NVFP4 operands only"),
    (dict(mode=0), 3, "mode"),
    (dict(mode=3), 3, "mode"),
    (dict(mode=2, fmt=0x10), 3, "BSQ_GROUP_M only"),
    (dict(c_dtype=5), 3, "c_dtype"),
    (dict(groups=-1), 2, "negative"),
    (dict(K=48), 2, "multiple of 32"),
    (dict(groups=(1 << 24) + 1), 2, "too many groups"),
    (dict(offs=None), 1, "offsets"),
    (dict(c=None), 1, "c is NULL"),
    (dict(bc=None), 1, "operand"),
    (dict(sa=None), 1, "tensor-scale"),
    (dict(offs=FAKE + 4), 6, "8-byte"),
    (dict(ac=FAKE + 8), 6, "aligned"),
])
def test_grouped_gemm_validation(L, kw, status, needle):
    assert gg(L, **kw) == status
    assert needle in last(L)


def test_grouped_gemm_empty_is_a_no_op(L):
    assert gg(L, groups=0, offs=None, c=None) == 0
    assert gg(L, M=0, offs=None) == 0
    assert gg(L, fmt=1, sa=None, sb=None, N=0) == 0


def test_linear_sizes(L):
    T, K, N = 256, 512, 384
    saved = L.nvfp4_linear_saved_bytes(T, K)
    ws = L.nvfp4_linear_workspace_bytes(T, K, N)
    assert saved >= T * K * 9 // 16 + 16 and saved < T * K * 2
    # workspace holds the forward operands of X and W, or dY (both directions) and W's columnwise
    assert ws >= max((T + N) * K * 9 // 16, 2 * T * N * 9 // 16 + N * K * 9 // 16)
    assert L.nvfp4_linear_saved_bytes(-1, 4) == -1 and L.nvfp4_linear_workspace_bytes(1, -1, 1) == -1


def test_linear_validation(L):
    fwd, bwd = L.nvfp4_linear_forward, L.nvfp4_linear_backward
    assert fwd(FAKE, FAKE, 48, 64, 64, 0, FAKE, FAKE, FAKE, FAKE, None) == 2 and "multiples of 32" in last(L)
    assert fwd(FAKE, FAKE, 0, 64, 64, 0, FAKE, FAKE, FAKE, FAKE, None) == 2 and "empty" in last(L)
    assert fwd(FAKE, FAKE, 64, 64, 64, 0, None, FAKE, FAKE, FAKE, None) == 1
    assert fwd(FAKE, FAKE, 64, 64, 64, 0, FAKE, FAKE, FAKE + 8, FAKE, None) == 6
    assert bwd(FAKE, FAKE, FAKE, 64, 64, 40, 0, FAKE, FAKE, FAKE, FAKE, None) == 2
    # tokens are the wgrad GEMM's contraction length: bounded like any NVFP4 K
    assert fwd(FAKE, FAKE, 1 << 24, 64, 64, 0, FAKE, FAKE, FAKE, FAKE, None) == 2 and "below" in last(L)
    assert bwd(FAKE, FAKE, FAKE, 64, 64, 1 << 24, 0, FAKE, FAKE, FAKE, FAKE, None) == 2 and "below" in last(L)
    assert bwd(FAKE, FAKE, None, 64, 64, 64, 0, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert bwd(FAKE, FAKE, FAKE, 64, 64, 64, 0, FAKE, FAKE, FAKE, FAKE + 4, None) == 6


def rq(L, x=FAKE, rows=64, cols=256, rounding=0, signs=None, codes=FAKE, scales=FAKE, amax=FAKE, senc=FAKE):
    return L.nvfp4_quantize_rowscaled(x, rows, cols, rounding, 0, 0, signs, codes, scales, amax, senc, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(rounding=3), 3, "rounding"),
    (dict(rows=-2), 2, "negative"),
    (dict(cols=40), 2, "multiple of 16"),
    (dict(amax=None), 1, "amax_rows"),
    (dict(senc=None), 1, "amax_rows"),
    (dict(x=None), 1, "NULL"),
    (dict(codes=None), 1, "NULL"),
    (dict(scales=None), 1, "NULL"),
    (dict(x=FAKE + 4), 6, "aligned"),
    (dict(codes=FAKE + 8), 6, "aligned"),
    (dict(signs=FAKE + 1), 6, "aligned"),
])
def test_nvfp4_quantize_rowscaled_validation(L, kw, status, needle):
    assert rq(L, **kw) == status
    assert needle in last(L)


def test_nvfp4_quantize_rowscaled_empty_is_a_no_op(L):
    assert rq(L, rows=0, x=None, codes=None, scales=None, amax=None, senc=None) == 0


def test_dequantize_validation(L):
    f = L.nvfp4_dequantize
    assert f(FAKE, FAKE, FAKE, 4, 24, FAKE, None) == 2
    assert f(None, FAKE, FAKE, 4, 32, FAKE, None) == 1
    assert f(FAKE, FAKE, FAKE, 0, 32, FAKE, None) == 0


def test_error_cleared_on_success(L):
    assert q(L, direction=0) == 3
    assert last(L) != ""
    assert L.blockscaled_gemm(0, 0, 8, 64, *([FAKE] * 7), 0, None) == 0
    assert last(L) == ""


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import block_scaled_precision_nvfp4_amd as bsq
    monkeypatch.setattr(bsq, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(bsq, "_lib", None)
    with pytest.raises(RuntimeError, match="libbsq.so not found"):
        bsq.lib()
