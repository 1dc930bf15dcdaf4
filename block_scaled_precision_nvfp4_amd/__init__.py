"""Python binding of libbsq: block-scaled (NVFP4 / MXFP8) quantization and GEMM on MI355X.

Thin ctypes marshalling over the C ABI in include/bsq.h: every step of the computation
runs in the library's HIP kernels.  PyTorch only provides device memory (output
tensors are allocated with torch.empty) and the current HIP stream.  The functions
have the names of the C entry points.  Importing works without a GPU; calling a
compute function needs libbsq.so (built by ``python -m
block_scaled_precision_nvfp4_amd.build``) and fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

import torch

ROW, COL = 1, 2
MX_SLAB = 4   # OR'ed into an MXFP8 cast's direction: codes in the slab layout
RNE, SR = 0, 1
FMT_NVFP4, FMT_MXFP8 = 0, 1
FMT_A_ROWSCALED, FMT_B_ROWSCALED = 0x10, 0x20
FMT_MX_SLAB_A, FMT_MX_SLAB_B = 0x40, 0x80   # OR'ed into FMT_MXFP8: that operand's codes in the slab layout
FMT_MX_SLAB = FMT_MX_SLAB_A | FMT_MX_SLAB_B
GROUP_M, GROUP_K = 1, 2
OUT_BF16, OUT_F32 = 0, 1
NVFP4_QUANTIZE_WORKSPACE_BYTES = 8192   # BSQ_NVFP4_QUANTIZE_WORKSPACE_BYTES

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsq.so")

_ERRORS = {1: "null pointer", 2: "shape", 3: "argument", 4: "unsupported", 5: "HIP", 6: "alignment"}


class BsqError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed (%s error %d): %s" % (fn, _ERRORS.get(status, "?"), status, msg))
        self.status = status


_lib = None


def lib():
    """Load libbsq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libbsq.so not found at %s; build it with "
                               "`python -m block_scaled_precision_nvfp4_amd.build`" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        vp, i64, i32, u32, u64 = C.c_void_p, C.c_int64, C.c_int, C.c_uint32, C.c_uint64
        L.nvfp4_quantize.argtypes = [vp, i64, i64, i32, i32, u64, u32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.nvfp4_quantize_noalloc.argtypes = [vp, i64, i64, i32, i32, u64, u32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.nvfp4_quantize_fprop_wgrad.argtypes = [vp, i64, i64, i32, u64, u32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.nvfp4_col_mxfp8_row_quantize.argtypes = [vp, i64, i64, i32, u64, u32, vp, vp, vp, vp, vp, vp, i32,
                                                   vp, vp, vp]
        L.nvfp4_quantize_rowscaled.argtypes = [vp, i64, i64, i32, u64, u32, vp, vp, vp, vp, vp, vp]
        L.nvfp4_dequantize.argtypes = [vp, vp, vp, i64, i64, vp, vp]
        L.mxfp8_quantize.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp, vp]
        L.mxfp8_requantize_nvfp4.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, vp, vp, vp]
        L.rht_apply.argtypes = [vp, i64, i64, i32, vp, vp, vp]
        L.blockscaled_gemm.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp]
        L.blockscaled_grouped_gemm.argtypes = [i32, i32, i64, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp]
        L.nvfp4_linear_workspace_bytes.argtypes = [i64, i64, i64]
        L.nvfp4_linear_workspace_bytes.restype = C.c_int64
        L.nvfp4_linear_saved_bytes.argtypes = [i64, i64]
        L.nvfp4_linear_saved_bytes.restype = C.c_int64
        L.nvfp4_linear_forward.argtypes = [vp, vp, i64, i64, i64, u64, vp, vp, vp, vp, vp]
        L.nvfp4_linear_backward.argtypes = [vp, vp, vp, i64, i64, i64, u64, vp, vp, vp, vp, vp]
        for f in ("nvfp4_linear_forward", "nvfp4_linear_backward", "nvfp4_quantize", "nvfp4_quantize_noalloc",
                  "nvfp4_col_mxfp8_row_quantize", "nvfp4_quantize_fprop_wgrad", "nvfp4_quantize_rowscaled",
                  "nvfp4_dequantize", "mxfp8_quantize", "mxfp8_requantize_nvfp4", "rht_apply",
                  "blockscaled_gemm", "blockscaled_grouped_gemm", "bsq_version"):
            getattr(L, f).restype = C.c_int
        L.bsq_last_error.argtypes = []
        L.bsq_last_error.restype = C.c_char_p
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise BsqError(fn, status, lib().bsq_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev_tensor(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA/HIP tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    """The caller's scratch tensor (checked for size and device), or a new one."""
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != torch.device(device):
        raise TypeError("workspace must be a device tensor on %s" % (device,))
    if not ws.is_contiguous() or ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace must be contiguous and hold at least %d bytes" % nbytes)
    return ws


def _signs(rht_signs, device):
    if rht_signs is None:
        return None
    s = rht_signs
    if not isinstance(s, torch.Tensor):
        s = torch.tensor(s, dtype=torch.int8)
    s = s.to(device=device, dtype=torch.int8).contiguous()
    if s.numel() != 16:
        raise ValueError("rht_signs must have 16 entries")
    return s


def nvfp4_quantize(x: torch.Tensor, direction: int = ROW, rounding: int = RNE, sr_seed: int = 0,
                   sr_stream: int = 0, rht_signs=None, workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """NVFP4-quantize a bf16 [rows, cols] device tensor.  Returns the requested directions'
    ``{row,col}_codes`` / ``{row,col}_scales`` (uint8) and ``amax`` / ``s_enc`` (float32[2],
    index 0 rowwise, 1 columnwise), all on x's device.  ``workspace`` (a device tensor of at
    least NVFP4_QUANTIZE_WORKSPACE_BYTES bytes) is the call's scratch; one is allocated when
    none is given."""
    _dev_tensor(x, torch.bfloat16, "x")
    R, Cc = x.shape
    dev = x.device
    out: Dict[str, torch.Tensor] = {}
    u8 = dict(dtype=torch.uint8, device=dev)
    if direction & ROW:
        out["row_codes"] = torch.empty((R, Cc // 2), **u8)
        out["row_scales"] = torch.empty((R, Cc // 16), **u8)
    if direction & COL:
        out["col_codes"] = torch.empty((Cc, R // 2), **u8)
        out["col_scales"] = torch.empty((Cc, R // 16), **u8)
    out["amax"] = torch.empty(2, dtype=torch.float32, device=dev)
    out["s_enc"] = torch.empty(2, dtype=torch.float32, device=dev)
    ws = _workspace(workspace, NVFP4_QUANTIZE_WORKSPACE_BYTES, dev)
    sg = _signs(rht_signs, dev)
    _check("nvfp4_quantize", lib().nvfp4_quantize(
        x.data_ptr(), R, Cc, direction, rounding, sr_seed & (2 ** 64 - 1), sr_stream, _ptr(sg),
        _ptr(out.get("row_codes")), _ptr(out.get("row_scales")), _ptr(out.get("col_codes")),
        _ptr(out.get("col_scales")), out["amax"].data_ptr(), out["s_enc"].data_ptr(), ws.data_ptr(), _stream(dev)))
    return out


def nvfp4_quantize_fprop_wgrad(x: torch.Tensor, rounding: int = RNE, sr_seed: int = 0, sr_stream: int = 0,
                               rht_signs=None, workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """One pass over a bf16 [rows, cols] activation that writes its rowwise forward operand (RNE,
    no transform: ``row_codes``, ``row_scales``) and its columnwise wgrad operand (the given
    rounding and transform: ``col_codes``, ``col_scales``); ``amax`` / ``s_enc`` as for
    ``nvfp4_quantize`` (index 0 rowwise, 1 columnwise)."""
    _dev_tensor(x, torch.bfloat16, "x")
    R, Cc = x.shape
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    out = {"row_codes": torch.empty((R, Cc // 2), **u8), "row_scales": torch.empty((R, Cc // 16), **u8),
           "col_codes": torch.empty((Cc, R // 2), **u8), "col_scales": torch.empty((Cc, R // 16), **u8),
           "amax": torch.empty(2, dtype=torch.float32, device=dev),
           "s_enc": torch.empty(2, dtype=torch.float32, device=dev)}
    ws = _workspace(workspace, NVFP4_QUANTIZE_WORKSPACE_BYTES, dev)
    sg = _signs(rht_signs, dev)
    _check("nvfp4_quantize_fprop_wgrad", lib().nvfp4_quantize_fprop_wgrad(
        x.data_ptr(), R, Cc, rounding, sr_seed & (2 ** 64 - 1), sr_stream, _ptr(sg), out["row_codes"].data_ptr(),
        out["row_scales"].data_ptr(), out["col_codes"].data_ptr(), out["col_scales"].data_ptr(),
        out["amax"].data_ptr(), out["s_enc"].data_ptr(), ws.data_ptr(), _stream(dev)))
    return out


def nvfp4_col_mxfp8_row_quantize(x: torch.Tensor, rounding: int = RNE, sr_seed: int = 0, sr_stream: int = 0,
                                 rht_signs=None, mx_slab: bool = False,
                                 workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """One pass over a bf16 [rows, cols] device tensor that writes NVFP4 columnwise (as
    ``nvfp4_quantize(x, COL, ...)``: ``col_codes``, ``col_scales``, ``amax``, ``s_enc``) and
    MXFP8 rowwise (as ``mxfp8_quantize(x, ROW | (MX_SLAB if mx_slab else 0))``:
    ``mx_row_codes``, ``mx_row_scales``).  RHT and SR apply to the NVFP4 part only."""
    _dev_tensor(x, torch.bfloat16, "x")
    R, Cc = x.shape
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    out = {"col_codes": torch.empty((Cc, R // 2), **u8), "col_scales": torch.empty((Cc, R // 16), **u8),
           "amax": torch.empty(2, dtype=torch.float32, device=dev),
           "s_enc": torch.empty(2, dtype=torch.float32, device=dev),
           "mx_row_codes": torch.empty((R, Cc), **u8), "mx_row_scales": torch.empty((R, Cc // 32), **u8)}
    ws = _workspace(workspace, NVFP4_QUANTIZE_WORKSPACE_BYTES, dev)
    sg = _signs(rht_signs, dev)
    _check("nvfp4_col_mxfp8_row_quantize", lib().nvfp4_col_mxfp8_row_quantize(
        x.data_ptr(), R, Cc, rounding, sr_seed & (2 ** 64 - 1), sr_stream, _ptr(sg), out["col_codes"].data_ptr(),
        out["col_scales"].data_ptr(), out["amax"].data_ptr(), out["s_enc"].data_ptr(), ws.data_ptr(),
        MX_SLAB if mx_slab else 0, out["mx_row_codes"].data_ptr(), out["mx_row_scales"].data_ptr(),
        _stream(dev)))
    return out


def nvfp4_quantize_rowscaled(x: torch.Tensor, rounding: int = RNE, sr_seed: int = 0, sr_stream: int = 0,
                             rht_signs=None) -> Dict[str, torch.Tensor]:
    """Rowwise NVFP4 with one outer scale per row.  Returns ``codes`` [rows, cols/2],
    ``scales`` [rows, cols/16] (uint8), ``amax`` and ``s_enc`` (float32[rows])."""
    _dev_tensor(x, torch.bfloat16, "x")
    R, Cc = x.shape
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    out = {"codes": torch.empty((R, Cc // 2), **u8), "scales": torch.empty((R, Cc // 16), **u8),
           "amax": torch.empty(R, dtype=torch.float32, device=dev),
           "s_enc": torch.empty(R, dtype=torch.float32, device=dev)}
    sg = _signs(rht_signs, dev)
    _check("nvfp4_quantize_rowscaled", lib().nvfp4_quantize_rowscaled(
        x.data_ptr(), R, Cc, rounding, sr_seed & (2 ** 64 - 1), sr_stream, _ptr(sg), out["codes"].data_ptr(),
        out["scales"].data_ptr(), out["amax"].data_ptr(), out["s_enc"].data_ptr(), _stream(dev)))
    return out


def nvfp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, s_enc: torch.Tensor) -> torch.Tensor:
    """bf16 [rows, cols] value of NVFP4 codes [rows, cols/2] with scales [rows, cols/16] and
    tensor scale ``s_enc`` (a 1-element float32 device tensor)."""
    _dev_tensor(codes, torch.uint8, "codes")
    _dev_tensor(scales, torch.uint8, "scales")
    _dev_tensor(s_enc, torch.float32, "s_enc")
    rows, half = codes.shape
    out = torch.empty((rows, half * 2), dtype=torch.bfloat16, device=codes.device)
    _check("nvfp4_dequantize", lib().nvfp4_dequantize(codes.data_ptr(), scales.data_ptr(), s_enc.data_ptr(),
                                                      rows, half * 2, out.data_ptr(), _stream(codes.device)))
    return out


def mxfp8_quantize(x: torch.Tensor, direction: int = ROW) -> Dict[str, torch.Tensor]:
    """MXFP8-cast a bf16 [rows, cols] device tensor (E4M3 codes, E8M0 scale per 32)."""
    _dev_tensor(x, torch.bfloat16, "x")
    R, Cc = x.shape
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    out: Dict[str, torch.Tensor] = {}
    if direction & ROW:
        out["row_codes"] = torch.empty((R, Cc), **u8)
        out["row_scales"] = torch.empty((R, Cc // 32), **u8)
    if direction & COL:
        out["col_codes"] = torch.empty((Cc, R), **u8)
        out["col_scales"] = torch.empty((Cc, R // 32), **u8)
    _check("mxfp8_quantize", lib().mxfp8_quantize(
        x.data_ptr(), R, Cc, direction, _ptr(out.get("row_codes")), _ptr(out.get("row_scales")),
        _ptr(out.get("col_codes")), _ptr(out.get("col_scales")), _stream(dev)))
    return out


def mxfp8_requantize_nvfp4(codes: torch.Tensor, scales: torch.Tensor, s_enc: torch.Tensor,
                           direction: int = COL) -> Dict[str, torch.Tensor]:
    """MXFP8 cast of the rowwise-dequantized value of an NVFP4 rowwise tensor (``codes``
    [rows, cols/2], ``scales`` [rows, cols/16], 1-element float32 ``s_enc``), without the
    bf16 intermediate; bit-identical to ``mxfp8_quantize(nvfp4_dequantize(...))``."""
    _dev_tensor(codes, torch.uint8, "codes")
    _dev_tensor(scales, torch.uint8, "scales")
    _dev_tensor(s_enc, torch.float32, "s_enc")
    R, Cc = codes.shape[0], codes.shape[1] * 2
    if tuple(scales.shape) != (R, Cc // 16):
        raise ValueError("scales must be [rows, cols/16]")
    dev = codes.device
    u8 = dict(dtype=torch.uint8, device=dev)
    out: Dict[str, torch.Tensor] = {}
    if direction & ROW:
        out["row_codes"] = torch.empty((R, Cc), **u8)
        out["row_scales"] = torch.empty((R, Cc // 32), **u8)
    if direction & COL:
        out["col_codes"] = torch.empty((Cc, R), **u8)
        out["col_scales"] = torch.empty((Cc, R // 32), **u8)
    _check("mxfp8_requantize_nvfp4", lib().mxfp8_requantize_nvfp4(
        codes.data_ptr(), scales.data_ptr(), s_enc.data_ptr(), R, Cc, direction, _ptr(out.get("row_codes")),
        _ptr(out.get("row_scales")), _ptr(out.get("col_codes")), _ptr(out.get("col_scales")), _stream(dev)))
    return out


def rht_apply(x: torch.Tensor, axis: int, rht_signs) -> torch.Tensor:
    """float32 16-point random Hadamard transform of a bf16 tensor along ``axis``."""
    _dev_tensor(x, torch.bfloat16, "x")
    R, Cc = x.shape
    sg = _signs(rht_signs, x.device)
    out = torch.empty((R, Cc), dtype=torch.float32, device=x.device)
    _check("rht_apply", lib().rht_apply(x.data_ptr(), R, Cc, axis, sg.data_ptr(), out.data_ptr(),
                                        _stream(x.device)))
    return out


def blockscaled_gemm(fmt: int, a_codes: torch.Tensor, a_scales: torch.Tensor, a_s_enc: Optional[torch.Tensor],
                     b_codes: torch.Tensor, b_scales: torch.Tensor, b_s_enc: Optional[torch.Tensor],
                     out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[M, N] = A[M, K] B[N, K]^T on NVFP4 (fmt 0) or MXFP8 (fmt 1) operands, fp32 accumulate.
    ``fmt`` may carry FMT_A_ROWSCALED / FMT_B_ROWSCALED (NVFP4): that operand's ``s_enc`` then
    holds one float per row."""
    _dev_tensor(a_codes, torch.uint8, "a_codes")
    _dev_tensor(b_codes, torch.uint8, "b_codes")
    _dev_tensor(a_scales, torch.uint8, "a_scales")
    _dev_tensor(b_scales, torch.uint8, "b_scales")
    M, N = a_codes.shape[0], b_codes.shape[0]
    base = fmt & ~(FMT_A_ROWSCALED | FMT_B_ROWSCALED)
    K = a_codes.shape[1] * (2 if base == FMT_NVFP4 else 1)
    for flag, t, n, name in ((FMT_A_ROWSCALED, a_s_enc, M, "a_s_enc"), (FMT_B_ROWSCALED, b_s_enc, N, "b_s_enc")):
        if base == FMT_NVFP4 and t is not None:
            _dev_tensor(t, torch.float32, name)
            want = n if fmt & flag else 1
            if t.numel() < want:
                raise ValueError("%s has %d entries, needs %d" % (name, t.numel(), want))
    if b_codes.shape[1] != a_codes.shape[1]:
        raise ValueError("operands disagree on K")
    c_dtype = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    else:
        _dev_tensor(out, out_dtype, "out")
        if tuple(out.shape) != (M, N):
            raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), (M, N)))
    _check("blockscaled_gemm", lib().blockscaled_gemm(
        fmt, M, N, K, a_codes.data_ptr(), a_scales.data_ptr(), _ptr(a_s_enc), b_codes.data_ptr(),
        b_scales.data_ptr(), _ptr(b_s_enc), out.data_ptr(), c_dtype, _stream(a_codes.device)))
    return out


def blockscaled_grouped_gemm(fmt: int, mode: int, offsets: torch.Tensor, a_codes: torch.Tensor,
                             a_scales: torch.Tensor, a_s_enc: Optional[torch.Tensor], b_codes: torch.Tensor,
                             b_scales: torch.Tensor, b_s_enc: Optional[torch.Tensor],
                             out_dtype: torch.dtype = torch.bfloat16,
                             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One block-scaled GEMM per group; ``offsets`` is an int64 device tensor of groups + 1
    boundaries.  GROUP_M: A [M, K] (rows grouped), B [groups, N, K] (codes as [groups, N,
    K/2] or [groups * N, K/2] for NVFP4), C [M, N] (rows outside every group untouched).
    GROUP_K: A [M, K] and B [N, K] grouped along K, C [groups, M, N]."""
    _dev_tensor(offsets, torch.int64, "offsets")
    for t, nm in ((a_codes, "a_codes"), (b_codes, "b_codes"), (a_scales, "a_scales"), (b_scales, "b_scales")):
        _dev_tensor(t, torch.uint8, nm)
    for t, nm in ((a_s_enc, "a_s_enc"), (b_s_enc, "b_s_enc")):
        if t is not None:
            _dev_tensor(t, torch.float32, nm)
    G = offsets.numel() - 1
    if G < 0:
        raise ValueError("offsets needs groups + 1 entries")
    base = fmt & ~(FMT_A_ROWSCALED | FMT_B_ROWSCALED)
    epb = 2 if base == FMT_NVFP4 else 1
    M, K = a_codes.shape[0], a_codes.shape[-1] * epb
    if mode == GROUP_M:
        N = b_codes.shape[-2] if b_codes.dim() == 3 else (b_codes.shape[0] // G if G else 0)
        shape = (M, N)
    else:
        N = b_codes.shape[0]
        shape = (G, M, N)
    if b_codes.shape[-1] * epb != K:
        raise ValueError("operands disagree on K")
    c_dtype = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32}[out_dtype]
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=a_codes.device)
    else:
        _dev_tensor(out, out_dtype, "out")
        if tuple(out.shape) != shape:
            raise ValueError("out has shape %s, expected %s" % (tuple(out.shape), shape))
    _check("blockscaled_grouped_gemm", lib().blockscaled_grouped_gemm(
        fmt, mode, G, offsets.data_ptr(), M, N, K, a_codes.data_ptr(), a_scales.data_ptr(), _ptr(a_s_enc),
        b_codes.data_ptr(), b_scales.data_ptr(), _ptr(b_s_enc), out.data_ptr(), c_dtype, _stream(a_codes.device)))
    return out


def nvfp4_linear_forward(x: torch.Tensor, w: torch.Tensor, sr_seed: int, rht_signs,
                         workspace: Optional[torch.Tensor] = None):
    """NVFP4 linear forward: returns (y [T, N] bf16, saved) where ``saved`` (a uint8 device
    tensor) holds the quantized activation that nvfp4_linear_backward needs."""
    _dev_tensor(x, torch.bfloat16, "x")
    _dev_tensor(w, torch.bfloat16, "w")
    T, K = x.shape
    N = w.shape[0]
    dev = x.device
    L = lib()
    saved = torch.empty(L.nvfp4_linear_saved_bytes(T, K), dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = torch.empty(L.nvfp4_linear_workspace_bytes(T, K, N), dtype=torch.uint8, device=dev)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    sg = _signs(rht_signs, dev)
    _check("nvfp4_linear_forward", L.nvfp4_linear_forward(
        x.data_ptr(), w.data_ptr(), T, K, N, sr_seed & (2 ** 64 - 1), sg.data_ptr(), saved.data_ptr(),
        workspace.data_ptr(), y.data_ptr(), _stream(dev)))
    return y, saved


def nvfp4_linear_backward(dy: torch.Tensor, w: torch.Tensor, saved: torch.Tensor, sr_seed: int, rht_signs,
                          workspace: Optional[torch.Tensor] = None):
    """NVFP4 linear backward: returns (dx [T, K] bf16, dw [N, K] fp32)."""
    _dev_tensor(dy, torch.bfloat16, "dy")
    _dev_tensor(w, torch.bfloat16, "w")
    _dev_tensor(saved, torch.uint8, "saved")
    T, N = dy.shape
    K = w.shape[1]
    dev = dy.device
    L = lib()
    if saved.numel() < L.nvfp4_linear_saved_bytes(T, K):
        raise ValueError("saved buffer is too small for this layer")
    if workspace is None:
        workspace = torch.empty(L.nvfp4_linear_workspace_bytes(T, K, N), dtype=torch.uint8, device=dev)
    dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((N, K), dtype=torch.float32, device=dev)
    sg = _signs(rht_signs, dev)
    _check("nvfp4_linear_backward", L.nvfp4_linear_backward(
        dy.data_ptr(), w.data_ptr(), saved.data_ptr(), T, K, N, sr_seed & (2 ** 64 - 1), sg.data_ptr(),
        workspace.data_ptr(), dx.data_ptr(), dw.data_ptr(), _stream(dev)))
    return dx, dw
