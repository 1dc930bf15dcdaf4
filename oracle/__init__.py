"""CPU oracle of block-scaled quantization and the block-scaled GEMM (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``oracle.c`` (plain C, built
with gcc) through ctypes and works on numpy arrays; it shares nothing with the
HIP library.  See ``oracle.c`` for the definitions and their sources.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")

ROW, COL = 1, 2
RNE, SR = 0, 1
FMT_NVFP4, FMT_MXFP8 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c into _build/liboracle.so with gcc (OpenMP, strict IEEE binary32)."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build(force=False)
        L = C.CDLL(path)
        u8p = C.POINTER(C.c_uint8)
        u16p = C.POINTER(C.c_uint16)
        f32p = C.POINTER(C.c_float)
        f64p = C.POINTER(C.c_double)
        i8p = C.POINTER(C.c_int8)
        i64p = C.POINTER(C.c_int64)
        u32p = C.POINTER(C.c_uint32)
        L.or_bf16_to_f32.argtypes = [C.c_uint16]; L.or_bf16_to_f32.restype = C.c_float
        L.or_f32_to_bf16_rne.argtypes = [C.c_float]; L.or_f32_to_bf16_rne.restype = C.c_uint16
        L.or_e2m1_decode.argtypes = [C.c_uint8]; L.or_e2m1_decode.restype = C.c_float
        L.or_e2m1_encode_rne.argtypes = [C.c_float]; L.or_e2m1_encode_rne.restype = C.c_uint8
        L.or_e2m1_encode_sr.argtypes = [C.c_float, C.c_uint32]; L.or_e2m1_encode_sr.restype = C.c_uint8
        L.or_e4m3_decode.argtypes = [C.c_uint8]; L.or_e4m3_decode.restype = C.c_float
        L.or_e4m3_encode_rne_sat.argtypes = [C.c_float]; L.or_e4m3_encode_rne_sat.restype = C.c_uint8
        L.or_e8m0_decode.argtypes = [C.c_uint8]; L.or_e8m0_decode.restype = C.c_float
        L.or_philox4x32_10.argtypes = [u32p, u32p, u32p]; L.or_philox4x32_10.restype = None
        L.or_sr_word.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, C.c_uint64]
        L.or_sr_word.restype = C.c_uint32
        L.or_rht16.argtypes = [f32p, i8p, f32p]; L.or_rht16.restype = None
        L.or_nvfp4_tensor_scale.argtypes = [C.c_float]; L.or_nvfp4_tensor_scale.restype = C.c_float
        L.or_nvfp4_block_scale.argtypes = [C.c_float, C.c_float]; L.or_nvfp4_block_scale.restype = C.c_uint8
        L.or_mxfp8_scale_byte.argtypes = [C.c_float]; L.or_mxfp8_scale_byte.restype = C.c_uint8
        L.or_nvfp4_quantize.argtypes = [u16p, C.c_int64, C.c_int64, C.c_int, C.c_int, C.c_uint64,
                                        C.c_uint32, i8p, u8p, u8p, u8p, u8p, f32p, f32p]
        L.or_nvfp4_quantize.restype = C.c_int
        L.or_nvfp4_dequantize.argtypes = [u8p, u8p, C.c_float, C.c_int64, C.c_int64, u16p]
        L.or_nvfp4_dequantize.restype = None
        L.or_mxfp8_quantize.argtypes = [u16p, C.c_int64, C.c_int64, C.c_int, u8p, u8p, u8p, u8p]
        L.or_mxfp8_quantize.restype = C.c_int
        L.or_rht_apply.argtypes = [u16p, C.c_int64, C.c_int64, C.c_int, i8p, f32p]
        L.or_rht_apply.restype = C.c_int
        L.or_blockscaled_gemm.argtypes = [C.c_int, C.c_int64, C.c_int64, C.c_int64,
                                          u8p, u8p, C.c_float, u8p, u8p, C.c_float,
                                          i64p, C.c_int64, i64p, C.c_int64, f64p]
        L.or_blockscaled_gemm.restype = C.c_int
        L.or_nvfp4_quantize_rowscaled.argtypes = [u16p, C.c_int64, C.c_int64, C.c_int, C.c_uint64, C.c_uint32,
                                                  i8p, u8p, u8p, f32p, f32p]
        L.or_nvfp4_quantize_rowscaled.restype = C.c_int
        L.or_blockscaled_gemm_rows.argtypes = [C.c_int, C.c_int64, C.c_int64, C.c_int64,
                                               u8p, u8p, f32p, C.c_int, u8p, u8p, f32p, C.c_int,
                                               i64p, C.c_int64, i64p, C.c_int64, f64p, f64p]
        L.or_blockscaled_gemm_rows.restype = C.c_int
        L.or_num_threads.argtypes = []; L.or_num_threads.restype = C.c_int
        L.or_set_num_threads.argtypes = [C.c_int]; L.or_set_num_threads.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.POINTER(ctype))


def _bits(x) -> np.ndarray:
    """bf16 input as a contiguous uint16 numpy array (accepts a torch bf16 tensor or uint16 array)."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch  # only for accepting torch CPU tensors
    assert x.dtype == torch.bfloat16
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _signs(signs):
    if signs is None:
        return None
    s = np.ascontiguousarray(np.asarray(signs, dtype=np.int8).reshape(16))
    assert np.all(np.abs(s.astype(np.int32)) == 1), "sign vector entries must be +-1"
    return s


def num_threads() -> int:
    return lib().or_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (OpenMP); the results do not depend on it."""
    lib().or_set_num_threads(int(n))


# ---------------------------------------------------------------- scalar codecs

def e2m1_decode(code: int) -> float:
    return lib().or_e2m1_decode(code)


def e2m1_encode_rne(v: float) -> int:
    return lib().or_e2m1_encode_rne(v)


def e2m1_encode_sr(v: float, u: int) -> int:
    return lib().or_e2m1_encode_sr(v, u)


def e4m3_decode(code: int) -> float:
    return lib().or_e4m3_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().or_e4m3_encode_rne_sat(v)


def e8m0_decode(b: int) -> float:
    return lib().or_e8m0_decode(b)


def philox4x32_10(counter, key):
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint32).reshape(4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.zeros(4, dtype=np.uint32)
    lib().or_philox4x32_10(_p(c, C.c_uint32), _p(k, C.c_uint32), _p(out, C.c_uint32))
    return out


def sr_word(seed: int, stream: int, direction: int, i: int) -> int:
    return lib().or_sr_word(seed & (2**64 - 1), stream, direction, i)


def rht16(x, signs) -> np.ndarray:
    xi = np.ascontiguousarray(np.asarray(x, dtype=np.float32).reshape(16))
    out = np.zeros(16, dtype=np.float32)
    lib().or_rht16(_p(xi, C.c_float), _p(_signs(signs), C.c_int8), _p(out, C.c_float))
    return out


def nvfp4_tensor_scale(amax: float) -> float:
    return lib().or_nvfp4_tensor_scale(amax)


def nvfp4_block_scale(block_amax: float, s_enc: float) -> int:
    return lib().or_nvfp4_block_scale(block_amax, s_enc)


def mxfp8_scale_byte(block_amax: float) -> int:
    return lib().or_mxfp8_scale_byte(block_amax)


def f32_to_bf16_rne(v: float) -> int:
    return lib().or_f32_to_bf16_rne(v)


# ---------------------------------------------------------------- tensor ops

def nvfp4_quantize(x, direction: int = ROW, rounding: int = RNE, sr_seed: int = 0,
                   sr_stream: int = 0, signs=None) -> dict:
    """NVFP4 quantization of bf16 x[R][C].  Returns a dict with the requested
    directions' codes/scales and amax[2], s_enc[2] ([0] rowwise, [1] columnwise)."""
    xb = _bits(x)
    R, Cc = xb.shape
    out = {}
    rc = rs = cc = cs = None
    if direction & ROW:
        rc = np.zeros((R, Cc // 2), np.uint8); rs = np.zeros((R, Cc // 16), np.uint8)
    if direction & COL:
        cc = np.zeros((Cc, R // 2), np.uint8); cs = np.zeros((Cc, R // 16), np.uint8)
    amax = np.zeros(2, np.float32)
    s_enc = np.zeros(2, np.float32)
    sg = _signs(signs)
    u8 = C.c_uint8
    nullu8 = C.POINTER(C.c_uint8)()
    st = lib().or_nvfp4_quantize(
        _p(xb, C.c_uint16), R, Cc, direction, rounding, sr_seed & (2**64 - 1), sr_stream,
        _p(sg, C.c_int8) if sg is not None else C.POINTER(C.c_int8)(),
        _p(rc, u8) if rc is not None else nullu8, _p(rs, u8) if rs is not None else nullu8,
        _p(cc, u8) if cc is not None else nullu8, _p(cs, u8) if cs is not None else nullu8,
        _p(amax, C.c_float), _p(s_enc, C.c_float))
    if st != 0:
        raise ValueError("oracle nvfp4_quantize failed with status %d" % st)
    if rc is not None:
        out["row_codes"], out["row_scales"] = rc, rs
    if cc is not None:
        out["col_codes"], out["col_scales"] = cc, cs
    out["amax"], out["s_enc"] = amax, s_enc
    return out


def nvfp4_quantize_rowscaled(x, rounding: int = RNE, sr_seed: int = 0, sr_stream: int = 0, signs=None) -> dict:
    """Row-scaled NVFP4 (rowwise, one amax and tensor scale per row) of bf16 x[R][C].
    Returns codes [R][C/2], scales [R][C/16], amax[R], s_enc[R]."""
    xb = _bits(x)
    R, Cc = xb.shape
    codes = np.zeros((R, Cc // 2), np.uint8)
    scales = np.zeros((R, Cc // 16), np.uint8)
    amax = np.zeros(R, np.float32)
    s_enc = np.zeros(R, np.float32)
    sg = _signs(signs)
    u8 = C.c_uint8
    st = lib().or_nvfp4_quantize_rowscaled(
        _p(xb, C.c_uint16), R, Cc, rounding, sr_seed & (2**64 - 1), sr_stream,
        _p(sg, C.c_int8) if sg is not None else C.POINTER(C.c_int8)(),
        _p(codes, u8), _p(scales, u8), _p(amax, C.c_float), _p(s_enc, C.c_float))
    if st != 0:
        raise ValueError("oracle nvfp4_quantize_rowscaled failed with status %d" % st)
    return {"codes": codes, "scales": scales, "amax": amax, "s_enc": s_enc}


def nvfp4_dequantize(codes: np.ndarray, scales: np.ndarray, s_enc: float) -> np.ndarray:
    """bf16 bits [rows][cols] of the dequantized NVFP4 tensor."""
    rows, half = codes.shape
    cols = half * 2
    out = np.zeros((rows, cols), np.uint16)
    lib().or_nvfp4_dequantize(_p(np.ascontiguousarray(codes), C.c_uint8),
                              _p(np.ascontiguousarray(scales), C.c_uint8), float(s_enc),
                              rows, cols, _p(out, C.c_uint16))
    return out


def mxfp8_quantize(x, direction: int = ROW) -> dict:
    xb = _bits(x)
    R, Cc = xb.shape
    rc = rs = cc = cs = None
    if direction & ROW:
        rc = np.zeros((R, Cc), np.uint8); rs = np.zeros((R, Cc // 32), np.uint8)
    if direction & COL:
        cc = np.zeros((Cc, R), np.uint8); cs = np.zeros((Cc, R // 32), np.uint8)
    u8 = C.c_uint8
    nullu8 = C.POINTER(C.c_uint8)()
    st = lib().or_mxfp8_quantize(
        _p(xb, C.c_uint16), R, Cc, direction,
        _p(rc, u8) if rc is not None else nullu8, _p(rs, u8) if rs is not None else nullu8,
        _p(cc, u8) if cc is not None else nullu8, _p(cs, u8) if cs is not None else nullu8)
    if st != 0:
        raise ValueError("oracle mxfp8_quantize failed with status %d" % st)
    out = {}
    if rc is not None:
        out["row_codes"], out["row_scales"] = rc, rs
    if cc is not None:
        out["col_codes"], out["col_scales"] = cc, cs
    return out


def rht_apply(x, axis: int, signs) -> np.ndarray:
    xb = _bits(x)
    R, Cc = xb.shape
    out = np.zeros((R, Cc), np.float32)
    st = lib().or_rht_apply(_p(xb, C.c_uint16), R, Cc, axis, _p(_signs(signs), C.c_int8),
                            _p(out, C.c_float))
    if st != 0:
        raise ValueError("oracle rht_apply failed with status %d" % st)
    return out


def blockscaled_gemm(fmt: int, a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc,
                     rows=None, cols=None, with_abs: bool = False):
    """binary64 C = A B^T of the dequantized operands (optionally only rows x cols of C).
    An NVFP4 tensor scale is a number (per-tensor) or an array with one scale per row of
    that operand (row-scaled).  With ``with_abs`` the result is (C, S), S[m][n] =
    sum_k |A[m][k] B[n][k]| (what bounds the rounding error of a finite-precision C)."""
    M = a_codes.shape[0]
    N = b_codes.shape[0]
    K = a_codes.shape[1] * (2 if fmt == FMT_NVFP4 else 1)
    mi = np.ascontiguousarray(np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, np.int64))
    ni = np.ascontiguousarray(np.arange(N, dtype=np.int64) if cols is None else np.asarray(cols, np.int64))
    out = np.zeros((mi.size, ni.size), np.float64)
    out_abs = np.zeros((mi.size, ni.size), np.float64) if with_abs else None
    u8 = C.c_uint8
    sa = np.ascontiguousarray(np.atleast_1d(np.asarray(a_s_enc, np.float32)))
    sb = np.ascontiguousarray(np.atleast_1d(np.asarray(b_s_enc, np.float32)))
    a_rows, b_rows = int(sa.size > 1 or (sa.size == M and M > 1)), int(sb.size > 1 or (sb.size == N and N > 1))
    if a_rows and sa.size != M or b_rows and sb.size != N:
        raise ValueError("per-row tensor scales must have one entry per operand row")
    st = lib().or_blockscaled_gemm_rows(
        fmt, M, N, K,
        _p(np.ascontiguousarray(a_codes), u8), _p(np.ascontiguousarray(a_scales), u8), _p(sa, C.c_float), a_rows,
        _p(np.ascontiguousarray(b_codes), u8), _p(np.ascontiguousarray(b_scales), u8), _p(sb, C.c_float), b_rows,
        _p(mi, C.c_int64), mi.size, _p(ni, C.c_int64), ni.size, _p(out, C.c_double),
        None if out_abs is None else _p(out_abs, C.c_double))
    if st != 0:
        raise ValueError("oracle blockscaled_gemm failed with status %d" % st)
    return (out, out_abs) if with_abs else out


GROUP_M, GROUP_K = 1, 2


def _group_bounds(offsets, g: int, extent: int):
    """Boundaries of group g clamped to [0, extent], the upper one raised to the lower."""
    a = min(max(int(offsets[g]), 0), extent)
    b = min(max(int(offsets[g + 1]), a), extent)
    return a, b


def blockscaled_grouped_gemm(fmt: int, mode: int, offsets, a_codes, a_scales, a_s_enc, b_codes, b_scales,
                             b_s_enc, a_rows: bool = False, b_rows: bool = False, with_abs: bool = False):
    """One block-scaled GEMM per group, group g covering offsets[g] .. offsets[g+1] of the
    grouped dimension (the grouped GEMM of a mixture-of-experts linear layer: the
    general_grouped_gemm step of the GroupedLinear path in the dispatch flowchart of the page
    "[Pytorch][Common] Hybrid quantization").  Each group is the plain GEMM of its slices.
      GROUP_M: rows of A [M][K] and C [M][N]; B is stacked per group, b_codes [G][N][K/epb];
               returns C [M][N] in float64, NaN in rows outside every group.
      GROUP_K: columns of A [M][K] and B [N][K]; returns C [G][M][N].  A group whose
               boundaries are not multiples of 32 is empty (its C_g is 0), as the library
               documents.
    NVFP4 tensor scales: one per group, or (GROUP_M, a_rows / b_rows) one per row of A / of
    the stacked B.  MXFP8 ignores them.  With ``with_abs`` the result is (C, S) with S the
    sums of absolute products, as blockscaled_gemm gives them."""
    G = len(offsets) - 1
    epb = 2 if fmt == FMT_NVFP4 else 1
    blk = 16 if fmt == FMT_NVFP4 else 32
    M = a_codes.shape[0]
    nv = fmt == FMT_NVFP4
    sa = np.atleast_1d(np.asarray(a_s_enc, np.float32)) if nv else None
    sb = np.atleast_1d(np.asarray(b_s_enc, np.float32)) if nv else None
    if mode == GROUP_M:
        N = b_codes.shape[1]
        out = np.full((M, N), np.nan)
        out_abs = np.full((M, N), np.nan)
        for g in range(G):
            o0, o1 = _group_bounds(offsets, g, M)
            if o1 == o0:
                continue
            s_a = (sa[o0:o1] if a_rows else float(sa[g])) if nv else 1.0
            s_b = (sb[g * N:(g + 1) * N] if b_rows else float(sb[g])) if nv else 1.0
            out[o0:o1], out_abs[o0:o1] = blockscaled_gemm(fmt, a_codes[o0:o1], a_scales[o0:o1], s_a,
                                                          b_codes[g], b_scales[g], s_b, with_abs=True)
        return (out, out_abs) if with_abs else out
    K = a_codes.shape[1] * epb
    N = b_codes.shape[0]
    out = np.zeros((G, M, N))
    out_abs = np.zeros((G, M, N))
    for g in range(G):
        o0, o1 = _group_bounds(offsets, g, K)
        if o1 == o0 or o0 % 32 or (o1 - o0) % 32:
            continue
        cs, ss = slice(o0 // epb, o1 // epb), slice(o0 // blk, o1 // blk)
        out[g], out_abs[g] = blockscaled_gemm(
            fmt, np.ascontiguousarray(a_codes[:, cs]), np.ascontiguousarray(a_scales[:, ss]),
            float(sa[g]) if nv else 1.0, np.ascontiguousarray(b_codes[:, cs]),
            np.ascontiguousarray(b_scales[:, ss]), float(sb[g]) if nv else 1.0, with_abs=True)
    return (out, out_abs) if with_abs else out


if __name__ == "__main__":
    print(build(force=True), file=sys.stderr)
