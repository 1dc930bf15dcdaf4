"""Pins of the oracle's grouped block-scaled GEMM (one GEMM per group: the grouped GEMM of a
mixture-of-experts linear layer on the page "[Pytorch][Common] Hybrid quantization",
GroupedLinear path of the dispatch flowchart).

The grouped oracle slices the operands and calls the plain oracle GEMM per group; these tests
tie its slicing to things it does not compute itself: a brute-force float64 product of
operands decoded here from the closed-form E2M1 / E4M3 / E8M0 definitions, the linearity of
the contraction (the K-groups of a tiling of [0, K) sum to the whole-K GEMM), row
independence (M-groups against identical experts are rows of one GEMM), and the documented
edge rules (empty groups, clamped boundaries, K-group boundaries that are not multiples
of 32).
"""
import numpy as np
import pytest
import torch

from synthetic import gaussian_bf16, outlier_bf16

E2M1 = [0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6]


def e4m3_py(b: int) -> float:
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    v = m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -v if s else v


def deq_nv(codes, scales, s_rows):
    R, half = codes.shape
    out = np.zeros((R, 2 * half))
    for r in range(R):
        for k in range(2 * half):
            byte = int(codes[r, k // 2])
            c = byte & 0xF if k % 2 == 0 else byte >> 4
            out[r, k] = E2M1[c] * e4m3_py(int(scales[r, k // 16])) / float(s_rows[r])
    return out


def deq_mx(codes, scales):
    R, K = codes.shape
    out = np.zeros((R, K))
    for r in range(R):
        for k in range(K):
            out[r, k] = e4m3_py(int(codes[r, k])) * 2.0 ** (int(scales[r, k // 32]) - 127)
    return out


def nv_rows(orc, x):
    q = orc.nvfp4_quantize(x, direction=orc.ROW)
    return q["row_codes"], q["row_scales"], float(q["s_enc"][0])


def test_m_grouped_nvfp4_brute_force(orc):
    """Three experts, one of them empty, rows before the first and after the last group;
    per-group A scales (each group quantized on its own) and per-expert B scales."""
    K, N = 64, 5
    offs = [2, 9, 9, 20]
    x = outlier_bf16((23, K), seed=1, mask_seed=2)
    a_codes = np.zeros((23, K // 2), np.uint8)
    a_scales = np.zeros((23, K // 16), np.uint8)
    sa = np.zeros(3, np.float32)
    for g in range(3):
        if offs[g + 1] > offs[g]:
            c, s, S = nv_rows(orc, x[offs[g]:offs[g + 1]])
            a_codes[offs[g]:offs[g + 1]], a_scales[offs[g]:offs[g + 1]], sa[g] = c, s, S
        else:
            sa[g] = 1.0
    bq = [nv_rows(orc, gaussian_bf16((N, K), 0.05 * (g + 1), 10 + g)) for g in range(3)]
    b_codes = np.stack([q[0] for q in bq])
    b_scales = np.stack([q[1] for q in bq])
    sb = np.array([q[2] for q in bq], np.float32)
    got = orc.blockscaled_grouped_gemm(orc.FMT_NVFP4, orc.GROUP_M, offs, a_codes, a_scales, sa,
                                       b_codes, b_scales, sb)
    assert np.all(np.isnan(got[:2])) and np.all(np.isnan(got[20:]))
    for g in range(3):
        o0, o1 = offs[g], offs[g + 1]
        if o1 == o0:
            continue
        ref = deq_nv(a_codes[o0:o1], a_scales[o0:o1], np.full(o1 - o0, sa[g])) @ deq_nv(
            b_codes[g], b_scales[g], np.full(N, sb[g])).T
        assert np.allclose(got[o0:o1], ref, rtol=1e-12, atol=0)


def test_m_grouped_rowscaled_a_and_b(orc):
    K, N, G = 32, 3, 2
    offs = [0, 4, 7]
    x = outlier_bf16((7, K), seed=5, mask_seed=6)
    qa = orc.nvfp4_quantize_rowscaled(x)
    qb = [orc.nvfp4_quantize_rowscaled(gaussian_bf16((N, K), 1.0, 20 + g)) for g in range(G)]
    got = orc.blockscaled_grouped_gemm(orc.FMT_NVFP4, orc.GROUP_M, offs, qa["codes"], qa["scales"], qa["s_enc"],
                                       np.stack([q["codes"] for q in qb]), np.stack([q["scales"] for q in qb]),
                                       np.concatenate([q["s_enc"] for q in qb]), a_rows=True, b_rows=True)
    for g in range(G):
        o0, o1 = offs[g], offs[g + 1]
        ref = deq_nv(qa["codes"][o0:o1], qa["scales"][o0:o1], qa["s_enc"][o0:o1]) @ deq_nv(
            qb[g]["codes"], qb[g]["scales"], qb[g]["s_enc"]).T
        assert np.allclose(got[o0:o1], ref, rtol=1e-12, atol=0)


def test_m_grouped_identical_experts_are_rows_of_one_gemm(orc):
    K, N = 96, 7
    x = gaussian_bf16((40, K), 1.0, 30)
    w = gaussian_bf16((N, K), 0.1, 31)
    c, s, S = nv_rows(orc, x)
    wc, ws, wS = nv_rows(orc, w)
    offs = [0, 13, 13, 29, 40]
    got = orc.blockscaled_grouped_gemm(orc.FMT_NVFP4, orc.GROUP_M, offs, c, s, np.full(4, S, np.float32),
                                       np.stack([wc] * 4), np.stack([ws] * 4), np.full(4, wS, np.float32))
    assert np.array_equal(got, orc.blockscaled_gemm(orc.FMT_NVFP4, c, s, S, wc, ws, wS))


def mx_cols(orc, t):
    q = orc.mxfp8_quantize(t, direction=orc.COL)
    return q["col_codes"], q["col_scales"]


def test_k_grouped_mxfp8_brute_force_and_linearity(orc):
    """wgrad shape: dY [T, M] and X [T, N] quantized columnwise over all T tokens; groups of
    tokens (one empty) tile [0, T)."""
    T, M, N = 160, 6, 4
    dy = outlier_bf16((T, M), seed=40, mask_seed=41)
    x = gaussian_bf16((T, N), 1.0, 42)
    ac, as_ = mx_cols(orc, dy)
    bc, bs = mx_cols(orc, x)
    offs = [0, 64, 64, 96, 160]
    got = orc.blockscaled_grouped_gemm(orc.FMT_MXFP8, orc.GROUP_K, offs, ac, as_, None, bc, bs, None)
    A, B = deq_mx(ac, as_), deq_mx(bc, bs)
    for g in range(4):
        o0, o1 = offs[g], offs[g + 1]
        assert np.allclose(got[g], A[:, o0:o1] @ B[:, o0:o1].T, rtol=1e-12, atol=0)
    assert not got[1].any()
    whole = orc.blockscaled_gemm(orc.FMT_MXFP8, ac, as_, 1.0, bc, bs, 1.0)
    assert np.allclose(got.sum(axis=0), whole, rtol=1e-12, atol=1e-300)


def test_k_grouped_nvfp4_per_group_scales(orc):
    """NVFP4 wgrad operands quantized per group (each group its own tensor scale), laid out
    along the grouped dimension."""
    T, M, N = 96, 4, 3
    offs = [0, 32, 96]
    dy = gaussian_bf16((T, M), 1.0, 50)
    x = outlier_bf16((T, N), seed=51, mask_seed=52)
    parts = []
    for g in range(2):
        qa = orc.nvfp4_quantize(dy[offs[g]:offs[g + 1]], direction=orc.COL)
        qb = orc.nvfp4_quantize(x[offs[g]:offs[g + 1]], direction=orc.COL)
        parts.append((qa, qb))
    cat = lambda k, w: np.ascontiguousarray(np.concatenate([p[w][k] for p in parts], axis=1))
    sa = np.array([p[0]["s_enc"][1] for p in parts], np.float32)
    sb = np.array([p[1]["s_enc"][1] for p in parts], np.float32)
    got = orc.blockscaled_grouped_gemm(orc.FMT_NVFP4, orc.GROUP_K, offs, cat("col_codes", 0), cat("col_scales", 0),
                                       sa, cat("col_codes", 1), cat("col_scales", 1), sb)
    for g in range(2):
        qa, qb = parts[g]
        ref = deq_nv(qa["col_codes"], qa["col_scales"], np.full(M, sa[g])) @ deq_nv(
            qb["col_codes"], qb["col_scales"], np.full(N, sb[g])).T
        assert np.allclose(got[g], ref, rtol=1e-12, atol=0)


def test_edge_rules(orc):
    """A group's start is clamped to [0, extent] and its end to [start, extent]; a K-group
    whose boundaries are not multiples of 32 is empty."""
    T, M, N = 128, 3, 2
    ac, as_ = mx_cols(orc, gaussian_bf16((T, M), 1.0, 60))
    bc, bs = mx_cols(orc, gaussian_bf16((T, N), 1.0, 61))
    got = orc.blockscaled_grouped_gemm(orc.FMT_MXFP8, orc.GROUP_K, [-64, 32, 48, 16, 500], ac, as_, None, bc, bs,
                                       None)
    whole = lambda o0, o1: orc.blockscaled_gemm(orc.FMT_MXFP8, np.ascontiguousarray(ac[:, o0:o1]),
                                                np.ascontiguousarray(as_[:, o0 // 32:o1 // 32]), 1.0,
                                                np.ascontiguousarray(bc[:, o0:o1]),
                                                np.ascontiguousarray(bs[:, o0 // 32:o1 // 32]), 1.0)
    assert np.array_equal(got[0], whole(0, 32))       # -64 clamped to 0
    assert not got[1].any()                           # 32..48: not a multiple of 32
    assert not got[2].any()                           # 48..16 raised to 48..48: empty
    assert not got[3].any()                           # 16..128 (500 clamped): 16 not aligned
    got2 = orc.blockscaled_grouped_gemm(orc.FMT_MXFP8, orc.GROUP_K, [0, 64, 500], ac, as_, None, bc, bs, None)
    assert np.array_equal(got2[1], whole(64, 128))   # 500 clamped to T


def test_split_quantize_of_the_grouped_recipe_is_the_whole_tensor_call(orc):
    """Row-scaled NVFP4 (RNE) and MXFP8 of each token split equal the whole-tensor
    quantization restricted to the split when the splits are multiples of 32 (rows are
    independent, MXFP8 has no tensor scale) -- so the grouped recipe's split-quantize needs
    no per-split launch."""
    T, K = 224, 96
    offs = [0, 64, 64, 160, 224]
    x = outlier_bf16((T, K), seed=70, mask_seed=71)
    rs = orc.nvfp4_quantize_rowscaled(x)
    mx = orc.mxfp8_quantize(x, direction=orc.ROW | orc.COL)
    for g in range(4):
        o0, o1 = offs[g], offs[g + 1]
        if o1 == o0:
            continue
        part = x[o0:o1].contiguous()
        p_rs = orc.nvfp4_quantize_rowscaled(part)
        assert np.array_equal(p_rs["codes"], rs["codes"][o0:o1]) and np.array_equal(p_rs["s_enc"], rs["s_enc"][o0:o1])
        assert np.array_equal(p_rs["scales"], rs["scales"][o0:o1])
        p_mx = orc.mxfp8_quantize(part, direction=orc.ROW | orc.COL)
        assert np.array_equal(p_mx["row_codes"], mx["row_codes"][o0:o1])
        assert np.array_equal(p_mx["col_codes"], mx["col_codes"][:, o0:o1])
        assert np.array_equal(p_mx["col_scales"], mx["col_scales"][:, o0 // 32:o1 // 32])
