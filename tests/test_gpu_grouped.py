"""GPU parity of the grouped block-scaled GEMM (one GEMM per group in one launch, group
boundaries read on the device) against the CPU oracle, through the C ABI.

M-grouped (per-expert fprop / dgrad): ragged group sizes including empty groups, rows before
the first and after the last group (which must stay untouched), K a multiple of 256 (NVFP4
kernel with scale records) and not (per-slice scales), per-group and per-row (row-scaled) NVFP4
tensor scales, MXFP8, and more than 64 groups (the device-side scan takes several chunks).
K-grouped (per-expert wgrad): MXFP8 operands quantized columnwise over all tokens (row-major
or slab-layout codes, and the full-size mixture-of-experts wgrad sampled), NVFP4
operands quantized per group, empty and misaligned groups (computed as empty).  Operands
are quantized on the GPU and by the oracle from the same bf16 inputs and must agree bit for
bit before the GEMMs are compared (relative Frobenius error <= 2e-3 against the oracle
output rounded as the GPU stores it, and every element within the rounding-error bound of
fp32 accumulation)."""
import numpy as np
import pytest
import torch

import block_scaled_precision_nvfp4_amd as bsq
from synthetic import STD_W, gaussian_bf16, outlier_bf16
from tests.gpu_common import (GEMM_TOL, assert_bytes_equal, assert_f32_equal, assert_gemm_elements, bf16_round,
                              from_slab, mxfp8_mfma_model, note, rel_fro, stratified)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def splits_to_offsets(first, sizes):
    return [first] + list(first + np.cumsum(sizes))


def check_close(got64, ref64, out_dtype, what, sabs, K, model=None):
    want = bf16_round(ref64) if out_dtype == torch.bfloat16 else ref64
    err = rel_fro(got64, want)
    note("  %s rel_fro = %.3e" % (what, err))
    assert err <= GEMM_TOL, (what, err)
    assert_gemm_elements(got64, ref64, sabs, K, out_dtype == torch.bfloat16, what, model=model)


def nv_experts(G, N, K, seed):
    """Per-expert NVFP4 weights, each quantized on its own (GPU and oracle)."""
    import oracle
    ws = [gaussian_bf16((N, K), STD_W * (1 + g), seed + g) for g in range(G)]
    q = [bsq.nvfp4_quantize(w.to(DEV), direction=bsq.ROW) for w in ws]
    r = [oracle.nvfp4_quantize(w, direction=oracle.ROW) for w in ws]
    for qq, rr in zip(q, r):
        assert_bytes_equal(qq["row_codes"], rr["row_codes"], "expert codes")
    gpu = (torch.stack([x["row_codes"] for x in q]).contiguous(), torch.stack([x["row_scales"] for x in q]).contiguous(),
           torch.cat([x["s_enc"][0:1] for x in q]).contiguous())
    ref = (np.stack([x["row_codes"] for x in r]), np.stack([x["row_scales"] for x in r]),
           np.array([x["s_enc"][0] for x in r], np.float32))
    return gpu, ref


def nv_tokens_per_group(x, offs):
    """Expert inputs quantized per group (each group its own tensor scale), in one buffer."""
    import oracle
    M, K = x.shape
    G = len(offs) - 1
    gc = torch.zeros((M, K // 2), dtype=torch.uint8, device=DEV)
    gs = torch.zeros((M, K // 16), dtype=torch.uint8, device=DEV)
    gS = torch.ones(G, dtype=torch.float32, device=DEV)
    rc = np.zeros((M, K // 2), np.uint8)
    rs = np.zeros((M, K // 16), np.uint8)
    rS = np.ones(G, np.float32)
    for g in range(G):
        o0, o1 = offs[g], offs[g + 1]
        if o1 == o0:
            continue
        q = bsq.nvfp4_quantize(x[o0:o1].contiguous().to(DEV), direction=bsq.ROW)
        r = oracle.nvfp4_quantize(x[o0:o1].contiguous(), direction=oracle.ROW)
        gc[o0:o1], gs[o0:o1], gS[g:g + 1] = q["row_codes"], q["row_scales"], q["s_enc"][0:1]
        rc[o0:o1], rs[o0:o1], rS[g] = r["row_codes"], r["row_scales"], r["s_enc"][0]
    torch.cuda.synchronize()
    assert_bytes_equal(gc, rc, "per-group A codes")
    assert_f32_equal(gS, rS, "per-group A s_enc")
    return (gc, gs, gS), (rc, rs, rS)


def run_m_grouped(fmt, a_gpu, a_ref, b_gpu, b_ref, offs, M, N, out_dtype, a_rows=False, label="", layout=0):
    import oracle
    note("grouped M %s fmt=%d M=%d N=%d groups=%d out=%s" % (label, fmt, M, N, len(offs) - 1, out_dtype))
    o = torch.tensor(offs, dtype=torch.int64, device=DEV)
    out = torch.full((M, N), 1.0, dtype=out_dtype, device=DEV)
    f = fmt | (bsq.FMT_A_ROWSCALED if a_rows else 0) | layout
    bsq.blockscaled_grouped_gemm(f, bsq.GROUP_M, o, *a_gpu, *b_gpu, out_dtype=out_dtype, out=out)
    torch.cuda.synchronize()
    ref, sabs = oracle.blockscaled_grouped_gemm(fmt, oracle.GROUP_M, offs, *a_ref, *b_ref, a_rows=a_rows,
                                                with_abs=True)
    got = out.float().cpu().numpy().astype(np.float64)
    inside = ~np.isnan(ref[:, 0])
    assert np.all(got[~inside] == 1.0), "rows outside every group were written"
    K = a_ref[0].shape[1] * (2 if fmt == bsq.FMT_NVFP4 else 1)
    if inside.any():
        model = None
        if fmt == bsq.FMT_MXFP8:
            # the FP8 MFMA instruction model, group by group: that group's rows of A against its B
            model = np.full(ref.shape, np.nan)
            for g in range(len(offs) - 1):
                o0, o1 = offs[g], offs[g + 1]
                if o1 > o0:
                    model[o0:o1] = mxfp8_mfma_model(a_ref[0][o0:o1], a_ref[1][o0:o1], b_ref[0][g], b_ref[1][g])
            model = model[inside]
        check_close(got[inside], ref[inside], out_dtype, label, sabs[inside], K, model=model)


@pytest.mark.parametrize("K", [512, 160])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_m_grouped_nvfp4_per_group_scales(K, out_dtype):
    sizes = [300, 0, 517, 211]
    offs = splits_to_offsets(16, sizes)
    M, N = offs[-1] + 9, 384
    x = outlier_bf16((M, K), seed=K, mask_seed=K + 1)
    a_gpu, a_ref = nv_tokens_per_group(x, offs)
    b_gpu, b_ref = nv_experts(len(sizes), N, K, 100)
    run_m_grouped(bsq.FMT_NVFP4, a_gpu, a_ref, b_gpu, b_ref, offs, M, N, out_dtype, label="nvfp4 per-group")


def test_m_grouped_nvfp4_rowscaled_inputs():
    """The Composer-style grouped fprop: row-scaled NVFP4 expert inputs (one call over all
    tokens: rows are independent), per-tensor NVFP4 experts."""
    import oracle
    sizes = [640, 37, 0, 1100, 256]
    offs = splits_to_offsets(0, sizes)
    M, N, K = offs[-1], 512, 1024
    x = (gaussian_bf16((M, K), 1.0, 7).float() * torch.logspace(-2, 2, M).reshape(M, 1)).to(torch.bfloat16)
    q = bsq.nvfp4_quantize_rowscaled(x.to(DEV))
    r = oracle.nvfp4_quantize_rowscaled(x)
    torch.cuda.synchronize()
    assert_bytes_equal(q["codes"], r["codes"], "row-scaled codes")
    assert_f32_equal(q["s_enc"], r["s_enc"], "row-scaled s_enc")
    b_gpu, b_ref = nv_experts(len(sizes), N, K, 200)
    run_m_grouped(bsq.FMT_NVFP4, (q["codes"], q["scales"], q["s_enc"]), (r["codes"], r["scales"], r["s_enc"]),
                  b_gpu, b_ref, offs, M, N, torch.bfloat16, a_rows=True, label="row-scaled fprop")


def test_m_grouped_mxfp8_dgrad():
    import oracle
    sizes = [96, 500, 0, 333]
    offs = splits_to_offsets(5, sizes)
    M, N, K = offs[-1] + 3, 320, 512
    dy = gaussian_bf16((M, K), 1e-3, 11)
    qa = bsq.mxfp8_quantize(dy.to(DEV), direction=bsq.ROW)
    ra = oracle.mxfp8_quantize(dy, direction=oracle.ROW)
    ws = [gaussian_bf16((N, K), STD_W, 300 + g) for g in range(len(sizes))]
    qb = [bsq.mxfp8_quantize(w.to(DEV), direction=bsq.ROW) for w in ws]
    rb = [oracle.mxfp8_quantize(w, direction=oracle.ROW) for w in ws]
    torch.cuda.synchronize()
    assert_bytes_equal(qa["row_codes"], ra["row_codes"], "dY codes")
    b_gpu = (torch.stack([x["row_codes"] for x in qb]).contiguous(), torch.stack([x["row_scales"] for x in qb]).contiguous(), None)
    b_ref = (np.stack([x["row_codes"] for x in rb]), np.stack([x["row_scales"] for x in rb]), None)
    run_m_grouped(bsq.FMT_MXFP8, (qa["row_codes"], qa["row_scales"], None), (ra["row_codes"], ra["row_scales"], None),
                  b_gpu, b_ref, offs, M, N, torch.bfloat16, label="mxfp8 dgrad")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_m_grouped_mxfp8_dgrad_slab_b(out_dtype):
    """M-grouped MXFP8 dgrad with each expert's codes in the slab layout (a ragged last band:
    N = 320), the token operand row-major, K = 1536: the slab bytes hold exactly the oracle's
    codes and the GEMM matches the oracle's."""
    import oracle
    sizes = [96, 500, 0, 333]
    offs = splits_to_offsets(5, sizes)
    M, N, K = offs[-1] + 3, 320, 1536
    dy = gaussian_bf16((M, K), 1e-3, 12)
    qa = bsq.mxfp8_quantize(dy.to(DEV), direction=bsq.ROW)
    ra = oracle.mxfp8_quantize(dy, direction=oracle.ROW)
    ws = [gaussian_bf16((N, K), STD_W, 310 + g) for g in range(len(sizes))]
    qb = [bsq.mxfp8_quantize(w.to(DEV), direction=bsq.ROW | bsq.MX_SLAB) for w in ws]
    rb = [oracle.mxfp8_quantize(w, direction=oracle.ROW) for w in ws]
    torch.cuda.synchronize()
    assert_bytes_equal(qa["row_codes"], ra["row_codes"], "dY codes")
    for g, (x, r) in enumerate(zip(qb, rb)):
        assert np.array_equal(from_slab(x["row_codes"], N, K), r["row_codes"]), "expert %d slab codes" % g
    b_gpu = (torch.stack([x["row_codes"] for x in qb]).contiguous(), torch.stack([x["row_scales"] for x in qb]).contiguous(), None)
    b_ref = (np.stack([x["row_codes"] for x in rb]), np.stack([x["row_scales"] for x in rb]), None)
    run_m_grouped(bsq.FMT_MXFP8, (qa["row_codes"], qa["row_scales"], None), (ra["row_codes"], ra["row_scales"], None),
                  b_gpu, b_ref, offs, M, N, out_dtype, label="mxfp8 dgrad slab B", layout=bsq.FMT_MX_SLAB_B)


def test_m_grouped_many_groups():
    """100 groups of 0..40 rows: the device-side scan walks two 64-group chunks."""
    rng = np.random.default_rng(12)
    sizes = rng.integers(0, 41, 100)
    sizes[[3, 64, 65, 99]] = 0
    offs = splits_to_offsets(0, sizes)
    M, N, K = offs[-1], 128, 256
    x = gaussian_bf16((M, K), 1.0, 13)
    a_gpu, a_ref = nv_tokens_per_group(x, offs)
    b_gpu, b_ref = nv_experts(100, N, K, 400)
    run_m_grouped(bsq.FMT_NVFP4, a_gpu, a_ref, b_gpu, b_ref, offs, M, N, torch.bfloat16, label="100 groups")


def run_k_grouped(fmt, a_gpu, a_ref, b_gpu, b_ref, offs, M, N, label="", layout=0):
    import oracle
    note("grouped K %s fmt=%d M=%d N=%d groups=%d layout=%#x" % (label, fmt, M, N, len(offs) - 1, layout))
    o = torch.tensor(offs, dtype=torch.int64, device=DEV)
    out = bsq.blockscaled_grouped_gemm(fmt | layout, bsq.GROUP_K, o, *a_gpu, *b_gpu, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, sabs = oracle.blockscaled_grouped_gemm(fmt, oracle.GROUP_K, offs, *a_ref, *b_ref, with_abs=True)
    got = out.cpu().numpy().astype(np.float64)
    for g in range(len(offs) - 1):
        o0, o1 = offs[g], offs[g + 1]
        if not ref[g].any():
            assert not got[g].any(), "group %d should be zero" % g
        else:
            model = None
            if fmt == bsq.FMT_MXFP8:   # the group's K range of the whole-token operands
                model = mxfp8_mfma_model(a_ref[0][:, o0:o1], a_ref[1][:, o0 // 32:o1 // 32],
                                         b_ref[0][:, o0:o1], b_ref[1][:, o0 // 32:o1 // 32])
            check_close(got[g], ref[g], torch.float32, "%s group %d" % (label, g), sabs[g], o1 - o0, model=model)


def test_k_grouped_mxfp8_wgrad():
    """dW_g = dY_g^T X_g over token groups, both operands MXFP8 columnwise over all tokens: an
    empty group, groups of 32 and 64 tokens, two misaligned groups (empty by definition), and
    groups whose length is a multiple of 512 (scale-record path, at offset 0 and inside the
    rows) next to ones that are not."""
    import oracle
    offs = [0, 512, 512, 544, 1000, 1024, 1536, 1984, 2048]
    T, M, N = 2048, 320, 192
    dy = gaussian_bf16((T, M), 1e-3, 21)
    x = outlier_bf16((T, N), seed=22, mask_seed=23)
    qa = bsq.mxfp8_quantize(dy.to(DEV), direction=bsq.COL)
    qb = bsq.mxfp8_quantize(x.to(DEV), direction=bsq.COL)
    ra = oracle.mxfp8_quantize(dy, direction=oracle.COL)
    rb = oracle.mxfp8_quantize(x, direction=oracle.COL)
    torch.cuda.synchronize()
    assert_bytes_equal(qa["col_codes"], ra["col_codes"], "dY col codes")
    assert_bytes_equal(qb["col_codes"], rb["col_codes"], "X col codes")
    run_k_grouped(bsq.FMT_MXFP8, (qa["col_codes"], qa["col_scales"], None), (ra["col_codes"], ra["col_scales"], None),
                  (qb["col_codes"], qb["col_scales"], None), (rb["col_codes"], rb["col_scales"], None),
                  offs, M, N, label="mxfp8 wgrad")


@pytest.mark.parametrize("layout", [0, bsq.FMT_MX_SLAB_A, bsq.FMT_MX_SLAB_B, bsq.FMT_MX_SLAB])
def test_k_grouped_mxfp8_offset_records(layout):
    """K-grouped MXFP8 wgrad whose groups start at many byte offsets inside a 16-byte scale
    record (starts at multiples of 32 tokens), with odd numbers of K-blocks (the last K slice
    half outside the group), one group spanning several 8-slice record groups, and NaN scale
    bytes in the two columns after the last group (a misaligned group, computed as empty),
    which must not reach the last group's sums.  With the slab flags the operands' codes come
    from casts with MX_SLAB (groups starting half-way into a 64-token slab take its second
    half and the next slab's first; ragged last bands: M = 320, N = 192)."""
    import oracle
    kblocks = [3, 17, 1, 37, 5, 2, 41]
    offs = [0]
    for n in kblocks:
        offs.append(offs[-1] + 32 * n)
    end = offs[-1]
    offs += [end + 8, 4096]
    T, M, N = 4096, 320, 192
    dy = gaussian_bf16((T, M), 1e-3, 81)
    x = outlier_bf16((T, N), seed=82, mask_seed=83)
    slab_a = bsq.MX_SLAB if layout & bsq.FMT_MX_SLAB_A else 0
    slab_b = bsq.MX_SLAB if layout & bsq.FMT_MX_SLAB_B else 0
    qa = bsq.mxfp8_quantize(dy.to(DEV), direction=bsq.COL | slab_a)
    qb = bsq.mxfp8_quantize(x.to(DEV), direction=bsq.COL | slab_b)
    ra = oracle.mxfp8_quantize(dy, direction=oracle.COL)
    rb = oracle.mxfp8_quantize(x, direction=oracle.COL)
    torch.cuda.synchronize()
    for q, r, nm, sl, rows in ((qa, ra, "dY", slab_a, M), (qb, rb, "X", slab_b, N)):
        codes = torch.from_numpy(from_slab(q["col_codes"], rows, T)) if sl else q["col_codes"]
        assert_bytes_equal(codes, r["col_codes"], nm + " col codes")
        assert_bytes_equal(q["col_scales"], r["col_scales"], nm + " col scales")
    nan_cols = slice(end // 32, end // 32 + 2)
    for t in (qa["col_scales"], qb["col_scales"]):
        t[:, nan_cols] = 255
    for r in (ra, rb):
        r["col_scales"] = np.array(r["col_scales"], copy=True)
        r["col_scales"][:, nan_cols] = 255
    run_k_grouped(bsq.FMT_MXFP8, (qa["col_codes"], qa["col_scales"], None), (ra["col_codes"], ra["col_scales"], None),
                  (qb["col_codes"], qb["col_scales"], None), (rb["col_codes"], rb["col_scales"], None),
                  offs, M, N, label="mxfp8 offset records", layout=layout)


@pytest.mark.parametrize("layout", [0, bsq.FMT_MX_SLAB, bsq.FMT_MX_SLAB_B])
def test_k_grouped_mxfp8_many_groups(layout):
    """40 groups of a [520, 264] wgrad output (3 x 2 tiles, ragged in both dimensions; 320
    workgroups with the padding to 8 per group): group lengths at random multiples of 32
    including empty groups and one that is not a multiple of 32 (it and the next group are
    computed as empty), on row-major, both-slab or B-only slab codes."""
    import oracle
    rng = np.random.default_rng(91)
    sizes = list(rng.integers(0, 7, 40) * 32)
    sizes[5] = 0
    sizes[17] = 48   # misaligned: this group and the next (which realigns) are empty
    sizes[18] = 80
    offs = splits_to_offsets(0, sizes)
    T = 4096
    assert offs[-1] <= T
    M, N = 520, 264
    dy = gaussian_bf16((T, M), 1e-3, 92)
    x = outlier_bf16((T, N), seed=93, mask_seed=94)
    slab_a = bsq.MX_SLAB if layout & bsq.FMT_MX_SLAB_A else 0
    slab_b = bsq.MX_SLAB if layout & bsq.FMT_MX_SLAB_B else 0
    qa = bsq.mxfp8_quantize(dy.to(DEV), direction=bsq.COL | slab_a)
    qb = bsq.mxfp8_quantize(x.to(DEV), direction=bsq.COL | slab_b)
    ra = oracle.mxfp8_quantize(dy, direction=oracle.COL)
    rb = oracle.mxfp8_quantize(x, direction=oracle.COL)
    torch.cuda.synchronize()
    for q, r, nm, sl, rows in ((qa, ra, "dY", slab_a, M), (qb, rb, "X", slab_b, N)):
        codes = torch.from_numpy(from_slab(q["col_codes"], rows, T)) if sl else q["col_codes"]
        assert_bytes_equal(codes, r["col_codes"], nm + " col codes")
    run_k_grouped(bsq.FMT_MXFP8, (qa["col_codes"], qa["col_scales"], None), (ra["col_codes"], ra["col_scales"], None),
                  (qb["col_codes"], qb["col_scales"], None), (rb["col_codes"], rb["col_scales"], None),
                  offs, M, N, label="mxfp8 many groups", layout=layout)


@pytest.mark.parametrize("offs,M,N", [
    ([0, 256, 288, 288, 800], 288, 160),
    # groups starting at odd multiples of 32 tokens (scale bytes 2 bytes into a dword), lengths
    # that end inside a 128-token slice, a 32-token group and one over many slices
    ([0, 96, 1056, 1088, 2400, 2400, 4064, 4096], 320, 192),
])
def test_k_grouped_nvfp4_per_group_scales(offs, M, N):
    """NVFP4 wgrad operands quantized columnwise per group (each group its own tensor scale)
    and laid out along the token dimension."""
    import oracle
    T = offs[-1]
    dy = gaussian_bf16((T, M), 1e-3, 31)
    x = gaussian_bf16((T, N), 1.0, 32)
    G = len(offs) - 1
    parts_q, parts_r = [], []
    for g in range(G):
        o0, o1 = offs[g], offs[g + 1]
        if o1 == o0:
            parts_q.append(None)
            parts_r.append(None)
            continue
        parts_q.append([bsq.nvfp4_quantize(t[o0:o1].contiguous().to(DEV), direction=bsq.COL) for t in (dy, x)])
        parts_r.append([oracle.nvfp4_quantize(t[o0:o1].contiguous(), direction=oracle.COL) for t in (dy, x)])
    torch.cuda.synchronize()

    def cat_gpu(i, key):
        return torch.cat([p[i][key] for p in parts_q if p is not None], dim=1).contiguous()

    def cat_ref(i, key):
        return np.ascontiguousarray(np.concatenate([p[i][key] for p in parts_r if p is not None], axis=1))

    def s_gpu(i):
        return torch.cat([p[i]["s_enc"][1:2] if p is not None else torch.ones(1, device=DEV) for p in parts_q]).contiguous()

    def s_ref(i):
        return np.array([p[i]["s_enc"][1] if p is not None else 1.0 for p in parts_r], np.float32)

    for i in (0, 1):
        assert_bytes_equal(cat_gpu(i, "col_codes"), cat_ref(i, "col_codes"), "col codes %d" % i)
        assert_f32_equal(s_gpu(i), s_ref(i), "per-group s_enc %d" % i)
    run_k_grouped(bsq.FMT_NVFP4, (cat_gpu(0, "col_codes"), cat_gpu(0, "col_scales"), s_gpu(0)),
                  (cat_ref(0, "col_codes"), cat_ref(0, "col_scales"), s_ref(0)),
                  (cat_gpu(1, "col_codes"), cat_gpu(1, "col_scales"), s_gpu(1)),
                  (cat_ref(1, "col_codes"), cat_ref(1, "col_scales"), s_ref(1)), offs, M, N, label="nvfp4 wgrad")


def test_grouped_moe_fprop_sampled():
    """A mixture-of-experts fprop at a realistic size: 8 experts, 16384 routed tokens,
    K = 4096, N = 2048, row-scaled NVFP4 inputs; compared on rows x columns that include the
    first and last row and column of every 256-wide band of each group's output (every output
    tile of every group)."""
    import oracle
    G, T, N, K = 8, 16384, 2048, 4096
    rng = np.random.default_rng(41)
    cuts = np.sort(rng.choice(np.arange(1, T), G - 1, replace=False))
    offs = [0] + [int(c) for c in cuts] + [T]
    note("grouped M moe fprop sampled offs=%s" % offs)
    x = gaussian_bf16((T, K), 1.0, 42)
    q = bsq.nvfp4_quantize_rowscaled(x.to(DEV))
    b_gpu, b_ref = nv_experts(G, N, K, 500)
    o = torch.tensor(offs, dtype=torch.int64, device=DEV)
    y = bsq.blockscaled_grouped_gemm(bsq.FMT_NVFP4 | bsq.FMT_A_ROWSCALED, bsq.GROUP_M, o, q["codes"], q["scales"],
                                     q["s_enc"], *b_gpu)
    torch.cuda.synchronize()
    r = oracle.nvfp4_quantize_rowscaled(x)
    assert_bytes_equal(q["codes"], r["codes"], "row-scaled codes")
    cols = stratified(N, 43)
    for g in range(G):
        o0, o1 = offs[g], offs[g + 1]
        rows = o0 + stratified(o1 - o0, 44 + g)
        yc = y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].float().cpu().numpy()
        ref, sabs = oracle.blockscaled_gemm(oracle.FMT_NVFP4, r["codes"][o0:o1], r["scales"][o0:o1],
                                            r["s_enc"][o0:o1], b_ref[0][g], b_ref[1][g], float(b_ref[2][g]),
                                            rows=rows - o0, cols=cols, with_abs=True)
        check_close(yc.astype(np.float64), ref, torch.bfloat16, "expert %d" % g, sabs, K)


def test_grouped_moe_wgrad_mxfp8_slab_sampled():
    """The mixture-of-experts wgrad at full size: 8 experts over 16384 tokens (boundaries at
    random multiples of 32), dW_g [14336, 4096] = dY_g^T X_g from MXFP8 columnwise casts of dY
    [16384, 14336] and X [16384, 4096] with slab-layout codes, fp32 out; the casts are checked
    whole against the oracle, the GEMM on rows x columns that include the first and last of
    every 256-wide band of each group's output (every output tile of every group)."""
    import oracle
    G, T, M, N = 8, 16384, 14336, 4096
    rng = np.random.default_rng(2024)
    cuts = np.sort(rng.choice(np.arange(1, T // 32), G - 1, replace=False)) * 32
    offs = [0] + [int(c) for c in cuts] + [T]
    note("grouped K moe wgrad slab sampled offs=%s" % offs)
    dy = gaussian_bf16((T, M), 1e-4, 61)
    x = gaussian_bf16((T, N), 1.0, 62)
    qa = bsq.mxfp8_quantize(dy.to(DEV), direction=bsq.COL | bsq.MX_SLAB)
    qb = bsq.mxfp8_quantize(x.to(DEV), direction=bsq.COL | bsq.MX_SLAB)
    o = torch.tensor(offs, dtype=torch.int64, device=DEV)
    dw = bsq.blockscaled_grouped_gemm(bsq.FMT_MXFP8 | bsq.FMT_MX_SLAB, bsq.GROUP_K, o, qa["col_codes"],
                                      qa["col_scales"], None, qb["col_codes"], qb["col_scales"], None,
                                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    ra = oracle.mxfp8_quantize(dy, direction=oracle.COL)
    rb = oracle.mxfp8_quantize(x, direction=oracle.COL)
    del dy, x
    assert np.array_equal(from_slab(qa["col_codes"], M, T), ra["col_codes"]), "dY slab codes"
    assert np.array_equal(from_slab(qb["col_codes"], N, T), rb["col_codes"]), "X slab codes"
    assert_bytes_equal(qa["col_scales"], ra["col_scales"], "dY col scales")
    assert_bytes_equal(qb["col_scales"], rb["col_scales"], "X col scales")
    del qa, qb
    for g in range(G):
        o0, o1 = offs[g], offs[g + 1]
        rows, cols = stratified(M, 70 + g), stratified(N, 80 + g)
        got = dw[g][torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].cpu().numpy()
        a = (np.ascontiguousarray(ra["col_codes"][rows, o0:o1]), np.ascontiguousarray(ra["col_scales"][rows, o0 // 32:o1 // 32]))
        b = (np.ascontiguousarray(rb["col_codes"][cols, o0:o1]), np.ascontiguousarray(rb["col_scales"][cols, o0 // 32:o1 // 32]))
        ref, sabs = oracle.blockscaled_gemm(oracle.FMT_MXFP8, a[0], a[1], 1.0, b[0], b[1], 1.0, with_abs=True)
        model = mxfp8_mfma_model(a[0], a[1], b[0], b[1])
        check_close(got.astype(np.float64), ref, torch.float32, "expert %d" % g, sabs, o1 - o0, model=model)
