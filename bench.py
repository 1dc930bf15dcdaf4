"""Benchmark: one training step of a block-scaled quantized linear layer at the Llama-3-8B
FFN up-projection shape (tokens M = 16384, out features N = 14336, in features K = 4096)
on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic bf16 inputs already
resident in HBM:
  fwd    NVFP4 rowwise (RNE) of X[16384,4096] and W[14336,4096]; Y = X W^T (bf16)
  wgrad  16-point RHT + Philox SR, NVFP4 columnwise of dY[16384,14336] and X;
         dW = dY^T X (fp32)
  dgrad  per-direction (hybrid) recipe: MXFP8 rowwise of dY, MXFP8 columnwise of
         bf16(dequant(NVFP4 rowwise W)) (one fused call from W's NVFP4 codes); dX = dY W (bf16)
value = the step's GEMM FLOPs (3 x 2MNK) / step time, in TFLOP/s.  The line also carries
the NVFP4 quantize GB/s and the NVFP4 GEMM TFLOP/s of the forward pass, the roofline of
the dominant kernel (the NVFP4 GEMM) timed with HIP events on its own stream, and the CPU
oracle timed on a token-sample of the same step.

The roofline's `traffic` (HBM bytes per launch of the forward NVFP4 GEMM) comes from a
hardware-counter summary under profiles/ (FETCH_SIZE and WRITE_SIZE, each scaled by the
ratio the same counter shows for a plain copy of known size, which `--copy-calibration`
runs); it is reported only while the GEMM sources still hash to the values recorded there.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-side-figures]
       python bench.py --copy-calibration      (a 1 GiB device-to-device copy, for the counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

M_TOK, N_OUT, K_IN = 16384, 14336, 4096
HBM_PEAK_GBPS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0
FP8_MFMA_PEAK_TFLOPS = 5000.0

# algorithmic bytes per element of one NVFP4 quantization direction: 2 B bf16 read,
# 0.5 B codes + 1/16 B scale written.
NVFP4_BYTES_PER_ELT = 2.0 + 0.5 + 1.0 / 16


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=2048)
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--no-side-figures", action="store_true",
                   help="skip the row-scaled, grouped and linear-layer figures (for counter runs)")
    p.add_argument("--mx-row-major", action="store_true",
                   help="MXFP8 GEMM operands in row-major instead of slab layout (for comparison)")
    p.add_argument("--quant-only", action="store_true",
                   help="only the quantize-only workload's casts (for kernel traces and counters)")
    return p.parse_args()


GEMM_SOURCES = ("block_scaled_precision_nvfp4_amd/csrc/gemm.hip",
                "block_scaled_precision_nvfp4_amd/csrc/device_common.hpp")
QUANT_SOURCES = ("block_scaled_precision_nvfp4_amd/csrc/quantize.hip",
                 "block_scaled_precision_nvfp4_amd/csrc/device_common.hpp")
# HBM traffic per launch (hardware counters) of the kernels the line reports a roofline for:
# the summary under profiles/ and the sources it was taken on
TRAFFIC = {
    "gemm_fwd_nvfp4": ("profiles/gemm_nvfp4_fwd_llama3_8b_hbm_traffic.md", GEMM_SOURCES),
    "gemm_wgrad_nvfp4": ("profiles/gemm_nvfp4_wgrad_llama3_8b_hbm_traffic.md", GEMM_SOURCES),
    "quant_dy_hybrid": ("profiles/nvfp4_col_mxfp8_row_dy_llama3_8b_hbm_traffic.md", QUANT_SOURCES),
}


def source_hash(files=GEMM_SOURCES, root: str = ROOT) -> str:
    """SHA-256 of kernel sources with comments and blank lines dropped: counters taken on the
    same code stay valid across comment edits."""
    h = hashlib.sha256()
    for rel in files:
        with open(os.path.join(root, rel)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(key: str):
    """HBM bytes per launch of a kernel (group) from its committed counter summary, or None
    when the summary is absent or was taken on other sources."""
    rel, files = TRAFFIC[key]
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
    if rec is None or rec.get("source_sha256") != source_hash(files):
        return None
    return rec


def copy_calibration(iters: int = 5):
    """A plain device-to-device copy of 1 GiB, the known-size kernel the HBM counters are
    scaled by (the copy reads 1 GiB and writes 1 GiB per launch)."""
    import torch
    n = 1 << 29   # bf16 elements = 1 GiB
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    print(json.dumps({"copy_bytes_each_way": 2 * n, "launches": iters, "ms": round(ms, 4),
                      "GBps_read_plus_write": round(4 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


class Step:
    """Buffers and launches of one step; every kernel runs on torch's current stream."""

    def __init__(self, dev, mx_rows: bool = False):
        import torch
        import block_scaled_precision_nvfp4_amd as bsq
        from synthetic import (SEED_DY, SEED_SIGNS, SEED_W, SEED_X, STD_DY, STD_W, gaussian_bf16, rht_signs)
        self.bsq, self.torch = bsq, torch
        self.X = gaussian_bf16((M_TOK, K_IN), 1.0, SEED_X).to(dev)
        self.W = gaussian_bf16((N_OUT, K_IN), STD_W, SEED_W).to(dev)
        self.dY = gaussian_bf16((M_TOK, N_OUT), STD_DY, SEED_DY).to(dev)
        self.signs = rht_signs(SEED_SIGNS).to(dev)
        self.seed = 42
        self.dev = dev
        # scratch of the NVFP4 quantize calls (their per-workgroup partial maxima); the step's
        # calls run in stream order, so one workspace serves them all
        self.qws = torch.empty(bsq.NVFP4_QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
        self.mx_rows = mx_rows
        self.ev = {}

    def _ev(self, name):
        torch = self.torch
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.ev.setdefault(name, []).append(e)

    def run(self, marks=()):
        """One step.  Event pairs are recorded around the kernel groups named in ``marks``
        (each pair is a stream barrier, so the throughput loop records only the pairs around
        the two NVFP4 GEMMs):
          q_fwd    X in one pass (NVFP4 rowwise RNE for fprop, columnwise RHT + SR for
                   wgrad) and W NVFP4 rowwise RNE
          g_fwd    forward NVFP4 GEMM
          q_dy     dY in one pass (NVFP4 columnwise RHT + SR for wgrad, MXFP8 rowwise for dgrad)
          g_wgrad  wgrad NVFP4 GEMM
          q_mx     MXFP8 columnwise W from its NVFP4 codes
          g_dgrad  dgrad MXFP8 GEMM"""
        bsq, torch = self.bsq, self.torch
        mark = (lambda name: self._ev(name) if name[:-1] in marks else None)
        # fwd
        mark("q_fwd0")
        ws = self.qws
        # X's forward operand and its saved wgrad operand from one pass over X
        qx = bsq.nvfp4_quantize_fprop_wgrad(self.X, rounding=bsq.SR, sr_seed=self.seed, sr_stream=1,
                                            rht_signs=self.signs, workspace=ws)
        qw = bsq.nvfp4_quantize(self.W, direction=bsq.ROW, workspace=ws)
        mark("q_fwd1")
        mark("g_fwd0")
        y = bsq.blockscaled_gemm(bsq.FMT_NVFP4, qx["row_codes"], qx["row_scales"], qx["s_enc"][0:1],
                                 qw["row_codes"], qw["row_scales"], qw["s_enc"][0:1], out_dtype=torch.bfloat16)
        mark("g_fwd1")
        # backward operands of dY: NVFP4 columnwise (RHT + SR) for wgrad and MXFP8 rowwise for
        # dgrad from one pass over dY; MXFP8 codes in the GEMM's slab layout unless the
        # row-major layout is asked for
        lay, fmx = (0, bsq.FMT_MXFP8) if self.mx_rows else (bsq.MX_SLAB, bsq.FMT_MXFP8 | bsq.FMT_MX_SLAB)
        mark("q_dy0")
        qdy = bsq.nvfp4_col_mxfp8_row_quantize(self.dY, rounding=bsq.SR, sr_seed=self.seed, sr_stream=0,
                                               rht_signs=self.signs, mx_slab=not self.mx_rows, workspace=ws)
        mark("q_dy1")
        mark("g_wgrad0")
        dw = bsq.blockscaled_gemm(bsq.FMT_NVFP4, qdy["col_codes"], qdy["col_scales"], qdy["s_enc"][1:2],
                                  qx["col_codes"], qx["col_scales"], qx["s_enc"][1:2], out_dtype=torch.float32)
        mark("g_wgrad1")
        # dgrad (MXFP8 operands; W from its rowwise-dequantized NVFP4 value)
        mark("q_mx0")
        mw = bsq.mxfp8_requantize_nvfp4(qw["row_codes"], qw["row_scales"], qw["s_enc"][0:1], direction=bsq.COL | lay)
        mark("q_mx1")
        mark("g_dgrad0")
        dx = bsq.blockscaled_gemm(fmx, qdy["mx_row_codes"], qdy["mx_row_scales"], None,
                                  mw["col_codes"], mw["col_scales"], None, out_dtype=torch.bfloat16)
        mark("g_dgrad1")
        return y, dw, dx

    def avg_ms(self, name):
        a, b = self.ev[name + "0"], self.ev[name + "1"]
        return sum(x.elapsed_time(y) for x, y in zip(a, b)) / len(a)


def measured_peaks(dev):
    """The rates this GPU sustains, beside the published peaks: a 512 MiB device-to-device copy
    (read + write bytes over time) and register-only MFMA loops (libbsq_peak.so) for the f16
    32x32x16 and the FP8 scaled 32x32x64 instructions, at one and two waves per SIMD."""
    import ctypes
    import torch
    import block_scaled_precision_nvfp4_amd as bsq
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    path = os.path.join(os.path.dirname(bsq.LIB_PATH), "libbsq_peak.so")
    L = ctypes.CDLL(path)
    L.bsq_peak_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    L.bsq_peak_mfma_loop.restype = ctypes.c_int
    stream = torch.cuda.current_stream(dev).cuda_stream
    out = {"copy_GBps": round(copy_gbps, 1)}
    for kind, name, flop in ((0, "mfma_f16_32x32x16_TFLOPs", 2.0 * 32 * 32 * 16),
                             (1, "mfma_fp8_32x32x64_TFLOPs", 2.0 * 32 * 32 * 64)):
        best = 0.0
        for wgs in (256 * 4, 256 * 8):          # one and two waves per SIMD
            iters = 4096 if kind == 0 else 2048
            sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
            assert L.bsq_peak_mfma_loop(kind, wgs, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream)) == 0
            torch.cuda.synchronize()
            e0.record()
            assert L.bsq_peak_mfma_loop(kind, wgs, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream)) == 0
            e1.record()
            torch.cuda.synchronize()
            flops = wgs * 4 * iters * 8 * flop
            best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        out[name] = round(best, 1)
    return out


def quant_only_figures(dev, peaks, iters: int = 10):
    """Side figure outside the step: the quantize-only workload, [8192, 4096] N(0,1) bf16 with 1 %
    of entries x100, each cast timed alone over ``iters`` launches that rotate over 4 copies of
    the input (so no launch reads what the previous one just read).  GB/s are algorithmic: the
    input read once plus the outputs written."""
    import torch
    import block_scaled_precision_nvfp4_amd as bsq
    from synthetic import outlier_bf16
    R, C = 8192, 4096
    base = outlier_bf16((R, C)).to(dev)
    xs = [base.clone() for _ in range(4)]
    ws = torch.empty(bsq.NVFP4_QUANTIZE_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    n = R * C
    cases = {
        "nvfp4_row_rne": (lambda x: bsq.nvfp4_quantize(x, direction=bsq.ROW, workspace=ws), 2.0 + 0.5625),
        "nvfp4_col_rne": (lambda x: bsq.nvfp4_quantize(x, direction=bsq.COL, workspace=ws), 2.0 + 0.5625),
        "nvfp4_row_col_rne": (lambda x: bsq.nvfp4_quantize(x, direction=bsq.ROW | bsq.COL, workspace=ws),
                              2.0 + 2 * 0.5625),
        "mxfp8_row": (lambda x: bsq.mxfp8_quantize(x, direction=bsq.ROW), 2.0 + 1.03125),
        "mxfp8_col": (lambda x: bsq.mxfp8_quantize(x, direction=bsq.COL), 2.0 + 1.03125),
    }
    out = {"shape": [R, C]}
    for name, (fn, bpe) in cases.items():
        us = spin_timed_us(torch, lambda i: fn(xs[i % 4]), iters)
        gbps = bpe * n / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 2), "GBps": round(gbps, 1), "of_8TBps": round(gbps / HBM_PEAK_GBPS, 4),
                     "of_measured_copy": round(gbps / peaks["copy_GBps"], 4)}
    return out


_SPIN_CYCLES_PER_MS = []


def spin_timed_us(torch, fn, iters: int) -> float:
    """Mean us per launch of ``fn(i)``, i = 0 .. iters-1, with the host's work kept out of the
    timed region.  A cast of ~20-50 us runs shorter than the binding's host work per call (output
    allocation and argument marshalling), so back-to-back calls would time the host: a spin
    kernel queued first holds the stream until every timed launch is enqueued, and the events
    then bracket the kernels alone."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not _SPIN_CYCLES_PER_MS:
        torch.cuda._sleep(1 << 20)
        e0.record()
        torch.cuda._sleep(1 << 24)
        e1.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS.append((1 << 24) / max(e0.elapsed_time(e1), 1e-3))
    backlog = int(_SPIN_CYCLES_PER_MS[0] * max(5.0, 0.25 * iters))
    fn(0)
    torch.cuda.synchronize()
    torch.cuda._sleep(backlog)
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters * 1e3


def timed_ms(torch, fn, iters: int) -> float:
    """Mean ms of ``fn`` over ``iters`` back-to-back calls, after ``iters`` untimed calls that
    bring the shader clock up (after a pause it takes ~10 ms of dense work to ramp: the first
    calls of a GEMM run up to 15 % slower)."""
    for _ in range(iters):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def rowscaled_figures(step, iters: int):
    """Side figures outside the step: row-scaled NVFP4 (one outer scale per row) of X, timed
    behind a spin kernel over ``iters`` launches rotating over 4 copies of X (as the
    quantize-only casts), and the forward GEMM with row-scaled X over ``iters`` back-to-back
    launches."""
    bsq, torch = step.bsq, step.torch
    qw = bsq.nvfp4_quantize(step.W, direction=bsq.ROW)
    qx = bsq.nvfp4_quantize_rowscaled(step.X)
    fmt = bsq.FMT_NVFP4 | bsq.FMT_A_ROWSCALED
    y = bsq.blockscaled_gemm(fmt, qx["codes"], qx["scales"], qx["s_enc"], qw["row_codes"], qw["row_scales"],
                             qw["s_enc"][0:1])
    xs = [step.X] + [step.X.clone() for _ in range(3)]
    for i in range(iters):   # bring the shader clock up, as timed_ms does
        bsq.nvfp4_quantize_rowscaled(xs[i % 4])
    q_ms = spin_timed_us(torch, lambda i: bsq.nvfp4_quantize_rowscaled(xs[i % 4]), iters) * 1e-3
    del xs
    g_ms = timed_ms(torch, lambda: bsq.blockscaled_gemm(fmt, qx["codes"], qx["scales"], qx["s_enc"], qw["row_codes"],
                                                        qw["row_scales"], qw["s_enc"][0:1], out=y), iters)
    q_bytes = M_TOK * K_IN * NVFP4_BYTES_PER_ELT + 8.0 * M_TOK   # + amax and S per row
    return {"nvfp4_rowscaled_quant_X_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
            "nvfp4_rowscaled_quant_X_ms": round(q_ms, 4),
            "gemm_fwd_rowscaled_X_TFLOPs": round(2.0 * M_TOK * N_OUT * K_IN / (g_ms * 1e-3) / 1e12, 2)}


def linear_layer_figures(step, iters: int):
    """Side figure outside the step: the NVFP4 linear layer entry points (forward saving the
    quantized activation, backward with RHT + SR on every backward operand and NVFP4 dgrad),
    forward + backward timed over ``iters`` iterations with a preallocated workspace."""
    bsq, torch = step.bsq, step.torch
    L = bsq.lib()
    ws = torch.empty(L.nvfp4_linear_workspace_bytes(M_TOK, K_IN, N_OUT), dtype=torch.uint8, device=step.dev)
    y, saved = bsq.nvfp4_linear_forward(step.X, step.W, step.seed, step.signs, workspace=ws)

    def fwd_bwd():
        _, sv = bsq.nvfp4_linear_forward(step.X, step.W, step.seed, step.signs, workspace=ws)
        bsq.nvfp4_linear_backward(step.dY, step.W, sv, step.seed, step.signs, workspace=ws)
    ms = timed_ms(torch, fwd_bwd, iters)
    return {"ms": round(ms, 4), "TFLOPs": round(3 * 2.0 * M_TOK * N_OUT * K_IN / (ms * 1e-3) / 1e12, 2),
            "saved_activation_bytes": int(saved.numel()), "bf16_activation_bytes": 2 * M_TOK * K_IN}


QWEN_TOK, QWEN_N, QWEN_K = 65536, 12288, 4096


def qwen3_8b_hybrid_figures(dev, iters: int, mx_rows: bool = False):
    """Side figure outside the step: the per-direction (hybrid) recipe at the Qwen3-8B FFN shape,
    X [65536, 4096], W [12288, 4096], dY [65536, 12288] -- forward NVFP4 rowwise GEMM; MXFP8
    rowwise dY, MXFP8 columnwise dY and X from the bf16 originals and W from its rowwise-
    dequantized NVFP4 value; dgrad dX = dY W (bf16) and wgrad dW = dY^T X (fp32) on MXFP8.
    Inputs are drawn as the step's are (CPU generator, seeds X 1234, W 1235, dY 1236, the same
    standard deviations), at these shapes."""
    import torch
    import block_scaled_precision_nvfp4_amd as bsq
    from synthetic import SEED_DY, SEED_W, SEED_X, STD_DY, STD_W, gaussian_bf16
    X = gaussian_bf16((QWEN_TOK, QWEN_K), 1.0, SEED_X).to(dev)
    W = gaussian_bf16((QWEN_N, QWEN_K), STD_W, SEED_W).to(dev)
    dY = gaussian_bf16((QWEN_TOK, QWEN_N), STD_DY, SEED_DY).to(dev)
    lay, fmx = (0, bsq.FMT_MXFP8) if mx_rows else (bsq.MX_SLAB, bsq.FMT_MXFP8 | bsq.FMT_MX_SLAB)
    def run():
        qx = bsq.nvfp4_quantize(X, direction=bsq.ROW)
        qw = bsq.nvfp4_quantize(W, direction=bsq.ROW)
        y = bsq.blockscaled_gemm(bsq.FMT_NVFP4, qx["row_codes"], qx["row_scales"], qx["s_enc"][0:1],
                                 qw["row_codes"], qw["row_scales"], qw["s_enc"][0:1])
        mdy = bsq.mxfp8_quantize(dY, direction=bsq.ROW | bsq.COL | lay)
        mx = bsq.mxfp8_quantize(X, direction=bsq.COL | lay)
        mw = bsq.mxfp8_requantize_nvfp4(qw["row_codes"], qw["row_scales"], qw["s_enc"][0:1], direction=bsq.COL | lay)
        dx = bsq.blockscaled_gemm(fmx, mdy["row_codes"], mdy["row_scales"], None, mw["col_codes"],
                                  mw["col_scales"], None)
        dw = bsq.blockscaled_gemm(fmx, mdy["col_codes"], mdy["col_scales"], None, mx["col_codes"],
                                  mx["col_scales"], None, out_dtype=torch.float32)
        return y, dx, dw
    ms = timed_ms(torch, run, iters)
    flops = 3 * 2.0 * QWEN_TOK * QWEN_N * QWEN_K
    return {"shape": "X[%d,%d] W[%d,%d]" % (QWEN_TOK, QWEN_K, QWEN_N, QWEN_K), "ms_per_step": round(ms, 3),
            "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1)}


MOE_EXPERTS = 8


def grouped_figures(step, iters: int):
    """Side figures outside the step: the same layer's tokens routed to MOE_EXPERTS experts
    of the same shape (seeded random split), run as grouped GEMMs in the Composer-style
    grouped recipe -- fprop on row-scaled NVFP4 inputs and per-expert NVFP4 weights, dgrad and
    wgrad on MXFP8 -- each timed over ``iters`` launches.  Total flops equal the dense GEMM's."""
    import numpy as np
    bsq, torch = step.bsq, step.torch
    G = MOE_EXPERTS
    rng = np.random.default_rng(2024)
    cuts = np.sort(rng.choice(np.arange(1, M_TOK // 32), G - 1, replace=False)) * 32   # wgrad needs 32-multiples
    offs_l = [0] + [int(c) for c in cuts] + [M_TOK]
    offs = torch.tensor(offs_l, dtype=torch.int64, device=step.dev)
    qx = bsq.nvfp4_quantize_rowscaled(step.X)
    w_codes = torch.empty((G, N_OUT, K_IN // 2), dtype=torch.uint8, device=step.dev)
    w_scales = torch.empty((G, N_OUT, K_IN // 16), dtype=torch.uint8, device=step.dev)
    w_s = torch.empty(G, dtype=torch.float32, device=step.dev)
    mw_codes = torch.empty((G, K_IN, N_OUT), dtype=torch.uint8, device=step.dev)
    mw_scales = torch.empty((G, K_IN, N_OUT // 32), dtype=torch.uint8, device=step.dev)
    for g in range(G):   # experts: W scaled per expert so that every expert has its own tensor scale
        wg = (step.W.float() * (1.0 + 0.1 * g)).to(torch.bfloat16)
        q = bsq.nvfp4_quantize(wg, direction=bsq.ROW)
        w_codes[g], w_scales[g], w_s[g:g + 1] = q["row_codes"], q["row_scales"], q["s_enc"][0:1]
        m = bsq.mxfp8_requantize_nvfp4(q["row_codes"], q["row_scales"], q["s_enc"][0:1],
                                       direction=bsq.COL | (0 if step.mx_rows else bsq.MX_SLAB))
        mw_codes[g], mw_scales[g] = m["col_codes"], m["col_scales"]
    # wgrad operands: columnwise casts over all tokens, slab-layout codes unless the row-major
    # layout is asked for; dgrad's token operand is M-grouped, so row-major
    lay = 0 if step.mx_rows else bsq.MX_SLAB
    mdy = bsq.mxfp8_quantize(step.dY, direction=bsq.ROW)
    mdy.update(bsq.mxfp8_quantize(step.dY, direction=bsq.COL | lay))
    mx = bsq.mxfp8_quantize(step.X, direction=bsq.COL | lay)
    fwd_fmt = bsq.FMT_NVFP4 | bsq.FMT_A_ROWSCALED
    y = torch.empty((M_TOK, N_OUT), dtype=torch.bfloat16, device=step.dev)
    dx = torch.empty((M_TOK, K_IN), dtype=torch.bfloat16, device=step.dev)
    dw = torch.empty((G, N_OUT, K_IN), dtype=torch.float32, device=step.dev)
    launches = {
        "fprop": lambda: bsq.blockscaled_grouped_gemm(fwd_fmt, bsq.GROUP_M, offs, qx["codes"], qx["scales"],
                                                      qx["s_enc"], w_codes, w_scales, w_s, out=y),
        "dgrad": lambda: bsq.blockscaled_grouped_gemm(bsq.FMT_MXFP8 | (0 if step.mx_rows else bsq.FMT_MX_SLAB_B),
                                                      bsq.GROUP_M, offs, mdy["row_codes"],
                                                      mdy["row_scales"], None, mw_codes, mw_scales, None, out=dx),
        "wgrad": lambda: bsq.blockscaled_grouped_gemm(bsq.FMT_MXFP8 | (0 if step.mx_rows else bsq.FMT_MX_SLAB),
                                                      bsq.GROUP_K, offs, mdy["col_codes"],
                                                      mdy["col_scales"], None, mx["col_codes"], mx["col_scales"],
                                                      None, out_dtype=torch.float32, out=dw),
    }
    # the same wgrad on NVFP4: dY and X quantized columnwise per expert (each expert's tokens
    # its own tensor scale), codes and scales laid out along all tokens
    nv = [[bsq.nvfp4_quantize(t[offs_l[g]:offs_l[g + 1]].contiguous(), direction=bsq.COL) for t in (step.dY, step.X)]
          for g in range(G)]
    ncat = lambda i, key: torch.cat([q[i][key] for q in nv], dim=1).contiguous()
    ns = lambda i: torch.cat([q[i]["s_enc"][1:2] for q in nv]).contiguous()
    na = (ncat(0, "col_codes"), ncat(0, "col_scales"), ns(0))
    nb = (ncat(1, "col_codes"), ncat(1, "col_scales"), ns(1))
    del nv
    launches["wgrad_nvfp4"] = lambda: bsq.blockscaled_grouped_gemm(bsq.FMT_NVFP4, bsq.GROUP_K, offs, *na, *nb,
                                                                   out_dtype=torch.float32, out=dw)
    out = {"experts": G, "tokens_per_expert": [offs_l[i + 1] - offs_l[i] for i in range(G)]}
    flops = 2.0 * M_TOK * N_OUT * K_IN
    for name, fn in launches.items():
        ms = timed_ms(torch, fn, iters)
        out["grouped_%s_TFLOPs" % name] = round(flops / (ms * 1e-3) / 1e12, 2)
    return out


def odd_k_figures(step, iters: int):
    """Side figure outside the step: the forward NVFP4 GEMM with K = 4032 (the first 4032
    columns of X and W), whose scale rows are not 16 bytes apart, so that the GEMM takes its
    per-slice scale path."""
    bsq, torch = step.bsq, step.torch
    K = 4032
    qx = bsq.nvfp4_quantize(step.X[:, :K].contiguous(), direction=bsq.ROW)
    qw = bsq.nvfp4_quantize(step.W[:, :K].contiguous(), direction=bsq.ROW)
    y = torch.empty((M_TOK, N_OUT), dtype=torch.bfloat16, device=step.dev)
    ms = timed_ms(torch, lambda: bsq.blockscaled_gemm(bsq.FMT_NVFP4, qx["row_codes"], qx["row_scales"],
                                                      qx["s_enc"][0:1], qw["row_codes"], qw["row_scales"],
                                                      qw["s_enc"][0:1], out=y), iters)
    return {"shape": [M_TOK, N_OUT, K], "ms": round(ms, 4), "TFLOPs": round(2.0 * M_TOK * N_OUT * K / (ms * 1e-3) / 1e12, 1)}


def cpu_baseline(tokens: int):
    """The oracle on the host cores: (1) the step on a token sample (the same operations with
    M = tokens; all threads), the headline value; (2) the full quantize-only workload
    ([8192, 4096] with 1 % outliers: NVFP4 rowwise, NVFP4 columnwise, MXFP8 rowwise) with all
    threads and with one.  GB/s are the algorithmic bytes of the GPU figures."""
    import oracle
    from synthetic import (SEED_DY, SEED_SIGNS, SEED_W, SEED_X, STD_DY, STD_W, gaussian_bf16, outlier_bf16,
                           rht_signs)
    threads = oracle.num_threads()
    X = gaussian_bf16((tokens, K_IN), 1.0, SEED_X)
    W = gaussian_bf16((N_OUT, K_IN), STD_W, SEED_W)
    dY = gaussian_bf16((tokens, N_OUT), STD_DY, SEED_DY)
    d = rht_signs(SEED_SIGNS).numpy()
    t0 = time.perf_counter()
    qx = oracle.nvfp4_quantize(X, direction=oracle.ROW)
    qw = oracle.nvfp4_quantize(W, direction=oracle.ROW)
    oracle.blockscaled_gemm(oracle.FMT_NVFP4, qx["row_codes"], qx["row_scales"], qx["s_enc"][0],
                            qw["row_codes"], qw["row_scales"], qw["s_enc"][0])
    qdy = oracle.nvfp4_quantize(dY, direction=oracle.COL, rounding=oracle.SR, sr_seed=42, sr_stream=0, signs=d)
    qxc = oracle.nvfp4_quantize(X, direction=oracle.COL, rounding=oracle.SR, sr_seed=42, sr_stream=1, signs=d)
    oracle.blockscaled_gemm(oracle.FMT_NVFP4, qdy["col_codes"], qdy["col_scales"], qdy["s_enc"][1],
                            qxc["col_codes"], qxc["col_scales"], qxc["s_enc"][1])
    mdy = oracle.mxfp8_quantize(dY, direction=oracle.ROW)
    wdq = oracle.nvfp4_dequantize(qw["row_codes"], qw["row_scales"], float(qw["s_enc"][0]))
    mw = oracle.mxfp8_quantize(wdq, direction=oracle.COL)
    oracle.blockscaled_gemm(oracle.FMT_MXFP8, mdy["row_codes"], mdy["row_scales"], 1.0,
                            mw["col_codes"], mw["col_scales"], 1.0)
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * tokens * N_OUT * K_IN

    xq = outlier_bf16((8192, 4096))
    n = xq.numel()
    casts = (("nvfp4_row", lambda: oracle.nvfp4_quantize(xq, direction=oracle.ROW), 2.5625),
             ("nvfp4_col", lambda: oracle.nvfp4_quantize(xq, direction=oracle.COL), 2.5625),
             ("mxfp8_row", lambda: oracle.mxfp8_quantize(xq, direction=oracle.ROW), 2.0 + 1.03125))

    def quant_only(nthreads):
        oracle.set_num_threads(nthreads)
        out = {"threads": oracle.num_threads()}
        for name, fn, bpe in casts:
            t = time.perf_counter()
            fn()
            sec = time.perf_counter() - t
            out[name] = {"s": round(sec, 3), "GBps": round(bpe * n / sec / 1e9, 2)}
        return out
    q_all = quant_only(threads)
    q_one = quant_only(1)
    oracle.set_num_threads(threads)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "the full step with %d of %d tokens (M = %d), %d threads; %.1f s" % (tokens, M_TOK, tokens, threads, dt),
            "host_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
            "quant_only_full": {"shape": [8192, 4096], "all_threads": q_all, "one_thread": q_one}}


def roofline_entry(bound, achieved, peak, unit, kernel, algorithmic_bytes, traffic_key=None, **extra):
    """One roofline object: achieved / peak for a kernel, with the counter-measured HBM traffic
    per launch when a summary taken on the current sources exists."""
    tr = measured_traffic(traffic_key) if traffic_key else None
    e = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": None if tr is None else tr["traffic_bytes"],
         "algorithmic_bytes": int(algorithmic_bytes), "kernel": kernel}
    e.update(extra)
    return e


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the path here has no multi-GPU implementation (--gpus %d requested)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    import block_scaled_precision_nvfp4_amd as bsq
    bsq.lib()
    dev = torch.device("cuda:0")
    if args.quant_only:
        print(json.dumps(quant_only_figures(dev, {"copy_GBps": float("nan")}, iters=args.steps)), flush=True)
        return
    step = Step(dev, args.mx_row_major)
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for _ in range(args.steps):
        step.run(marks=("g_fwd", "g_wgrad"))
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    gemm_flops = 2.0 * M_TOK * N_OUT * K_IN
    value = 3 * gemm_flops / (ms_step * 1e-3) / 1e12
    # the two NVFP4 GEMMs (the longest kernels of the step), timed inside the timed steps
    g_fwd = step.avg_ms("g_fwd")
    g_wgrad = step.avg_ms("g_wgrad")

    # per-group breakdown in separate, untimed steps (the marker barriers would add gaps)
    for _ in range(max(2, args.steps // 2)):
        step.run(marks=("q_fwd", "q_dy", "q_mx", "g_dgrad"))
    torch.cuda.synchronize()
    g_dgrad = step.avg_ms("g_dgrad")
    q_fwd, q_dy, q_mx = (step.avg_ms(k) for k in ("q_fwd", "q_dy", "q_mx"))
    # the forward quantization: X read once and written in both directions, W rowwise
    q_bytes = (NVFP4_BYTES_PER_ELT + 0.5625) * M_TOK * K_IN + NVFP4_BYTES_PER_ELT * N_OUT * K_IN
    # ... against the two-pass floor (each tensor read twice: amax pass and encode pass)
    q_floor = q_bytes + 2.0 * (M_TOK + N_OUT) * K_IN
    # dY's one-pass cast: dY read once, NVFP4 columnwise and MXFP8 rowwise written
    dy_bytes = (NVFP4_BYTES_PER_ELT + 1.03125) * M_TOK * N_OUT
    # the metric's quantization half: the forward operands alone, NVFP4 rowwise RNE of X and W
    # as two plain calls (the step makes X's rowwise operand together with its columnwise one)
    # (timed behind a spin kernel: two binding calls cost about as much host time as their ~90 us
    # of kernels, so back-to-back timing could measure the host)
    ws = step.qws
    rne_ms = spin_timed_us(torch, lambda i: (bsq.nvfp4_quantize(step.X, direction=bsq.ROW, workspace=ws),
                                             bsq.nvfp4_quantize(step.W, direction=bsq.ROW, workspace=ws)),
                           max(4, args.steps)) * 1e-3
    rne_bytes = NVFP4_BYTES_PER_ELT * (M_TOK + N_OUT) * K_IN
    peaks = measured_peaks(dev)
    side = moe = layer = qwen = quant_only = odd_k = None
    if not args.no_side_figures:
        quant_only = quant_only_figures(dev, peaks)
        side = rowscaled_figures(step, max(3, args.steps // 2))
        moe = grouped_figures(step, max(3, args.steps // 2))
        odd_k = odd_k_figures(step, max(3, args.steps // 2))
        layer = linear_layer_figures(step, max(3, args.steps // 2))
        qwen = qwen3_8b_hybrid_figures(dev, 3, args.mx_row_major)
    tflops = lambda ms: gemm_flops / (ms * 1e-3) / 1e12
    gbps = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    # algorithmic bytes of one GEMM launch: both operands' codes and scales once, C once
    nv_op = 0.5 + 1.0 / 16
    algo = {"fwd": (M_TOK + N_OUT) * K_IN * nv_op + 2.0 * M_TOK * N_OUT,
            "wgrad": (N_OUT + K_IN) * M_TOK * nv_op + 4.0 * N_OUT * K_IN,
            "dgrad": (M_TOK + K_IN) * N_OUT * 1.03125 + 2.0 * M_TOK * K_IN}
    gemms = {
        "fwd_nvfp4": roofline_entry("mfma", tflops(g_fwd), F16_MFMA_PEAK_TFLOPS, "TFLOP/s",
                                    "gemm_nvp_kernel<false, false>: NVFP4 fwd Y = X W^T, persistent, f16 MFMA with in-register dequant",
                                    algo["fwd"], "gemm_fwd_nvfp4", ms=round(g_fwd, 4),
                                    frac_of_measured=round(tflops(g_fwd) / peaks["mfma_f16_32x32x16_TFLOPs"], 4)),
        "wgrad_nvfp4": roofline_entry("mfma", tflops(g_wgrad), F16_MFMA_PEAK_TFLOPS, "TFLOP/s",
                                      "gemm_nvp_kernel<true, false>: NVFP4 wgrad dW = dY^T X (fp32 out), persistent, f16 MFMA",
                                      algo["wgrad"], "gemm_wgrad_nvfp4", ms=round(g_wgrad, 4),
                                      frac_of_measured=round(tflops(g_wgrad) / peaks["mfma_f16_32x32x16_TFLOPs"], 4)),
        "dgrad_mxfp8": roofline_entry("mfma", tflops(g_dgrad), FP8_MFMA_PEAK_TFLOPS, "TFLOP/s",
                                      "gemm_kernel<1,0,0>: MXFP8 dgrad dX = dY W, scaled fp8 MFMA", algo["dgrad"],
                                      ms=round(g_dgrad, 4),
                                      frac_of_measured=round(tflops(g_dgrad) / peaks["mfma_fp8_32x32x64_TFLOPs"], 4)),
    }
    # the roofline of the dominant kernel: the NVFP4 GEMM with the longer average launch
    dominant = "wgrad_nvfp4" if g_wgrad >= g_fwd else "fwd_nvfp4"
    roofline = dict(gemms[dominant])
    roofline["measured_peak"] = peaks["mfma_f16_32x32x16_TFLOPs"]
    # quantization rooflines: HBM-bound; an NVFP4 cast with a per-tensor amax reads its input
    # twice (amax pass, encode pass), so besides the fraction of 8 TB/s the entry gives the
    # fraction of what two reads + one write allow at 8 TB/s
    two_pass = lambda bpe_write: (2.0 + bpe_write) / (4.0 + bpe_write)
    quant = {
        "dy_col_rht_sr_mx_row": roofline_entry(
            "hbm", gbps(dy_bytes, q_dy), HBM_PEAK_GBPS, "GB/s",
            "nvfp4_amax_rht_kernel<2,false> + nvfp4_encode_kernel<2,true,true,true,false>: dY[16384,14336] in one encode "
            "pass, NVFP4 columnwise RHT16 + Philox SR and MXFP8 rowwise", dy_bytes, "quant_dy_hybrid",
            us=round(q_dy * 1e3, 2),
            two_pass_bound_frac=round(gbps(dy_bytes, q_dy) / (HBM_PEAK_GBPS * two_pass(0.5625 + 1.03125)), 4)),
        "fwd_X_both_W_row": roofline_entry(
            "hbm", gbps(q_bytes, q_fwd), HBM_PEAK_GBPS, "GB/s",
            "nvfp4_amax_rht_kernel<3,true> + nvfp4_encode_kernel<3,true,true,false,true>: X[16384,4096] rowwise RNE "
            "and columnwise RHT16 + SR in one encode pass; W rowwise RNE (amax + streaming encode)", q_bytes,
            us=round(q_fwd * 1e3, 2),
            two_pass_bound_frac=round(gbps(q_bytes, q_fwd) / (HBM_PEAK_GBPS * q_bytes / q_floor), 4)),
        "mx_w_requant": roofline_entry(
            "hbm", gbps(N_OUT * K_IN * (0.5625 + 1.03125), q_mx), HBM_PEAK_GBPS, "GB/s",
            "MXFP8 columnwise of W from its NVFP4 rowwise codes (one pass)",
            N_OUT * K_IN * (0.5625 + 1.03125), us=round(q_mx * 1e3, 2)),
    }
    if quant_only is not None:
        for name, e in quant_only.items():
            if name.startswith("nvfp4") and isinstance(e, dict):
                w = 2 * 0.5625 if name == "nvfp4_row_col_rne" else 0.5625
                e["two_pass_bound_frac"] = round(e["GBps"] / (HBM_PEAK_GBPS * two_pass(w)), 4)
    line = {
        "metric": "NVFP4 quant GB/s + block-scaled GEMM TFLOP/s at Llama-3-8B FFN shape",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "nvfp4/mxfp8 operands, f16/fp8 MFMA, fp32 accumulate", "data": "synthetic",
        "config": {"workload": "quantized linear fwd+wgrad+dgrad step, Llama-3-8B FFN up-proj",
                   "tokens": M_TOK, "in_features": K_IN, "out_features": N_OUT,
                   "fwd": "NVFP4 row RNE", "wgrad": "NVFP4 col RHT16+SR", "dgrad": "MXFP8 (W from rowwise-dequantized)",
                   "mxfp8_code_layout": "row-major" if args.mx_row_major else "slab"},
        "nvfp4_quant_GBps": round(gbps(rne_bytes, rne_ms), 1),
        "nvfp4_quant_frac": {"of_peak_8TBps": round(gbps(rne_bytes, rne_ms) / HBM_PEAK_GBPS, 4),
                             "of_measured_copy": round(gbps(rne_bytes, rne_ms) / peaks["copy_GBps"], 4),
                             "of_two_pass_bound": round(gbps(rne_bytes, rne_ms) / (HBM_PEAK_GBPS * two_pass(0.5625)), 4),
                             "what": "NVFP4 rowwise RNE of X[16384,4096] and W[14336,4096], two calls, "
                                     "timed apart from the step"},
        "nvfp4_gemm_TFLOPs": round(tflops(g_fwd), 2),
        "kernel_ms": {"nvfp4_quant_X_both_W_row": round(q_fwd, 4), "dy_nvfp4_col_mxfp8_row": round(q_dy, 4),
                      "mxfp8_requant_w": round(q_mx, 4),
                      "gemm_fwd_nvfp4": round(g_fwd, 4), "gemm_wgrad_nvfp4": round(g_wgrad, 4),
                      "gemm_dgrad_mxfp8": round(g_dgrad, 4)},
        "mxfp8_gemm_TFLOPs": round(tflops(g_dgrad), 2),
        "mxfp8_gemm_frac": {"of_peak": round(tflops(g_dgrad) / FP8_MFMA_PEAK_TFLOPS, 4),
                            "of_measured": round(tflops(g_dgrad) / peaks["mfma_fp8_32x32x64_TFLOPs"], 4)},
        "measured_peaks": peaks,
        "quant_only": quant_only,
        "row_scaled": side,
        "nvfp4_gemm_k4032": odd_k,
        "moe_grouped": moe,
        "nvfp4_linear_layer": layer,
        "qwen3_8b_hybrid": qwen,
        "gemm_rooflines": gemms,
        "quant_rooflines": quant,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_sample_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
