"""Helpers shared by the GPU parity tests (imported only by tests marked gpu)."""
import sys

import numpy as np
import torch


def note(msg: str):
    """Name the case on stdout before a GPU step, so a failing run shows where it was."""
    print("[gpu-case] " + msg, flush=True)
    sys.stdout.flush()


def cpu_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_bytes_equal(gpu: torch.Tensor, ref: np.ndarray, what: str):
    g = cpu_u8(gpu)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    if not np.array_equal(g, ref):
        bad = np.argwhere(g != ref)
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d bytes differ; first at %s: gpu %#x oracle %#x"
                             % (what, len(bad), g.size, i, int(g[i]), int(ref[i])))


def assert_f32_equal(gpu: torch.Tensor, ref: np.ndarray, what: str):
    g = gpu.detach().cpu().numpy()
    assert g.shape == ref.shape
    gb, rb = g.view(np.uint32), np.ascontiguousarray(ref, np.float32).view(np.uint32)
    if not np.array_equal(gb, rb):
        bad = np.argwhere(gb != rb)
        i = tuple(bad[0])
        raise AssertionError("%s: %d values differ; first at %s: gpu %r oracle %r" % (what, len(bad), i, g[i], ref[i]))


def bf16_round(y64: np.ndarray) -> np.ndarray:
    """Oracle output rounded as the GPU output is stored (bf16 RNE), back in float64."""
    return torch.from_numpy(y64).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


GEMM_TOL = 2e-3


def from_slab(t: torch.Tensor, rows: int, K: int) -> np.ndarray:
    """The row-major [rows][K] codes held by a buffer in the slab layout: rows in bands of 256,
    band b from byte 256 b K holding its n rows as K/64 slabs of n x 64 bytes."""
    flat = t.cpu().numpy().reshape(-1)
    assert flat.size == rows * K
    out = np.empty((rows, K), np.uint8)
    for b0 in range(0, rows, 256):
        n = min(256, rows - b0)
        out[b0:b0 + n] = flat[b0 * K:(b0 + n) * K].reshape(K // 64, n, 64).transpose(1, 0, 2).reshape(n, K)
    return out
