"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth

TOL = 1e-4   # |y_gpu - y| <= TOL * sum_k |w x| for every output


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def x_host(x: torch.Tensor) -> np.ndarray:
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def check_dequant(qtype, w_rep, rows, cols, gguf_rows_host, row_idx, where):
    """Repacked weights on the device dequantise bit-exactly (+0 == -0) to the oracle's fp32 values."""
    Wg = kq.dequant(qtype, w_rep, rows, cols)
    torch.cuda.synchronize()
    Wg = Wg[torch.as_tensor(row_idx, device=Wg.device)].cpu().numpy()
    Wo = O.dequant_f32(qtype, len(row_idx), cols, gguf_rows_host)
    bad = Wg != Wo
    assert not bad.any(), f"{where}: {int(bad.sum())} dequantised weights differ, first at {np.argwhere(bad)[0]}"


def check_y(yg: np.ndarray, yo: np.ndarray, ao: np.ndarray, where: str):
    err = np.abs(yg.astype(np.float64) - yo)
    bad = err > TOL * ao
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {int(bad.sum())} outputs over tolerance; first {tuple(i)}: gpu {yg[tuple(i)]!r} "
                             f"oracle {yo[tuple(i)]!r} bound {TOL * ao[tuple(i)]!r}")
    return float(np.max(err / np.where(ao > 0, ao, 1.0)))


def sample_rows(rows: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 62, 63, 64, 65, rows // 2, rows - 65, rows - 64, rows - 2, rows - 1]
    pick = set(r for r in fixed if 0 <= r < rows)
    pick.update(rng.integers(0, rows, size=min(n, rows)).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def oracle_rows(qtype, gguf_dev: torch.Tensor, row_idx, cols, x: torch.Tensor):
    g = gguf_dev[torch.as_tensor(row_idx, device=gguf_dev.device)].cpu().numpy()
    y, a = O.gemv(qtype, len(row_idx), cols, g, x_host(x))
    return g, y, a
