"""Shared helpers of the GPU parity tests: host copies of device tensors, the oracle run on
exactly the bytes the GPU consumed, and the comparison bars.

Bars: gamma, packed bytes, int8 codes, absmax and int32 accumulators bit-exact; y within
1e-5 relative of the oracle's fp64 rescale, and exactly 0 where the oracle's is 0."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

Y_RTOL = 1e-5


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def acts_host_f32(x: torch.Tensor) -> np.ndarray:
    """The activations as the oracle sees them (bf16 widened by the oracle itself)."""
    if x.dtype == torch.bfloat16:
        bits = x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return oracle.bf16_bits_to_f32(bits)
    return host(x.float())


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = "y") -> None:
    y = y_gpu.astype(np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    zero = y_ref == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero where the oracle is 0"
    bad = np.abs(y - y_ref) > Y_RTOL * np.abs(y_ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} entries beyond {Y_RTOL} rel, e.g. "
                             + ", ".join(f"{tuple(i)}: {y[tuple(i)]} vs {y_ref[tuple(i)]}" for i in idx))


def check_equal(a: np.ndarray, b: np.ndarray, what: str) -> None:
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if not np.array_equal(a, b):
        diff = np.argwhere(a != b)
        raise AssertionError(f"{what}: {len(diff)} mismatches, first at {tuple(diff[0])}: "
                             f"{a[tuple(diff[0])]} vs {b[tuple(diff[0])]}")


def gamma_bits(g) -> int:
    return int(np.asarray(g, dtype=np.float32).reshape(-1)[0:1].view(np.uint32)[0])


def host_threads() -> int:
    """Host threads for the oracle: the CPUs this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_forward_rows(q: np.ndarray, gamma, xq: np.ndarray, absmax: np.ndarray, k: int):
    """oracle.forward on every token row, the rows split into contiguous slices computed
    on host threads at once (the oracle's C routines run outside the interpreter lock).
    Each row's result depends on that row alone, so the slices concatenate to the
    single-call result."""
    m = xq.shape[0]
    parts = max(1, min(host_threads(), m))
    bounds = [m * i // parts for i in range(parts + 1)]
    def one(i):
        lo, hi = bounds[i], bounds[i + 1]
        return oracle.forward(q, gamma, np.ascontiguousarray(xq[lo:hi]), np.ascontiguousarray(absmax[lo:hi]), k)
    with ThreadPoolExecutor(parts) as pool:
        res = list(pool.map(one, range(parts)))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])
