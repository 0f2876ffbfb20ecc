"""Helpers shared by the GPU tests: progress lines, error measures, and the
device-side cases (workloads.device) that run the library through its C ABI."""
from __future__ import annotations

import sys

import numpy as np

import gqa_attention_paged_amd as gq  # noqa: F401  (the library; fails loudly when it is not built)
from workloads.device import (DeviceChunk, DeviceDecode, DevicePrefill, bits_to_tensor,  # noqa: F401
                              tensor_to_f64)


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def max_abs_err(a: np.ndarray, b: np.ndarray) -> float:
    if a.size == 0:
        return 0.0
    d = np.abs(a - b)
    if np.isnan(d).any():
        return float("inf")
    return float(d.max())


def lse_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |a - b| over finite entries; inf if the -inf pattern differs or NaN appears."""
    if np.isnan(gpu).any():
        return float("inf")
    if not np.array_equal(np.isneginf(gpu), np.isneginf(ref)):
        return float("inf")
    fin = np.isfinite(ref)
    return float(np.abs(gpu[fin] - ref[fin]).max()) if fin.any() else 0.0


def lse_within(gpu: np.ndarray, ref: np.ndarray, bound) -> bool:
    """|gpu - ref| <= bound (a scalar or an array shaped like ref) on every
    finite entry, the same -inf pattern, and no NaN."""
    if np.isnan(gpu).any() or not np.array_equal(np.isneginf(gpu), np.isneginf(ref)):
        return False
    fin = np.isfinite(ref)
    b = np.broadcast_to(np.asarray(bound, np.float64), ref.shape)
    return bool(np.all(np.abs(gpu[fin] - ref[fin]) <= b[fin]))
