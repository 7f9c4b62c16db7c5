"""Helpers for the GPU parity tests: upload seeded inputs, run the library, compare
with the oracle at the stated tolerances."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import workloads as W

# Tolerances for O and LSE against the fp64 oracle.
TOL_FP32_MAX = 1e-5
TOL_BF16_MAX = 1e-2
TOL_BF16_MEAN = 1e-3
TOL_LSE = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(x.copy()).cuda()


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """o_*: [..., d] arrays of the same shape; lse_*: matching row arrays."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    empty = ~np.isfinite(lse_ref)
    assert np.array_equal(empty, ~np.isfinite(lse_gpu)), f"{what}: empty-row pattern differs"
    assert np.all(lse_gpu[empty] == -np.inf), f"{what}: empty rows must have LSE = -inf"
    err = np.abs(o_gpu - o_ref)
    if dtype == "fp32":
        assert err.max() <= TOL_FP32_MAX, f"{what}: max|dO| {err.max():.3e}"
    else:
        assert err.max() <= TOL_BF16_MAX, f"{what}: max|dO| {err.max():.3e}"
        assert err.mean() <= TOL_BF16_MEAN, f"{what}: mean|dO| {err.mean():.3e}"
    if (~empty).any():
        le = np.abs(lse_gpu[~empty] - lse_ref[~empty]).max()
        assert le <= TOL_LSE, f"{what}: max|dLSE| {le:.3e}"
    return float(err.max()), float(err.mean())


def qkv_case(seed, B, nq, nk, H, d, dtype, amp=1.0):
    q = W.gen_tensor(seed, W.TENSOR_Q, B, nq, H, d, amp, dtype)
    k = W.gen_tensor(seed, W.TENSOR_K, B, nk, H, d, amp, dtype)
    v = W.gen_tensor(seed, W.TENSOR_V, B, nk, H, d, amp, dtype)
    return q, k, v


def e4m3_half_spacing(x):
    """Half the gap between neighbouring E4M3 values around x >= 0 (the largest
    error of rounding x to nearest): 2^(e - 4) for normal x in [2^e, 2^(e+1)),
    2^-10 below 2^-6 (subnormals, spacing 2^-9)."""
    x = np.asarray(x, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -6)))
    return np.where(x < 2.0 ** -6, 2.0 ** -10, np.exp2(e - 4))


def oracle_map(fn, items):
    """fn over items on a thread pool the size of the usable cores (at most 16): the
    oracle's numpy work releases the interpreter lock, so independent (batch, head)
    problems run side by side. Results come back in the order of items."""
    items = list(items)
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(items)))
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))
