"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module holds shapes, seeds and random-number generation only. It contains
none of the attention arithmetic, so that the CPU oracle and the GPU path can
both draw their inputs from it without sharing any of the computation.

Inputs are drawn per (tensor, batch, head) slice from
``numpy.random.default_rng([seed, tensor_id, b, h])``. Any slice can therefore
be regenerated on its own, which lets the oracle check sampled outputs of the
large workloads without materialising every tensor on the host.

bf16 values are produced by rounding float32 draws to the nearest bf16 (ties to
even) with integer bit operations, and are carried as uint16 bit patterns. The
exact same bits are uploaded to the device and upcast for the oracle, so input
quantisation is never counted as error.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
BF16_NAN_BITS = 0x7FC0


# --------------------------------------------------------------------------
# bf16 bit helpers (storage format only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (float32, uint16 bf16 bits or uint8 E4M3 codes) -> float64 values, exactly."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    if dtype == "fp8":
        return e4m3_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# fp8 E4M3 bit helpers (storage format only; OCP "E4M3FN": 1 sign bit, 4
# exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN,
# largest finite 448, smallest subnormal 2^-9)
# --------------------------------------------------------------------------
E4M3_MAX = 448.0
E4M3_NAN_BITS = 0x7F


def e4m3_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact values of E4M3 codes (uint8) as float32; NaN codes give NaN."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & ((b & 7) == 7), np.nan, mag)
    return (sign * mag).astype(np.float32)


_E4M3_POS = None


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to E4M3 (nearest, ties to the even code),
    saturating at +-448; returns uint8 codes."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = e4m3_bits_to_f32(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)  # 0 .. 448
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left").clip(0, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(x < 0, code | 0x80, code).astype(np.uint8)


# --------------------------------------------------------------------------
# Slice generator
# --------------------------------------------------------------------------
def gen_slice(seed: int, tensor_id: int, b: int, h: int, n: int, d: int,
              amp: float, dtype: str) -> np.ndarray:
    """One [n, d] slice of tensor ``tensor_id`` for (batch b, head h).

    Returns float32 values (dtype "fp32") or uint16 bf16 bits (dtype "bf16").
    """
    rng = np.random.default_rng([int(seed), int(tensor_id), int(b), int(h)])
    x = rng.standard_normal((n, d), dtype=np.float32)
    if amp != 1.0:
        x *= np.float32(amp)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp32":
        return x
    if dtype == "fp8":
        return f32_to_e4m3_bits(x)
    raise ValueError(dtype)


def gen_tensor(seed: int, tensor_id: int, B: int, N: int, H: int, d: int,
               amp: float, dtype: str) -> np.ndarray:
    """A [B, N, H, d] tensor assembled from its per-(b, h) slices."""
    out = np.empty((B, N, H, d), dtype={"bf16": np.uint16, "fp8": np.uint8}.get(dtype, np.float32))
    for b in range(B):
        for h in range(H):
            out[b, :, h, :] = gen_slice(seed, tensor_id, b, h, N, d, amp, dtype)
    return out


def gen_block_table(seed: int, batch: int, pages_per_seq: int, pool_pages: int) -> np.ndarray:
    """Distinct physical page ids for every (sequence, logical page): a seeded permutation."""
    if pool_pages < batch * pages_per_seq:
        raise ValueError("pool too small")
    perm = np.random.default_rng(seed).permutation(pool_pages)[: batch * pages_per_seq]
    return perm.reshape(batch, pages_per_seq).astype(np.int32)


def scatter_pages(pool: np.ndarray, block_table: np.ndarray, b: int, h: int,
                  x: np.ndarray, page_size: int) -> None:
    """Write logical rows x[t] (t < len(x)) of (b, h) into pool[page, t % ps, h, :].

    Storage placement only (a copy); the oracle's own gather is separate.
    """
    n = x.shape[0]
    npages = (n + page_size - 1) // page_size
    for p in range(npages):
        t0 = p * page_size
        t1 = min(n, t0 + page_size)
        pool[block_table[b, p], 0:t1 - t0, h, :] = x[t0:t1]


def alibi_slopes(H: int) -> np.ndarray:
    """Per-head ALiBi slopes 2^(-8(h+1)/H), h 0-based (the workload's stated choice)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    amp: float = 1.0
    causal: bool = False
    window_left: int = -1
    window_right: int = -1
    alibi: bool = False
    softcap: float = 0.0
    paged: bool = False
    page_size: int = 0
    pool_factor: float = 0.0
    num_splits: int = 1
    seed: int = 0
    table_seed: int = 104
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def pages_per_seq(self) -> int:
        return (self.Nk + self.page_size - 1) // self.page_size

    @property
    def pool_pages(self) -> int:
        return int(math.ceil(self.pool_factor * self.B * self.pages_per_seq))

    def slopes(self):
        return alibi_slopes(self.H) if self.alibi else None


WORKLOADS = {
    1: Workload(1, "tiny_fp32_noncausal", B=1, H=2, Nq=128, Nk=128, d=64, dtype="fp32", seed=1),
    2: Workload(2, "gpt_causal_prefill", B=4, H=16, Nq=2048, Nk=2048, d=128, dtype="bf16",
                causal=True, seed=2),
    3: Workload(3, "sliding_window_16k", B=1, H=16, Nq=16384, Nk=16384, d=64, dtype="bf16",
                causal=True, window_left=4096, window_right=0, seed=3),
    4: Workload(4, "paged_splitkv_decode", B=8, H=32, Nq=1, Nk=32768, d=128, dtype="bf16",
                causal=True, paged=True, page_size=256, pool_factor=1.2, num_splits=16, seed=4),
    5: Workload(5, "alibi_softcap_nq_ne_nk", B=2, H=8, Nq=512, Nk=4096, d=128, dtype="bf16",
                amp=2.0, causal=True, alibi=True, softcap=30.0, seed=5),
}


def gen_qkv(w: Workload):
    """Contiguous Q [B,Nq,H,d], K and V [B,Nk,H,d] in storage form."""
    q = gen_tensor(w.seed, TENSOR_Q, w.B, w.Nq, w.H, w.d, w.amp, w.dtype)
    k = gen_tensor(w.seed, TENSOR_K, w.B, w.Nk, w.H, w.d, w.amp, w.dtype)
    v = gen_tensor(w.seed, TENSOR_V, w.B, w.Nk, w.H, w.d, w.amp, w.dtype)
    return q, k, v


def gen_paged(w: Workload, poison_unused: bool = True, seqlens=None):
    """Q plus a paged K/V pool [pool_pages, page_size, H, d] and its block table.

    Every sequence holds pages for w.Nk keys. With `seqlens`, sequence b stores
    only its first seqlens[b] keys (the first seqlens[b] rows of the same
    slices). With poison_unused, every pool row that holds no stored key (pages
    no sequence references, and rows past a sequence's length) is NaN (bf16,
    float32 or the E4M3 NaN code), so a wrong gather or a read past a length
    shows up as NaN. For w.dtype "fp8" the pool holds E4M3 codes and Q is bf16.
    """
    # An E4M3 cache ("fp8") is read with bf16 queries.
    q = gen_tensor(w.seed, TENSOR_Q, w.B, w.Nq, w.H, w.d, w.amp,
                   "bf16" if w.dtype == "fp8" else w.dtype)
    bt = gen_block_table(w.table_seed, w.B, w.pages_per_seq, w.pool_pages)
    st = {"bf16": np.uint16, "fp8": np.uint8}.get(w.dtype, np.float32)
    shape = (w.pool_pages, w.page_size, w.H, w.d)
    nan = {"bf16": BF16_NAN_BITS, "fp8": E4M3_NAN_BITS}.get(w.dtype, np.float32("nan"))
    kc = np.full(shape, nan if poison_unused else 0, dtype=st)
    vc = np.full(shape, nan if poison_unused else 0, dtype=st)
    for b in range(w.B):
        n = w.Nk if seqlens is None else int(seqlens[b])
        for h in range(w.H):
            ks = gen_slice(w.seed, TENSOR_K, b, h, w.Nk, w.d, w.amp, w.dtype)[:n]
            vs = gen_slice(w.seed, TENSOR_V, b, h, w.Nk, w.d, w.amp, w.dtype)[:n]
            scatter_pages(kc, bt, b, h, ks, w.page_size)
            scatter_pages(vc, bt, b, h, vs, w.page_size)
    return q, kc, vc, bt


# --------------------------------------------------------------------------
# Packed variable-length batches
# --------------------------------------------------------------------------
def cu_seqlens(lengths) -> np.ndarray:
    """Cumulative offsets [0, l0, l0 + l1, ...] as int32."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def varlen_lengths(seed: int, batch: int, max_len: int, min_len: int = 1) -> np.ndarray:
    """Seeded sequence lengths, uniform in [min_len, max_len]."""
    rng = np.random.default_rng([int(seed), 7])
    return rng.integers(min_len, max_len + 1, size=batch).astype(np.int64)


def gen_varlen(seed: int, lens_q, lens_k, H: int, d: int, amp: float, dtype: str):
    """Packed Q [sum(lens_q), H, d], K and V [sum(lens_k), H, d] plus cu_seqlens_q/k.

    Sequence b's rows are the slices gen_slice(seed, tensor, b, h, len, d), so a
    sequence of a pack equals batch entry b of a batched tensor of that length.
    """
    cq, ck = cu_seqlens(lens_q), cu_seqlens(lens_k)
    st = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((int(cq[-1]), H, d), dtype=st)
    k = np.empty((int(ck[-1]), H, d), dtype=st)
    v = np.empty((int(ck[-1]), H, d), dtype=st)
    for b in range(len(lens_q)):
        for h in range(H):
            q[cq[b]:cq[b + 1], h] = gen_slice(seed, TENSOR_Q, b, h, int(lens_q[b]), d, amp, dtype)
            k[ck[b]:ck[b + 1], h] = gen_slice(seed, TENSOR_K, b, h, int(lens_k[b]), d, amp, dtype)
            v[ck[b]:ck[b + 1], h] = gen_slice(seed, TENSOR_V, b, h, int(lens_k[b]), d, amp, dtype)
    return q, k, v, cq, ck
