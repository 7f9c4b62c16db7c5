"""LDS pipeline hazard check: the forward kernels' multi-stage copy rings against a
single-buffered build of the same sources.

tests/hazard/libfa_serial_copies.so is built by build() from the same sources with
FA_SERIAL_COPIES: each K/V tile is copied into one buffer, waited for and fenced by
barriers on both sides, so no copy overlaps any compute. The arithmetic and its order
are unchanged, so every output must agree bit for bit with libfa.so; a copy that
overwrote a stage still being read, or a read of a stage not yet written, would show
up as a difference. Covered: the contiguous forward (whole key range, batched and
packed), its key splits, the paged multi-row pass with page-aligned tiles, with
per-wavefront slabs of 16-key pages and with rows gathered one by one, the FP8 forward (whole key range, key splits, and a paged
cache in whole tiles, in per-wavefront slabs and in row gathers) at both head sizes, and the
backward (the dK/dV kernels' query-block rings at both head sizes, including the two-role
exchange of P' at head_dim 128, and the dQ kernel's key-tile buffers), batched and packed.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import exact_tiled_attention_05_amd as fa
import workloads as W
from gpu_common import say, to_dev

pytestmark = pytest.mark.gpu

SERIAL = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hazard", "libfa_serial_copies.so")


@pytest.fixture(scope="module")
def serial_lib():
    if not os.path.exists(SERIAL):
        pytest.fail(f"{SERIAL} missing: run __graft_entry__.build()")
    return fa.declare(ctypes.CDLL(SERIAL))


def both(serial_lib, fn, *args, **kw):
    """fn (a binding call) through libfa.so, then through the serial build."""
    main = fn(*args, **kw)
    saved = fa._lib
    fa._lib = serial_lib
    try:
        ser = fn(*args, **kw)
    finally:
        fa._lib = saved
    torch.cuda.synchronize()
    return main, ser


def assert_same(a, b, what):
    a = a if isinstance(a, (tuple, list)) else (a,)
    b = b if isinstance(b, (tuple, list)) else (b,)
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x, y), f"{what}: output {i} differs (max |diff| " \
                                  f"{(x.float() - y.float()).abs().max().item():.3e})"


def qkv(seed, B, nq, nk, H, d, amp=1.0):
    return [to_dev(W.gen_tensor(seed, t, B, n, H, d, amp, "bf16"), "bf16")
            for t, n in ((W.TENSOR_Q, nq), (W.TENSOR_K, nk), (W.TENSOR_V, nk))]


FWD_CASES = [
    # (B, H, nq, nk, d, causal, wl, wr, alibi, cap)
    (4, 16, 2048, 2048, 128, True, -1, -1, False, 0.0),     # the causal prefill shape
    (1, 16, 16384, 16384, 64, True, 4096, 0, False, 0.0),   # the 16K window shape
    (2, 8, 512, 4096, 128, True, -1, -1, True, 30.0),       # ALiBi + softcap, Nq != Nk
    (1, 3, 300, 1000, 64, False, 77, 30, True, 0.0),
    (2, 2, 129, 65, 128, False, -1, -1, False, 12.0),
    (1, 2, 1000, 333, 128, True, -1, -1, False, 0.0),       # rows with no key
]


@pytest.mark.parametrize("case", FWD_CASES)
def test_contiguous_forward_matches_serial_copies(serial_lib, case):
    B, H, nq, nk, d, causal, wl, wr, alibi, cap = case
    say(f"hazard fa_fwd {case}")
    q, k, v = qkv(7000 + FWD_CASES.index(case), B, nq, nk, H, d, 2.0 if cap else 1.0)
    ts = torch.from_numpy(W.alibi_slopes(H)).cuda() if alibi else None
    m, s = both(serial_lib, fa.attention, q, k, v, 1.0 / np.sqrt(d), causal, wl, wr, ts, cap)
    assert_same(m, s, f"fa_fwd {case}")


def test_packed_forward_matches_serial_copies(serial_lib):
    lens = W.varlen_lengths(91, 8, 2048)
    say(f"hazard fa_fwd_varlen {lens.tolist()}")
    q, k, v, cq, ck = W.gen_varlen(12500, lens, lens, 16, 128, 1.0, "bf16")
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    tcq, tck = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    n = int(lens.max())
    m, s = both(serial_lib, fa.attention_varlen, tq, tk, tv, tcq, tck, n, n, 1.0 / np.sqrt(128),
                True)
    assert_same(m, s, "fa_fwd_varlen")


@pytest.mark.parametrize("d,splits,alibi,cap", [(128, 8, True, 30.0), (64, 5, False, 0.0)])
def test_key_splits_match_serial_copies(serial_lib, d, splits, alibi, cap):
    say(f"hazard fa_fwd_split d{d} S{splits}")
    q, k, v = qkv(7100 + d, 2, 512, 4096, 8, d, 2.0 if cap else 1.0)
    ts = torch.from_numpy(W.alibi_slopes(8)).cuda() if alibi else None
    m, s = both(serial_lib, fa.attention_split_partials, q, k, v, splits,
                softmax_scale=1.0 / np.sqrt(d), causal=True, alibi_slopes=ts, softcap=cap)
    assert_same(m, s, f"fa_fwd_split d{d}")


@pytest.mark.parametrize("page_size", [256, 16, 7])  # page tiles, 16-row slabs, row gathers
def test_paged_multirow_matches_serial_copies(serial_lib, page_size):
    say(f"hazard fa_fwd_splitkv multi-row, page {page_size}")
    w = W.Workload(0, "hazard_paged", B=2, H=4, Nq=300, Nk=3000, d=128, dtype="bf16",
                   causal=True, paged=True, page_size=page_size, pool_factor=1.2, num_splits=4,
                   seed=7200 + page_size)
    q, kc, vc, bt = W.gen_paged(w)
    tq, tk, tv = to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16")
    tbt = torch.from_numpy(bt).cuda()
    m, s = both(serial_lib, fa.attention_paged_splitkv, tq, tk, tv, tbt, w.Nk, w.num_splits,
                w.scale, causal=True)
    assert_same(m, s, f"fa_fwd_splitkv page {page_size}")


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_forward_matches_serial_copies(serial_lib, d):
    say(f"hazard fa_fwd_fp8 d{d}")
    B, H, nq, nk = 2, 8, 1000, 3000
    q8, k8, v8 = (torch.from_numpy(W.gen_tensor(7300 + d, t, B, n, H, d, 1.0, "fp8")).cuda()
                  for t, n in ((W.TENSOR_Q, nq), (W.TENSOR_K, nk), (W.TENSOR_V, nk)))
    ts = torch.from_numpy(W.alibi_slopes(H)).cuda()
    m, s = both(serial_lib, fa.attention_fp8, q8, k8, v8, 0.5, 1.0, 2.0, 1.0 / np.sqrt(d), True,
                -1, -1, ts, 20.0)
    assert_same(m, s, f"fa_fwd_fp8 d{d}")


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_split_matches_serial_copies(serial_lib, d):
    say(f"hazard fa_fwd_split_fp8 d{d}")
    B, H, nq, nk = 2, 4, 600, 3000
    q8, k8, v8 = (torch.from_numpy(W.gen_tensor(7400 + d, t, B, n, H, d, 1.0, "fp8")).cuda()
                  for t, n in ((W.TENSOR_Q, nq), (W.TENSOR_K, nk), (W.TENSOR_V, nk)))
    ts = torch.from_numpy(W.alibi_slopes(H)).cuda()
    m, s = both(serial_lib, fa.attention_split_partials_fp8, q8, k8, v8, 5, 0.5, 1.0, 2.0,
                1.0 / np.sqrt(d), True, -1, -1, ts, 20.0)
    assert_same(m, s, f"fa_fwd_split_fp8 d{d}")


@pytest.mark.parametrize("d,page_size", [(128, 256), (64, 384), (128, 64), (128, 16), (64, 100)])
def test_fp8_paged_matches_serial_copies(serial_lib, d, page_size):
    say(f"hazard fa_fwd_paged_fp8 d{d} page {page_size}")
    w = W.Workload(0, "hazard_fp8_paged", B=2, H=4, Nq=300, Nk=3000, d=d, dtype="fp8",
                   causal=True, paged=True, page_size=page_size, pool_factor=1.2, num_splits=3,
                   seed=7500 + d)
    _, kc, vc, bt = W.gen_paged(w, seqlens=[3000, 1700])
    q8 = torch.from_numpy(W.gen_tensor(7500 + d, W.TENSOR_Q, 2, 300, 4, d, 1.0, "fp8")).cuda()
    tk, tv = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
    tbt = torch.from_numpy(bt).cuda()
    tsl = torch.tensor([3000, 1700], dtype=torch.int32).cuda()
    ts = torch.from_numpy(W.alibi_slopes(4)).cuda()
    m, s = both(serial_lib, fa.attention_paged_fp8, q8, tk, tv, tbt, w.Nk, 3, 0.5, 1.0, 2.0,
                1.0 / np.sqrt(d), True, -1, -1, ts, 20.0, cache_seqlens=tsl)
    assert_same(m, s, f"fa_fwd_paged_fp8 d{d}")



BWD_CASES = [
    # (B, H, nq, nk, d, causal, wl, wr, alibi, cap)
    (4, 16, 2048, 2048, 128, True, -1, -1, False, 0.0),     # the causal prefill shape
    (2, 8, 512, 4096, 128, True, -1, -1, True, 30.0),       # ALiBi + softcap, Nq != Nk
    (2, 4, 1000, 333, 128, True, -1, -1, False, 0.0),       # rows with no key
    (1, 3, 300, 1000, 128, False, 77, 30, True, 0.0),       # a window on both sides
    (2, 2, 129, 65, 128, False, -1, -1, False, 12.0),       # ragged blocks
    (2, 8, 1024, 1024, 64, True, -1, -1, False, 0.0),
    (1, 3, 300, 1000, 64, False, 77, 30, True, 10.0),
    (2, 2, 1000, 333, 64, True, -1, -1, False, 0.0),
]


@pytest.mark.parametrize("case", BWD_CASES)
def test_backward_matches_serial_copies(serial_lib, case):
    B, H, nq, nk, d, causal, wl, wr, alibi, cap = case
    say(f"hazard fa_bwd {case}")
    seed = 7600 + BWD_CASES.index(case)
    q, k, v = qkv(seed, B, nq, nk, H, d, 2.0 if cap else 1.0)
    dout = to_dev(W.gen_tensor(seed, W.TENSOR_V, B, nq, H, d, 1.0, "bf16"), "bf16")
    ts = torch.from_numpy(W.alibi_slopes(H)).cuda() if alibi else None
    o, lse = fa.attention(q, k, v, 1.0 / np.sqrt(d), causal, wl, wr, ts, cap)
    m, s = both(serial_lib, fa.attention_backward, q, k, v, o, lse, dout, 1.0 / np.sqrt(d),
                causal, wl, wr, ts, cap)
    assert_same(m, s, f"fa_bwd {case}")


@pytest.mark.parametrize("d", [128, 64])
def test_packed_backward_matches_serial_copies(serial_lib, d):
    lens = W.varlen_lengths(93, 6, 1500)
    say(f"hazard fa_bwd_varlen d{d} {lens.tolist()}")
    q, k, v, cq, ck = W.gen_varlen(12600 + d, lens, lens, 4, d, 1.0, "bf16")
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    tcq, tck = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    n = int(lens.max())
    o, lse = fa.attention_varlen(tq, tk, tv, tcq, tck, n, n, 1.0 / np.sqrt(d), True)
    dout = torch.randn(tq.shape, generator=torch.Generator().manual_seed(d)).bfloat16().cuda()
    m, s = both(serial_lib, fa.attention_varlen_backward, tq, tk, tv, o, lse, dout, tcq, tck, n,
                n, 1.0 / np.sqrt(d), True)
    assert_same(m, s, f"fa_bwd_varlen d{d}")
