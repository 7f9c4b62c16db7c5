"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Tolerances: fp32 inputs max|dO| <= 1e-5; bf16 inputs max|dO| <= 1e-2 and
mean|dO| <= 1e-3 (fp32 O); |dLSE| <= 1e-3; rows with no visible key must be
O = 0, LSE = -inf exactly. Gathers through the block table must be bit-exact.
"""
import itertools

import numpy as np
import pytest
import torch

import exact_tiled_attention_05_amd as fa
import oracle as O
import workloads as W
from gpu_common import TOL_LSE, check, oracle_map, qkv_case, say, to_dev

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, dtype, scale, causal, wl, wr, slopes, cap, out_dtype=torch.float32):
    B, nq, H, d = q.shape
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    ts = None if slopes is None else torch.from_numpy(np.asarray(slopes, np.float32)).cuda()
    o, lse = fa.attention(tq, tk, tv, scale, causal, wl, wr, ts, cap, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def oracle_fwd(q, k, v, dtype, scale, causal, wl, wr, slopes, cap, rows=None, bh=None):
    return O.attention_ref(W.to_float(q, dtype), W.to_float(k, dtype), W.to_float(v, dtype),
                           scale, causal, wl, wr, slopes, cap, rows=rows, bh=bh)


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------
def test_cfg1_tiny_fp32():
    w = W.WORKLOADS[1]
    say(f"cfg1 {w}")
    q, k, v = W.gen_qkv(w)
    o, lse = run_fwd(q, k, v, w.dtype, w.scale, w.causal, -1, -1, None, 0.0)
    ro, rl = oracle_fwd(q, k, v, w.dtype, w.scale, w.causal, -1, -1, None, 0.0)
    print(check(o, lse, ro, rl, "fp32", "cfg1"))


def test_cfg2_causal_prefill_full():
    w = W.WORKLOADS[2]
    say(f"cfg2 {w}")
    q, k, v = W.gen_qkv(w)
    o, lse = run_fwd(q, k, v, w.dtype, w.scale, True, -1, -1, None, 0.0)
    ro, rl = oracle_fwd(q, k, v, w.dtype, w.scale, True, -1, -1, None, 0.0)
    print(check(o, lse, ro, rl, "bf16", "cfg2"))


def test_cfg3_sliding_window_full():
    """Every row of every head (16 x 16384 rows), each against the oracle over the keys
    its window lets it see."""
    w = W.WORKLOADS[3]
    say(f"cfg3 {w}")
    q, k, v = W.gen_qkv(w)
    o, lse = run_fwd(q, k, v, w.dtype, w.scale, True, w.window_left, w.window_right, None, 0.0)
    qf, kf, vf = (W.to_float(x, w.dtype) for x in (q, k, v))
    del q, k, v
    say("cfg3: oracle, every row of every head")
    res = oracle_map(lambda h: O.attention_bh(qf[0, :, h], kf[0, :, h], vf[0, :, h],
                                              np.arange(w.Nq), w.Nq, w.scale, True,
                                              w.window_left, w.window_right), range(w.H))
    ro = np.stack([r[0] for r in res], axis=1)[None]
    rl = np.stack([r[1] for r in res])[None]
    print(check(o, lse, ro, rl, "bf16", "cfg3"))


def test_cfg5_alibi_softcap_full():
    w = W.WORKLOADS[5]
    say(f"cfg5 {w}")
    q, k, v = W.gen_qkv(w)
    slopes = w.slopes()
    o, lse = run_fwd(q, k, v, w.dtype, w.scale, True, -1, -1, slopes, w.softcap)
    ro, rl = oracle_fwd(q, k, v, w.dtype, w.scale, True, -1, -1, slopes, w.softcap)
    print(check(o, lse, ro, rl, "bf16", "cfg5"))


def test_cfg4_paged_decode_full_size():
    """The full decode workload: every (b, h) pair, combined and per split, against the
    oracle over keys regenerated from their seeded slices (not read back from the
    pool, so the scatter into pages is checked too)."""
    w = W.WORKLOADS[4]
    say(f"cfg4 {w}: generating inputs")
    q, kc, vc, bt = W.gen_paged(w)
    tq, tk, tv = to_dev(q, w.dtype), to_dev(kc, w.dtype), to_dev(vc, w.dtype)
    del kc, vc
    tbt = torch.from_numpy(bt).cuda()
    say("cfg4: split pass + combine")
    o_part, lse_part = fa.attention_paged_splitkv(tq, tk, tv, tbt, w.Nk, w.num_splits,
                                                  w.scale, causal=True)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    op, lp = o_part.cpu().numpy(), lse_part.cpu().numpy()
    assert not np.isnan(o).any() and not np.isnan(op).any()   # poisoned pages never read
    qf = W.to_float(q, w.dtype)
    splits = O.split_bounds(w.Nk, w.num_splits, w.page_size)

    def oracle_pair(bh):
        b, h = bh
        kb = W.to_float(W.gen_slice(w.seed, W.TENSOR_K, b, h, w.Nk, w.d, w.amp, w.dtype), w.dtype)
        vb = W.to_float(W.gen_slice(w.seed, W.TENSOR_V, b, h, w.Nk, w.d, w.amp, w.dtype), w.dtype)
        rows = np.arange(w.Nq)
        full = O.attention_bh(qf[b, :, h, :], kb, vb, rows, w.Nq, w.scale, True)
        parts = [O.attention_bh(qf[b, :, h, :], kb, vb, rows, w.Nq, w.scale, True, key_lo=lo,
                                key_hi=hi) for lo, hi in splits]
        return full, parts

    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    say(f"cfg4: oracle, all {len(pairs)} (b, h) pairs and their {len(splits)} splits")
    for (b, h), ((ro, rl), parts) in zip(pairs, oracle_map(oracle_pair, pairs)):
        check(o[b, :, h, :], lse[b, h, :], ro, rl, "bf16", f"cfg4 b{b} h{h}")
        for s, (so, sl) in enumerate(parts):
            check(op[s, b, h], lp[s, b, h], so, sl, "bf16", f"cfg4 split {s} b{b} h{h}")


def test_cfg4_gather_bit_exact_vs_identity_table():
    """Permuted pages + table == the same keys laid out contiguously (identity table)."""
    w = W.WORKLOADS[4]
    say("cfg4 gather: generating")
    q, kc, vc, bt = W.gen_paged(w)
    tq, tk, tv = to_dev(q, w.dtype), to_dev(kc, w.dtype), to_dev(vc, w.dtype)
    del kc, vc
    tbt = torch.from_numpy(bt).cuda()
    o1, l1 = fa.attention_paged_splitkv(tq, tk, tv, tbt, w.Nk, w.num_splits, w.scale, causal=True)
    torch.cuda.synchronize()
    o1, l1 = o1.cpu(), l1.cpu()
    del tk, tv
    k = W.gen_tensor(w.seed, W.TENSOR_K, w.B, w.Nk, w.H, w.d, w.amp, w.dtype)
    v = W.gen_tensor(w.seed, W.TENSOR_V, w.B, w.Nk, w.H, w.d, w.amp, w.dtype)
    pps = w.pages_per_seq
    ki = to_dev(k.reshape(w.B * pps, w.page_size, w.H, w.d), w.dtype)
    vi = to_dev(v.reshape(w.B * pps, w.page_size, w.H, w.d), w.dtype)
    del k, v
    bt_id = torch.arange(w.B * pps, dtype=torch.int32).reshape(w.B, pps).cuda()
    say("cfg4 gather: identity run")
    o2, l2 = fa.attention_paged_splitkv(tq, ki, vi, bt_id, w.Nk, w.num_splits, w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.cpu()) and torch.equal(l1, l2.cpu())


# --------------------------------------------------------------------------
# Brute-force sweep of small and ragged shapes
# --------------------------------------------------------------------------
SIZES = [1, 2, 3, 17, 64, 127, 128, 129, 255]


def mask_variants(nq, nk):
    return [(False, -1, -1), (True, -1, -1), (True, 5, -1), (False, 7, 3), (False, -1, 0),
            (True, max(0, nk // 3), 0)]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64), ("fp32", 128)])
def test_sweep_small_shapes(dtype, d):
    case = 0
    for nq, nk in itertools.product(SIZES, SIZES):
        for (causal, wl, wr) in mask_variants(nq, nk):
            alibi = case % 3 == 1
            cap = 7.5 if case % 4 == 2 else 0.0
            case += 1
            if (nq * nk) % 5 not in (0, 1) and dtype == "fp32":
                continue  # fp32 sweep on a deterministic subset (it is the slow kernel)
            B, H = 1 + case % 2, 2
            amp = 2.0 if cap else 1.0
            q, k, v = qkv_case(1000 + case, B, nq, nk, H, d, dtype, amp)
            slopes = W.alibi_slopes(H) if alibi else None
            scale = 1.0 / np.sqrt(d)
            what = f"{dtype} d{d} nq{nq} nk{nk} causal{causal} wl{wl} wr{wr} alibi{alibi} cap{cap}"
            say(what)
            o, lse = run_fwd(q, k, v, dtype, scale, causal, wl, wr, slopes, cap)
            ro, rl = oracle_fwd(q, k, v, dtype, scale, causal, wl, wr, slopes, cap)
            check(o, lse, ro, rl, dtype, what)


def test_bf16_output_is_rounded_fp32_output():
    q, k, v = qkv_case(77, 2, 200, 300, 4, 128, "bf16")
    o32, l32 = run_fwd(q, k, v, "bf16", 0.09, True, -1, -1, None, 0.0)
    o16, l16 = run_fwd(q, k, v, "bf16", 0.09, True, -1, -1, None, 0.0, out_dtype=torch.bfloat16)
    want = torch.from_numpy(o32).to(torch.bfloat16).float().numpy()
    bad = np.argwhere(o16 != want)
    assert len(bad) == 0, (f"{len(bad)} of {o16.size} bf16 outputs differ from the rounded fp32 "
                           f"output; first {bad[:4].tolist()}: {o16[tuple(bad[0])]} vs "
                           f"{want[tuple(bad[0])]} (fp32 {o32[tuple(bad[0])]!r})")
    badl = np.argwhere(l16 != l32)
    assert len(badl) == 0, f"{len(badl)} LSE values differ; first {badl[:4].tolist()}"


def test_determinism_bitwise():
    q, k, v = qkv_case(78, 2, 300, 700, 4, 128, "bf16")
    a = run_fwd(q, k, v, "bf16", 0.088, True, 100, 0, W.alibi_slopes(4), 20.0)
    b = run_fwd(q, k, v, "bf16", 0.088, True, 100, 0, W.alibi_slopes(4), 20.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_rows_exact():
    """Nq > Nk under causal: the first Nq - Nk rows see no key."""
    for dtype, d in [("bf16", 128), ("fp32", 64)]:
        q, k, v = qkv_case(79, 1, 300, 40, 2, d, dtype)
        o, lse = run_fwd(q, k, v, dtype, 0.1, True, -1, -1, None, 0.0)
        assert np.all(o[:, :260] == 0.0) and np.all(lse[:, :, :260] == -np.inf)
        ro, rl = oracle_fwd(q, k, v, dtype, 0.1, True, -1, -1, None, 0.0)
        check(o, lse, ro, rl, dtype, f"empty rows {dtype}")


# --------------------------------------------------------------------------
# Split-KV over paged caches: small cases
# --------------------------------------------------------------------------
SPLIT_CASES = [
    # (dtype, d, B, H, nq, nk, page_size, num_splits, causal, wl, wr, alibi, cap)
    ("bf16", 128, 2, 3, 1, 1000, 64, 4, True, -1, -1, False, 0.0),
    ("bf16", 128, 3, 2, 1, 777, 16, 16, True, -1, -1, True, 0.0),
    ("bf16", 64, 2, 2, 5, 300, 7, 3, True, 50, 0, False, 10.0),
    ("bf16", 128, 1, 4, 130, 400, 256, 2, True, -1, -1, True, 30.0),
    ("bf16", 64, 2, 1, 3, 50, 256, 8, False, -1, -1, False, 0.0),
    ("bf16", 128, 2, 2, 1, 4096, 256, 16, True, 1000, 0, False, 0.0),
    ("fp32", 64, 2, 2, 1, 500, 32, 5, True, -1, -1, False, 0.0),
    ("fp32", 128, 1, 3, 40, 200, 16, 3, True, -1, -1, True, 5.0),
]


@pytest.mark.parametrize("case", SPLIT_CASES)
def test_splitkv_paged_small(case):
    dtype, d, B, H, nq, nk, ps, S, causal, wl, wr, alibi, cap = case
    say(f"split {case}")
    w = W.Workload(0, "split", B=B, H=H, Nq=nq, Nk=nk, d=d, dtype=dtype, causal=causal,
                   paged=True, page_size=ps, pool_factor=1.5, num_splits=S, seed=hash(case) % 1000)
    q, kc, vc, bt = W.gen_paged(w)
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    scale = 1.0 / np.sqrt(d)
    o_part, lse_part = fa.attention_paged_splitkv(
        to_dev(q, dtype), to_dev(kc, dtype), to_dev(vc, dtype), torch.from_numpy(bt).cuda(), nk, S,
        scale, causal, wl, wr, ts, cap)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    qf = W.to_float(q, dtype)
    k = np.stack([O.paged_gather_ref(W.to_float(kc, dtype), bt, b, nk) for b in range(B)])
    v = np.stack([O.paged_gather_ref(W.to_float(vc, dtype), bt, b, nk) for b in range(B)])
    rop, rlp = O.splitkv_ref(qf, k, v, S, ps, scale, causal, wl, wr, slopes, cap)
    check(o_part.cpu().numpy(), lse_part.cpu().numpy(), rop, rlp, dtype, "partials")
    ro, rl = O.attention_ref(qf, k, v, scale, causal, wl, wr, slopes, cap)
    check(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, dtype, "combined")


def test_paged_gather_beyond_the_lds_page_table():
    """Row gathers whose workgroup spans more pages than the kernel stages in LDS read the
    block table directly: 64 bf16 rows over 30000 keys in 7-key pages (4286 pages; the
    bf16 multi-row pass stages 4096 ids at head_dim 128) and 64 E4M3 rows over 16000 keys
    (2286 pages; the FP8 pass stages 2048), one split each; the pools' unused rows are
    NaN."""
    d, H, nq, ps = 128, 2, 64, 7
    scale = 1.0 / np.sqrt(d)
    slopes = W.alibi_slopes(H)
    ts = torch.from_numpy(slopes).cuda()
    say("paged gather past the LDS page table: bf16, 30000 keys in 7-key pages")
    nk = 30000
    w = W.Workload(0, "gather_long", B=1, H=H, Nq=nq, Nk=nk, d=d, dtype="bf16", causal=True,
                   paged=True, page_size=ps, pool_factor=1.2, num_splits=1, seed=4400)
    q, kc, vc, bt = W.gen_paged(w)
    assert w.pages_per_seq > 4096
    o_part, lse_part = fa.attention_paged_splitkv(
        to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16"), torch.from_numpy(bt).cuda(), nk,
        1, scale, True, -1, -1, ts, 0.0)
    torch.cuda.synchronize()
    k = O.paged_gather_ref(W.to_float(kc, "bf16"), bt, 0, nk)[None]
    v = O.paged_gather_ref(W.to_float(vc, "bf16"), bt, 0, nk)[None]
    rop, rlp = O.splitkv_ref(W.to_float(q, "bf16"), k, v, 1, ps, scale, True, alibi_slopes=slopes)
    check(o_part.cpu().numpy(), lse_part.cpu().numpy(), rop, rlp, "bf16", "bf16 partials")

    say("paged gather past the LDS page table: E4M3, 16000 keys in 7-key pages")
    nk = 16000
    w = W.Workload(0, "gather_long_fp8", B=1, H=H, Nq=nq, Nk=nk, d=d, dtype="fp8", causal=True,
                   paged=True, page_size=ps, pool_factor=1.2, num_splits=1, seed=4401)
    _, kc, vc, bt = W.gen_paged(w)
    assert w.pages_per_seq > 2048
    q8 = W.gen_tensor(4401, W.TENSOR_Q, 1, nq, H, d, 1.0, "fp8")
    o_part, lse_part = fa.attention_paged_fp8(to_dev_fp8(q8), to_dev_fp8(kc), to_dev_fp8(vc),
                                              torch.from_numpy(bt).cuda(), nk, 1, 1.0, 1.0, 1.0,
                                              scale, True, -1, -1, ts, 0.0)
    torch.cuda.synchronize()
    k8 = O.paged_gather_ref(kc, bt, 0, nk)[None]
    v8 = O.paged_gather_ref(vc, bt, 0, nk)[None]
    check_fp8_partials(o_part.cpu().numpy(), lse_part.cpu().numpy(), q8, k8, v8, (1.0, 1.0, 1.0),
                       scale, True, -1, -1, slopes, 0.0, 1, "fp8 partials", align=ps)


# --------------------------------------------------------------------------
# Split-KV over contiguous K/V (fa_fwd_split): chunks of whole 64-key tiles
# --------------------------------------------------------------------------
CONTIG_SPLIT_CASES = [
    # (d, B, H, nq, nk, num_splits, causal, wl, wr, alibi, cap)
    (128, 2, 3, 70, 1000, 4, True, -1, -1, False, 0.0),
    (64, 1, 4, 200, 333, 3, False, -1, -1, True, 10.0),
    (128, 1, 2, 130, 130, 8, True, 40, 0, False, 0.0),
    (64, 2, 2, 300, 90, 2, True, -1, -1, False, 0.0),     # Nq > Nk: leading rows see no key
    (128, 1, 3, 1, 2000, 7, True, -1, -1, True, 30.0),
    (128, 2, 2, 64, 64, 16, False, -1, -1, False, 0.0),   # more splits than key tiles
]


@pytest.mark.parametrize("case", CONTIG_SPLIT_CASES)
def test_split_contiguous_small(case):
    d, B, H, nq, nk, S, causal, wl, wr, alibi, cap = case
    say(f"contig split {case}")
    q, k, v = qkv_case(4000 + CONTIG_SPLIT_CASES.index(case), B, nq, nk, H, d, "bf16",
                       2.0 if cap else 1.0)
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(np.asarray(slopes, np.float32)).cuda()
    scale = 1.0 / np.sqrt(d)
    o_part, lse_part = fa.attention_split_partials(to_dev(q, "bf16"), to_dev(k, "bf16"),
                                                   to_dev(v, "bf16"), S, scale, causal, wl, wr,
                                                   ts, cap)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    qf, kf, vf = (W.to_float(x, "bf16") for x in (q, k, v))
    assert fa.fa_split_chunk_len(nk, S, 64) == -(-(-(-nk // S)) // 64) * 64
    rop, rlp = O.splitkv_ref(qf, kf, vf, S, 64, scale, causal, wl, wr, slopes, cap)
    check(o_part.cpu().numpy(), lse_part.cpu().numpy(), rop, rlp, "bf16", "partials")
    ro, rl = O.attention_ref(qf, kf, vf, scale, causal, wl, wr, slopes, cap)
    check(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", "combined")


def test_cfg5_split_full():
    """ALiBi + softcap, Nq=512 over Nk=4096: 64 query tiles leave most CUs idle, so the
    key range is split 8 ways and merged by the combine kernel."""
    w = W.WORKLOADS[5]
    say(f"cfg5 split {w}")
    q, k, v = W.gen_qkv(w)
    slopes = w.slopes()
    ts = torch.from_numpy(np.asarray(slopes, np.float32)).cuda()
    o, lse = fa.attention_split(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), 8,
                                softmax_scale=w.scale, causal=True, alibi_slopes=ts,
                                softcap=w.softcap)
    torch.cuda.synchronize()
    ro, rl = oracle_fwd(q, k, v, w.dtype, w.scale, True, -1, -1, slopes, w.softcap)
    print(check(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, "bf16", "cfg5 split"))


def test_combine_matches_oracle_on_random_partials():
    rng = np.random.default_rng(5)
    S, B, H, nq, d = 6, 2, 3, 5, 128
    op = rng.standard_normal((S, B, H, nq, d)).astype(np.float32)
    lp = (rng.standard_normal((S, B, H, nq)) * 3).astype(np.float32)
    lp[1] = -np.inf                       # one empty split everywhere
    lp[:, 0, 0, 0] = -np.inf              # one row with every split empty
    o, lse = fa.combine(torch.from_numpy(op).cuda(), torch.from_numpy(lp).cuda())
    torch.cuda.synchronize()
    ro, rl = O.combine_ref(op, lp)        # [B, H, nq, d]
    check(o.cpu().numpy().transpose(0, 2, 1, 3), lse.cpu().numpy(), ro, rl, "fp32", "combine")




def _unaligned(t):
    """A copy of t whose data starts 4 bytes past a 16-byte boundary."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    u = buf[1:].view(t.shape)
    u.copy_(t)
    return u


@pytest.mark.parametrize("S,d", [(1, 128), (6, 64), (8, 128), (16, 128), (16, 64), (17, 64),
                                 (17, 128), (32, 128), (33, 128), (70, 64)])
def test_combine_forms(S, d):
    """Both combine forms (16-byte segments for up to d/4 splits on aligned buffers, one
    row per wavefront otherwise) against the oracle, on rows with some empty splits and
    rows with every split empty; in fp32 the two forms agree to within a few roundings,
    and each form's bf16 output is its fp32 output rounded to nearest even."""
    say(f"combine forms S={S} d={d}")
    rng = np.random.default_rng(1000 + 7 * S + d)
    B, H, nq = 2, 5, 37                   # 370 rows: a partial last workgroup in both forms
    op = rng.standard_normal((S, B, H, nq, d)).astype(np.float32)
    lp = (rng.standard_normal((S, B, H, nq)) * 4).astype(np.float32)
    lp[rng.random((S, B, H, nq)) < 0.2] = -np.inf
    lp[:, 1, 2, :5] = -np.inf              # rows with every split empty
    top = torch.from_numpy(op).cuda()
    tlp = torch.from_numpy(lp).cuda()
    ro, rl = O.combine_ref(op, lp)        # [B, H, nq, d]

    def run(aligned, out_dtype):
        o = torch.zeros((B, nq, H, d), dtype=out_dtype, device="cuda")
        if not aligned:
            o = _unaligned(o)
        lse = torch.empty((B, H, nq), dtype=torch.float32, device="cuda")
        fa._check(fa.fa_splitkv_combine(top if aligned else _unaligned(top), tlp, S, B, H, nq,
                                        d, o, lse, None), "fa_splitkv_combine")
        torch.cuda.synchronize()
        return o.contiguous(), lse

    res = {}
    for aligned in (True, False):
        o32, lse32 = run(aligned, torch.float32)
        o16, lse16 = run(aligned, torch.bfloat16)
        on = o32.cpu().numpy().transpose(0, 2, 1, 3)
        check(on, lse32.cpu().numpy(), ro, rl, "fp32", f"combine aligned={aligned}")
        assert np.all(on[1, 2, :5] == 0) and np.all(np.isneginf(lse32.cpu().numpy()[1, 2, :5]))
        assert torch.equal(o16.view(torch.int16), o32.bfloat16().view(torch.int16))
        assert torch.equal(lse16, lse32)
        res[aligned] = (o32, lse32)
    # The forms round the exponent arguments differently (one rounds lse*log2(e)
    # before subtracting the maximum, the other fuses the two), nothing else.
    (oa, la), (ou, lu) = res[True], res[False]
    assert torch.allclose(oa, ou, rtol=1e-5, atol=1e-6)
    fin = torch.isfinite(la)
    assert torch.equal(fin, torch.isfinite(lu))
    assert torch.allclose(la[fin], lu[fin], rtol=1e-6, atol=1e-6)


# --------------------------------------------------------------------------
# Variable sequence lengths: packed batches (fa_fwd_varlen)
# --------------------------------------------------------------------------
VARLEN_CASES = [
    # (dtype, d, H, [(nq, nk), ...], causal, wl, wr, alibi, cap)
    ("bf16", 128, 2, [(1, 1), (17, 300), (128, 128), (129, 64), (300, 1000), (0, 5), (7, 0),
                      (255, 257)], True, -1, -1, False, 0.0),
    ("bf16", 64, 3, [(64, 64), (130, 500), (1, 700), (200, 3), (33, 33)], True, 60, 0, True, 0.0),
    ("bf16", 128, 2, [(100, 100), (250, 140), (3, 400)], False, -1, -1, True, 20.0),
    ("bf16", 64, 2, [(129, 129), (0, 0), (90, 2000)], False, 30, 30, False, 8.0),
    ("fp32", 64, 2, [(1, 1), (33, 100), (70, 40), (0, 3), (5, 0)], True, -1, -1, False, 0.0),
    ("fp32", 128, 2, [(40, 90), (64, 64)], True, 20, 0, True, 5.0),
]


def run_varlen(q, k, v, cq, ck, dtype, maxq, maxk, scale, causal, wl, wr, slopes, cap,
               out_dtype=torch.float32):
    ts = None if slopes is None else torch.from_numpy(np.asarray(slopes, np.float32)).cuda()
    o, lse = fa.attention_varlen(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype),
                                 torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), maxq,
                                 maxk, scale, causal, wl, wr, ts, cap, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", VARLEN_CASES)
def test_varlen_packed_small(case):
    dtype, d, H, lens, causal, wl, wr, alibi, cap = case
    say(f"varlen {case}")
    lq, lk = [a for a, _ in lens], [b for _, b in lens]
    q, k, v, cq, ck = W.gen_varlen(5000 + VARLEN_CASES.index(case), lq, lk, H, d,
                                   2.0 if cap else 1.0, dtype)
    slopes = W.alibi_slopes(H) if alibi else None
    scale = 1.0 / np.sqrt(d)
    o, lse = run_varlen(q, k, v, cq, ck, dtype, max(lq), max(lk), scale, causal, wl, wr,
                        slopes, cap)
    ro, rl = O.attention_varlen_ref(W.to_float(q, dtype), W.to_float(k, dtype),
                                    W.to_float(v, dtype), cq, ck, scale, causal, wl, wr, slopes,
                                    cap)
    check(o, lse, ro, rl, dtype, f"varlen {case}")


def test_varlen_equal_lengths_bitwise_equals_batched():
    """A pack of equal-length sequences is the batched problem: the same kernel
    computes the same tiles, so O and LSE match fa_fwd bit for bit."""
    B, nq, nk, H, d = 3, 200, 333, 4, 128
    q, k, v = qkv_case(90, B, nq, nk, H, d, "bf16")
    ob, lb = run_fwd(q, k, v, "bf16", 0.09, True, 100, 0, W.alibi_slopes(H), 0.0)
    cq, ck = W.cu_seqlens([nq] * B), W.cu_seqlens([nk] * B)
    ov, lv = run_varlen(q.reshape(B * nq, H, d), k.reshape(B * nk, H, d),
                        v.reshape(B * nk, H, d), cq, ck, "bf16", nq, nk, 0.09, True, 100, 0,
                        W.alibi_slopes(H), 0.0)
    assert np.array_equal(ov, ob.reshape(B * nq, H, d))
    assert np.array_equal(lv, lb.transpose(1, 0, 2).reshape(H, B * nq))


def test_varlen_mixed_lengths_sampled_heads():
    """Eight causal sequences of seeded lengths up to 2048 at the prefill head
    shape (16 heads of 128): every row of two heads against the oracle."""
    H, d = 16, 128
    lens = W.varlen_lengths(91, 8, 2048)
    say(f"varlen mixed lengths {lens.tolist()}")
    q, k, v, cq, ck = W.gen_varlen(91, lens, lens, H, d, 1.0, "bf16")
    o, lse = run_varlen(q, k, v, cq, ck, "bf16", int(lens.max()), int(lens.max()),
                        1.0 / np.sqrt(d), True, -1, -1, None, 0.0)
    heads = [0, 11]
    ro, rl = O.attention_varlen_ref(W.to_float(q, "bf16"), W.to_float(k, "bf16"),
                                    W.to_float(v, "bf16"), cq, ck, 1.0 / np.sqrt(d), True,
                                    heads=heads)
    check(o[:, heads], lse[heads], ro[:, heads], rl[heads], "bf16", "varlen mixed")
    assert not np.isnan(o).any() and not np.isnan(lse).any()


# --------------------------------------------------------------------------
# Per-sequence cache lengths in the split pass (fa_fwd_splitkv_seqlens)
# --------------------------------------------------------------------------
SEQLENS_CASES = [
    # (dtype, d, H, nq, max_k, page_size, num_splits, seqlens, causal, wl, wr, alibi, cap)
    ("bf16", 128, 2, 1, 1000, 64, 4, [1000, 0, 1, 513, 64, 999], True, -1, -1, False, 0.0),
    ("bf16", 64, 3, 1, 777, 16, 16, [777, 5, 300, 0], True, 100, 0, True, 0.0),
    ("bf16", 128, 2, 1, 4096, 256, 16, [4096, 2047, 2048, 1, 3000], True, -1, -1, True, 30.0),
    ("bf16", 128, 2, 5, 300, 7, 3, [300, 4, 0, 150], True, 50, 0, False, 10.0),
    ("bf16", 64, 2, 130, 400, 64, 2, [400, 100, 129, 0], True, -1, -1, True, 0.0),
    ("bf16", 128, 1, 40, 256, 256, 4, [256, 17, 39, 40, 41], False, -1, -1, False, 0.0),
    ("fp32", 64, 2, 1, 500, 32, 5, [500, 0, 77], True, -1, -1, False, 0.0),
    ("fp32", 128, 2, 20, 200, 16, 3, [200, 10, 25], True, -1, -1, True, 5.0),
]


@pytest.mark.parametrize("case", SEQLENS_CASES)
def test_splitkv_seqlens_small(case):
    dtype, d, H, nq, nk, ps, S, seqlens, causal, wl, wr, alibi, cap = case
    say(f"split seqlens {case}")
    B = len(seqlens)
    w = W.Workload(0, "split_seqlens", B=B, H=H, Nq=nq, Nk=nk, d=d, dtype=dtype, causal=causal,
                   paged=True, page_size=ps, pool_factor=1.3, num_splits=S,
                   seed=6000 + SEQLENS_CASES.index(case))
    q, kc, vc, bt = W.gen_paged(w, seqlens=seqlens)   # every row past a length is NaN
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    scale = 1.0 / np.sqrt(d)
    tsl = torch.tensor(seqlens, dtype=torch.int32).cuda()
    o_part, lse_part = fa.attention_paged_splitkv(
        to_dev(q, dtype), to_dev(kc, dtype), to_dev(vc, dtype), torch.from_numpy(bt).cuda(), nk, S,
        scale, causal, wl, wr, ts, cap, cache_seqlens=tsl)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    qf = W.to_float(q, dtype)
    k = np.zeros((B, nk, H, d))
    v = np.zeros((B, nk, H, d))
    for b, n in enumerate(seqlens):
        k[b, :n] = O.paged_gather_ref(W.to_float(kc, dtype), bt, b, n)
        v[b, :n] = O.paged_gather_ref(W.to_float(vc, dtype), bt, b, n)
    rop, rlp = O.splitkv_ref(qf, k, v, S, ps, scale, causal, wl, wr, slopes, cap,
                             seqlens_k=seqlens)
    check(o_part.cpu().numpy(), lse_part.cpu().numpy(), rop, rlp, dtype, "partials")
    ro, rl = O.combine_ref(rop, rlp)
    check(o.cpu().numpy().transpose(0, 2, 1, 3), lse.cpu().numpy(), ro, rl, dtype, "combined")


def test_splitkv_seqlens_decode_full_size():
    """The paged decode shape (8 x 32 heads, 32768-key capacity, 256-key pages,
    16 splits) with per-sequence lengths from 0 to the capacity; every row past a
    length is NaN. Sampled (b, h) pairs against the oracle."""
    w = W.WORKLOADS[4]
    seqlens = [32768, 1, 0, 20000, 256, 255, 31000, 12345]
    say(f"cfg4 seqlens {seqlens}: generating inputs")
    q, kc, vc, bt = W.gen_paged(w, seqlens=seqlens)
    tq, tk, tv = to_dev(q, w.dtype), to_dev(kc, w.dtype), to_dev(vc, w.dtype)
    del kc, vc
    tbt = torch.from_numpy(bt).cuda()
    tsl = torch.tensor(seqlens, dtype=torch.int32).cuda()
    o, lse = fa.decode_paged(tq, tk, tv, tbt, w.Nk, w.num_splits, softmax_scale=w.scale,
                             causal=True, cache_seqlens=tsl)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert not np.isnan(o).any()
    qf = W.to_float(q, w.dtype)
    for b, h in [(0, 3), (1, 0), (2, 31), (3, 17), (4, 5), (5, 30), (6, 9), (7, 22)]:
        n = seqlens[b]
        kb = W.to_float(W.gen_slice(w.seed, W.TENSOR_K, b, h, w.Nk, w.d, w.amp, w.dtype)[:n], w.dtype)
        vb = W.to_float(W.gen_slice(w.seed, W.TENSOR_V, b, h, w.Nk, w.d, w.amp, w.dtype)[:n], w.dtype)
        ro, rl = O.attention_bh(qf[b, :, h, :], kb, vb, np.arange(1), 1, w.scale, True)
        check(o[b, :, h, :], lse[b, h, :], ro, rl, "bf16", f"cfg4 seqlens b{b} h{h}")


@pytest.mark.parametrize("dtype,d,nq", [("bf16", 128, 1), ("bf16", 64, 1), ("bf16", 128, 6),
                                        ("fp32", 64, 3)])
def test_splitkv_seqlens_uniform_bitwise_equals_splitkv(dtype, d, nq):
    """Lengths all equal to the capacity reproduce fa_fwd_splitkv bit for bit."""
    w = W.Workload(0, "uniform", B=3, H=4, Nq=nq, Nk=3000, d=d, dtype=dtype, causal=True,
                   paged=True, page_size=64, pool_factor=1.2, num_splits=5, seed=92)
    say(f"seqlens uniform {dtype} d{d} nq{nq}")
    q, kc, vc, bt = W.gen_paged(w)
    tq, tk, tv = to_dev(q, dtype), to_dev(kc, dtype), to_dev(vc, dtype)
    tbt = torch.from_numpy(bt).cuda()
    full = torch.full((w.B,), w.Nk, dtype=torch.int32).cuda()
    ts = torch.from_numpy(W.alibi_slopes(w.H)).cuda()
    a = fa.attention_paged_splitkv(tq, tk, tv, tbt, w.Nk, w.num_splits, w.scale, True, 500, 0, ts,
                                   cache_seqlens=full)
    c = fa.attention_paged_splitkv(tq, tk, tv, tbt, w.Nk, w.num_splits, w.scale, True, 500, 0, ts)
    torch.cuda.synchronize()
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])


# --------------------------------------------------------------------------
# Appending the new keys to the paged cache (fa_fwd_splitkv_append)
# --------------------------------------------------------------------------
APPEND_CASES = [
    # (dtype, d, H, nq, max_k, page_size, num_splits, seqlens, causal, wl, wr, alibi, cap)
    ("bf16", 128, 2, 1, 1000, 64, 4, [999, 0, 1, 511, 63, 700], True, -1, -1, False, 0.0),
    ("bf16", 64, 3, 1, 777, 16, 16, [776, 5, 300, 0], True, 100, 0, True, 0.0),
    ("bf16", 128, 2, 1, 4096, 256, 16, [4095, 2047, 255, 1], True, -1, -1, True, 30.0),
    ("bf16", 128, 2, 5, 300, 7, 3, [295, 4, 0, 150], True, 50, 0, False, 10.0),
    ("bf16", 64, 2, 130, 400, 64, 2, [270, 100, 0], True, -1, -1, True, 0.0),
    ("bf16", 128, 3, 40, 1000, 16, 4, [960, 500, 0, 1], True, -1, -1, True, 30.0),
    ("fp32", 64, 2, 1, 500, 32, 5, [499, 0, 77], True, -1, -1, False, 0.0),
    ("fp32", 128, 2, 20, 200, 16, 3, [180, 10, 0], True, -1, -1, True, 5.0),
]


def bits(x):
    return x.view(np.uint16) if x.dtype == np.uint16 else x.view(np.uint32)


def from_dev(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


@pytest.mark.parametrize("case", APPEND_CASES)
def test_splitkv_append_small(case):
    dtype, d, H, nq, nk, ps, S, seqlens, causal, wl, wr, alibi, cap = case
    say(f"append {case}")
    B = len(seqlens)
    seed = 7000 + APPEND_CASES.index(case)
    w = W.Workload(0, "append", B=B, H=H, Nq=nq, Nk=nk, d=d, dtype=dtype, causal=causal,
                   paged=True, page_size=ps, pool_factor=1.3, num_splits=S, seed=seed)
    q, kc, vc, bt = W.gen_paged(w, seqlens=seqlens)    # rows past each length are NaN
    kn = W.gen_tensor(seed + 500, W.TENSOR_K, B, nq, H, d, 1.0, dtype)
    vn = W.gen_tensor(seed + 500, W.TENSOR_V, B, nq, H, d, 1.0, dtype)
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    scale = 1.0 / np.sqrt(d)
    tkc, tvc = to_dev(kc, dtype), to_dev(vc, dtype)
    o_part, lse_part = fa.attention_paged_append(
        to_dev(q, dtype), to_dev(kn, dtype), to_dev(vn, dtype), tkc, tvc,
        torch.from_numpy(bt).cuda(), torch.tensor(seqlens, dtype=torch.int32).cuda(), nk, S,
        scale, causal, wl, wr, ts, cap)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    # The cache now holds the new keys, bit for bit, and nothing else changed.
    want_k, want_v = O.kvcache_append_ref(kc, vc, bt, seqlens, kn, vn)
    assert np.array_equal(bits(from_dev(tkc, dtype)), bits(want_k))
    assert np.array_equal(bits(from_dev(tvc, dtype)), bits(want_v))
    qf = W.to_float(q, dtype)
    k = np.zeros((B, nk, H, d))
    v = np.zeros((B, nk, H, d))
    for b, n in enumerate(seqlens):
        k[b, :n] = O.paged_gather_ref(W.to_float(kc, dtype), bt, b, n)
        v[b, :n] = O.paged_gather_ref(W.to_float(vc, dtype), bt, b, n)
    rop, rlp = O.splitkv_append_ref(qf, k, v, W.to_float(kn, dtype), W.to_float(vn, dtype),
                                    seqlens, S, ps, scale, causal, wl, wr, slopes, cap)
    check(o_part.cpu().numpy(), lse_part.cpu().numpy(), rop, rlp, dtype, "partials")
    ro, rl = O.combine_ref(rop, rlp)
    check(o.cpu().numpy().transpose(0, 2, 1, 3), lse.cpu().numpy(), ro, rl, dtype, "combined")


@pytest.mark.parametrize("d,ps", [(128, 16), (64, 64)])
def test_multirow_append_bitwise_equals_append_then_seqlens(d, ps):
    """Several appended rows over pages of a multiple of 16 keys: the call appends in a
    launch of its own and then runs the slab pass over the cache, so its partials equal
    bit for bit those of fa_fwd_splitkv_seqlens over a cache appended beforehand (by
    the oracle) with every count raised by the appended rows."""
    B, H, nq, nk, S = 3, 2, 60, 700, 3
    seqlens = [640, 200, 0]
    say(f"multi-row append vs append-then-seqlens d{d} page {ps}")
    w = W.Workload(0, "append_eq", B=B, H=H, Nq=nq, Nk=nk, d=d, dtype="bf16", causal=True,
                   paged=True, page_size=ps, pool_factor=1.3, num_splits=S, seed=7800 + ps)
    q, kc, vc, bt = W.gen_paged(w, seqlens=seqlens)
    kn = W.gen_tensor(7801 + ps, W.TENSOR_K, B, nq, H, d, 1.0, "bf16")
    vn = W.gen_tensor(7801 + ps, W.TENSOR_V, B, nq, H, d, 1.0, "bf16")
    tq, tbt = to_dev(q, "bf16"), torch.from_numpy(bt).cuda()
    tkc, tvc = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    op1, lp1 = fa.attention_paged_append(tq, to_dev(kn, "bf16"), to_dev(vn, "bf16"), tkc, tvc, tbt,
                                         torch.tensor(seqlens, dtype=torch.int32).cuda(), nk, S,
                                         1.0 / np.sqrt(d), True)
    want_k, want_v = O.kvcache_append_ref(kc, vc, bt, seqlens, kn, vn)
    op2, lp2 = fa.attention_paged_splitkv(
        tq, to_dev(want_k, "bf16"), to_dev(want_v, "bf16"), tbt, nk, S, 1.0 / np.sqrt(d), True,
        cache_seqlens=torch.tensor([n + nq for n in seqlens], dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    assert torch.equal(op1, op2) and torch.equal(lp1, lp2)


@pytest.mark.parametrize("dtype,nq", [("fp32", 1), ("fp32", 5), ("bf16", 1), ("bf16", 70)])
def test_alibi_far_splits_keep_fp32_precision(dtype, nq):
    """Splits thousands of keys away from the query rows under a strong ALiBi
    slope (0.5 per key): each split's partial output is still held to its input's
    bound (fp32: 1e-5), i.e. the bias of the keys that carry a split's weight
    is not swamped by the distance to the query."""
    B, H, d, nk, ps, S = 1, 2, 64, 4000, 64, 4
    say(f"alibi far splits {dtype} nq{nq}")
    w = W.Workload(0, "far", B=B, H=H, Nq=nq, Nk=nk, d=d, dtype=dtype, causal=True, paged=True,
                   page_size=ps, pool_factor=1.1, num_splits=S, seed=7700 + nq)
    q, kc, vc, bt = W.gen_paged(w)
    slopes = np.array([0.5, 0.125], dtype=np.float32)
    scale = 1.0 / np.sqrt(d)
    o_part, lse_part = fa.attention_paged_splitkv(
        to_dev(q, dtype), to_dev(kc, dtype), to_dev(vc, dtype), torch.from_numpy(bt).cuda(), nk,
        S, scale, True, -1, -1, torch.from_numpy(slopes).cuda(), 0.0)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    k = np.zeros((B, nk, H, d))
    v = np.zeros((B, nk, H, d))
    k[0] = O.paged_gather_ref(W.to_float(kc, dtype), bt, 0, nk)
    v[0] = O.paged_gather_ref(W.to_float(vc, dtype), bt, 0, nk)
    rop, rlp = O.splitkv_ref(W.to_float(q, dtype), k, v, S, ps, scale, True, -1, -1, slopes, 0.0)
    assert np.isfinite(rlp).all() and rlp.min() < -1000  # far splits: tiny but nonzero weight
    check(o_part.cpu().numpy(), lse_part.cpu().numpy(), rop, rlp, dtype, "far partials")
    ro, rl = O.combine_ref(rop, rlp)
    check(o.cpu().numpy().transpose(0, 2, 1, 3), lse.cpu().numpy(), ro, rl, dtype, "combined")


WIDE_CASES = [
    # (H, seqlens or None, window_left, alibi, softcap, append one key per sequence)
    (33, None, -1, False, 0.0, False),
    (32, [8192, 5000, 1, 0], 3000, True, 30.0, False),
    (31, [8000, 4095, 0, 8191], -1, True, 0.0, True),
]


@pytest.mark.parametrize("case", WIDE_CASES)
def test_decode_wide_head_groups(case):
    """Decode launches large enough for two 256-byte heads per workgroup (at least
    256 workgroups and 1024 keys per split): odd head counts (the last group holds
    one head), per-sequence lengths, a window, ALiBi, softcap and appended keys;
    the partials and the combined output against the oracle."""
    H, seqlens, wl, alibi, cap, append = case
    B, nk, d, ps, S = 4, 8192, 128, 256, 8
    assert (H + 1) // 2 * B * S >= 256 and nk // S >= 1024  # the launch takes wide groups
    seed = 7600 + WIDE_CASES.index(case)
    say(f"wide decode {case}")
    w = W.Workload(0, "wide", B=B, H=H, Nq=1, Nk=nk, d=d, dtype="bf16", causal=True, paged=True,
                   page_size=ps, pool_factor=1.2, num_splits=S, seed=seed)
    lens = seqlens if seqlens is not None else [nk] * B
    q, kc, vc, bt = W.gen_paged(w, seqlens=lens)
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    scale = 1.0 / np.sqrt(d)
    tq, tkc, tvc, tbt = to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16"), torch.from_numpy(bt).cuda()
    tsl = torch.tensor(lens, dtype=torch.int32).cuda()
    if append:
        kn = W.gen_tensor(seed + 500, W.TENSOR_K, B, 1, H, d, 1.0, "bf16")
        vn = W.gen_tensor(seed + 500, W.TENSOR_V, B, 1, H, d, 1.0, "bf16")
        o_part, lse_part = fa.attention_paged_append(tq, to_dev(kn, "bf16"), to_dev(vn, "bf16"), tkc,
                                                     tvc, tbt, tsl, nk, S, scale, True, wl, -1, ts, cap)
    else:
        o_part, lse_part = fa.attention_paged_splitkv(tq, tkc, tvc, tbt, nk, S, scale, True, wl, -1,
                                                      ts, cap, cache_seqlens=tsl)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    qf = W.to_float(q, "bf16")
    k = np.zeros((B, nk, H, d), dtype=np.float32)
    v = np.zeros((B, nk, H, d), dtype=np.float32)
    for b, n in enumerate(lens):
        k[b, :n] = W.to_float(O.paged_gather_ref(kc, bt, b, n), "bf16")
        v[b, :n] = W.to_float(O.paged_gather_ref(vc, bt, b, n), "bf16")
    if append:
        want_k, want_v = O.kvcache_append_ref(kc, vc, bt, lens, kn, vn)
        assert np.array_equal(bits(from_dev(tkc, "bf16")), bits(want_k))
        assert np.array_equal(bits(from_dev(tvc, "bf16")), bits(want_v))
        rop, rlp = O.splitkv_append_ref(qf, k, v, W.to_float(kn, "bf16"), W.to_float(vn, "bf16"),
                                        lens, S, ps, scale, True, wl, -1, slopes, cap)
    else:
        rop, rlp = O.splitkv_ref(qf, k, v, S, ps, scale, True, wl, -1, slopes, cap, seqlens_k=lens)
    check(o_part.cpu().numpy(), lse_part.cpu().numpy(), rop, rlp, "bf16", "wide partials")
    ro, rl = O.combine_ref(rop, rlp)
    check(o.cpu().numpy().transpose(0, 2, 1, 3), lse.cpu().numpy(), ro, rl, "bf16", "wide combined")


def test_incremental_decode_three_steps():
    """Three decode steps, each appending one token per sequence and attending
    over everything cached so far, against the oracle on the growing cache."""
    B, H, d, nk, ps, S = 3, 4, 128, 600, 32, 8
    start = [0, 97, 590]
    w = W.Workload(0, "incremental", B=B, H=H, Nq=1, Nk=nk, d=d, dtype="bf16", causal=True,
                   paged=True, page_size=ps, pool_factor=1.25, num_splits=S, seed=93)
    _, kc, vc, bt = W.gen_paged(w, seqlens=start)
    tkc, tvc = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    tbt = torch.from_numpy(bt).cuda()
    kf, vf = W.to_float(kc, "bf16"), W.to_float(vc, "bf16")
    for step in range(3):
        say(f"incremental decode step {step}")
        lens = [n + step for n in start]
        q = W.gen_tensor(940 + step, W.TENSOR_Q, B, 1, H, d, 1.0, "bf16")
        kn = W.gen_tensor(940 + step, W.TENSOR_K, B, 1, H, d, 1.0, "bf16")
        vn = W.gen_tensor(940 + step, W.TENSOR_V, B, 1, H, d, 1.0, "bf16")
        o_part, lse_part = fa.attention_paged_append(
            to_dev(q, "bf16"), to_dev(kn, "bf16"), to_dev(vn, "bf16"), tkc, tvc, tbt,
            torch.tensor(lens, dtype=torch.int32).cuda(), nk, S, causal=True)
        o, lse = fa.combine(o_part, lse_part)
        torch.cuda.synchronize()
        kf, vf = O.kvcache_append_ref(kf, vf, bt, lens, W.to_float(kn, "bf16"),
                                      W.to_float(vn, "bf16"))
        for b, n in enumerate(lens):
            kb = O.paged_gather_ref(kf, bt, b, n + 1)
            vb = O.paged_gather_ref(vf, bt, b, n + 1)
            for h in range(H):
                ro, rl = O.attention_bh(W.to_float(q, "bf16")[b, :, h], kb[:, h], vb[:, h],
                                        np.arange(1), 1, 1.0 / np.sqrt(d), True)
                check(o.cpu().numpy()[b, :, h], lse.cpu().numpy()[b, h], ro, rl, "bf16",
                      f"step {step} b{b} h{h}")


# --------------------------------------------------------------------------
# Backward pass (fa_bwd)
# --------------------------------------------------------------------------
# The tolerance follows from the arithmetic: the kernels round P and dZ to bf16
# (nearest even: relative error at most 2^-8, the unit roundoff of an 8-bit
# significand) as matrix-core operands and do everything else in fp32. A
# relative change r of every P and dZ entry moves dV by at most r P^T|dO|, dK by
# r scale |dZ|^T|Q| and dQ by r scale |dZ||K| (the oracle's bound terms); the
# test allows r = 2^-8. dP_ij = dO_i.v_j and D_i = dO_i.O_i are fp32 sums over
# head_dim terms, so each errs by up to about d 2^-24 times the sum of the
# absolute values of its terms, |dO_i||v_j| and |dO_i|.|O_i|, before dP - D
# cancels (to exactly 0 where a row sees a single key); carried through P into
# dQ and dK that gives the oracle's cancellation magnitudes
# scale (P (|dO||V|^T + |dO|.|O|)) |K| and its transpose with |Q|, and the test
# allows 2^-16 (>= 2 d 2^-24 for d <= 128) times them, plus 2e-5 of the largest
# gradient for the remaining fp32 arithmetic. The oracle's pins check that these
# magnitudes are the worst cases of those perturbations and cover a simulated
# rounding. O and LSE come from the oracle, so the forward's rounding stays out.
U_BF16 = 2.0 ** -8
E_CANCEL = 2.0 ** -16
BWD_CASES = [
    # (d, B, H, nq, nk, causal, wl, wr, alibi, cap)
    (128, 1, 2, 128, 128, True, -1, -1, False, 0.0),
    (128, 2, 2, 200, 333, True, -1, -1, False, 0.0),
    (64, 1, 3, 300, 90, True, -1, -1, False, 0.0),       # Nq > Nk: rows with no key
    (128, 1, 2, 257, 257, False, -1, -1, True, 0.0),
    (64, 2, 2, 150, 400, True, 50, 0, False, 10.0),
    (128, 1, 2, 100, 300, False, 40, 20, True, 20.0),
    (64, 1, 2, 1, 129, True, -1, -1, True, 0.0),
    (128, 1, 1, 129, 1, False, -1, -1, False, 0.0),
    (128, 1, 2, 64, 1000, True, 100, 0, True, 30.0),
]


def check_grad(g, ref, bound, what, cancel=0.0, out_bf16=False):
    """Elementwise: |g - ref| <= 2^-8 bound + 2^-16 cancel + 2e-5 max|ref| (+ 2^-8 |g| for
    gradients stored in bf16: rounding the output itself)."""
    g = np.asarray(g, dtype=np.float64)
    assert not np.isnan(g).any(), f"{what}: NaN"
    err = np.abs(g - ref)
    tol = U_BF16 * bound + E_CANCEL * cancel + 2e-5 * max(float(np.abs(ref).max()), 1e-30)
    if out_bf16:
        tol = tol + U_BF16 * np.abs(g)
    bad = np.argwhere(err > tol)
    assert len(bad) == 0, (f"{what}: {len(bad)} entries over the bound; first {bad[0].tolist()}: "
                           f"{g[tuple(bad[0])]} vs {ref[tuple(bad[0])]} (tol {tol[tuple(bad[0])]:.3e})")
    return float(err.max())


def bwd_inputs(seed, B, nq, nk, H, d, amp):
    q, k, v = qkv_case(seed, B, nq, nk, H, d, "bf16", amp)
    do = W.gen_tensor(seed, 3, B, nq, H, d, 1.0, "bf16")
    return q, k, v, do


@pytest.mark.parametrize("case", BWD_CASES)
def test_bwd_small(case):
    d, B, H, nq, nk, causal, wl, wr, alibi, cap = case
    say(f"bwd {case}")
    q, k, v, do = bwd_inputs(8000 + BWD_CASES.index(case), B, nq, nk, H, d, 2.0 if cap else 1.0)
    qf, kf, vf, gf = (W.to_float(x, "bf16") for x in (q, k, v, do))
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    scale = 1.0 / np.sqrt(d)
    o_ref, l_ref = O.attention_ref(qf, kf, vf, scale, causal, wl, wr, slopes, cap)
    dq, dk, dv = fa.attention_backward(
        to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
        torch.from_numpy(o_ref.astype(np.float32)).cuda(),
        torch.from_numpy(l_ref.astype(np.float32)).cuda(), to_dev(do, "bf16"), scale, causal, wl,
        wr, ts, cap)
    torch.cuda.synchronize()
    rq, rk, rv, _, bd = O.attention_bwd_ref(qf, kf, vf, gf, scale, causal, wl, wr, slopes, cap,
                                             with_bounds=True)
    print(check_grad(dq.cpu().numpy(), rq, bd["dq"], "dQ", bd["dq_cancel"]),
          check_grad(dk.cpu().numpy(), rk, bd["dk"], "dK", bd["dk_cancel"]),
          check_grad(dv.cpu().numpy(), rv, bd["dv"], "dV"))


def test_bwd_deterministic_and_bf16_output():
    """Two calls give identical bits; bf16 gradients are the fp32 ones rounded."""
    B, nq, nk, H, d = 2, 300, 500, 4, 128
    q, k, v, do = bwd_inputs(8100, B, nq, nk, H, d, 1.0)
    tq, tk, tv, tg = (to_dev(x, "bf16") for x in (q, k, v, do))
    ts = torch.from_numpy(W.alibi_slopes(H)).cuda()
    o, lse = fa.attention(tq, tk, tv, 0.09, True, 200, 0, ts, 15.0)
    a = fa.attention_backward(tq, tk, tv, o, lse, tg, 0.09, True, 200, 0, ts, 15.0)
    b = fa.attention_backward(tq, tk, tv, o, lse, tg, 0.09, True, 200, 0, ts, 15.0)
    c = fa.attention_backward(tq, tk, tv, o, lse, tg, 0.09, True, 200, 0, ts, 15.0,
                              grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y)
        assert torch.equal(x.to(torch.bfloat16), z)


def oracle_bwd_pairs(q, k, v, do, pairs, scale, causal=True, wl=-1, wr=-1, slopes=None, cap=0.0):
    """Oracle forward (O, LSE) and backward with its bound magnitudes, per (b, h) pair
    of bf16 [B, N, H, d] inputs, on the thread pool."""
    def one(bh):
        b, h = bh
        sl = lambda x: W.to_float(x[b, :, h], "bf16")  # noqa: E731
        qb, kb, vb, gb = sl(q), sl(k), sl(v), sl(do)
        slope = None if slopes is None else float(slopes[h])
        nq = qb.shape[0]
        fwd = O.attention_bh(qb, kb, vb, np.arange(nq), nq, scale, causal, wl, wr, slope, cap)
        return fwd, O.attention_bwd_bh(qb, kb, vb, gb, nq, scale, causal, wl, wr, slope, cap,
                                       with_bounds=True)
    return oracle_map(one, pairs)


def test_bwd_causal_prefill_full_size():
    """The causal prefill shape (B4 H16 N2048 d128): every gradient element of every
    (b, h) within the oracle's bound, with O and LSE from the oracle (so the forward's
    rounding stays out, as in the small cases). Then end to end from the GPU forward's
    O and LSE, whose D inherits the forward's bf16 rounding of P: sampled pairs within
    1e-2 of the oracle in relative Frobenius norm."""
    w = W.WORKLOADS[2]
    say(f"bwd full size {w}")
    q, k, v = W.gen_qkv(w)
    do = W.gen_tensor(w.seed, 3, w.B, w.Nq, w.H, w.d, 1.0, "bf16")
    tq, tk, tv, tg = (to_dev(x, "bf16") for x in (q, k, v, do))
    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]
    say("bwd full size: oracle forward and backward, every (b, h)")
    ref = oracle_bwd_pairs(q, k, v, do, pairs, w.scale)
    o_ref = np.zeros((w.B, w.Nq, w.H, w.d), np.float32)
    l_ref = np.zeros((w.B, w.H, w.Nq), np.float32)
    for (b, h), ((ro, rl), _) in zip(pairs, ref):
        o_ref[b, :, h], l_ref[b, h] = ro, rl
    dq, dk, dv = fa.attention_backward(tq, tk, tv, torch.from_numpy(o_ref).cuda(),
                                       torch.from_numpy(l_ref).cuda(), tg, w.scale, True)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    worst = [0.0, 0.0, 0.0]
    for (b, h), (_, (rq, rk, rv, _, bd)) in zip(pairs, ref):
        e = (check_grad(dq[b, :, h], rq, bd["dq"], f"b{b} h{h} dQ", bd["dq_cancel"]),
             check_grad(dk[b, :, h], rk, bd["dk"], f"b{b} h{h} dK", bd["dk_cancel"]),
             check_grad(dv[b, :, h], rv, bd["dv"], f"b{b} h{h} dV"))
        worst = [max(x, y) for x, y in zip(worst, e)]
    say(f"  elementwise max |error| dQ {worst[0]:.2e} dK {worst[1]:.2e} dV {worst[2]:.2e}")

    o, lse = fa.attention(tq, tk, tv, w.scale, True)
    dq, dk, dv = fa.attention_backward(tq, tk, tv, o, lse, tg, w.scale, True)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    assert not (np.isnan(dq).any() or np.isnan(dk).any() or np.isnan(dv).any())
    for (b, h), (_, (rq, rk, rv, _, _)) in zip(pairs, ref):
        if (b, h) not in [(0, 0), (3, 15), (2, 7)]:
            continue
        for got, r, name in ((dq[b, :, h], rq, "dQ"), (dk[b, :, h], rk, "dK"), (dv[b, :, h], rv, "dV")):
            rel = np.linalg.norm(got - r) / np.linalg.norm(r)
            say(f"  end to end b{b} h{h} {name}: relative error {rel:.2e}")
            assert rel <= 1e-2, (b, h, name, rel)


# --------------------------------------------------------------------------
# FP8 forward (fa_fwd_fp8)
# --------------------------------------------------------------------------
# Tolerance from the arithmetic: the kernel rounds 2^8 P to E4M3 (nearest; the
# error is at most half the format's spacing there) for the output product and
# normalises by the unrounded row sum, so O_i moves by at most
# sum_j halfspacing(2^8 P_ij) / 2^8 |v_j| (the oracle's weighted bound). The test
# allows twice that (fp32 rounding of P can move a value across a tie), plus
# 1e-5 of max|O| for the fp32 products; LSE (from the unrounded sum) within 1e-3.
FP8_CASES = [
    # (B, H, nq, nk, causal, wl, wr, alibi, cap, q_ds, k_ds, v_ds)
    (1, 2, 128, 128, True, -1, -1, False, 0.0, 1.0, 1.0, 1.0),
    (2, 2, 200, 333, True, -1, -1, False, 0.0, 0.5, 0.25, 2.0),
    (1, 3, 300, 90, True, -1, -1, False, 0.0, 1.0, 1.0, 1.0),      # Nq > Nk: rows with no key
    (1, 2, 257, 257, False, -1, -1, True, 0.0, 0.125, 1.0, 0.5),
    (2, 2, 150, 400, True, 50, 0, False, 10.0, 1.0, 0.5, 1.0),
    (1, 2, 100, 300, False, 40, 20, True, 20.0, 2.0, 0.5, 4.0),
    (1, 4, 1, 1000, True, -1, -1, False, 0.0, 1.0, 1.0, 1.0),
    (1, 1, 129, 1, False, -1, -1, False, 0.0, 1.0, 1.0, 1.0),
]


def fp8_case(seed, B, nq, nk, H, d=128):
    return (W.gen_tensor(seed, W.TENSOR_Q, B, nq, H, d, 1.0, "fp8"),
            W.gen_tensor(seed, W.TENSOR_K, B, nk, H, d, 1.0, "fp8"),
            W.gen_tensor(seed, W.TENSOR_V, B, nk, H, d, 1.0, "fp8"))


def check_fp8(o, lse, q8, k8, v8, ds, scale, causal, wl, wr, slopes, cap, what, bh=None, rows=None):
    from gpu_common import e4m3_half_spacing
    qf = W.to_float(q8, "fp8") * ds[0]
    kf = W.to_float(k8, "fp8") * ds[1]
    vf = W.to_float(v8, "fp8") * ds[2]
    ro, rl = O.attention_ref(qf, kf, vf, scale, causal, wl, wr, slopes, cap, bh=bh)
    bound = O.prob_weighted_abs_ref(qf, kf, vf, scale, causal, wl, wr, slopes, cap, bh=bh,
                                    weight=lambda pp: e4m3_half_spacing(256.0 * pp) / 256.0)
    sel = [(b, h) for b in range(q8.shape[0]) for h in range(q8.shape[2])] if bh is None else bh
    for b, h in sel:
        og, rg, bd = o[b, :, h], ro[b, :, h], bound[b, :, h]
        assert not np.isnan(og).any(), f"{what}: NaN"
        empty = ~np.isfinite(rl[b, h])
        assert np.array_equal(empty, ~np.isfinite(lse[b, h])), f"{what}: empty-row pattern"
        err = np.abs(og - rg)
        tol = 2.0 * bd + 1e-5 * max(float(np.abs(rg).max()), 1e-30)
        bad = np.argwhere(err > tol)
        assert len(bad) == 0, (f"{what} b{b} h{h}: {len(bad)} over the bound, first {bad[0].tolist()}"
                               f" {og[tuple(bad[0])]} vs {rg[tuple(bad[0])]} tol {tol[tuple(bad[0])]:.3e}")
        if (~empty).any():
            assert np.abs(lse[b, h][~empty] - rl[b, h][~empty]).max() <= TOL_LSE, what
    return float(np.abs(o - ro)[np.isfinite(ro)].max()) if bh is None else 0.0


def to_dev_fp8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", FP8_CASES)
def test_fp8_small(case, d):
    B, H, nq, nk, causal, wl, wr, alibi, cap, qd, kd, vd = case
    say(f"fp8 d{d} {case}")
    q8, k8, v8 = fp8_case(9000 + FP8_CASES.index(case) + 50 * (d == 64), B, nq, nk, H, d)
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.attention_fp8(to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8), qd, kd, vd, scale,
                              causal, wl, wr, ts, cap)
    torch.cuda.synchronize()
    print(check_fp8(o.cpu().numpy(), lse.cpu().numpy(), q8, k8, v8, (qd, kd, vd), scale, causal,
                    wl, wr, slopes, cap, f"fp8 {case}"))


def test_fp8_bf16_output_and_determinism():
    q8, k8, v8 = fp8_case(9100, 2, 300, 500, 4)
    tq, tk, tv = to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8)
    a = fa.attention_fp8(tq, tk, tv, 0.5, 0.5, 1.0, 0.09, True)
    b = fa.attention_fp8(tq, tk, tv, 0.5, 0.5, 1.0, 0.09, True)
    c = fa.attention_fp8(tq, tk, tv, 0.5, 0.5, 1.0, 0.09, True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[0].to(torch.bfloat16), c[0]) and torch.equal(a[1], c[1])


def test_fp8_causal_prefill_sampled_heads():
    """The causal prefill shape (B4 H16 N2048 d128) in FP8: three (b, h) pairs
    against the oracle on the dequantised inputs."""
    w = W.WORKLOADS[2]
    say("fp8 causal prefill")
    q8, k8, v8 = (W.gen_tensor(w.seed, t, w.B, w.Nq, w.H, w.d, 1.0, "fp8")
                  for t in (W.TENSOR_Q, W.TENSOR_K, W.TENSOR_V))
    o, lse = fa.attention_fp8(to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8), 1.0, 1.0, 1.0,
                              w.scale, True)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert not np.isnan(o).any()
    check_fp8(o, lse, q8, k8, v8, (1.0, 1.0, 1.0), w.scale, True, -1, -1, None, 0.0,
              "fp8 prefill", bh=[(0, 0), (3, 15), (2, 7)])


def test_fp8_sliding_window_head_dim_64():
    """The 16K sliding-window shape (B1 H16 N16384 d64, causal, window 4096) in FP8:
    three heads, every row, against the oracle on the dequantised inputs."""
    w = W.WORKLOADS[3]
    say("fp8 sliding window d64")
    q8, k8, v8 = (W.gen_tensor(w.seed, t, w.B, w.Nq, w.H, w.d, 1.0, "fp8")
                  for t in (W.TENSOR_Q, W.TENSOR_K, W.TENSOR_V))
    o, lse = fa.attention_fp8(to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8), 1.0, 1.0, 1.0,
                              w.scale, True, w.window_left, w.window_right)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    assert not np.isnan(o).any()
    check_fp8(o, lse, q8, k8, v8, (1.0, 1.0, 1.0), w.scale, True, w.window_left,
              w.window_right, None, 0.0, "fp8 window", bh=[(0, 0), (0, 9), (0, 15)])


# (B, H, nq, nk, splits, causal, wl, wr, alibi, cap, q/k/v descales)
FP8_SPLIT_CASES = [
    (2, 3, 200, 1000, 4, True, -1, -1, False, 0.0, 1.0, 1.0, 1.0),
    (1, 2, 64, 3000, 7, True, -1, -1, True, 30.0, 0.5, 2.0, 0.25),   # ALiBi far from the row
    (1, 2, 300, 300, 3, False, 50, 20, True, 0.0, 1.0, 1.0, 1.0),
    (2, 2, 500, 90, 2, True, -1, -1, False, 10.0, 1.0, 1.0, 1.0),    # Nq > Nk: rows with no key
    (1, 2, 5, 129, 6, False, -1, -1, False, 0.0, 1.0, 1.0, 1.0),     # more splits than key tiles
]


def check_fp8_partials(o_part, lse_part, q8, k8, v8, ds, scale, causal, wl, wr, slopes, cap, S,
                       what, align=128):
    """Each split's partial against the oracle's split partial on the dequantised inputs,
    within twice the E4M3 rounding bound over that split's own keys (chunks of whole
    multiples of `align` keys)."""
    from gpu_common import e4m3_half_spacing
    qf = W.to_float(q8, "fp8") * ds[0]
    kf = W.to_float(k8, "fp8") * ds[1]
    vf = W.to_float(v8, "fp8") * ds[2]
    nk = k8.shape[1]
    rop, rlp = O.splitkv_ref(qf, kf, vf, S, align, scale, causal, wl, wr, slopes, cap)
    for si, (lo, hi) in enumerate(O.split_bounds(nk, S, align)):
        bound = O.prob_weighted_abs_ref(qf, kf, vf, scale, causal, wl, wr, slopes, cap,
                                        weight=lambda pp: e4m3_half_spacing(256.0 * pp) / 256.0,
                                        key_lo=lo, key_hi=hi)
        for b in range(q8.shape[0]):
            for h in range(q8.shape[2]):
                og, rg = o_part[si, b, h], rop[si, b, h]
                empty = ~np.isfinite(rlp[si, b, h])
                assert np.array_equal(empty, ~np.isfinite(lse_part[si, b, h])), \
                    f"{what} split {si}: empty-row pattern"
                assert not np.isnan(og).any(), f"{what} split {si}: NaN"
                assert np.all(og[empty] == 0.0), f"{what} split {si}: empty rows not zero"
                tol = 2.0 * bound[b, :, h] + 1e-5 * max(float(np.abs(rg).max()), 1e-30)
                bad = np.argwhere(np.abs(og - rg) > tol)
                assert len(bad) == 0, f"{what} split {si} b{b} h{h}: {len(bad)} over the bound"
                if (~empty).any():
                    dl = np.abs(lse_part[si, b, h][~empty] - rlp[si, b, h][~empty]).max()
                    assert dl <= TOL_LSE, f"{what} split {si}: lse {dl:.2e}"


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", FP8_SPLIT_CASES)
def test_fp8_split_partials_and_combined(case, d):
    B, H, nq, nk, S, causal, wl, wr, alibi, cap, qd, kd, vd = case
    say(f"fp8 split d{d} {case}")
    q8, k8, v8 = fp8_case(9500 + FP8_SPLIT_CASES.index(case) + 50 * (d == 64), B, nq, nk, H, d)
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    scale = 1.0 / np.sqrt(d)
    tq, tk, tv = to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8)
    o_part, lse_part = fa.attention_split_partials_fp8(tq, tk, tv, S, qd, kd, vd, scale, causal,
                                                       wl, wr, ts, cap)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    assert fa.fa_split_chunk_len(nk, S, 128) == -(-(-(-nk // S)) // 128) * 128
    check_fp8_partials(o_part.cpu().numpy(), lse_part.cpu().numpy(), q8, k8, v8, (qd, kd, vd),
                       scale, causal, wl, wr, slopes, cap, S, f"fp8 split {case}")
    print(check_fp8(o.cpu().numpy(), lse.cpu().numpy(), q8, k8, v8, (qd, kd, vd), scale, causal,
                    wl, wr, slopes, cap, f"fp8 split combined {case}"))


# fa_fwd_paged_fp8: E4M3 queries over a paged E4M3 cache (pages of a multiple of 32
# keys copied in per-wavefront slabs of the 128-key tiles, other page sizes row by row). Each sequence's partials are checked against the oracle's split partials over
# its gathered, dequantised keys, within the E4M3 rounding bound over each split's keys;
# the pool's unused rows are NaN codes, so any read outside a sequence's keys shows.
FP8_PAGED_CASES = [
    # (B, H, nq, nk, page_size, S, seqlens or None, causal, wl, wr, alibi, cap, qd, kd, vd)
    (2, 3, 300, 1000, 128, 3, None, True, -1, -1, False, 0.0, 1.0, 1.0, 1.0),
    (3, 2, 129, 700, 256, 2, [700, 129, 1], False, 100, 30, True, 0.0, 0.5, 2.0, 1.5),
    (3, 2, 200, 1500, 384, 4, [1500, 999, 200], True, -1, -1, True, 20.0, 1.0, 0.5, 2.0),
    (2, 2, 64, 2000, 512, 5, [2000, 0], True, 300, 0, False, 10.0, 1.0, 1.0, 0.25),
    (1, 4, 500, 4096, 256, 8, None, True, -1, -1, True, 30.0, 0.75, 1.25, 1.0),
    # Row gathers: pages of 16, 64, 7 and 200 keys.
    (2, 3, 300, 1000, 16, 4, [1000, 333], True, -1, -1, True, 0.0, 1.0, 1.0, 1.0),
    (2, 2, 129, 900, 64, 3, None, False, 200, 50, False, 15.0, 0.5, 1.0, 2.0),
    (3, 2, 100, 500, 7, 5, [500, 1, 0], True, 64, 0, True, 30.0, 1.0, 0.5, 1.0),
    (1, 3, 256, 3000, 200, 6, None, True, -1, -1, False, 0.0, 1.0, 2.0, 0.5),
]


def fp8_paged_case(case, seed, d):
    B, H, nq, nk, ps, S, seqlens, causal, wl, wr, alibi, cap, qd, kd, vd = case
    w = W.Workload(0, "fp8_paged", B=B, H=H, Nq=nq, Nk=nk, d=d, dtype="fp8", causal=causal,
                   paged=True, page_size=ps, pool_factor=1.3, num_splits=S, seed=seed)
    _, kc, vc, bt = W.gen_paged(w, seqlens=seqlens)
    q8 = W.gen_tensor(seed, W.TENSOR_Q, B, nq, H, d, 1.0, "fp8")
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    tsl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32).cuda()
    o_part, lse_part = fa.attention_paged_fp8(
        to_dev_fp8(q8), to_dev_fp8(kc), to_dev_fp8(vc), torch.from_numpy(bt).cuda(), nk, S, qd,
        kd, vd, 1.0 / np.sqrt(d), causal, wl, wr, ts, cap, cache_seqlens=tsl)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    return q8, kc, vc, bt, slopes, o_part.cpu().numpy(), lse_part.cpu().numpy(), \
        o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", FP8_PAGED_CASES)
def test_fp8_paged_partials_and_combined(case, d):
    B, H, nq, nk, ps, S, seqlens, causal, wl, wr, alibi, cap, qd, kd, vd = case
    say(f"fp8 paged d{d} {case}")
    seed = 9700 + FP8_PAGED_CASES.index(case) + 50 * (d == 64)
    q8, kc, vc, bt, slopes, op, lp, o, lse = fp8_paged_case(case, seed, d)
    assert not np.isnan(op).any() and not np.isnan(o).any(), "NaN: a poisoned pool row was read"
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        n = nk if seqlens is None else seqlens[b]
        if n == 0:  # no key: every split empty
            assert np.all(op[:, b] == 0.0) and np.all(lp[:, b] == -np.inf)
            assert np.all(o[b] == 0.0) and np.all(lse[b] == -np.inf)
            continue
        k8 = O.paged_gather_ref(kc, bt, b, n)[None]
        v8 = O.paged_gather_ref(vc, bt, b, n)[None]
        check_fp8_partials(op[:, b:b + 1], lp[:, b:b + 1], q8[b:b + 1], k8, v8, (qd, kd, vd),
                           scale, causal, wl, wr, slopes, cap, S, f"fp8 paged b{b} {case}",
                           align=ps)
        print(check_fp8(o[b:b + 1], lse[b:b + 1], q8[b:b + 1], k8, v8, (qd, kd, vd), scale,
                        causal, wl, wr, slopes, cap, f"fp8 paged combined b{b} {case}"))


@pytest.mark.parametrize("d,ps,nk,S,alibi,cap", [(128, 128, 1000, 3, True, 30.0),
                                                  (64, 256, 2048, 4, False, 0.0),
                                                  (128, 512, 4096, 8, False, 20.0),
                                                  (128, 64, 2048, 4, True, 0.0),    # slabs
                                                  (64, 32, 2048, 4, False, 0.0),    # slabs
                                                  (64, 16, 1000, 1, False, 10.0),   # gathers
                                                  (128, 48, 1152, 3, True, 20.0)])  # gathers
def test_fp8_paged_is_bitwise_fa_fwd_split_fp8(d, ps, nk, S, alibi, cap):
    """With chunks that coincide (equal key counts; chunk lengths a multiple of 128
    either way) the paged pass reads the same 128-key tiles in the same order as
    fa_fwd_split_fp8 over the gathered keys, whether its pages travel as tiles or row
    by row: partials bit for bit."""
    say(f"fp8 paged == split d{d} page {ps} nk {nk} S{S}")
    B, H, nq = 2, 3, 257
    case = (B, H, nq, nk, ps, S, None, True, -1, -1, alibi, cap, 0.5, 1.5, 2.0)
    seed = 9800 + d + ps
    q8, kc, vc, bt, slopes, op, lp, _, _ = fp8_paged_case(case, seed, d)
    assert O.split_bounds(nk, S, ps) == O.split_bounds(nk, S, 128)
    k8 = np.stack([O.paged_gather_ref(kc, bt, b, nk) for b in range(B)])
    v8 = np.stack([O.paged_gather_ref(vc, bt, b, nk) for b in range(B)])
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    op2, lp2 = fa.attention_split_partials_fp8(to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8), S,
                                               0.5, 1.5, 2.0, 1.0 / np.sqrt(d), True, -1, -1,
                                               ts, cap)
    torch.cuda.synchronize()
    assert np.array_equal(op, op2.cpu().numpy()) and np.array_equal(lp, lp2.cpu().numpy())


@pytest.mark.parametrize("d,alibi,cap", [(128, True, 30.0), (64, False, 0.0)])
def test_fp8_one_split_is_bitwise_fa_fwd_fp8(d, alibi, cap):
    """One split covers every key with the same tiles in the same order: its partial is
    fa_fwd_fp8's fp32 output and LSE bit for bit."""
    q8, k8, v8 = fp8_case(9600 + d, 2, 300, 700, 4, d)
    ts = torch.from_numpy(W.alibi_slopes(4)).cuda() if alibi else None
    tq, tk, tv = to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8)
    o, lse = fa.attention_fp8(tq, tk, tv, 0.5, 1.5, 2.0, 0.1, True, -1, -1, ts, cap)
    o_part, lse_part = fa.attention_split_partials_fp8(tq, tk, tv, 1, 0.5, 1.5, 2.0, 0.1, True,
                                                       -1, -1, ts, cap)
    torch.cuda.synchronize()
    assert torch.equal(o_part[0], o.permute(0, 2, 1, 3)) and torch.equal(lse_part[0], lse)


def test_fp8_split_alibi_softcap_shape():
    """The ALiBi + softcap set (B2 H8 Nq512 Nk4096 d128, amplitude 2, causal) in E4M3
    through 8 key splits and the combine kernel, every head and row."""
    w = W.WORKLOADS[5]
    say("fp8 split alibi softcap shape")
    q8, k8, v8 = (W.gen_tensor(w.seed, t, w.B, n, w.H, w.d, w.amp, "fp8")
                  for t, n in ((W.TENSOR_Q, w.Nq), (W.TENSOR_K, w.Nk), (W.TENSOR_V, w.Nk)))
    slopes = w.slopes()
    ts = torch.from_numpy(np.asarray(slopes, np.float32)).cuda()
    o, lse = fa.attention_split_fp8(to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8), 8,
                                    softmax_scale=w.scale, causal=True, alibi_slopes=ts,
                                    softcap=w.softcap)
    torch.cuda.synchronize()
    print(check_fp8(o.cpu().numpy(), lse.cpu().numpy(), q8, k8, v8, (1.0, 1.0, 1.0), w.scale,
                    True, -1, -1, slopes, w.softcap, "fp8 split cfg5 shape"))


# --------------------------------------------------------------------------
# Brute-force sweeps of small and ragged shapes: backward and FP8
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d", [128, 64])
def test_bwd_sweep_small_shapes(d):
    case = 0
    for nq, nk in itertools.product(SIZES, SIZES):
        for (causal, wl, wr) in mask_variants(nq, nk):
            case += 1
            if (nq + 2 * nk + case) % 3:
                continue  # a deterministic third of the grid (every size and mask still occurs)
            alibi = case % 3 == 1
            cap = 7.5 if case % 4 == 2 else 0.0
            what = f"bwd d{d} nq{nq} nk{nk} causal{causal} wl{wl} wr{wr} alibi{alibi} cap{cap}"
            say(what)
            q, k, v, do = bwd_inputs(20000 + case, 1, nq, nk, 2, d, 2.0 if cap else 1.0)
            qf, kf, vf, gf = (W.to_float(x, "bf16") for x in (q, k, v, do))
            slopes = W.alibi_slopes(2) if alibi else None
            ts = None if slopes is None else torch.from_numpy(slopes).cuda()
            scale = 1.0 / np.sqrt(d)
            o_ref, l_ref = O.attention_ref(qf, kf, vf, scale, causal, wl, wr, slopes, cap)
            dq, dk, dv = fa.attention_backward(
                to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                torch.from_numpy(o_ref.astype(np.float32)).cuda(),
                torch.from_numpy(l_ref.astype(np.float32)).cuda(), to_dev(do, "bf16"), scale,
                causal, wl, wr, ts, cap)
            torch.cuda.synchronize()
            rq, rk, rv, _, bd = O.attention_bwd_ref(qf, kf, vf, gf, scale, causal, wl, wr, slopes,
                                                    cap, with_bounds=True)
            check_grad(dq.cpu().numpy(), rq, bd["dq"], what + " dQ", bd["dq_cancel"])
            check_grad(dk.cpu().numpy(), rk, bd["dk"], what + " dK", bd["dk_cancel"])
            check_grad(dv.cpu().numpy(), rv, bd["dv"], what + " dV")


@pytest.mark.parametrize("d", [128, 64])
def test_fp8_sweep_small_shapes(d):
    case = 0
    for nq, nk in itertools.product(SIZES, SIZES):
        for (causal, wl, wr) in mask_variants(nq, nk):
            case += 1
            if (2 * nq + nk + case) % 3:
                continue
            alibi = case % 3 == 1
            cap = 7.5 if case % 4 == 2 else 0.0
            ds = (0.5, 2.0, 0.25) if case % 5 == 0 else (1.0, 1.0, 1.0)
            what = f"fp8 d{d} nq{nq} nk{nk} causal{causal} wl{wl} wr{wr} alibi{alibi} cap{cap} ds{ds}"
            say(what)
            q8, k8, v8 = fp8_case(30000 + case + 5000 * (d == 64), 1 + case % 2, nq, nk, 2, d)
            slopes = W.alibi_slopes(2) if alibi else None
            ts = None if slopes is None else torch.from_numpy(slopes).cuda()
            scale = 1.0 / np.sqrt(d)
            o, lse = fa.attention_fp8(to_dev_fp8(q8), to_dev_fp8(k8), to_dev_fp8(v8), *ds, scale,
                                      causal, wl, wr, ts, cap)
            torch.cuda.synchronize()
            check_fp8(o.cpu().numpy(), lse.cpu().numpy(), q8, k8, v8, ds, scale, causal, wl, wr,
                      slopes, cap, what)


def test_varlen_random_packs():
    """Seeded random packs (0-300 rows per sequence, empty sequences included)
    across head sizes, dtypes and mask / score variants."""
    rng = np.random.default_rng(95)
    for case in range(24):
        dtype, d = [("bf16", 128), ("bf16", 64), ("fp32", 64), ("fp32", 128)][case % 4]
        B = int(rng.integers(1, 7))
        lq = rng.integers(0, 301, B)
        lk = rng.integers(0, 301, B)
        if case % 3 == 0:
            lq[rng.integers(0, B)] = 0
        causal, wl, wr = [(True, -1, -1), (False, -1, -1), (True, 40, 0), (False, 17, 9)][(case // 4) % 4]
        alibi, cap = case % 5 == 1, (6.0 if case % 7 == 3 else 0.0)
        if lq.sum() == 0:
            lq[0] = 5
        what = f"varlen random {case}: {dtype} d{d} lq{lq.tolist()} lk{lk.tolist()} {causal} {wl} {wr} {alibi} {cap}"
        say(what)
        q, k, v, cq, ck = W.gen_varlen(9500 + case, lq, lk, 2, d, 2.0 if cap else 1.0, dtype)
        slopes = W.alibi_slopes(2) if alibi else None
        scale = 1.0 / np.sqrt(d)
        o, lse = run_varlen(q, k, v, cq, ck, dtype, int(lq.max()), int(max(lk.max(), 0)), scale,
                            causal, wl, wr, slopes, cap)
        ro, rl = O.attention_varlen_ref(W.to_float(q, dtype), W.to_float(k, dtype),
                                        W.to_float(v, dtype), cq, ck, scale, causal, wl, wr,
                                        slopes, cap)
        check(o, lse, ro, rl, dtype, what)


def test_splitkv_seqlens_random():
    """Seeded random per-sequence cache lengths, page sizes and split counts,
    for the decode kernel (Nq = 1) and the multi-row paged kernel."""
    rng = np.random.default_rng(96)
    for case in range(16):
        dtype, d = [("bf16", 128), ("bf16", 64), ("fp32", 64), ("bf16", 128)][case % 4]
        nq = [1, 1, 3, 33][case % 4]
        ps = int([16, 64, 7, 256][case % 4])
        nk = int(rng.integers(100, 1500))
        B = int(rng.integers(1, 6))
        S = int(rng.integers(1, 12))
        seqlens = rng.integers(0, nk + 1, B).tolist()
        causal, wl = [(True, -1), (True, 200), (False, -1), (True, -1)][case % 4]
        alibi, cap = case % 3 == 2, (12.0 if case % 5 == 4 else 0.0)
        what = f"seqlens random {case}: {dtype} d{d} nq{nq} nk{nk} ps{ps} S{S} {seqlens} {causal} {wl}"
        say(what)
        w = W.Workload(0, "rand", B=B, H=2, Nq=nq, Nk=nk, d=d, dtype=dtype, causal=causal,
                       paged=True, page_size=ps, pool_factor=1.25, num_splits=S, seed=9600 + case)
        q, kc, vc, bt = W.gen_paged(w, seqlens=seqlens)
        slopes = W.alibi_slopes(2) if alibi else None
        ts = None if slopes is None else torch.from_numpy(slopes).cuda()
        scale = 1.0 / np.sqrt(d)
        o_part, lse_part = fa.attention_paged_splitkv(
            to_dev(q, dtype), to_dev(kc, dtype), to_dev(vc, dtype), torch.from_numpy(bt).cuda(), nk,
            S, scale, causal, wl, 0 if causal else -1, ts, cap,
            cache_seqlens=torch.tensor(seqlens, dtype=torch.int32).cuda())
        torch.cuda.synchronize()
        k = np.zeros((B, nk, 2, d))
        v = np.zeros((B, nk, 2, d))
        for b, n in enumerate(seqlens):
            k[b, :n] = O.paged_gather_ref(W.to_float(kc, dtype), bt, b, n)
            v[b, :n] = O.paged_gather_ref(W.to_float(vc, dtype), bt, b, n)
        rop, rlp = O.splitkv_ref(W.to_float(q, dtype), k, v, S, ps, scale, causal, wl,
                                 0 if causal else -1, slopes, cap, seqlens_k=seqlens)
        check(o_part.cpu().numpy(), lse_part.cpu().numpy(), rop, rlp, dtype, what)


# --------------------------------------------------------------------------
# Large shapes (index arithmetic far from the workloads' sizes)
# --------------------------------------------------------------------------
def test_many_heads_and_large_batch():
    """4096 heads (2 MiB rows between keys of one head) and a batch of 2048;
    sampled (b, h) pairs against the oracle."""
    for B, H, nq, nk, d in [(1, 4096, 65, 130, 128), (2048, 2, 3, 70, 64)]:
        say(f"large B/H: B{B} H{H} nq{nq} nk{nk} d{d}")
        q, k, v = qkv_case(97, B, nq, nk, H, d, "bf16")
        o, lse = run_fwd(q, k, v, "bf16", 0.1, True, -1, -1, None, 0.0)
        pairs = [(0, 0), (B - 1, H - 1), (B // 2, H // 3), (B - 1, 0)]
        ro, rl = oracle_fwd(q, k, v, "bf16", 0.1, True, -1, -1, None, 0.0, bh=pairs)
        for b, h in pairs:
            check(o[b, :, h], lse[b, h], ro[b, :, h], rl[b, h], "bf16", f"B{B} H{H} b{b} h{h}")


def test_long_window_sequence():
    """65536 keys with a 2048-key causal window (sampled rows across the range)."""
    B, H, n, d = 1, 2, 65536, 64
    say("long window sequence")
    q, k, v = qkv_case(98, B, n, n, H, d, "bf16")
    o, lse = run_fwd(q, k, v, "bf16", 0.125, True, 2048, 0, None, 0.0)
    rows = np.array([0, 1, 2047, 2048, 2049, 32767, 32768, 65534, 65535, 40000, 12345])
    ro, rl = oracle_fwd(q, k, v, "bf16", 0.125, True, 2048, 0, None, 0.0, rows=rows)
    check(o[:, rows], lse[:, :, rows], ro, rl, "bf16", "long window")


def test_decode_over_a_quarter_million_keys():
    """One query row over 262144 cached keys in 256-key pages, 64 splits."""
    w = W.Workload(0, "long_decode", B=1, H=2, Nq=1, Nk=262144, d=128, dtype="bf16", causal=True,
                   paged=True, page_size=256, pool_factor=1.1, num_splits=64, seed=99)
    say("decode over 262144 keys")
    q, kc, vc, bt = W.gen_paged(w)
    o, lse = fa.decode_paged(to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16"),
                             torch.from_numpy(bt).cuda(), w.Nk, w.num_splits, softmax_scale=w.scale,
                             causal=True)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    qf = W.to_float(q, "bf16")
    for h in range(w.H):
        kb = W.to_float(W.gen_slice(w.seed, W.TENSOR_K, 0, h, w.Nk, w.d, 1.0, "bf16"), "bf16")
        vb = W.to_float(W.gen_slice(w.seed, W.TENSOR_V, 0, h, w.Nk, w.d, 1.0, "bf16"), "bf16")
        ro, rl = O.attention_bh(qf[0, :, h], kb, vb, np.arange(1), 1, w.scale, True)
        check(o[0, :, h], lse[0, h], ro, rl, "bf16", f"long decode h{h}")


def test_tensors_over_4_gib():
    """K and V of 4 GiB each (262144 keys x 64 heads x 128 bf16 = 2^31 elements), so
    element and byte offsets pass 2^31 and 2^32. Heads 0, 37 and 63 hold seeded
    N(0,1) slices checked against the oracle (head 63's last keys sit at the top
    of the range); the other heads are filled on the device. Covered: the prefill
    (64 query rows over every key), the same bytes as a paged cache of 1024
    permuted 256-key pages (one query row, and the 64-row page-tile pass), and the
    backward (bf16 gradients, relative norm)."""
    B, H, nk, d, nq, ps = 1, 64, 262144, 128, 64, 256
    heads = (0, 37, 63)
    seed, scale = 4100, 1.0 / np.sqrt(128)
    say("over 4 GiB: filling K and V on the device")
    g = torch.Generator(device="cuda").manual_seed(seed)
    k = torch.randn((B, nk, H, d), generator=g, device="cuda", dtype=torch.bfloat16)
    v = torch.randn((B, nk, H, d), generator=g, device="cuda", dtype=torch.bfloat16)
    assert k.numel() == 2 ** 31
    ks, vs = {}, {}
    for h in heads:
        ks[h] = W.gen_slice(seed, W.TENSOR_K, 0, h, nk, d, 1.0, "bf16")
        vs[h] = W.gen_slice(seed, W.TENSOR_V, 0, h, nk, d, 1.0, "bf16")
        k[0, :, h] = to_dev(ks[h], "bf16")
        v[0, :, h] = to_dev(vs[h], "bf16")
    q = W.gen_tensor(seed, W.TENSOR_Q, B, nq, H, d, 1.0, "bf16")
    do = W.gen_tensor(seed, 3, B, nq, H, d, 1.0, "bf16")
    tq, tg = to_dev(q, "bf16"), to_dev(do, "bf16")
    perm = np.random.default_rng(seed).permutation(nk // ps).astype(np.int32)
    bt = torch.from_numpy(perm[None, :].copy()).cuda()
    # Logical key t of the paged view lives at page perm[t // ps], row t % ps.
    logical = (perm.astype(np.int64)[:, None] * ps + np.arange(ps)).reshape(-1)
    kc, vc = k.view(nk // ps, ps, H, d), v.view(nk // ps, ps, H, d)

    say("over 4 GiB: prefill, paged decode, paged 64-row pass")
    o, lse = fa.attention(tq, k, v, scale, True)
    od, lsed = fa.decode_paged(tq[:, :1].contiguous(), kc, vc, bt, nk, softmax_scale=scale,
                               causal=True)
    op, lsep = fa.decode_paged(tq, kc, vc, bt, nk, softmax_scale=scale, causal=True)
    torch.cuda.synchronize()
    say("over 4 GiB: backward from the GPU forward")
    g1 = fa.attention_backward(tq, k, v, o, lse, tg, scale, True, grad_dtype=torch.bfloat16)
    o_in, lse_in = o.clone(), lse.clone()
    torch.cuda.synchronize()
    o, lse, od, lsed, op, lsep = (x.float().cpu().numpy() for x in (o, lse, od, lsed, op, lsep))
    for h in heads:
        say(f"over 4 GiB: oracle forward for head {h}")
        qf = W.to_float(q[0, :, h], "bf16")
        kf, vf = W.to_float(ks[h], "bf16"), W.to_float(vs[h], "bf16")
        ro, rl = O.attention_bh(qf, kf, vf, np.arange(nq), nq, scale, True)
        check(o[0, :, h], lse[0, h], ro, rl, "bf16", f"prefill h{h}")
        o_in[0, :, h] = torch.from_numpy(ro.astype(np.float32)).cuda()
        lse_in[0, h] = torch.from_numpy(rl.astype(np.float32)).cuda()
        kl, vl = kf[logical], vf[logical]
        ro, rl = O.attention_bh(qf[:1], kl, vl, np.arange(1), 1, scale, True)
        check(od[0, :, h], lsed[0, h], ro, rl, "bf16", f"paged decode h{h}")
        ro, rl = O.attention_bh(qf, kl, vl, np.arange(nq), nq, scale, True)
        check(op[0, :, h], lsep[0, h], ro, rl, "bf16", f"paged 64 rows h{h}")
        del kl, vl
    say("over 4 GiB: backward from the oracle's O and LSE")
    g2 = fa.attention_backward(tq, k, v, o_in, lse_in, tg, scale, True, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for h in heads:
        say(f"over 4 GiB: oracle backward for head {h}")
        qf = W.to_float(q[0, :, h], "bf16")
        kf, vf = W.to_float(ks[h], "bf16"), W.to_float(vs[h], "bf16")
        rq, rk, rv, _, bd = O.attention_bwd_bh(qf, kf, vf, W.to_float(do[0, :, h], "bf16"), nq,
                                               scale, True, with_bounds=True)
        got1 = [x[0, :, h].float().cpu().numpy() for x in g1]
        got2 = [x[0, :, h].float().cpu().numpy() for x in g2]
        for x, ref, name in zip(got1, (rq, rk, rv), ("dQ", "dK", "dV")):
            rel = np.linalg.norm(x - ref) / np.linalg.norm(ref)
            assert rel <= 1e-2, (h, name, rel)
        check_grad(got2[0], rq, bd["dq"], f"h{h} dQ", bd["dq_cancel"], out_bf16=True)
        check_grad(got2[1], rk, bd["dk"], f"h{h} dK", bd["dk_cancel"], out_bf16=True)
        check_grad(got2[2], rv, bd["dv"], f"h{h} dV", out_bf16=True)
        del got1, got2, rq, rk, rv, bd


def test_bwd_many_heads():
    """The backward with 1024 heads (its row-term workspace and tile decode at large H):
    every head elementwise within the oracle's bound, O and LSE from the oracle."""
    B, H, nq, nk, d = 1, 1024, 40, 150, 128
    say("bwd many heads")
    q, k, v, do = bwd_inputs(8200, B, nq, nk, H, d, 1.0)
    tq, tk, tv, tg = (to_dev(x, "bf16") for x in (q, k, v, do))
    pairs = [(0, h) for h in range(H)]
    ref = oracle_bwd_pairs(q, k, v, do, pairs, 0.1)
    o_ref = np.stack([r[0][0] for r in ref], axis=1)[None].astype(np.float32)
    l_ref = np.stack([r[0][1] for r in ref])[None].astype(np.float32)
    dq, dk, dv = fa.attention_backward(tq, tk, tv, torch.from_numpy(o_ref).cuda(),
                                       torch.from_numpy(l_ref).cuda(), tg, 0.1, True)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()
    for (_, h), (_, (rq, rk, rv, _, bd)) in zip(pairs, ref):
        check_grad(dq[0, :, h], rq, bd["dq"], f"h{h} dQ", bd["dq_cancel"])
        check_grad(dk[0, :, h], rk, bd["dk"], f"h{h} dK", bd["dk_cancel"])
        check_grad(dv[0, :, h], rv, bd["dv"], f"h{h} dV")


# --------------------------------------------------------------------------
# Backward of packed batches (fa_bwd_varlen)
# --------------------------------------------------------------------------
VARLEN_BWD_CASES = [
    # (d, H, [(nq, nk), ...], causal, wl, wr, alibi, cap)
    (128, 2, [(1, 1), (17, 300), (128, 128), (129, 64), (300, 1000), (0, 5), (7, 0),
              (255, 257)], True, -1, -1, False, 0.0),
    (64, 3, [(64, 64), (130, 500), (1, 700), (200, 3), (33, 33), (0, 40)], True, 60, 0, True,
     0.0),
    (128, 2, [(100, 100), (250, 140), (3, 400), (0, 0)], False, -1, -1, True, 20.0),
    (64, 2, [(129, 129), (40, 0), (90, 600)], False, 30, 30, False, 8.0),
    (128, 1, [(300, 90), (1, 129), (129, 1)], True, -1, -1, False, 0.0),
]


def varlen_bwd_inputs(seed, lq, lk, H, d, amp):
    q, k, v, cq, ck = W.gen_varlen(seed, lq, lk, H, d, amp, "bf16")
    do = W.gen_tensor(seed, 3, 1, int(cq[-1]), H, d, 1.0, "bf16")[0]
    return q, k, v, do, cq, ck


def run_varlen_bwd(q, k, v, o, lse, do, cq, ck, maxq, maxk, scale, causal, wl, wr, slopes, cap,
                   grad_dtype=torch.float32):
    ts = None if slopes is None else torch.from_numpy(np.asarray(slopes, np.float32)).cuda()
    g = fa.attention_varlen_backward(
        to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
        torch.from_numpy(np.asarray(o, np.float32)).cuda(),
        torch.from_numpy(np.asarray(lse, np.float32)).cuda(), to_dev(do, "bf16"),
        torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), maxq, maxk, scale, causal, wl,
        wr, ts, cap, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in g]


def check_varlen_bwd(seed, lq, lk, H, d, causal, wl, wr, alibi, cap, what):
    q, k, v, do, cq, ck = varlen_bwd_inputs(seed, lq, lk, H, d, 2.0 if cap else 1.0)
    qf, kf, vf, gf = (W.to_float(x, "bf16") for x in (q, k, v, do))
    slopes = W.alibi_slopes(H) if alibi else None
    scale = 1.0 / np.sqrt(d)
    ro, rl = O.attention_varlen_ref(qf, kf, vf, cq, ck, scale, causal, wl, wr, slopes, cap)
    dq, dk, dv = run_varlen_bwd(q, k, v, ro, rl, do, cq, ck, max(int(max(lq)), 1),
                                int(max(lk)), scale, causal, wl, wr, slopes, cap)
    rq, rk, rv, bd = O.attention_varlen_bwd_ref(qf, kf, vf, gf, cq, ck, scale, causal, wl, wr,
                                                slopes, cap, with_bounds=True)
    return (check_grad(dq, rq, bd["dq"], what + " dQ", bd["dq_cancel"]),
            check_grad(dk, rk, bd["dk"], what + " dK", bd["dk_cancel"]),
            check_grad(dv, rv, bd["dv"], what + " dV"))


@pytest.mark.parametrize("case", VARLEN_BWD_CASES)
def test_varlen_bwd_packed_small(case):
    """Packs with empty sequences (no query: dK = dV = 0; no key: dQ = 0),
    Nq > Nk per sequence and every mask / score variant, against the oracle."""
    d, H, lens, causal, wl, wr, alibi, cap = case
    what = f"varlen bwd {case}"
    say(what)
    lq, lk = [a for a, _ in lens], [b for _, b in lens]
    print(check_varlen_bwd(12000 + VARLEN_BWD_CASES.index(case), lq, lk, H, d, causal, wl, wr,
                           alibi, cap, what))


def test_varlen_bwd_equal_lengths_bitwise_equals_batched():
    """A pack of equal-length sequences is the batched problem: the same
    kernels compute the same tiles, so the gradients match fa_bwd bit for bit."""
    B, nq, nk, H, d = 3, 200, 333, 4, 128
    say("varlen bwd bitwise vs batched")
    q, k, v, do = bwd_inputs(12100, B, nq, nk, H, d, 1.0)
    tq, tk, tv, tg = (to_dev(x, "bf16") for x in (q, k, v, do))
    ts = torch.from_numpy(W.alibi_slopes(H)).cuda()
    o, lse = fa.attention(tq, tk, tv, 0.09, True, 100, 0, ts, 12.0)
    gb = fa.attention_backward(tq, tk, tv, o, lse, tg, 0.09, True, 100, 0, ts, 12.0)
    cq = torch.from_numpy(W.cu_seqlens([nq] * B)).cuda()
    ck = torch.from_numpy(W.cu_seqlens([nk] * B)).cuda()
    pk = lambda x, n: x.reshape(B * n, H, d)  # noqa: E731
    gv = fa.attention_varlen_backward(
        pk(tq, nq), pk(tk, nk), pk(tv, nk), pk(o, nq),
        lse.permute(1, 0, 2).reshape(H, B * nq).contiguous(), pk(tg, nq), cq, ck, nq, nk, 0.09,
        True, 100, 0, ts, 12.0)
    torch.cuda.synchronize()
    for a, b, n in zip(gb, gv, (nq, nk, nk)):
        assert torch.equal(pk(a, n), b)


def test_varlen_bwd_random_packs():
    """Seeded random packs (0-300 rows per sequence, empty sequences included)
    across head sizes and mask / score variants; bf16 gradients are the fp32
    ones rounded."""
    rng = np.random.default_rng(121)
    for case in range(12):
        d = (128, 64)[case % 2]
        B = int(rng.integers(1, 6))
        lq = rng.integers(0, 301, B)
        lk = rng.integers(0, 301, B)
        if case % 3 == 0:
            lq[rng.integers(0, B)] = 0
        if lq.sum() == 0:
            lq[0] = 5
        causal, wl, wr = [(True, -1, -1), (False, -1, -1), (True, 40, 0), (False, 17, 9)][(case // 2) % 4]
        alibi, cap = case % 5 == 1, (6.0 if case % 7 == 3 else 0.0)
        what = f"varlen bwd random {case}: d{d} lq{lq.tolist()} lk{lk.tolist()} {causal} {wl} {wr} {alibi} {cap}"
        say(what)
        check_varlen_bwd(12200 + case, lq.tolist(), lk.tolist(), 2, d, causal, wl, wr, alibi, cap,
                         what)


def test_varlen_bwd_deterministic_and_bf16_output():
    lens = [300, 0, 77, 513]
    q, k, v, do, cq, ck = varlen_bwd_inputs(12300, lens, [400, 10, 77, 513], 4, 128, 1.0)
    tq, tk, tv, tg = (to_dev(x, "bf16") for x in (q, k, v, do))
    tcq, tck = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    say("varlen bwd determinism")
    o, lse = fa.attention_varlen(tq, tk, tv, tcq, tck, 513, 513, 0.1, True)
    a = fa.attention_varlen_backward(tq, tk, tv, o, lse, tg, tcq, tck, 513, 513, 0.1, True)
    b = fa.attention_varlen_backward(tq, tk, tv, o, lse, tg, tcq, tck, 513, 513, 0.1, True)
    c = fa.attention_varlen_backward(tq, tk, tv, o, lse, tg, tcq, tck, 513, 513, 0.1, True,
                                     grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y)
        assert torch.equal(x.to(torch.bfloat16), z)


def test_varlen_bwd_mixed_lengths():
    """Eight causal sequences of seeded lengths up to 2048 at the prefill head shape
    (16 heads of 128): every head of every sequence elementwise within the oracle's
    bound, O and LSE from the oracle; then end to end from the GPU forward's O and
    LSE, two heads of every sequence within 1e-2 in relative norm."""
    H, d = 16, 128
    lens = W.varlen_lengths(91, 8, 2048)
    say(f"varlen bwd mixed lengths {lens.tolist()}")
    q, k, v, do, cq, ck = varlen_bwd_inputs(12400, lens, lens, H, d, 1.0)
    assert np.array_equal(cq, ck)  # self-attention lengths: one row range per sequence
    tq, tk, tv, tg = (to_dev(x, "bf16") for x in (q, k, v, do))
    tcq, tck = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    n = int(lens.max())
    scale = 1.0 / np.sqrt(d)
    items = [(b, h) for b in range(len(lens)) for h in range(H)]

    def one(bh):
        b, h = bh
        r = slice(int(cq[b]), int(cq[b + 1]))
        sl = lambda x: W.to_float(x[r, h], "bf16")  # noqa: E731
        nb = int(lens[b])
        return (O.attention_bh(sl(q), sl(k), sl(v), np.arange(nb), nb, scale, True),
                O.attention_bwd_bh(sl(q), sl(k), sl(v), sl(do), nb, scale, True, with_bounds=True))

    say("varlen bwd: oracle forward and backward, every head of every sequence")
    ref = oracle_map(one, items)
    o_ref = np.zeros((int(cq[-1]), H, d), np.float32)
    l_ref = np.zeros((H, int(cq[-1])), np.float32)
    for (b, h), ((ro, rl), _) in zip(items, ref):
        o_ref[cq[b]:cq[b + 1], h], l_ref[h, cq[b]:cq[b + 1]] = ro, rl
    dq, dk, dv = (x.cpu().numpy() for x in fa.attention_varlen_backward(
        tq, tk, tv, torch.from_numpy(o_ref).cuda(), torch.from_numpy(l_ref).cuda(), tg, tcq, tck,
        n, n, scale, True))
    for (b, h), (_, (rq, rk, rv, _, bd)) in zip(items, ref):
        r = slice(int(cq[b]), int(cq[b + 1]))
        check_grad(dq[r, h], rq, bd["dq"], f"seq {b} h{h} dQ", bd["dq_cancel"])
        check_grad(dk[r, h], rk, bd["dk"], f"seq {b} h{h} dK", bd["dk_cancel"])
        check_grad(dv[r, h], rv, bd["dv"], f"seq {b} h{h} dV")

    o, lse = fa.attention_varlen(tq, tk, tv, tcq, tck, n, n, scale, True)
    dq, dk, dv = (x.cpu().numpy() for x in
                  fa.attention_varlen_backward(tq, tk, tv, o, lse, tg, tcq, tck, n, n, scale, True))
    assert not (np.isnan(dq).any() or np.isnan(dk).any() or np.isnan(dv).any())
    for (b, h), (_, (rq, rk, rv, _, _)) in zip(items, ref):
        if h not in (b % H, (5 * b + 3) % H):
            continue
        r = slice(int(cq[b]), int(cq[b + 1]))
        for got, rr, name in ((dq[r, h], rq, "dQ"), (dk[r, h], rk, "dK"), (dv[r, h], rv, "dV")):
            rel = np.linalg.norm(got - rr) / max(np.linalg.norm(rr), 1e-30)
            assert rel <= 1e-2, (b, h, name, rel)


# --------------------------------------------------------------------------
# Decode over an E4M3 paged cache (fa_fwd_splitkv_fp8)
# --------------------------------------------------------------------------
# The kernel widens the codes exactly and works in fp32 with unrounded
# probabilities, as the bf16 decode does, so O is held to the fp32 bound after
# dividing by V's descale (the output scales with it), and LSE to the usual one.
FP8_DECODE_CASES = [
    # (d, H, max_k, page_size, num_splits, seqlens or None, causal, wl, wr, alibi, cap, kd, vd)
    (128, 2, 1000, 64, 4, [1000, 0, 1, 513, 64, 999], True, -1, -1, False, 0.0, 1.0, 1.0),
    (64, 3, 777, 16, 16, [777, 5, 300, 0], True, 100, 0, True, 0.0, 0.5, 2.0),
    (128, 2, 4096, 256, 16, None, True, -1, -1, True, 30.0, 0.25, 0.125),
    (128, 2, 300, 7, 3, [300, 4, 0, 150], True, 50, 0, False, 10.0, 1.0, 1.0),
    (64, 2, 500, 32, 5, None, False, -1, -1, False, 0.0, 3.0, 1.0),
    (128, 1, 2000, 128, 7, [2000, 1999, 1000], False, 300, 40, True, 0.0, 0.75, 0.5),
    # Large enough for four heads per workgroup (at least 256 workgroups, 1024 keys per split);
    # 33 and 31 heads leave a partial last group.
    (128, 33, 8192, 256, 8, [8192, 5000, 1, 0], True, 3000, 0, True, 30.0, 0.5, 0.25),
    (128, 31, 8192, 256, 8, [8192] * 4, True, -1, -1, False, 0.0, 1.0, 1.0),
]


def fp8_decode_case(case, seed, B=None):
    d, H, nk, ps, S, seqlens, causal, wl, wr, alibi, cap, kd, vd = case
    B = len(seqlens) if seqlens else (B or 3)
    w = W.Workload(0, "fp8_decode", B=B, H=H, Nq=1, Nk=nk, d=d, dtype="fp8", causal=causal,
                   paged=True, page_size=ps, pool_factor=1.3, num_splits=S, seed=seed)
    q, kc, vc, bt = W.gen_paged(w, seqlens=seqlens)
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    tsl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32).cuda()
    scale = 1.0 / np.sqrt(d)
    o_part, lse_part = fa.attention_paged_splitkv_fp8(
        to_dev(q, "bf16"), torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(), kd, vd,
        torch.from_numpy(bt).cuda(), nk, S, scale, causal, wl, wr, ts, cap, cache_seqlens=tsl)
    o, lse = fa.combine(o_part, lse_part)
    torch.cuda.synchronize()
    return w, q, kc, vc, bt, slopes, scale, o_part.cpu().numpy(), lse_part.cpu().numpy(), \
        o.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("case", FP8_DECODE_CASES)
def test_fp8_decode_small(case):
    d, H, nk, ps, S, seqlens, causal, wl, wr, alibi, cap, kd, vd = case
    say(f"fp8 decode {case}")
    w, q, kc, vc, bt, slopes, scale, op, lp, o, lse = fp8_decode_case(
        case, 13000 + FP8_DECODE_CASES.index(case))
    lens = seqlens or [nk] * w.B
    kf, vf = W.to_float(kc, "fp8") * kd, W.to_float(vc, "fp8") * vd
    k = np.zeros((w.B, nk, H, d))
    v = np.zeros((w.B, nk, H, d))
    for b, n in enumerate(lens):
        k[b, :n] = O.paged_gather_ref(kf, bt, b, n)
        v[b, :n] = O.paged_gather_ref(vf, bt, b, n)
    rop, rlp = O.splitkv_ref(W.to_float(q, "bf16"), k, v, S, ps, scale, causal, wl, wr, slopes,
                             cap, seqlens_k=seqlens)
    check(op / vd, lp, rop / vd, rlp, "fp32", "partials")
    ro, rl = O.combine_ref(rop, rlp)
    check(o.transpose(0, 2, 1, 3) / vd, lse, ro / vd, rl, "fp32", "combined")


def test_fp8_decode_long_cache_sampled():
    """32768 keys per sequence in 256-key pages, 16 splits, head_dim 128:
    sampled (b, h) pairs against the oracle; no NaN from the poisoned pool."""
    case = (128, 4, 32768, 256, 16, [32768, 20000, 1, 0], True, -1, -1, False, 0.0, 0.5, 0.25)
    say("fp8 decode long cache")
    w, q, kc, vc, bt, slopes, scale, op, lp, o, lse = fp8_decode_case(case, 13100)
    assert not np.isnan(op).any() and not np.isnan(o).any()
    kd, vd = 0.5, 0.25
    for b, h in [(0, 0), (0, 3), (1, 2), (2, 1), (3, 1)]:
        n = case[5][b]
        qf = W.to_float(q[b, :, h], "bf16")
        k = np.zeros((1, w.Nk, 1, w.d))
        v = np.zeros((1, w.Nk, 1, w.d))
        k[0, :n, 0] = O.paged_gather_ref(W.to_float(kc[:, :, h:h + 1], "fp8") * kd, bt, b, n)[:, 0]
        v[0, :n, 0] = O.paged_gather_ref(W.to_float(vc[:, :, h:h + 1], "fp8") * vd, bt, b, n)[:, 0]
        rop, rlp = O.splitkv_ref(qf[None, :, None], k, v, w.num_splits, w.page_size, scale, True,
                                 seqlens_k=[n])
        check(op[:, b:b + 1, h:h + 1] / vd, lp[:, b:b + 1, h:h + 1], rop / vd, rlp, "fp32",
              f"partials b{b} h{h}")


def test_fp8_decode_every_code():
    """A cache whose keys and values cycle through all 254 finite E4M3 codes
    (subnormals, +-0 and +-448 included), read with small descales so the scores
    stay moderate: the kernel's widening of every code matches the oracle's."""
    d, H, nk, ps, S = 128, 2, 1024, 64, 4
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert len(codes) == 254
    rng = np.random.default_rng(13200)
    B = 2
    pages = nk // ps
    pool = B * pages + 3
    kc = np.full((pool, ps, H, d), W.E4M3_NAN_BITS, dtype=np.uint8)
    vc = np.full((pool, ps, H, d), W.E4M3_NAN_BITS, dtype=np.uint8)
    bt = rng.permutation(pool)[: B * pages].reshape(B, pages).astype(np.int32)
    for b in range(B):
        for h in range(H):
            ks = codes[(np.arange(nk * d) * 7 + 31 * b + 5 * h) % 254].reshape(nk, d)
            vs = codes[(np.arange(nk * d) * 11 + 17 * b + 3 * h) % 254].reshape(nk, d)
            W.scatter_pages(kc, bt, b, h, ks, ps)
            W.scatter_pages(vc, bt, b, h, vs, ps)
    q = W.gen_tensor(13201, W.TENSOR_Q, B, 1, H, d, 1.0, "bf16")
    kd, vd = 2.0 ** -10, 2.0 ** -6
    scale = 1.0 / np.sqrt(d)
    say("fp8 decode every code")
    o_part, lse_part = fa.attention_paged_splitkv_fp8(
        to_dev(q, "bf16"), torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(), kd, vd,
        torch.from_numpy(bt).cuda(), nk, S, scale, True)
    torch.cuda.synchronize()
    k = np.stack([O.paged_gather_ref(W.to_float(kc, "fp8") * kd, bt, b, nk) for b in range(B)])
    v = np.stack([O.paged_gather_ref(W.to_float(vc, "fp8") * vd, bt, b, nk) for b in range(B)])
    rop, rlp = O.splitkv_ref(W.to_float(q, "bf16"), k, v, S, ps, scale, True)
    # fp32 arithmetic on values up to 448 vd: the bound is relative to max|v|.
    vmax = float(np.abs(v).max())
    assert vmax == 448.0 * vd
    check(o_part.cpu().numpy() / vmax, lse_part.cpu().numpy(), rop / vmax, rlp, "fp32", "every code")


# --------------------------------------------------------------------------
# Capture in a HIP graph: a serving step (cache append + split pass + combine)
# --------------------------------------------------------------------------
def test_decode_step_replays_from_a_hip_graph():
    """The library allocates and clears nothing, so a decode step (append of the
    step's key and value, split pass, combine) captures as three kernel nodes.
    Every replay, with eager work and synchronisations in between, equals the
    eager call bit for bit (the append rewrites the same rows each time)."""
    w = W.Workload(0, "graph_step", B=3, H=4, Nq=1, Nk=3000, d=128, dtype="bf16", causal=True,
                   paged=True, page_size=64, pool_factor=1.3, num_splits=8, seed=14000)
    seqlens = [2999, 1500, 0]
    q, kc, vc, bt = W.gen_paged(w, seqlens=seqlens)
    kn = W.gen_tensor(14001, W.TENSOR_K, w.B, 1, w.H, w.d, 1.0, "bf16")
    vn = W.gen_tensor(14001, W.TENSOR_V, w.B, 1, w.H, w.d, 1.0, "bf16")
    tq, tkn, tvn = to_dev(q, "bf16"), to_dev(kn, "bf16"), to_dev(vn, "bf16")
    tk, tv = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    tbt = torch.from_numpy(bt).cuda()
    tsl = torch.tensor(seqlens, dtype=torch.int32).cuda()
    S = w.num_splits
    op = torch.empty((S, w.B, w.H, 1, w.d), dtype=torch.float32, device="cuda")
    lp = torch.empty((S, w.B, w.H, 1), dtype=torch.float32, device="cuda")
    o = torch.empty((w.B, 1, w.H, w.d), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.H, 1), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def step():
        st = fa.fa_fwd_splitkv_append(tq, tkn, tvn, tk, tv, tbt, tbt.shape[1], w.page_size, tsl,
                                      op, lp, S, w.B, w.H, 1, w.Nk, w.d, w.scale, True,
                                      stream=stream)
        assert st == 0, st
        assert fa.fa_splitkv_combine(op, lp, S, w.B, w.H, 1, w.d, o, lse, stream=stream) == 0

    say("hip graph: eager step")
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step()
    stream.synchronize()
    o_ref, lse_ref, k_ref = o.clone(), lse.clone(), tk.clone()
    g = torch.cuda.CUDAGraph()
    say("hip graph: capture")
    with torch.cuda.graph(g, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        o.fill_(float("nan"))
        lse.fill_(0.0)
        op.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"hip graph: replay {rep}")
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep
        assert torch.equal(tk.view(torch.int16), k_ref.view(torch.int16)), rep
    # and the eager result is the oracle's
    kf = W.to_float(kc, "bf16")
    vf = W.to_float(vc, "bf16")
    k2, v2 = O.kvcache_append_ref(kf, vf, bt, seqlens, W.to_float(kn, "bf16"), W.to_float(vn, "bf16"))
    k = np.zeros((w.B, w.Nk, w.H, w.d))
    v = np.zeros((w.B, w.Nk, w.H, w.d))
    for b, n in enumerate(seqlens):
        k[b, :n + 1] = O.paged_gather_ref(k2, bt, b, n + 1)
        v[b, :n + 1] = O.paged_gather_ref(v2, bt, b, n + 1)
    rop, rlp = O.splitkv_ref(W.to_float(q, "bf16"), k, v, S, w.page_size, w.scale, True,
                             seqlens_k=[n + 1 for n in seqlens])
    ro, rl = O.combine_ref(rop, rlp)
    check(o_ref.cpu().numpy().transpose(0, 2, 1, 3), lse_ref.cpu().numpy(), ro, rl, "bf16",
          "graph step")


def test_num_splits_from_the_device():
    """fa_num_splits with no compute-unit count asks the device (the same answer
    as with its count given), and the helpers use it when num_splits is None."""
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    for args in [(1, 32, 1, 4096, 128, 256), (2, 8, 512, 4096, 128, 64), (3, 5, 1, 1000, 64, 16)]:
        assert fa.fa_num_splits(*args) == fa.fa_num_splits(*args, num_cus=cus) > 0
    w = W.Workload(0, "auto_split", B=2, H=4, Nq=1, Nk=2000, d=128, dtype="bf16", causal=True,
                   paged=True, page_size=64, pool_factor=1.2, num_splits=1, seed=14100)
    q, kc, vc, bt = W.gen_paged(w)
    tq, tk, tv, tbt = to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16"), torch.from_numpy(bt).cuda()
    S = fa.fa_num_splits(w.B, w.H, 1, w.Nk, w.d, w.page_size)
    op_auto, lp_auto = fa.attention_paged_splitkv(tq, tk, tv, tbt, w.Nk)
    op, lp = fa.attention_paged_splitkv(tq, tk, tv, tbt, w.Nk, S)
    torch.cuda.synchronize()
    assert op_auto.shape[0] == S
    assert torch.equal(op_auto, op) and torch.equal(lp_auto, lp)


@pytest.mark.parametrize("d,alibi,cap,ps,nk", [(128, False, 0.0, 64, 1000), (64, True, 0.0, 64, 1000),
                                               (128, True, 20.0, 64, 1000),
                                               (128, False, 0.0, 16, 1152), (64, True, 0.0, 48, 1152),
                                               (128, True, 20.0, 32, 1152)])
def test_paged_tiles_bitwise_equal_contiguous_split(d, alibi, cap, ps, nk):
    """With pages of a multiple of 16 keys every wavefront's 16-row slab of a 64-key
    tile comes from one page, and with these key counts the paged split chunks are
    fa_fwd_split's: the multi-row paged pass runs the contiguous loop on
    per-wavefront addresses, so the partials are equal bit for bit to those over
    the same keys stored contiguously."""
    B, H, nq, S = 2, 3, 200, 3
    say(f"paged tiles vs contiguous d{d} alibi{alibi} cap{cap} page {ps}")
    assert O.split_bounds(nk, S, ps) == O.split_bounds(nk, S, 64)
    w = W.Workload(0, "ptiles", B=B, H=H, Nq=nq, Nk=nk, d=d, dtype="bf16", causal=True,
                   paged=True, page_size=ps, pool_factor=1.4, num_splits=S, seed=14200 + d + ps)
    q, kc, vc, bt = W.gen_paged(w)
    slopes = W.alibi_slopes(H) if alibi else None
    ts = None if slopes is None else torch.from_numpy(slopes).cuda()
    scale = 1.0 / np.sqrt(d)
    op, lp = fa.attention_paged_splitkv(to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16"),
                                        torch.from_numpy(bt).cuda(), nk, S, scale, True, 100, 0,
                                        ts, cap)
    k = np.stack([O.paged_gather_ref(kc, bt, b, nk) for b in range(B)])  # bf16 bits, contiguous
    v = np.stack([O.paged_gather_ref(vc, bt, b, nk) for b in range(B)])
    oc, lc = fa.attention_split_partials(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                         S, scale, True, 100, 0, ts, cap)
    torch.cuda.synchronize()
    assert torch.equal(op, oc) and torch.equal(lp, lc)


def test_concurrent_streams_match_sequential():
    """The library keeps no state between calls: a prefill, a paged decode and a
    backward launched on three streams at once give the bits they give one after
    another on the default stream."""
    q, k, v = qkv_case(14300, 2, 300, 500, 4, 128, "bf16")
    tq, tk, tv = (to_dev(x, "bf16") for x in (q, k, v))
    w = W.Workload(0, "streams", B=2, H=4, Nq=1, Nk=3000, d=128, dtype="bf16", causal=True,
                   paged=True, page_size=64, pool_factor=1.2, num_splits=6, seed=14301)
    dq, kc, vc, bt = W.gen_paged(w)
    tdq, tkc, tvc, tbt = to_dev(dq, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16"), torch.from_numpy(bt).cuda()
    tg = to_dev(W.gen_tensor(14302, 3, 2, 300, 4, 128, 1.0, "bf16"), "bf16")
    o0, l0 = fa.attention(tq, tk, tv, 0.1, True)

    def work(streams):
        s1, s2, s3 = streams
        with torch.cuda.stream(s1):
            a = fa.attention(tq, tk, tv, 0.1, True, stream=s1)
        with torch.cuda.stream(s2):
            b = fa.decode_paged(tdq, tkc, tvc, tbt, w.Nk, w.num_splits, causal=True, stream=s2)
        with torch.cuda.stream(s3):
            c = fa.attention_backward(tq, tk, tv, o0, l0, tg, 0.1, True, stream=s3)
        torch.cuda.synchronize()
        return [*a, *b, *c]

    say("streams: sequential")
    d = torch.cuda.default_stream()
    ref = work((d, d, d))
    say("streams: concurrent")
    streams = (torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream())
    for _ in range(3):
        got = work(streams)
        for x, y in zip(got, ref):
            assert torch.equal(x, y)
