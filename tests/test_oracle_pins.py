"""Pins for the CPU fp64 oracle: checks against facts that do not come from the oracle.

Each test names what it pins. Together they are chosen so that a plausible slip
in the oracle (a dropped transform, a wrong sign, a shifted diagonal, a
transposed operand, a wrong log base, a wrong split rule) fails at least one.
All CPU, float64.
"""
import importlib
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_examples.json")

MASKS = [  # (causal, window_left, window_right)
    (False, -1, -1), (True, -1, -1), (False, 3, -1), (False, -1, 2), (False, 2, 5),
    (True, 4, -1), (True, 0, -1), (False, 0, 0), (True, 1, 0),
]


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def interval(i, nq, nk, causal, wl, wr):
    """Closed-form allowed key interval [lo, hi] of row i (bottom-right anchored)."""
    ip = i + nk - nq
    lo, hi = 0, nk - 1
    if causal:
        hi = min(hi, ip)
    if wl >= 0:
        lo = max(lo, ip - wl)
    if wr >= 0:
        hi = min(hi, ip + wr)
    return lo, hi


# T1 -----------------------------------------------------------------------
@pytest.mark.parametrize("causal,wl,wr", MASKS)
def test_t1_softmax_rows_sum_to_one(causal, wl, wr):
    nq, nk, d = 7, 11, 5
    q, k = rnd(1, nq, d), rnd(2, nk, d)
    rows = np.arange(nq)
    s = O.scores_ref(q, k, rows, nq, 0.3, causal, wl, wr, slope=0.25, softcap=2.0)
    p, m, l = O.softmax_rows(s)
    ok = O.allowed_mask(nq, nk, rows, causal, wl, wr)
    assert np.all(p >= 0)
    assert np.all(p[~ok] == 0)
    nonempty = ok.any(axis=1)
    np.testing.assert_allclose(p[nonempty].sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[~nonempty] == 0)


# T2 / T4 ------------------------------------------------------------------
@pytest.mark.parametrize("causal,wl,wr", MASKS)
@pytest.mark.parametrize("nq,nk", [(5, 5), (3, 9), (9, 4), (1, 6), (6, 1)])
def test_t2_zero_query_gives_log_count_and_mean(causal, wl, wr, nq, nk):
    """Q = 0: every allowed score is 0, so LSE_i = ln(n_i) and O_i = mean of allowed V."""
    d = 4
    q = np.zeros((1, nq, 1, d))
    k = rnd(3, 1, nk, 1, d)
    v = rnd(4, 1, nk, 1, d)
    o, lse = O.attention_ref(q, k, v, 0.7, causal, wl, wr)
    for i in range(nq):
        lo, hi = interval(i, nq, nk, causal, wl, wr)
        n = max(0, hi - lo + 1)
        if n == 0:
            assert lse[0, 0, i] == -math.inf
            assert np.all(o[0, i, 0] == 0.0)
        else:
            assert abs(lse[0, 0, i] - math.log(n)) <= 1e-12
            np.testing.assert_allclose(o[0, i, 0], v[0, lo:hi + 1, 0].mean(axis=0), atol=1e-12)


def test_t4_bottom_right_counts():
    """Causal counts: Nq=Nk -> i+1; Nq<Nk -> i+off+1; Nq>Nk -> first Nq-Nk rows empty."""
    d = 3
    for nq, nk in [(6, 6), (3, 8), (8, 3)]:
        q = np.zeros((1, nq, 1, d))
        k, v = rnd(5, 1, nk, 1, d), rnd(6, 1, nk, 1, d)
        _, lse = O.attention_ref(q, k, v, 1.0, causal=True)
        off = nk - nq
        for i in range(nq):
            n = i + off + 1
            if n <= 0:
                assert lse[0, 0, i] == -math.inf
            else:
                assert abs(lse[0, 0, i] - math.log(min(n, nk))) < 1e-12


# T3 -----------------------------------------------------------------------
def test_t3_decode_query_sees_all_keys_golden():
    g = json.load(open(GOLDEN))["decode_query_sees_all_keys"]
    d = 8
    for n_cached in g["cached_tokens_N"]:
        nk = n_cached + 1
        q, k, v = rnd(7, 2, 1, 3, d), rnd(8, 2, nk, 3, d), rnd(9, 2, nk, 3, d)
        oc, lc = O.attention_ref(q, k, v, 0.35, causal=True)
        on, ln_ = O.attention_ref(q, k, v, 0.35, causal=False)
        assert np.array_equal(oc, on) and np.array_equal(lc, ln_)
        ok = O.allowed_mask(1, nk, np.arange(1), True, -1, -1)
        assert ok.sum() == nk


# T5 -----------------------------------------------------------------------
@pytest.mark.parametrize("nq,nk", [(5, 5), (4, 9)])
def test_t5_zero_window_selects_diagonal(nq, nk):
    d = 6
    q, k, v = rnd(10, 1, nq, 1, d), rnd(11, 1, nk, 1, d), rnd(12, 1, nk, 1, d)
    o, lse = O.attention_ref(q, k, v, 0.4, False, 0, 0)
    off = nk - nq
    for i in range(nq):
        assert np.array_equal(o[0, i, 0], v[0, i + off, 0])
        s_diag = 0.4 * float(np.dot(q[0, i, 0], k[0, i + off, 0]))
        assert abs(lse[0, 0, i] - s_diag) < 1e-12


def test_t5_wide_window_equals_causal():
    d, nq, nk = 5, 6, 10
    q, k, v = rnd(13, 1, nq, 2, d), rnd(14, 1, nk, 2, d), rnd(15, 1, nk, 2, d)
    a = O.attention_ref(q, k, v, 0.5, True, nk, 0)
    b = O.attention_ref(q, k, v, 0.5, True, -1, -1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# T6 -----------------------------------------------------------------------
@pytest.mark.parametrize("softcap", [0.0, 0.5])
def test_t6_alibi_zero_query_geometric_closed_form(softcap):
    """Q = 0 and causal: the weights are r^k with r = e^-slope over distances k = 0..n-1.

    With softcap on, Q = 0 still gives capped score 0, so the closed form must hold
    unchanged: this fails if the cap were applied after the bias.
    """
    nq, nk, d = 4, 9, 3
    slopes = np.array([0.5, 0.125])
    q = np.zeros((1, nq, 2, d))
    k, v = rnd(16, 1, nk, 2, d), rnd(17, 1, nk, 2, d)
    o, lse = O.attention_ref(q, k, v, 1.0, True, alibi_slopes=slopes, softcap=softcap)
    off = nk - nq
    for h in range(2):
        r = math.exp(-slopes[h])
        for i in range(nq):
            n = i + off + 1
            assert abs(lse[0, h, i] - math.log((1 - r ** n) / (1 - r))) < 1e-12
            w = np.array([r ** kk for kk in range(n)])
            want = sum(w[kk] * v[0, i + off - kk, h] for kk in range(n)) / w.sum()
            np.testing.assert_allclose(o[0, i, h], want, atol=1e-12)


def test_t6_alibi_symmetric_when_not_causal():
    nq = nk = 5
    q = np.zeros((1, nq, 1, 2))
    k, v = rnd(18, 1, nk, 1, 2), rnd(19, 1, nk, 1, 2)
    slope = 0.3
    _, lse = O.attention_ref(q, k, v, 1.0, False, alibi_slopes=[slope])
    for i in range(nq):
        want = math.log(sum(math.exp(-slope * abs(i - j)) for j in range(nk)))
        assert abs(lse[0, 0, i] - want) < 1e-12


# T7 -----------------------------------------------------------------------
def test_t7_zero_slopes_equal_no_alibi():
    q, k, v = rnd(20, 2, 5, 3, 4), rnd(21, 2, 7, 3, 4), rnd(22, 2, 7, 3, 4)
    a = O.attention_ref(q, k, v, 0.5, True, alibi_slopes=np.zeros(3))
    b = O.attention_ref(q, k, v, 0.5, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# T8 -----------------------------------------------------------------------
def test_t8_softcap_bounds_limit_and_value():
    nq, nk, d = 6, 8, 4
    q, k = rnd(23, nq, d) * 1.5, rnd(24, nk, d) * 1.5
    rows = np.arange(nq)
    cap = 3.0
    s = O.scores_ref(q, k, rows, nq, 1.0, softcap=cap)
    assert np.all(np.abs(s) < cap)
    raw = O.scores_ref(q, k, rows, nq, 1.0)
    # order preserved, odd symmetry
    assert np.all(np.argsort(s, axis=1) == np.argsort(raw, axis=1))
    s_neg = O.scores_ref(-q, k, rows, nq, 1.0, softcap=cap)
    np.testing.assert_allclose(s_neg, -s, atol=1e-15)
    # huge cap -> no cap
    s_big = O.scores_ref(q, k, rows, nq, 1.0, softcap=1e12)
    np.testing.assert_allclose(s_big, raw, rtol=0, atol=1e-12)
    # a scaled score equal to the cap maps to cap * tanh(1); tanh(1) = 0.76159415595576488812 (tables)
    one = O.scores_ref(np.array([[2.0]]), np.array([[3.0]]), np.arange(1), 1, 0.5, softcap=3.0)
    assert abs(one[0, 0] - 3.0 * 0.76159415595576488812) < 1e-14
    # small-score regime matches the series s - s^3 / (3 cap^2) to O(s^5)
    tiny = O.scores_ref(np.array([[1e-3]]), np.array([[1.0]]), np.arange(1), 1, 1.0, softcap=2.0)
    assert abs(tiny[0, 0] - (1e-3 - 1e-9 / 12.0)) < 1e-16


def test_t8_softcap_scale_applied_before_cap():
    """Scaling is inside the cap: cap(scale*qk) differs from scale*cap(qk)."""
    q, k = np.array([[4.0]]), np.array([[1.0]])
    s = O.scores_ref(q, k, np.arange(1), 1, 0.25, softcap=1.0)
    assert abs(s[0, 0] - 0.76159415595576488812) < 1e-14


# T9 -----------------------------------------------------------------------
def online_softmax_tiled(q, k, v, rows, nq, scale, causal, wl, wr, slope, cap, bm, bn):
    """Independent tiled streaming softmax (running max / running sum), fp64."""
    nk, d = k.shape[0], v.shape[1]
    off = nk - nq
    o_all = np.zeros((len(rows), d))
    lse_all = np.zeros(len(rows))
    for r0 in range(0, len(rows), bm):
        rr = rows[r0:r0 + bm]
        m = np.full(len(rr), -np.inf)
        l = np.zeros(len(rr))
        acc = np.zeros((len(rr), d))
        for j0 in range(0, nk, bn):
            jj = np.arange(j0, min(nk, j0 + bn))
            s = scale * (q[rr] @ k[jj].T)
            if cap > 0:
                s = cap * np.tanh(s / cap)
            for a, i in enumerate(rr):
                for b, j in enumerate(jj):
                    ip = i + off
                    if slope is not None:
                        s[a, b] -= slope * abs(ip - j)
                    bad = (causal and j > ip) or (wl >= 0 and j < ip - wl) or (wr >= 0 and j > ip + wr)
                    if bad:
                        s[a, b] = -np.inf
            m_new = np.maximum(m, s.max(axis=1))
            base = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
            p = np.exp(s - base[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[jj]
            m = m_new
        for a in range(len(rr)):
            if l[a] > 0:
                o_all[r0 + a] = acc[a] / l[a]
                lse_all[r0 + a] = m[a] + math.log(l[a])
            else:
                lse_all[r0 + a] = -np.inf
    return o_all, lse_all


@pytest.mark.parametrize("nq,nk", [(1, 1), (3, 2), (2, 9), (9, 9), (5, 17), (17, 5), (33, 33)])
def test_t9_tiled_online_softmax_equals_materialised(nq, nk):
    d = 4
    q, k, v = rnd(25, nq, d), rnd(26, nk, d), rnd(27, nk, d)
    rows = np.arange(nq)
    for (causal, wl, wr), slope, cap in itertools.product(MASKS, [None, 0.3], [0.0, 1.5]):
        want_o, want_l = O.attention_bh(q, k, v, rows, nq, 0.6, causal, wl, wr, slope, cap)
        for bm, bn in [(2, 3), (4, 5)]:
            got_o, got_l = online_softmax_tiled(q, k, v, rows, nq, 0.6, causal, wl, wr, slope, cap, bm, bn)
            np.testing.assert_allclose(got_o, want_o, atol=1e-12)
            fin = np.isfinite(want_l)
            assert np.array_equal(fin, np.isfinite(got_l))
            np.testing.assert_allclose(got_l[fin], want_l[fin], atol=1e-12)


# T10 ----------------------------------------------------------------------
@pytest.mark.parametrize("num_splits,page", [(1, 1), (2, 1), (3, 2), (4, 4), (7, 1), (16, 2)])
@pytest.mark.parametrize("causal,wl,wr", [(False, -1, -1), (True, -1, -1), (True, 3, 0)])
def test_t10_combine_of_splits_equals_unsplit(num_splits, page, causal, wl, wr):
    B, nq, nk, H, d = 2, 3, 13, 2, 5
    q, k, v = rnd(28, B, nq, H, d), rnd(29, B, nk, H, d), rnd(30, B, nk, H, d)
    slopes = np.array([0.2, 0.05])
    op, lp = O.splitkv_ref(q, k, v, num_splits, page, 0.45, causal, wl, wr, slopes, 4.0)
    oc, lc = O.combine_ref(op, lp)
    ou, lu = O.attention_ref(q, k, v, 0.45, causal, wl, wr, slopes, 4.0)
    np.testing.assert_allclose(oc, np.transpose(ou, (0, 2, 1, 3)), atol=1e-12)
    np.testing.assert_allclose(lc, lu, atol=1e-12)


def test_t10_combine_with_empty_splits_and_all_empty():
    o = np.array([[1.0, 2.0], [3.0, 4.0], [9.0, 9.0]])
    lse = np.array([math.log(1.0), math.log(3.0), -math.inf])
    oc, lc = O.combine_ref(o[:, None, :], lse[:, None])
    np.testing.assert_allclose(oc[0], [0.25 * 1 + 0.75 * 3, 0.25 * 2 + 0.75 * 4], atol=1e-15)
    assert abs(lc[0] - math.log(4.0)) < 1e-15
    oe, le = O.combine_ref(np.ones((3, 1, 2)), np.full((3, 1), -math.inf))
    assert np.all(oe == 0) and le[0] == -math.inf


def test_split_bounds_golden_and_rules():
    g = json.load(open(GOLDEN))["split_two_blocks_of_1000"]
    assert O.split_bounds(g["seqlen_k"], g["num_splits"], 1) == [tuple(b) for b in g["bounds"]]
    # chunks cover [0, nk) contiguously, never cut a page, trailing ones may be empty
    for nk, s, ps in [(32768, 16, 256), (1000, 3, 64), (5, 8, 1), (300, 4, 256)]:
        b = O.split_bounds(nk, s, ps)
        assert b[0][0] == 0 and b[-1][1] == nk
        for (lo, hi), (lo2, _) in zip(b, b[1:]):
            assert hi == lo2 and lo <= hi
        for lo, _ in b:
            assert lo % ps == 0 or lo == nk
    assert O.split_bounds(32768, 16, 256) == [(2048 * s, 2048 * (s + 1)) for s in range(16)]


# T11 ----------------------------------------------------------------------
@pytest.mark.parametrize("causal,wl,wr", [m for m in MASKS if m != (True, 0, -1)])
@pytest.mark.parametrize("use_alibi", [False, True])
def test_t11_matches_torch_sdpa_fp64(causal, wl, wr, use_alibi):
    """torch's CPU scaled_dot_product_attention with an explicit float mask (fp64)."""
    B, nq, nk, H, d = 2, 6, 9, 3, 8
    q, k, v = rnd(31, B, nq, H, d), rnd(32, B, nk, H, d), rnd(33, B, nk, H, d)
    slopes = np.array([0.5, 0.25, 0.125]) if use_alibi else None
    scale = 0.3
    off = nk - nq
    bias = np.zeros((H, nq, nk))
    for h in range(H):
        for i in range(nq):
            for j in range(nk):
                ip = i + off
                if (causal and j > ip) or (wl >= 0 and j < ip - wl) or (wr >= 0 and j > ip + wr):
                    bias[h, i, j] = -np.inf
                elif use_alibi:
                    bias[h, i, j] = -slopes[h] * abs(ip - j)
    nonempty = np.isfinite(bias).any(axis=2)  # [H, nq]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    want = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.from_numpy(bias)[None], scale=scale).permute(0, 2, 1, 3).numpy()
    got, _ = O.attention_ref(q, k, v, scale, causal, wl, wr, slopes)
    for h in range(H):
        for i in range(nq):
            if nonempty[h, i]:
                np.testing.assert_allclose(got[:, i, h], want[:, i, h], atol=1e-12)


# T12 ----------------------------------------------------------------------
def test_t12_paged_gather_matches_loop_and_identity():
    ps, H, d, B, nk = 4, 2, 3, 2, 10
    npages = 8
    pool = rnd(34, npages, ps, H, d)
    bt = np.array([[5, 1, 7], [0, 6, 2]], dtype=np.int32)
    for b in range(B):
        g = O.paged_gather_ref(pool, bt, b, nk)
        loop = np.stack([pool[bt[b][t // ps], t % ps] for t in range(nk)])
        assert np.array_equal(g, loop)
    contig = rnd(35, B, 12, H, d)
    pool_id = contig.reshape(B * 3, ps, H, d)
    bt_id = np.arange(B * 3, dtype=np.int32).reshape(B, 3)
    for b in range(B):
        assert np.array_equal(O.paged_gather_ref(pool_id, bt_id, b, 12), contig[b])


def test_t12_workload_scatter_roundtrip():
    """The workload's page placement and the oracle's gather are inverses."""
    w = W.Workload(0, "t", B=2, H=3, Nq=1, Nk=37, d=4, dtype="bf16", paged=True,
                   page_size=8, pool_factor=1.5, seed=9)
    q, kc, vc, bt = W.gen_paged(w)
    for b in range(w.B):
        g = O.paged_gather_ref(kc, bt, b, w.Nk)
        for h in range(w.H):
            assert np.array_equal(g[:, h, :], W.gen_slice(w.seed, W.TENSOR_K, b, h, w.Nk, w.d, 1.0, "bf16"))


# T13 ----------------------------------------------------------------------
def test_t13_key_permutation_invariance():
    q, k, v = rnd(36, 1, 4, 2, 5), rnd(37, 1, 11, 2, 5), rnd(38, 1, 11, 2, 5)
    perm = np.random.default_rng(39).permutation(11)
    a = O.attention_ref(q, k, v, 0.5, softcap=2.0)
    b = O.attention_ref(q, k[:, perm], v[:, perm], 0.5, softcap=2.0)
    np.testing.assert_allclose(a[0], b[0], atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], atol=1e-12)


# T14 ----------------------------------------------------------------------
def test_t14_single_key():
    q, k, v = rnd(40, 1, 3, 1, 4), rnd(41, 1, 1, 1, 4), rnd(42, 1, 1, 1, 4)
    o, lse = O.attention_ref(q, k, v, 0.9)
    for i in range(3):
        assert np.array_equal(o[0, i, 0], v[0, 0, 0])
        assert abs(lse[0, 0, i] - 0.9 * float(q[0, i, 0] @ k[0, 0, 0])) < 1e-12


# T15 ----------------------------------------------------------------------
def test_t15_generator_reproducible_and_bf16_rounding():
    a = W.gen_slice(3, 1, 0, 2, 16, 8, 1.0, "bf16")
    b = W.gen_slice(3, 1, 0, 2, 16, 8, 1.0, "bf16")
    c = W.gen_slice(3, 1, 0, 3, 16, 8, 1.0, "bf16")
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # rounding matches torch's float32 -> bfloat16 conversion (nearest, ties to even)
    x = np.random.default_rng(0).standard_normal(4096).astype(np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0]  # exact ties
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), tb)
    assert np.array_equal(W.bf16_bits_to_f32(tb), torch.from_numpy(tb.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_golden_scores_at_4096_tokens():
    g = json.load(open(GOLDEN))["scores_at_4096_tokens"]
    n = g["seqlen"]
    s = O.scores_ref(np.ones((n, 1)), np.ones((n, 1)), np.arange(n), n, 1.0)
    assert s.size == n * n and s.size > g["more_than"]


# T16-T20: variable sequence lengths ----------------------------------------
# (Per-sequence lengths: every sequence is its own problem, aligned to its own
# bottom-right corner.)
VARLEN = [(3, 5), (0, 4), (4, 0), (5, 2), (1, 7), (6, 6), (2, 9)]


def pack(lens, H, d, seed):
    """Packed tensor [sum(lens), H, d] and its cumulative offsets."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return rnd(seed, int(cu[-1]), H, d), cu


@pytest.mark.parametrize("causal,wl,wr", MASKS)
def test_t16_varlen_zero_query_counts_per_sequence(causal, wl, wr):
    """Q = 0: LSE of row i of sequence b is ln(n_i) with sequence b's own lengths,
    and O is the mean of sequence b's own allowed V rows."""
    H, d = 2, 3
    lq = [a for a, _ in VARLEN]
    lk = [b for _, b in VARLEN]
    cq = np.concatenate([[0], np.cumsum(lq)])
    k, ck = pack(lk, H, d, 40)
    v, _ = pack(lk, H, d, 41)
    q = np.zeros((int(cq[-1]), H, d))
    o, lse = O.attention_varlen_ref(q, k, v, cq, ck, 0.9, causal, wl, wr)
    for b, (nq, nk) in enumerate(VARLEN):
        for h in range(H):
            for i in range(nq):
                lo, hi = interval(i, nq, nk, causal, wl, wr)
                n = max(0, hi - lo + 1)
                row = cq[b] + i
                if n == 0:
                    assert lse[h, row] == -math.inf and np.all(o[row, h] == 0.0)
                else:
                    assert abs(lse[h, row] - math.log(n)) <= 1e-12
                    np.testing.assert_allclose(o[row, h], v[ck[b] + lo:ck[b] + hi + 1, h].mean(axis=0),
                                               atol=1e-12)


def test_t17_varlen_brute_force_loops():
    """Pure-Python per-element loops over a tiny pack, with cap, ALiBi and a window."""
    H, d, scale, cap = 2, 3, 0.8, 1.7
    slopes = [0.3, 0.1]
    lens = [(2, 3), (3, 1), (1, 4), (4, 4)]
    q, cq = pack([a for a, _ in lens], H, d, 42)
    k, ck = pack([b for _, b in lens], H, d, 43)
    v, _ = pack([b for _, b in lens], H, d, 44)
    for causal, wl, wr in [(True, -1, -1), (False, 1, 2), (True, 2, -1)]:
        o, lse = O.attention_varlen_ref(q, k, v, cq, ck, scale, causal, wl, wr, slopes, cap)
        for b, (nq, nk) in enumerate(lens):
            for h in range(H):
                for i in range(nq):
                    ip = i + nk - nq
                    sc = []
                    for j in range(nk):
                        if (causal and j > ip) or (wl >= 0 and j < ip - wl) or (wr >= 0 and j > ip + wr):
                            continue
                        dot = sum(q[cq[b] + i, h, e] * k[ck[b] + j, h, e] for e in range(d))
                        x = cap * math.tanh(scale * dot / cap) - slopes[h] * abs(ip - j)
                        sc.append((x, j))
                    row = cq[b] + i
                    if not sc:
                        assert lse[h, row] == -math.inf
                        continue
                    den = sum(math.exp(x) for x, _ in sc)
                    assert abs(lse[h, row] - math.log(den)) < 1e-12
                    for e in range(d):
                        want = sum(math.exp(x) * v[ck[b] + j, h, e] for x, j in sc) / den
                        assert abs(o[row, h, e] - want) < 1e-12


def test_t18_varlen_independence_and_pack_order():
    """Changing one sequence's K/V changes only its rows; reversing the packing
    order permutes the outputs and nothing else."""
    H, d = 2, 4
    lq = [a for a, _ in VARLEN]
    lk = [b for _, b in VARLEN]
    q, cq = pack(lq, H, d, 45)
    k, ck = pack(lk, H, d, 46)
    v, _ = pack(lk, H, d, 47)
    o, lse = O.attention_varlen_ref(q, k, v, cq, ck, 0.5, True, 3, -1)
    k2, v2 = k.copy(), v.copy()
    b_hit = 4
    k2[ck[b_hit]:ck[b_hit + 1]] += 1.0
    v2[ck[b_hit]:ck[b_hit + 1]] *= -2.0
    o2, lse2 = O.attention_varlen_ref(q, k2, v2, cq, ck, 0.5, True, 3, -1)
    mine = np.zeros(q.shape[0], dtype=bool)
    mine[cq[b_hit]:cq[b_hit + 1]] = True
    assert np.array_equal(o2[~mine], o[~mine]) and np.array_equal(lse2[:, ~mine], lse[:, ~mine])
    assert not np.allclose(o2[mine], o[mine])
    # reversed order
    order = list(reversed(range(len(VARLEN))))
    qr = np.concatenate([q[cq[b]:cq[b + 1]] for b in order])
    kr = np.concatenate([k[ck[b]:ck[b + 1]] for b in order])
    vr = np.concatenate([v[ck[b]:ck[b + 1]] for b in order])
    cqr = np.concatenate([[0], np.cumsum([lq[b] for b in order])])
    ckr = np.concatenate([[0], np.cumsum([lk[b] for b in order])])
    orr, lr = O.attention_varlen_ref(qr, kr, vr, cqr, ckr, 0.5, True, 3, -1)
    for pos, b in enumerate(order):
        assert np.array_equal(orr[cqr[pos]:cqr[pos + 1]], o[cq[b]:cq[b + 1]])
        assert np.array_equal(lr[:, cqr[pos]:cqr[pos + 1]], lse[:, cq[b]:cq[b + 1]])


def test_t18_varlen_equal_lengths_is_the_batched_problem():
    B, nq, nk, H, d = 3, 4, 6, 2, 5
    q, k, v = rnd(48, B, nq, H, d), rnd(49, B, nk, H, d), rnd(50, B, nk, H, d)
    slopes = np.array([0.25, 0.5])
    ob, lb = O.attention_ref(q, k, v, 0.4, True, 2, 0, slopes, 3.0)
    cq, ck = np.arange(B + 1) * nq, np.arange(B + 1) * nk
    ov, lv = O.attention_varlen_ref(q.reshape(B * nq, H, d), k.reshape(B * nk, H, d),
                                    v.reshape(B * nk, H, d), cq, ck, 0.4, True, 2, 0, slopes, 3.0)
    np.testing.assert_allclose(ov, ob.reshape(B * nq, H, d), atol=1e-14)
    np.testing.assert_allclose(lv, np.transpose(lb, (1, 0, 2)).reshape(H, B * nq), atol=1e-14)


@pytest.mark.parametrize("num_splits,page", [(1, 1), (3, 2), (4, 4), (16, 2)])
@pytest.mark.parametrize("nq,causal,wl,wr", [(1, True, -1, -1), (3, True, -1, -1), (3, False, 2, 1),
                                            (5, True, 4, 0)])
def test_t19_seqlens_split_equals_truncated_cache(num_splits, page, nq, causal, wl, wr):
    """Per-sequence key counts: combining the splits gives the attention over the
    first seqlens[b] keys alone (later cache rows play no part)."""
    B, nk, H, d = 4, 13, 2, 3
    seqlens = [13, 0, 5, 8]
    q, k, v = rnd(51, B, nq, H, d), rnd(52, B, nk, H, d), rnd(53, B, nk, H, d)
    slopes = np.array([0.2, 0.07])
    op, lp = O.splitkv_ref(q, k, v, num_splits, page, 0.6, causal, wl, wr, slopes, 2.5,
                           seqlens_k=seqlens)
    oc, lc = O.combine_ref(op, lp)
    for b, n in enumerate(seqlens):
        kb, vb = k[b:b + 1, :n].copy(), v[b:b + 1, :n].copy()
        if n == 0:
            assert np.all(lc[b] == -math.inf) and np.all(oc[b] == 0.0)
            continue
        ou, lu = O.attention_ref(q[b:b + 1], kb, vb, 0.6, causal, wl, wr, slopes, 2.5)
        np.testing.assert_allclose(oc[b], np.transpose(ou[0], (1, 0, 2)), atol=1e-12)
        np.testing.assert_allclose(lc[b], lu[0], atol=1e-12)
    # Rows past seqlens[b] must not matter: poison them.
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(seqlens):
        k2[b, n:] = np.nan
        v2[b, n:] = np.nan
    op2, lp2 = O.splitkv_ref(q, k2, v2, num_splits, page, 0.6, causal, wl, wr, slopes, 2.5,
                             seqlens_k=seqlens)
    assert np.array_equal(op2, op) and np.array_equal(lp2, lp)


def test_t20_seqlens_chunks_and_decode_counts():
    """Q = 0 decode (Nq = 1, causal): split s of sequence b holds the keys of its
    own chunk, C_b = ceil(n_b / S) rounded up to the page, so its LSE is
    ln(#keys in that chunk); merged, LSE = ln(n_b)."""
    B, nk, H, d, S, ps = 5, 40, 1, 2, 4, 4
    seqlens = [40, 1, 0, 17, 33]
    q = np.zeros((B, 1, H, d))
    k, v = rnd(54, B, nk, H, d), rnd(55, B, nk, H, d)
    op, lp = O.splitkv_ref(q, k, v, S, ps, 1.0, True, seqlens_k=seqlens)
    want_chunks = {40: [12, 12, 12, 4], 1: [1, 0, 0, 0], 0: [0, 0, 0, 0], 17: [8, 8, 1, 0],
                   33: [12, 12, 9, 0]}
    for b, n in enumerate(seqlens):
        for s, cnt in enumerate(want_chunks[n]):
            if cnt == 0:
                assert lp[s, b, 0, 0] == -math.inf and np.all(op[s, b, 0, 0] == 0.0)
            else:
                assert abs(lp[s, b, 0, 0] - math.log(cnt)) < 1e-12
    _, lc = O.combine_ref(op, lp)
    for b, n in enumerate(seqlens):
        assert (lc[b, 0, 0] == -math.inf) if n == 0 else abs(lc[b, 0, 0] - math.log(n)) < 1e-12


# T21-T22: appending the new keys to a paged cache -----------------------------
def test_t21_kvcache_append_positions_by_hand():
    """Pages of 2 rows, sequence 0 mapped to pages [3, 0, 1] and holding 3 keys:
    its new keys 3 and 4 land in page 0 row 1 and page 1 row 0; sequence 1
    (pages [2, 4], 0 keys) gets new keys 0 and 1 in page 2 rows 0 and 1. No
    other pool row changes."""
    H, d = 1, 2
    pool = rnd(60, 5, 2, H, d)
    vpool = rnd(61, 5, 2, H, d)
    bt = np.array([[3, 0, 1], [2, 4, 4]])
    kn, vn = rnd(62, 2, 2, H, d), rnd(63, 2, 2, H, d)
    kc, vc = O.kvcache_append_ref(pool, vpool, bt, [3, 0], kn, vn)
    assert np.array_equal(kc[0, 1], kn[0, 0]) and np.array_equal(kc[1, 0], kn[0, 1])
    assert np.array_equal(kc[2, 0], kn[1, 0]) and np.array_equal(kc[2, 1], kn[1, 1])
    assert np.array_equal(vc[0, 1], vn[0, 0]) and np.array_equal(vc[2, 1], vn[1, 1])
    changed = {(0, 1), (1, 0), (2, 0), (2, 1)}
    for pg in range(5):
        for row in range(2):
            if (pg, row) not in changed:
                assert np.array_equal(kc[pg, row], pool[pg, row])
                assert np.array_equal(vc[pg, row], vpool[pg, row])


@pytest.mark.parametrize("nq,causal,wl,wr", [(1, True, -1, -1), (3, True, -1, -1), (2, False, 4, 1),
                                            (4, True, 2, 0)])
def test_t22_append_then_attend_equals_attention_over_the_joined_keys(nq, causal, wl, wr):
    B, nk, H, d, S, ps = 3, 12, 2, 3, 3, 2
    seqlens = [5, 0, 8]
    q = rnd(64, B, nq, H, d)
    k, v = rnd(65, B, nk, H, d), rnd(66, B, nk, H, d)
    kn, vn = rnd(67, B, nq, H, d), rnd(68, B, nq, H, d)
    slopes = np.array([0.3, 0.1])
    op, lp = O.splitkv_append_ref(q, k, v, kn, vn, seqlens, S, ps, 0.7, causal, wl, wr, slopes, 3.0)
    oc, lc = O.combine_ref(op, lp)
    for b, n in enumerate(seqlens):
        kj = np.concatenate([k[b, :n], kn[b]])[None]
        vj = np.concatenate([v[b, :n], vn[b]])[None]
        ou, lu = O.attention_ref(q[b:b + 1], kj, vj, 0.7, causal, wl, wr, slopes, 3.0)
        np.testing.assert_allclose(oc[b], np.transpose(ou[0], (1, 0, 2)), atol=1e-12)
        np.testing.assert_allclose(lc[b], lu[0], atol=1e-12)


def test_t22_decode_after_append_sees_every_key():
    """One new token per sequence, Q = 0, causal: it sees its n_b cached keys and
    itself, so LSE = ln(n_b + 1) and O is the mean of those n_b + 1 V rows."""
    B, nk, H, d = 4, 9, 1, 2
    seqlens = [0, 3, 8, 5]
    q = np.zeros((B, 1, H, d))
    k, v = rnd(69, B, nk, H, d), rnd(70, B, nk, H, d)
    kn, vn = rnd(71, B, 1, H, d), rnd(72, B, 1, H, d)
    op, lp = O.splitkv_append_ref(q, k, v, kn, vn, seqlens, 4, 1, 1.0, True)
    oc, lc = O.combine_ref(op, lp)
    for b, n in enumerate(seqlens):
        assert abs(lc[b, 0, 0] - math.log(n + 1)) < 1e-12
        want = np.concatenate([v[b, :n, 0], vn[b, :, 0]]).mean(axis=0)
        np.testing.assert_allclose(oc[b, 0, 0], want, atol=1e-12)


# T23-T26: the backward pass ------------------------------------------------------
BWD_VARIANTS = [  # (nq, nk, causal, wl, wr, slope, cap)
    (3, 5, False, -1, -1, None, 0.0), (4, 4, True, -1, -1, None, 0.0),
    (5, 3, True, -1, -1, 0.3, 0.0),          # Nq > Nk: the first rows see no key
    (3, 6, True, 2, 0, None, 1.5), (4, 5, False, 1, 2, 0.2, 2.0), (2, 7, True, -1, -1, 0.5, 0.8),
]


def _loss(q, k, v, g, scale, causal, wl, wr, slope, cap):
    o, _ = O.attention_bh(q, k, v, np.arange(q.shape[0]), q.shape[0], scale, causal, wl, wr,
                          slope, cap)
    return float((o * g).sum())


@pytest.mark.parametrize("nq,nk,causal,wl,wr,slope,cap", BWD_VARIANTS)
def test_t23_backward_matches_central_differences(nq, nk, causal, wl, wr, slope, cap):
    """L = sum(O * G): every entry of dQ, dK, dV against (L(x + e) - L(x - e)) / 2e of
    the forward oracle (float64, e = 1e-6)."""
    d, scale, eps = 3, 0.7, 1e-6
    q, k, v, g = rnd(80, nq, d), rnd(81, nk, d), rnd(82, nk, d), rnd(83, nq, d)
    dq, dk, dv, _ = O.attention_bwd_bh(q, k, v, g, nq, scale, causal, wl, wr, slope, cap)
    for x, grad in ((q, dq), (k, dk), (v, dv)):
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, g, scale, causal, wl, wr, slope, cap)
            x[idx] = old - eps
            lm = _loss(q, k, v, g, scale, causal, wl, wr, slope, cap)
            x[idx] = old
            assert abs((lp - lm) / (2 * eps) - grad[idx]) < 1e-7, (idx, grad[idx])


@pytest.mark.parametrize("causal,wl,wr,use_alibi,cap", [
    (False, -1, -1, False, 0.0), (True, -1, -1, True, 0.0), (True, 3, 0, False, 4.0),
    (False, 2, 5, True, 2.5)])
def test_t24_backward_matches_torch_autograd_fp64(causal, wl, wr, use_alibi, cap):
    """torch's own autograd through its float64 softmax and matmuls (CPU)."""
    B, nq, nk, H, d, scale = 2, 6, 9, 2, 4, 0.45
    q, k, v, g = rnd(84, B, nq, H, d), rnd(85, B, nk, H, d), rnd(86, B, nk, H, d), rnd(87, B, nq, H, d)
    slopes = np.array([0.25, 0.6]) if use_alibi else None
    dq, dk, dv, _ = O.attention_bwd_ref(q, k, v, g, scale, causal, wl, wr, slopes, cap)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = torch.einsum("bihd,bjhd->bhij", tq, tk) * scale
    if cap > 0:
        s = cap * torch.tanh(s / cap)
    i = torch.arange(nq)[:, None] + (nk - nq)
    j = torch.arange(nk)[None, :]
    if use_alibi:
        s = s - torch.tensor(slopes)[None, :, None, None] * (i - j).abs()
    ok = torch.ones(nq, nk, dtype=torch.bool)
    if causal:
        ok &= j <= i
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    s = s.masked_fill(~ok, float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(g))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal,wl,wr,slope", [(False, -1, -1, None), (True, -1, -1, 0.4),
                                                (True, 2, 0, None)])
def test_t25_backward_shift_invariances(causal, wl, wr, slope):
    """Adding one vector to every key moves each row's scores by a constant, which the
    softmax ignores, so the dK rows sum to 0; adding one vector to every value moves
    each non-empty row's output by it, so the dV rows sum to the dO of those rows."""
    nq, nk, d = 6, 8, 3
    q, k, v, g = rnd(88, nq, d), rnd(89, nk, d), rnd(90, nk, d), rnd(91, nq, d)
    dq, dk, dv, _ = O.attention_bwd_bh(q, k, v, g, nq, 0.8, causal, wl, wr, slope, 0.0)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    nonempty = O.allowed_mask(nq, nk, np.arange(nq), causal, wl, wr).any(axis=1)
    np.testing.assert_allclose(dv.sum(axis=0), g[nonempty].sum(axis=0), atol=1e-12)


def test_t26_backward_row_term_is_do_dot_o():
    B, nq, nk, H, d = 2, 5, 7, 2, 4
    q, k, v, g = rnd(92, B, nq, H, d), rnd(93, B, nk, H, d), rnd(94, B, nk, H, d), rnd(95, B, nq, H, d)
    o, _ = O.attention_ref(q, k, v, 0.5, True, -1, -1, np.array([0.1, 0.2]), 3.0)
    _, _, _, D = O.attention_bwd_ref(q, k, v, g, 0.5, True, -1, -1, np.array([0.1, 0.2]), 3.0)
    np.testing.assert_allclose(D, np.einsum("bihd,bihd->bhi", g, o), atol=1e-12)


# T31: the backward's tolerance magnitudes ------------------------------------------
def _loop_backward(q, k, v, g, scale, causal, wl, wr, slope, cap, p_pert=None, dz_pert=None,
                   dpd_pert=None):
    """dQ, dK, dV by pure-Python per-element loops, with optional perturbations of the
    intermediates the kernels round: p_pert(i, j) is added to P_ij where it enters
    dV = P^T dO, dpd_pert(i, j) to dP_ij - D_i, dz_pert(i, j) to dZ_ij where it enters
    dQ and dK. Also returns the unperturbed P, dZ, O, the cap derivative (1 - tanh^2)
    and the absolute-term sums of the two dot products, A_ij = sum_c |dO_ic v_jc| and
    B_i = sum_c |dO_ic O_ic|."""
    nq, d = len(q), len(q[0])
    nk = len(k)
    zero = lambda i, j: 0.0  # noqa: E731
    p_pert, dz_pert, dpd_pert = p_pert or zero, dz_pert or zero, dpd_pert or zero
    P = [[0.0] * nk for _ in range(nq)]
    T = [[1.0] * nk for _ in range(nq)]
    for i in range(nq):
        ip = i + nk - nq
        row = {}
        for j in range(nk):
            if (causal and j > ip) or (wl >= 0 and j < ip - wl) or (wr >= 0 and j > ip + wr):
                continue
            z = scale * sum(q[i][c] * k[j][c] for c in range(d))
            s = z
            if cap > 0:
                t = math.tanh(z / cap)
                s = cap * t
                T[i][j] = 1.0 - t * t
            if slope is not None:
                s -= slope * abs(ip - j)
            row[j] = s
        if row:
            m = max(row.values())
            den = sum(math.exp(x - m) for x in row.values())
            for j, x in row.items():
                P[i][j] = math.exp(x - m) / den
    O_ = [[sum(P[i][j] * v[j][c] for j in range(nk)) for c in range(d)] for i in range(nq)]
    A = [[sum(abs(g[i][c] * v[j][c]) for c in range(d)) for j in range(nk)] for i in range(nq)]
    B = [sum(abs(g[i][c] * O_[i][c]) for c in range(d)) for i in range(nq)]
    dz0 = [[0.0] * nk for _ in range(nq)]
    dz = [[0.0] * nk for _ in range(nq)]
    for i in range(nq):
        Di = sum(g[i][c] * O_[i][c] for c in range(d))
        for j in range(nk):
            dp = sum(g[i][c] * v[j][c] for c in range(d))
            dz0[i][j] = P[i][j] * (dp - Di) * T[i][j]
            dz[i][j] = P[i][j] * (dp - Di + dpd_pert(i, j)) * T[i][j] + dz_pert(i, j)
    dq = [[scale * sum(dz[i][j] * k[j][c] for j in range(nk)) for c in range(d)] for i in range(nq)]
    dk = [[scale * sum(dz[i][j] * q[i][c] for i in range(nq)) for c in range(d)] for j in range(nk)]
    dv = [[sum((P[i][j] + p_pert(i, j)) * g[i][c] for i in range(nq)) for c in range(d)]
          for j in range(nk)]
    return np.array(dq), np.array(dk), np.array(dv), P, dz0, T, A, B


@pytest.mark.parametrize("nq,nk,causal,wl,wr,slope,cap", [
    (3, 5, False, -1, -1, None, 0.0), (4, 4, True, -1, -1, 0.3, 0.0),
    (5, 3, True, -1, -1, None, 0.0),          # Nq > Nk: rows (and dQ bounds) that are 0
    (4, 5, False, 1, 2, 0.2, 0.0), (3, 6, True, 2, 0, None, 1.5), (4, 4, False, -1, -1, 0.4, 2.0)])
def test_t31_backward_bounds_are_the_worst_case_perturbations(nq, nk, causal, wl, wr, slope, cap):
    """The magnitudes that set the backward's tolerances, against their meaning rather
    than their formula. A relative change of at most r in every P_ij (where it meets dO)
    moves dV_jc by at most r * bound_dv; of every dZ_ij, dQ_ic and dK_jc by r * bound_dq
    and r * bound_dk; an error of at most e (A_ij + B_i) in dP_ij - D_i (the error bound
    of the two fp32 dot products: e times the sum of the absolute values of their terms)
    moves dQ_ic and dK_jc by at most e * the cancellation magnitudes. Each bound is found
    here as the largest change over every sign pattern of those perturbations (each
    output is linear in them, so the largest sits at a vertex), by loop backwards that
    share nothing with the oracle. Without a cap the bounds are attained exactly; with
    one the cancellation magnitudes take P where the perturbation meets P (1 - tanh^2),
    so they must be at least the largest change."""
    d, scale, r, e = 3, 0.7, 2.0 ** -8, 2.0 ** -16
    qa, ka, va, ga = rnd(96, nq, d), rnd(97, nk, d), rnd(98, nk, d), rnd(99, nq, d)
    q, k, v, g = (x.tolist() for x in (qa, ka, va, ga))
    args = (scale, causal, wl, wr, slope, cap)
    dq0, dk0, dv0, P, dz0, T, A, B = _loop_backward(q, k, v, g, *args)
    _, _, _, _, bd = O.attention_bwd_bh(qa, ka, va, ga, nq, *args, with_bounds=True)

    def worst(n_signs, make_pert, which):
        best = None
        for sig in itertools.product((-1.0, 1.0), repeat=n_signs):
            out = _loop_backward(q, k, v, g, *args, **make_pert(sig))
            ch = np.abs(out[which] - (dq0, dk0, dv0)[which])
            best = ch if best is None else np.maximum(best, ch)
        return best

    got = {
        "dq": worst(nk, lambda s: {"dz_pert": lambda i, j: r * s[j] * abs(dz0[i][j])}, 0) / r,
        "dk": worst(nq, lambda s: {"dz_pert": lambda i, j: r * s[i] * abs(dz0[i][j])}, 1) / r,
        "dv": worst(nq, lambda s: {"p_pert": lambda i, j: r * s[i] * P[i][j]}, 2) / r,
        "dq_cancel": worst(nk, lambda s: {"dpd_pert": lambda i, j: e * s[j] * (A[i][j] + B[i])},
                           0) / e,
        "dk_cancel": worst(nq, lambda s: {"dpd_pert": lambda i, j: e * s[i] * (A[i][j] + B[i])},
                           1) / e,
    }
    for name, want in got.items():
        tol = 1e-9 * max(float(np.abs(want).max()), 1e-12)
        if cap > 0 and name.endswith("cancel"):
            assert np.all(bd[name] >= want - tol), name
            assert np.all(bd[name] <= want / min(min(t) for t in T) + tol), name
        else:
            np.testing.assert_allclose(bd[name], want, rtol=1e-9, atol=tol, err_msg=name)
    assert max(float(np.abs(x).max()) for x in bd.values()) > 0


def _bf16(x):
    """Round float64 values to bf16 (nearest even) through float32, as torch does."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("causal,wl,wr,slope,cap", [(True, -1, -1, None, 0.0),
                                                    (False, 20, 5, 0.05, 0.0),
                                                    (True, -1, -1, 0.1, 8.0)])
def test_t31_backward_bounds_cover_simulated_rounding(causal, wl, wr, slope, cap):
    """The tolerance the GPU tests apply, 2^-8 * bound + 2^-16 * cancellation (bf16's unit
    roundoff on the P and dZ operands; fp32 dot products over 64 terms), covers a
    backward computed with exactly that rounding: P and dZ rounded to bf16 before the
    products, dP and D summed in float32."""
    nq, nk, d, scale = 40, 70, 64, 0.125
    q, k, v, g = (_bf16(rnd(s, n, d) * 2.0) for s, n in ((100, nq), (101, nk), (102, nk), (103, nq)))
    rq, rk, rv, _, bd = O.attention_bwd_bh(q, k, v, g, nq, scale, causal, wl, wr, slope, cap,
                                           with_bounds=True)
    s = O.scores_ref(q, k, np.arange(nq), nq, scale, causal, wl, wr, slope, cap)
    p, _, _ = O.softmax_rows(s)
    o = p @ v
    dp = (g.astype(np.float32) @ v.astype(np.float32).T).astype(np.float64)
    D = np.einsum("ic,ic->i", g.astype(np.float32), o.astype(np.float32)).astype(np.float64)
    dz = p * (dp - D[:, None])
    if cap > 0:
        t = np.tanh((q @ k.T) * scale / cap)
        dz = dz * (1.0 - t * t)
    pb, dzb = _bf16(p), _bf16(dz)
    sim = {"dq": scale * (dzb @ k), "dk": scale * (dzb.T @ q), "dv": pb.T @ g}
    for name, ref, cancel in (("dq", rq, bd["dq_cancel"]), ("dk", rk, bd["dk_cancel"]),
                              ("dv", rv, 0.0)):
        err = np.abs(sim[name] - ref)
        tol = 2.0 ** -8 * bd[name] + 2.0 ** -16 * cancel + 1e-12
        assert np.all(err <= tol), (name, float((err / tol).max()))
        assert float((err / tol).max()) > 1e-3, name   # the bound is not vacuous


# T32: evaluating a row block over its visible key span -----------------------------
@pytest.mark.parametrize("nq,nk", [(7, 7), (5, 12), (12, 5), (1, 9), (9, 1), (16, 40)])
def test_t32_visible_span_is_the_masks_visible_columns(nq, nk):
    """For every block of consecutive rows, visible_span is the first and one past the
    last key column the mask keeps for some row of the block (the mask itself decides;
    empty when it keeps none), for every mask and split range; for any subset of rows
    it contains every kept column."""
    rng = np.random.default_rng(104)
    for causal, wl, wr in MASKS:
        for key_lo, key_hi in [(0, None), (2, 6), (0, 3), (4, None)]:
            for r0 in range(nq):
                for r1 in range(r0 + 1, nq + 1):
                    rows = np.arange(r0, r1)
                    cols = np.flatnonzero(O.allowed_mask(nq, nk, rows, causal, wl, wr, key_lo,
                                                         key_hi).any(axis=0))
                    a, b = O.visible_span(nq, nk, rows, causal, wl, wr, key_lo, key_hi)
                    if len(cols) == 0:
                        assert b <= a or not O.allowed_mask(nq, nk, rows, causal, wl, wr, key_lo,
                                                            key_hi)[:, a:b].any()
                    else:
                        assert (a, b) == (cols[0], cols[-1] + 1), (causal, wl, wr, r0, r1)
            sub = np.sort(rng.choice(nq, size=min(nq, 3), replace=False))
            cols = np.flatnonzero(O.allowed_mask(nq, nk, sub, causal, wl, wr).any(axis=0))
            a, b = O.visible_span(nq, nk, sub, causal, wl, wr)
            assert len(cols) == 0 or (a <= cols[0] and cols[-1] < b)


@pytest.mark.parametrize("causal,wl,wr", MASKS)
def test_t32_span_evaluation_equals_every_key(causal, wl, wr, monkeypatch):
    """attention_bh (row blocks over their visible spans, blocks forced small) against
    the same rows over every key in one block: masked keys contribute exactly 0."""
    nq, nk, d = 23, 37, 5
    q, k, v = rnd(110, nq, d), rnd(111, nk, d), rnd(112, nk, d)
    for slope, cap in [(None, 0.0), (0.3, 2.0)]:
        rows = np.arange(nq)
        s = O.scores_ref(q, k, rows, nq, 0.6, causal, wl, wr, slope, cap)
        want_o, want_l = O.attend_rows(s, v)
        monkeypatch.setattr(importlib.import_module("oracle.attention_ref"), "_CHUNK_BYTES",
                            8 * nk * 3 * 4)  # blocks of 4 rows
        got_o, got_l = O.attention_bh(q, k, v, rows, nq, 0.6, causal, wl, wr, slope, cap)
        monkeypatch.undo()
        np.testing.assert_allclose(got_o, want_o, atol=1e-13)
        assert np.array_equal(np.isfinite(got_l), np.isfinite(want_l))
        np.testing.assert_allclose(got_l[np.isfinite(want_l)], want_l[np.isfinite(want_l)],
                                   atol=1e-13)
        # The probability-weighted bound over the spans against every key.
        p_all, _, _ = O.softmax_rows(s)
        for weight in (None, lambda x: 0.5 * np.sqrt(x)):
            want = (p_all if weight is None else np.where(p_all > 0, weight(p_all), 0.0)) @ np.abs(v)
            monkeypatch.setattr(importlib.import_module("oracle.attention_ref"), "_CHUNK_BYTES",
                                8 * nk * 3 * 4)
            got = O.prob_weighted_abs_ref(q[None, :, None], k[None, :, None], v[None, :, None], 0.6,
                                          causal, wl, wr, None if slope is None else [slope], cap,
                                          weight=weight)[0, :, 0]
            monkeypatch.undo()
            np.testing.assert_allclose(got, want, atol=1e-13)


# T27-T29: fp8 inputs ----------------------------------------------------------------
def test_t27_e4m3_decode_closed_form_and_torch():
    """E4M3 (1 sign, 4 exponent bits biased by 7, 3 mantissa bits, no infinities)."""
    dec = W.e4m3_bits_to_f32(np.arange(256, dtype=np.uint8)).astype(np.float64)
    assert dec[0x38] == 1.0 and dec[0x7E] == 448.0 and dec[0x01] == 2.0 ** -9
    assert dec[0x08] == 2.0 ** -6 and dec[0x07] == 7 * 2.0 ** -9 and dec[0x40] == 2.0
    assert dec[0x80] == 0.0 and math.copysign(1.0, dec[0x80]) == -1.0
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF]) and np.isfinite(dec[:0x7F]).all()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (dec == ref) | (np.isnan(dec) & np.isnan(ref))
    assert same.all()


def test_t28_e4m3_encode_is_round_to_nearest_even():
    x = np.random.default_rng(73).standard_normal(20000) * 30.0
    x = np.concatenate([x, [1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, -447.0, 0.0]])
    got = W.f32_to_e4m3_bits(x)
    want = torch.tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    assert W.f32_to_e4m3_bits(np.array([500.0, -1e6]))[0] == 0x7E          # saturates
    assert W.f32_to_e4m3_bits(np.array([-1e6]))[0] == 0xFE


def test_t29_probability_weighted_bound():
    """P|V| equals O when V >= 0 and bounds |O| otherwise; it is 0 for rows with no key."""
    B, nq, nk, H, d = 1, 5, 7, 2, 3
    q, k, v = rnd(74, B, nq, H, d), rnd(75, B, nk, H, d), rnd(76, B, nk, H, d)
    o, _ = O.attention_ref(q, k, np.abs(v), 0.6, True)
    np.testing.assert_allclose(O.prob_weighted_abs_ref(q, k, v, 0.6, True), o, atol=1e-14)
    o2, _ = O.attention_ref(q, k, v, 0.6, True, 2, 0, np.array([0.3, 0.1]), 2.0)
    bnd = O.prob_weighted_abs_ref(q, k, v, 0.6, True, 2, 0, np.array([0.3, 0.1]), 2.0)
    assert np.all(bnd >= np.abs(o2) - 1e-14)
    q3, k3, v3 = rnd(77, 1, 6, 1, 2), rnd(78, 1, 2, 1, 2), rnd(79, 1, 2, 1, 2)
    b3 = O.prob_weighted_abs_ref(q3, k3, v3, 1.0, True)                 # Nq > Nk: empty rows
    assert np.all(b3[0, :4] == 0.0)


def _loop_weighted_abs(q, k, v, scale, causal, wl, wr, slope, cap, lo, hi, weight):
    """sum_j w(P_ij) |v_j| with P the softmax over the keys [lo, hi) row i may see,
    written out key by key (mask, cap and ALiBi from their definitions)."""
    nq, nk = q.shape[0], k.shape[0]
    off = nk - nq
    out = np.zeros((nq, v.shape[1]))
    for i in range(nq):
        ip = i + off
        keys, sc = [], []
        for j in range(lo, hi):
            if (causal and j > ip) or (wl >= 0 and j < ip - wl) or (wr >= 0 and j > ip + wr):
                continue
            x = scale * float(np.dot(q[i], k[j]))
            if cap > 0:
                x = cap * math.tanh(x / cap)
            if slope is not None:
                x -= slope * abs(ip - j)
            keys.append(j)
            sc.append(x)
        if not keys:
            continue
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        tot = sum(e)
        for j, ej in zip(keys, e):
            out[i] += weight(ej / tot) * np.abs(v[j])
    return out


@pytest.mark.parametrize("causal,wl,wr,slope,cap", [(True, -1, -1, None, 0.0),
                                                   (False, 3, 2, 0.4, 2.0),
                                                   (True, 5, -1, 0.2, 0.0)])
def test_t29_probability_weighted_bound_over_a_key_range(causal, wl, wr, slope, cap):
    """Restricted to one split's keys [lo, hi), the bound is the split's own softmax
    weighting |V| (checked against a key-by-key loop), and over [0, Nk) it is the
    unrestricted bound."""
    nq, nk, d = 6, 11, 3
    q, k, v = rnd(81, 1, nq, 1, d), rnd(82, 1, nk, 1, d), rnd(83, 1, nk, 1, d)
    slopes = None if slope is None else np.array([slope])
    w = lambda pp: 0.25 * np.sqrt(pp)                  # any function of P; nonlinear on purpose
    for lo, hi in [(0, nk), (0, 4), (4, 8), (8, 11), (3, 3)]:
        got = O.prob_weighted_abs_ref(q, k, v, 0.7, causal, wl, wr, slopes, cap, weight=w,
                                      key_lo=lo, key_hi=hi)[0, :, 0]
        ref = _loop_weighted_abs(q[0, :, 0], k[0, :, 0], v[0, :, 0], 0.7, causal, wl, wr, slope,
                                 cap, lo, hi, lambda pp: 0.25 * math.sqrt(pp))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    full = O.prob_weighted_abs_ref(q, k, v, 0.7, causal, wl, wr, slopes, cap, weight=w)
    np.testing.assert_array_equal(full, O.prob_weighted_abs_ref(q, k, v, 0.7, causal, wl, wr,
                                                                 slopes, cap, weight=w,
                                                                 key_lo=0, key_hi=nk))


def test_t29_e4m3_half_spacing_matches_the_code_table():
    import gpu_common as G
    vals = W.e4m3_bits_to_f32(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)   # 0 .. 448
    for c in range(0x7E):
        lo, hi = vals[c], vals[c + 1]
        for x in (lo, 0.5 * (lo + hi), lo + 0.99 * (hi - lo)):
            assert G.e4m3_half_spacing(x) == (hi - lo) / 2, (c, x)
    # rounding to nearest never moves a value by more than it
    x = np.random.default_rng(80).uniform(0, 256, 5000)
    xr = W.e4m3_bits_to_f32(W.f32_to_e4m3_bits(x)).astype(np.float64)
    assert np.all(np.abs(xr - x) <= G.e4m3_half_spacing(x) * (1 + 1e-12))


def test_t30_varlen_backward_equals_batched_and_is_per_sequence():
    """Equal lengths: the batched backward; mixed lengths: each sequence's gradients
    depend on that sequence alone (checked against central differences of the
    packed forward for one entry per tensor and sequence)."""
    B, nq, nk, H, d = 2, 4, 6, 2, 3
    q, k, v, g = rnd(100, B, nq, H, d), rnd(101, B, nk, H, d), rnd(102, B, nk, H, d), rnd(103, B, nq, H, d)
    sl = np.array([0.2, 0.4])
    bq, bk, bv, _ = O.attention_bwd_ref(q, k, v, g, 0.6, True, 3, 0, sl, 2.0)
    cq, ck = np.arange(B + 1) * nq, np.arange(B + 1) * nk
    vq, vk, vv = O.attention_varlen_bwd_ref(q.reshape(-1, H, d), k.reshape(-1, H, d),
                                            v.reshape(-1, H, d), g.reshape(-1, H, d), cq, ck, 0.6,
                                            True, 3, 0, sl, 2.0)
    np.testing.assert_allclose(vq, bq.reshape(-1, H, d), atol=1e-14)
    np.testing.assert_allclose(vk, bk.reshape(-1, H, d), atol=1e-14)
    np.testing.assert_allclose(vv, bv.reshape(-1, H, d), atol=1e-14)
    lens = [(3, 5), (0, 2), (4, 1), (2, 0)]
    qp, cqp = pack([a for a, _ in lens], H, d, 104)
    kp, ckp = pack([b for _, b in lens], H, d, 105)
    vp_, _ = pack([b for _, b in lens], H, d, 106)
    gp, _ = pack([a for a, _ in lens], H, d, 107)
    dq, dk, dv = O.attention_varlen_bwd_ref(qp, kp, vp_, gp, cqp, ckp, 0.7, True)

    def loss():
        o, _ = O.attention_varlen_ref(qp, kp, vp_, cqp, ckp, 0.7, True)
        return float(np.nansum(o * gp))
    eps = 1e-6
    for x, grad, cu in ((qp, dq, cqp), (kp, dk, ckp), (vp_, dv, ckp)):
        for b in range(len(lens)):
            if cu[b + 1] == cu[b]:
                continue
            idx = (int(cu[b]), 1, 2)
            old = x[idx]
            x[idx] = old + eps
            lp = loss()
            x[idx] = old - eps
            lm = loss()
            x[idx] = old
            assert abs((lp - lm) / (2 * eps) - grad[idx]) < 1e-7
