"""CPU fp64 oracle for exact attention and its split-KV / paged-KV decode form.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this module; it
is called by the tests, by the smoke check and by the bench's CPU baseline leg.

The tiled method reaches, up to rounding order, the plain result of standard
attention, so the oracle is that plain definition written out: materialise the
score matrix S for one (batch, head), apply the score transforms and the mask,
take a row-wise softmax, multiply by V ("FlashAttention及变种改进", section 二.1,
the bottleneck of standard self-attention). Rows are
independent, so the oracle may compute any subset of query rows and may chunk
rows to bound host memory; no other blocking, fusion or reordering is done.

Variant definitions (the flash-attn v2.0-v2.7 update article, its v2.1 to v2.6
entries):

* causal mask aligned to the bottom-right corner of the score matrix: with
  off = Nk - Nq, query row i may see key j iff j <= i + off (v2.1 entry; the
  one-token decode query sees every cached key).
* sliding window (v2.3 entry): keys j in [i + off - window_left,
  i + off + window_right], inclusive; -1 means unbounded on that side.
* ALiBi (v2.4 entry): a linear position penalty, score -= slope_h * |i + off - j|.
* softcap (v2.6 entry): tanh cap on the scaled score,
  s <- softcap * tanh(s / softcap), applied before the bias and the mask.
* split-KV (v2.2 entry): keys are cut along the sequence into contiguous chunks,
  each chunk yields a normalised partial output and its log-sum-exp, and a
  separate reduce step merges the chunks.
* paged KV cache (v2.5 entry): logical key t of sequence b lives in physical page
  block_table[b, t // page_size], row t % page_size.

Variable sequence lengths ("FlashAttention深度解析：从算法创新到产业变革的全面影响",
the closing section on the roadmap, names them as a feature without defining
them). Reading taken here: every sequence of a batch is its own attention
problem over its own query rows and its own keys, with the v2.1 bottom-right
rule applied to that sequence's lengths (off_b = nk_b - nq_b). Two forms:

* a packed batch: sequence b owns query rows [cu_q[b], cu_q[b+1]) of a packed
  q and key rows [cu_k[b], cu_k[b+1]) of packed k and v;
* a paged cache with per-sequence key counts: sequence b uses only its first
  seqlens_k[b] cached keys, and its split chunks are cut from that count.

Appending to the cache ("解密FlashAttention：如何让大语言模型推理速度翻倍", the
sections on the key-value cache and on incremental processing of new tokens):
each step writes its new keys behind a sequence's cached ones and attends over
both, the new queries aligned with the new keys.

Conventions the pages leave open (each is stated with its reason where it is
used): LSE is the natural log of the row's sum of exp over allowed keys; a row
with no allowed key has O = 0 and LSE = -inf; split chunk length is
ceil(Nk / S) rounded up to a whole number of pages.

FP8 inputs ("IO感知技术革命: FlashAttention如何重塑大模型训练的经济学", the
section on FlashAttention-3 and H100 FP8; the deep-analysis page's roadmap):
the pages give no quantisation scheme. Reading taken here: Q, K, V arrive as
E4M3 codes with one descale factor per tensor, and the method computes exact
attention of the dequantised values, so the oracle is attention_ref on those
values; prob_weighted_abs_ref gives the bound that rounding the probabilities
to E4M3 inside the kernel may move O by.

All arithmetic is float64 on the exact input values.
"""
from __future__ import annotations

import numpy as np

NEG_INF = float("-inf")
_CHUNK_BYTES = 256 << 20


# --------------------------------------------------------------------------
# Mask geometry (flash-attn update article, v2.1 and v2.3 entries)
# --------------------------------------------------------------------------
def allowed_mask(nq: int, nk: int, rows: np.ndarray, causal: bool,
                 window_left: int, window_right: int,
                 key_lo: int = 0, key_hi: int | None = None) -> np.ndarray:
    """Boolean [len(rows), nk]: may query row i attend to key j.

    The diagonal is anchored at the bottom-right corner: i' = i + (nk - nq).
    Causal keeps j <= i'. A window keeps i' - window_left <= j <= i' + window_right
    (each side unbounded when negative). key_lo/key_hi further restrict the keys
    to one split chunk [key_lo, key_hi).
    """
    off = nk - nq
    ip = (np.asarray(rows, dtype=np.int64) + off)[:, None]
    j = np.arange(nk, dtype=np.int64)[None, :]
    ok = np.ones((ip.shape[0], nk), dtype=bool)
    if causal:
        ok &= j <= ip
    if window_left >= 0:
        ok &= j >= ip - window_left
    if window_right >= 0:
        ok &= j <= ip + window_right
    if key_lo > 0:
        ok &= j >= key_lo
    if key_hi is not None:
        ok &= j < key_hi
    return ok


# --------------------------------------------------------------------------
# Scores for one (batch, head)
# --------------------------------------------------------------------------
def scores_ref(q_bh: np.ndarray, k_bh: np.ndarray, rows: np.ndarray, nq: int,
               scale: float, causal: bool = False, window_left: int = -1,
               window_right: int = -1, slope: float | None = None,
               softcap: float = 0.0, key_lo: int = 0,
               key_hi: int | None = None, span: tuple | None = None) -> np.ndarray:
    """S[r, j] for the selected query rows: scaled, capped, biased, masked (-inf).

    q_bh: [len(rows), d] (the selected rows), k_bh: [nk, d]. span = (a, b): only the
    columns of keys a..b-1 are formed (S[:, j - a] for key j; positions stay absolute).
    """
    nk = k_bh.shape[0]
    a, b = (0, nk) if span is None else span
    s = (q_bh @ k_bh[a:b].T) * scale                  # standard attention: Q K^T, scaled
    if softcap > 0.0:                                 # v2.6: tanh cap on the scaled score
        s = softcap * np.tanh(s / softcap)
    if slope is not None:                             # v2.4: linear distance penalty
        off = nk - nq
        ip = (np.asarray(rows, dtype=np.int64) + off)[:, None]
        j = np.arange(a, b, dtype=np.int64)[None, :]
        s = s - slope * np.abs(ip - j).astype(np.float64)
    ok = allowed_mask(nq, nk, rows, causal, window_left, window_right, key_lo, key_hi)[:, a:b]
    return np.where(ok, s, NEG_INF)


def visible_span(nq: int, nk: int, rows: np.ndarray, causal: bool, window_left: int,
                 window_right: int, key_lo: int = 0, key_hi: int | None = None):
    """Keys [a, b) that at least one of `rows` may see (a >= b: none).

    Row i sees the interval [i' - window_left, i' + window_right] (i' = i + nk - nq;
    causal caps the right end at i'; -1 leaves a side open) cut to [key_lo, key_hi).
    Both ends grow with i, so every row's interval lies between the smallest row's
    left end and the largest row's right end (for consecutive rows, whose intervals
    touch, that is exactly their union). Keys outside it are masked for every row:
    their probabilities are exactly 0, so leaving them out changes no result.
    """
    rows = np.asarray(rows, dtype=np.int64)
    off = nk - nq
    hi_end = nk if key_hi is None else min(nk, key_hi)
    first, last = int(rows.min()) + off, int(rows.max()) + off
    a = key_lo if window_left < 0 else max(key_lo, first - window_left)
    b = hi_end
    if causal:
        b = min(b, last + 1)
    if window_right >= 0:
        b = min(b, last + window_right + 1)
    return max(0, a), max(0, b)


def softmax_rows(s: np.ndarray):
    """Row softmax of a masked score block. Returns (P, row max m, row sum l).

    A row whose every entry is -inf gets P = 0, m = -inf, l = 0.
    """
    m = s.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m_safe[:, None])                   # exp(-inf) = 0 for masked keys
    l = p.sum(axis=1)
    p = np.where(l[:, None] > 0, p / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return p, m, l


def attend_rows(s: np.ndarray, v_bh: np.ndarray):
    """O = softmax(S) V and LSE = m + ln l for one block of rows."""
    p, m, l = softmax_rows(s)
    o = p @ v_bh
    lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return o, lse


def _row_chunks(rows: np.ndarray, nk: int):
    step = max(1, _CHUNK_BYTES // (8 * max(1, nk) * 3))
    for c0 in range(0, len(rows), step):
        yield rows[c0:c0 + step]


def attention_bh(q_all, k_bh, v_bh, rows, nq, scale, causal=False, window_left=-1,
                 window_right=-1, slope=None, softcap=0.0, key_lo=0, key_hi=None):
    """O [len(rows), d] and LSE [len(rows)] for one (batch, head).

    q_all: [nq, d] (every query row of the head); only `rows` are computed.
    k_bh, v_bh: [nk, d]. key_lo/key_hi restrict the keys to one split chunk.
    """
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), v_bh.shape[1]), dtype=np.float64)
    lse = np.full(len(rows), NEG_INF, dtype=np.float64)
    if k_bh.shape[0] == 0:                            # no key at all: every row is empty
        return o, lse
    pos = 0
    for rc in _row_chunks(rows, k_bh.shape[0]):
        # Only the keys some row of the chunk may see (the others have P = 0).
        a, b = visible_span(nq, k_bh.shape[0], rc, causal, window_left, window_right, key_lo,
                            key_hi)
        if b > a:
            s = scores_ref(q_all[rc], k_bh, rc, nq, scale, causal, window_left,
                           window_right, slope, softcap, key_lo, key_hi, span=(a, b))
            oc, lc = attend_rows(s, v_bh[a:b])
            o[pos:pos + len(rc)] = oc
            lse[pos:pos + len(rc)] = lc
        pos += len(rc)
    return o, lse


def attention_ref(q, k, v, scale, causal=False, window_left=-1, window_right=-1,
                  alibi_slopes=None, softcap=0.0, rows=None, bh=None):
    """Exact attention forward over contiguous tensors.

    q [B, Nq, H, d], k and v [B, Nk, H, d] (any float dtype; computed in fp64).
    rows: optional subset of query rows; bh: optional list of (b, h) pairs.
    Returns O [B, len(rows), H, d] and LSE [B, H, len(rows)]; entries of pairs
    outside bh are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nq, H, _ = q.shape
    rows = np.arange(nq) if rows is None else np.asarray(rows, dtype=np.int64)
    pairs = [(b, h) for b in range(B) for h in range(H)] if bh is None else bh
    o = np.full((B, len(rows), H, v.shape[3]), np.nan)
    lse = np.full((B, H, len(rows)), np.nan)
    for b, h in pairs:
        slope = None if alibi_slopes is None else float(alibi_slopes[h])
        ob, lb = attention_bh(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :], rows, nq,
                              scale, causal, window_left, window_right, slope, softcap)
        o[b, :, h, :] = ob
        lse[b, h, :] = lb
    return o, lse


def prob_weighted_abs_ref(q, k, v, scale, causal=False, window_left=-1, window_right=-1,
                          alibi_slopes=None, softcap=0.0, bh=None, weight=None, key_lo=0,
                          key_hi=None):
    """sum_j w(P_ij) |v_j| per row and column, shaped like attention_ref's O
    (w = identity unless `weight` is given, a function applied to P elementwise).

    If every probability moves by at most w(P) (before the row is normalised by
    the unchanged sum), O_i moves by at most this; it is the bound used where
    probabilities are rounded to a short format (w(P) = r P for a relative
    error r, or half the format's spacing at P). key_lo/key_hi restrict the keys
    to one split chunk, P then being the chunk's own softmax (as in splitkv_ref).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nq, H, _ = q.shape
    pairs = [(b, h) for b in range(B) for h in range(H)] if bh is None else bh
    out = np.full((B, nq, H, v.shape[3]), np.nan)
    rows = np.arange(nq)
    for b, h in pairs:
        slope = None if alibi_slopes is None else float(alibi_slopes[h])
        if k.shape[1] == 0:
            out[b, :, h] = 0.0
            continue
        for rc in _row_chunks(rows, k.shape[1]):
            a, e = visible_span(nq, k.shape[1], rc, causal, window_left, window_right, key_lo,
                                key_hi)
            if e <= a:                                # no visible key: P = 0
                out[b, rc, h] = 0.0
                continue
            s = scores_ref(q[b, rc, h], k[b, :, h], rc, nq, scale, causal, window_left,
                           window_right, slope, softcap, key_lo, key_hi, span=(a, e))
            p, _, _ = softmax_rows(s)
            wp = p if weight is None else np.where(p > 0, weight(p), 0.0)
            out[b, rc, h] = wp @ np.abs(v[b, a:e, h])
    return out


# --------------------------------------------------------------------------
# Backward pass (gradients of the forward above)
# --------------------------------------------------------------------------
def attention_bwd_bh(q_bh, k_bh, v_bh, do_bh, nq, scale, causal=False, window_left=-1,
                     window_right=-1, slope=None, softcap=0.0, with_bounds=False):
    """dQ, dK, dV [n, d] and D [nq] for one (batch, head), by the chain rule.

    The forward is O = P V with P = softmax(S) over the allowed keys and
    S = T(scale * Q K^T), T the tanh cap then the ALiBi shift (a constant).
    With dO given: dV = P^T dO; dP = dO V^T; D_i = sum_j P_ij dP_ij (= dO_i . O_i);
    dS = P * (dP - D); through the cap dZ = dS * (1 - tanh^2(z / softcap));
    dQ = scale dZ K; dK = scale dZ^T Q. Rows with no allowed key have P = 0 and
    contribute nothing. (The pages call the training pass the backward pass and
    list a deterministic backward in the update article's v2.4 entry; the
    arithmetic is the derivative of standard attention, [Variants] section 二.1.)

    with_bounds: also return a dict of magnitudes that bound how rounding moves
    the gradients. "dq", "dk", "dv" = scale |dZ| |K|, scale |dZ|^T |Q|, P^T |dO|:
    a relative change r of every entry of P and dZ moves dQ, dK, dV by at most r
    times them. "dq_cancel", "dk_cancel" = the same products with |dZ| replaced
    by P (|dO| |V|^T + |dO|.|O|): dP_ij = dO_i . v_j and D_i = dO_i . O_i are sums
    over head_dim, and rounding such a sum errs by at most e times the sum of
    the absolute values of its terms (e about d times the unit roundoff), so an
    error of that size in dP - D moves dQ, dK by at most e times these.
    """
    rows = np.arange(nq)
    k_bh = np.asarray(k_bh, dtype=np.float64)
    q_bh = np.asarray(q_bh, dtype=np.float64)
    v_bh = np.asarray(v_bh, dtype=np.float64)
    do_bh = np.asarray(do_bh, dtype=np.float64)
    dq = np.zeros_like(q_bh)
    dk = np.zeros_like(k_bh)
    dv = np.zeros_like(v_bh)
    D = np.zeros(nq)
    if k_bh.shape[0] == 0 or nq == 0:
        if with_bounds:
            return dq, dk, dv, D, {"dq": np.zeros_like(dq), "dk": np.zeros_like(dk),
                                   "dv": np.zeros_like(dv), "dq_cancel": np.zeros_like(dq),
                                   "dk_cancel": np.zeros_like(dk)}
        return dq, dk, dv, D
    s = scores_ref(q_bh, k_bh, rows, nq, scale, causal, window_left, window_right, slope, softcap)
    p, _, _ = softmax_rows(s)
    dv = p.T @ do_bh
    dp = do_bh @ v_bh.T
    D = (p * dp).sum(axis=1)
    ds = p * (dp - D[:, None])
    if softcap > 0.0:
        t = np.tanh((q_bh @ k_bh.T) * scale / softcap)
        ds = ds * (1.0 - t * t)
    dq = scale * (ds @ k_bh)
    dk = scale * (ds.T @ q_bh)
    if with_bounds:
        a = np.abs(ds)
        o_bh = p @ v_bh
        c = p * (np.abs(do_bh) @ np.abs(v_bh).T + (np.abs(do_bh) * np.abs(o_bh)).sum(axis=1)[:, None])
        ak, aq = np.abs(k_bh), np.abs(q_bh)
        return dq, dk, dv, D, {"dq": scale * (a @ ak), "dk": scale * (a.T @ aq),
                               "dv": p.T @ np.abs(do_bh), "dq_cancel": scale * (c @ ak),
                               "dk_cancel": scale * (c.T @ aq)}
    return dq, dk, dv, D


def attention_bwd_ref(q, k, v, do, scale, causal=False, window_left=-1, window_right=-1,
                      alibi_slopes=None, softcap=0.0, bh=None, with_bounds=False):
    """Gradients of attention_ref's O with respect to q, k, v, given dO.

    q, do [B, Nq, H, d]; k, v [B, Nk, H, d]. Returns dq, dk, dv (shaped like
    q, k, v) and D [B, H, Nq] = rowsum(dO * O); pairs outside bh are NaN.
    with_bounds: also the bound magnitudes of attention_bwd_bh (a dict of arrays
    shaped like the gradient each bounds).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, nq, H, _ = q.shape
    pairs = [(b, h) for b in range(B) for h in range(H)] if bh is None else bh
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    D = np.full((B, H, nq), np.nan)
    like = {"dq": q, "dk": k, "dv": v, "dq_cancel": q, "dk_cancel": k}
    bounds = {n: np.full(x.shape, np.nan) for n, x in like.items()}
    for b, h in pairs:
        slope = None if alibi_slopes is None else float(alibi_slopes[h])
        g = attention_bwd_bh(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], nq, scale, causal,
                             window_left, window_right, slope, softcap, with_bounds)
        dq[b, :, h], dk[b, :, h], dv[b, :, h], D[b, h] = g[:4]
        if with_bounds:
            for n in bounds:
                bounds[n][b, :, h] = g[4][n]
    if with_bounds:
        return dq, dk, dv, D, bounds
    return dq, dk, dv, D


# --------------------------------------------------------------------------
# Packed variable-length batch (the deep-analysis page, roadmap section)
# --------------------------------------------------------------------------
def attention_varlen_ref(q, k, v, cu_seqlens_q, cu_seqlens_k, scale, causal=False,
                         window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                         seqs=None, heads=None):
    """Exact attention of each sequence of a packed batch, on its own.

    q [total_q, H, d], k and v [total_k, H, d]; sequence b owns query rows
    [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b],
    cu_seqlens_k[b+1]), and its mask and ALiBi distances are aligned to its own
    bottom-right corner. seqs / heads: optional subsets to compute.
    Returns O [total_q, H, d] and LSE [H, total_q]; entries not computed are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    H = q.shape[1]
    o = np.full((q.shape[0], H, v.shape[2]), np.nan)
    lse = np.full((H, q.shape[0]), np.nan)
    seqs = range(len(cq) - 1) if seqs is None else seqs
    heads = range(H) if heads is None else heads
    for b in seqs:
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        rows = np.arange(q1 - q0)
        for h in heads:
            slope = None if alibi_slopes is None else float(alibi_slopes[h])
            ob, lb = attention_bh(q[q0:q1, h, :], k[k0:k1, h, :], v[k0:k1, h, :], rows,
                                  q1 - q0, scale, causal, window_left, window_right, slope,
                                  softcap)
            o[q0:q1, h, :] = ob
            lse[h, q0:q1] = lb
    return o, lse


def attention_varlen_bwd_ref(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale, causal=False,
                             window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                             with_bounds=False):
    """Gradients of attention_varlen_ref: each sequence's own backward (attention_bwd_bh).

    q, do [total_q, H, d]; k, v [total_k, H, d]. Returns dq, dk, dv shaped like
    q, k, v (rows no sequence owns are 0), plus, with with_bounds, the bound
    magnitudes of attention_bwd_bh in a dict of arrays shaped the same way.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    cq = np.asarray(cu_seqlens_q, dtype=np.int64)
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    H = q.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    like = {"dq": q, "dk": k, "dv": v, "dq_cancel": q, "dk_cancel": k}
    bounds = {n: np.zeros(x.shape) for n, x in like.items()}
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        for h in range(H):
            slope = None if alibi_slopes is None else float(alibi_slopes[h])
            g = attention_bwd_bh(q[q0:q1, h], k[k0:k1, h], v[k0:k1, h], do[q0:q1, h], q1 - q0,
                                 scale, causal, window_left, window_right, slope, softcap,
                                 with_bounds)
            dq[q0:q1, h], dk[k0:k1, h], dv[k0:k1, h] = g[0], g[1], g[2]
            if with_bounds:
                for n in bounds:
                    rows = slice(q0, q1) if n.startswith("dq") else slice(k0, k1)
                    bounds[n][rows, h] = g[4][n]
    if with_bounds:
        return dq, dk, dv, bounds
    return dq, dk, dv


# --------------------------------------------------------------------------
# Paged KV cache (flash-attn update article, v2.5 entry)
# --------------------------------------------------------------------------
def paged_gather_ref(cache: np.ndarray, block_table: np.ndarray, b: int, nk: int) -> np.ndarray:
    """Logical keys [nk, H, d] of sequence b from a pool [num_pages, page_size, H, d].

    Key t sits in physical page block_table[b, t // page_size], row t % page_size.
    """
    ps = cache.shape[1]
    t = np.arange(nk)
    return cache[np.asarray(block_table)[b, t // ps], t % ps]


def kvcache_append_ref(k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                       seqlens, k_new: np.ndarray, v_new: np.ndarray):
    """Copies of the page pools with the new keys of every sequence written in.

    Row i of k_new[b] / v_new[b] ([B, n_new, H, d]) becomes logical key
    seqlens[b] + i of sequence b, i.e. pool row
    [block_table[b, t // page_size], t % page_size] with t = seqlens[b] + i
    (the update article's v2.5 entry for the page addressing; the inference
    article's incremental decoding for appending each step's keys to the cache).
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    ps = kc.shape[1]
    bt = np.asarray(block_table)
    for b in range(k_new.shape[0]):
        for i in range(k_new.shape[1]):
            t = int(seqlens[b]) + i
            kc[bt[b, t // ps], t % ps] = k_new[b, i]
            vc[bt[b, t // ps], t % ps] = v_new[b, i]
    return kc, vc


# --------------------------------------------------------------------------
# Split-KV and its reduce step (flash-attn update article, v2.2 entry)
# --------------------------------------------------------------------------
def split_bounds(nk: int, num_splits: int, page_size: int = 1):
    """Contiguous key chunks [lo, hi) for each split.

    The chunk length is ceil(nk / num_splits) rounded up to a whole number of
    pages, so a chunk never cuts a page; trailing chunks may be empty.
    """
    c = -(-nk // num_splits)
    c = -(-c // page_size) * page_size
    return [(min(nk, s * c), min(nk, (s + 1) * c)) for s in range(num_splits)]


def splitkv_ref(q, k, v, num_splits, page_size, scale, causal=False, window_left=-1,
                window_right=-1, alibi_slopes=None, softcap=0.0, bh=None, seqlens_k=None):
    """Per-split normalised outputs and log-sum-exps over contiguous logical K/V.

    seqlens_k: optional per-sequence key counts (each <= Nk); sequence b then
    uses keys [0, seqlens_k[b]) only, aligned to its own bottom-right corner,
    and its chunks are split_bounds(seqlens_k[b], ...).
    Returns o_part [S, B, H, Nq, d] and lse_part [S, B, H, Nq]; an empty chunk
    (or a row with no allowed key inside it) has o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nq, H, d = q.shape
    nk = k.shape[1]
    pairs = [(b, h) for b in range(B) for h in range(H)] if bh is None else bh
    o_part = np.full((num_splits, B, H, nq, v.shape[3]), np.nan)
    lse_part = np.full((num_splits, B, H, nq), np.nan)
    rows = np.arange(nq)
    for b, h in pairs:
        nk_b = nk if seqlens_k is None else int(seqlens_k[b])
        if not 0 <= nk_b <= nk:
            raise ValueError("seqlens_k entries must lie in [0, Nk]")
        slope = None if alibi_slopes is None else float(alibi_slopes[h])
        for s, (lo, hi) in enumerate(split_bounds(nk_b, num_splits, page_size)):
            ob, lb = attention_bh(q[b, :, h, :], k[b, :nk_b, h, :], v[b, :nk_b, h, :], rows, nq,
                                  scale, causal, window_left, window_right, slope,
                                  softcap, key_lo=lo, key_hi=hi)
            o_part[s, b, h] = ob
            lse_part[s, b, h] = lb
    return o_part, lse_part


def splitkv_append_ref(q, k, v, k_new, v_new, seqlens, num_splits, page_size, scale,
                       causal=False, window_left=-1, window_right=-1, alibi_slopes=None,
                       softcap=0.0, bh=None):
    """Split pass after appending each sequence's new keys to its cache.

    k, v [B, Nk, H, d]: logical cache contents (only keys [0, seqlens[b]) of
    sequence b are used); k_new, v_new [B, Nq, H, d]: one new key per query
    row. Sequence b attends over its seqlens[b] cached keys followed by its Nq
    new ones, so its queries line up with the new keys (bottom-right rule).
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nq = q.shape[0], q.shape[1]
    n_new = [int(n) + nq for n in seqlens]
    cap = max(n_new + [k.shape[1]])
    k2 = np.zeros((B, cap) + k.shape[2:])
    v2 = np.zeros((B, cap) + v.shape[2:])
    for b, n in enumerate(seqlens):
        n = int(n)
        k2[b, :n], v2[b, :n] = k[b, :n], v[b, :n]
        k2[b, n:n + nq], v2[b, n:n + nq] = k_new[b], v_new[b]
    return splitkv_ref(q, k2, v2, num_splits, page_size, scale, causal, window_left,
                       window_right, alibi_slopes, softcap, bh=bh, seqlens_k=n_new)


def combine_ref(o_part: np.ndarray, lse_part: np.ndarray):
    """Merge split partials: L = ln sum_s exp(lse_s), O = sum_s exp(lse_s - L) o_s.

    o_part [S, ..., d], lse_part [S, ...]. Where every split is empty: O = 0, L = -inf.
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    m = lse_part.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_part - m_safe[None])               # exp(-inf) = 0 for empty splits
    tot = w.sum(axis=0)
    L = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), NEG_INF)
    o = np.where((tot > 0)[..., None],
                 (w[..., None] * o_part).sum(axis=0) / np.where(tot > 0, tot, 1.0)[..., None],
                 0.0)
    return o, L
