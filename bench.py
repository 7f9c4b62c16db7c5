"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic input:
  1. fa_fwd on the GPT-style causal prefill (B=4, H=16, Nq=Nk=2048, d=128, bf16),
  2. fa_fwd_splitkv + fa_splitkv_combine on the paged decode
     (B=8, H=32, Nq=1, Nk=32768, d=128, bf16, 256-token pages, 16 splits),
  3. fa_fwd_split (8 key splits) + fa_splitkv_combine on the short query set
     with ALiBi and a tanh cap (B=2, H=8, Nq=512, Nk=4096, d=128, bf16),
  4. fa_fwd on the sliding-window prefill (B=1, H=16, Nq=Nk=16384, d=64, bf16,
     causal, window_left=4096: only the in-window pairs are computed),
  5. fa_fwd on the tiny fp32 case (B=1, H=2, Nq=Nk=128, d=64, fp32).
`value` is the prefill's algorithmic TFLOP/s (4*B*H*d*allowed pairs over the
prefill launch time); the decode's algorithmic GB/s, the split forward's and
the window's TFLOP/s (each with its roofline) and the tiny case's launch time
are reported beside it. After the timed steps, the variable-length
entry points are timed on their own (a packed causal prefill of 8 sequences of
seeded lengths, the decode with seeded per-sequence cache lengths, and the
decode step that appends one key per sequence before attending), the
backward pass of the causal prefill, its forward in FP8 and the window's forward
in FP8 (head_dim 64).
Inputs are resident in device memory before the timed region starts.

Prints ONE JSON line on stdout. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "exact_tiled_attention_05_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Source files each measured kernel is built from (a change voids its counters).
KERNEL_SOURCES = {
    "prefill": ["fa_fwd_bf16.hip", "fa_lds.h", "fa_device.h", "fa_params.h"],
    "decode_split": ["fa_decode.hip", "fa_device.h", "fa_params.h"],
    "window": ["fa_fwd_bf16.hip", "fa_lds.h", "fa_device.h", "fa_params.h"],
    "short_split": ["fa_fwd_bf16.hip", "fa_lds.h", "fa_device.h", "fa_params.h"],
}


def source_hash(kind):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kind):
    """HBM bytes per launch from the committed rocprofv3 counters, or None when the
    kernel's sources changed since they were taken (or none were taken)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)[kind]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha256") != source_hash(kind):
        return None
    return int(round((t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024))


def device_info(torch, dev):
    """CU count and maximum shader clock of the GPU agent as rocminfo reports them, and the
    dense bf16 MFMA rate they imply (4096 flop per clock per CU). `peak` in the roofline
    objects stays MI355X's published figure."""
    import subprocess
    prop = torch.cuda.get_device_properties(dev)
    out = {"name": prop.gcnArchName, "cus": int(prop.multi_processor_count), "max_sclk_mhz": None}
    try:
        text = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        for agent in text.split("Agent ")[1:]:
            if "gfx" not in agent or "Compute Unit" not in agent:
                continue
            for line in agent.splitlines():
                if "Max Clock Freq. (MHz)" in line:
                    out["max_sclk_mhz"] = int(line.split(":")[1].split()[0])
                elif line.strip().startswith("Compute Unit:"):
                    out["cus"] = int(line.split(":")[1].split()[0])
            break
    except (OSError, subprocess.SubprocessError, ValueError, IndexError):
        pass
    if out["max_sclk_mhz"]:
        out["bf16_peak_at_max_sclk_tflops"] = round(
            out["cus"] * out["max_sclk_mhz"] * 1e6 * 4096 / 1e12, 1)
    return out


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown cpu"


def allowed_pairs(nq, nk, causal, wl, wr):
    """Number of (query, key) pairs the mask keeps, summed over rows."""
    off = nk - nq
    i = np.arange(nq, dtype=np.int64) + off
    lo = np.zeros(nq, dtype=np.int64)
    hi = np.full(nq, nk - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, i)
    if wl >= 0:
        lo = np.maximum(lo, i - wl)
    if wr >= 0:
        hi = np.minimum(hi, i + wr)
    return int(np.maximum(0, hi - lo + 1).sum())


def window_sweep(fa, W, dev, up, args):
    """Time fa_fwd on the sliding-window shape (B1 H16 N16384 d64, causal) for window widths from
    256 keys to the whole causal range: with tiles outside each row's window skipped, the time
    follows the in-window pairs, not N^2 ([Updates] v2.3)."""
    import torch
    ww = W.WORKLOADS[3]
    q, k, v = (up(x, ww.dtype) for x in W.gen_qkv(ww))
    o = torch.empty((ww.B, ww.Nq, ww.H, ww.d), dtype=torch.float32, device=dev)
    lse = torch.empty((ww.B, ww.H, ww.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    n = max(args.steps, 5)
    for wl in (256, 512, 1024, 2048, 4096, 8192, -1):
        def call():
            st = fa.fa_fwd(q, k, v, o, lse, ww.B, ww.H, ww.Nq, ww.Nk, ww.d, ww.scale, True, wl, 0,
                           None, 0.0, stream)
            if st != 0:
                raise fa.FaError(st, "fa_fwd")
        for _ in range(max(args.warmup, 1)):
            call()
        torch.cuda.synchronize()
        times = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
        pairs = allowed_pairs(ww.Nq, ww.Nk, True, wl, 0)
        gflop = 4.0 * ww.B * ww.H * ww.d * pairs / 1e9
        us = float(np.median(times))
        print(json.dumps({"workload": f"sliding window B{ww.B} H{ww.H} N{ww.Nq} d{ww.d} causal",
                          "window_left": wl, "in_window_pairs_per_head": pairs,
                          "dense_fraction": round(pairs / (ww.Nq * ww.Nk), 4),
                          "gflop": round(gflop, 3), "us_median": round(us, 1),
                          "us_min": round(float(np.min(times)), 1),
                          "tflops": round(gflop / us * 1e3, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--print-source-hashes", action="store_true")
    ap.add_argument("--window-sweep", action="store_true",
                    help="only time fa_fwd on the 16K sliding-window shape at several window widths "
                         "(one JSON line per width: time against the in-window work)")
    args = ap.parse_args()
    if args.print_source_hashes:
        print(json.dumps({k: source_hash(k) for k in KERNEL_SOURCES}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on one device's share of the work).", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_05_amd as fa
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        x = torch.ones(1 << 28, device=dev)  # 1 GiB of fp32
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print("copied 3 x 1 GiB", flush=True)
        return
    fa.load_library()

    def up(x, dtype):
        x = np.ascontiguousarray(x)
        if dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    if args.window_sweep:
        window_sweep(fa, W, dev, up, args)
        return

    def up8(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # E4M3 codes as uint8

    # ---- prefill inputs
    wp = W.WORKLOADS[2]
    log(f"generating {wp.name}")
    q, k, v = W.gen_qkv(wp)
    pq, pk, pv = up(q, wp.dtype), up(k, wp.dtype), up(v, wp.dtype)
    del q, k, v
    po = torch.empty((wp.B, wp.Nq, wp.H, wp.d), dtype=torch.float32, device=dev)
    plse = torch.empty((wp.B, wp.H, wp.Nq), dtype=torch.float32, device=dev)
    pairs = allowed_pairs(wp.Nq, wp.Nk, True, -1, -1)
    prefill_flops = 4.0 * wp.B * wp.H * wp.d * pairs
    prefill_bytes = 3 * pq.numel() * 2 + po.numel() * 4 + plse.numel() * 4

    # ---- decode inputs
    wd = W.WORKLOADS[4]
    log(f"generating {wd.name}")
    dq_np, kc, vc, bt = W.gen_paged(wd)
    dq, dk, dv = up(dq_np, wd.dtype), up(kc, wd.dtype), up(vc, wd.dtype)
    del kc, vc
    dbt = torch.from_numpy(bt).to(dev)
    S = wd.num_splits
    o_part = torch.empty((S, wd.B, wd.H, wd.Nq, wd.d), dtype=torch.float32, device=dev)
    lse_part = torch.empty((S, wd.B, wd.H, wd.Nq), dtype=torch.float32, device=dev)
    do = torch.empty((wd.B, wd.Nq, wd.H, wd.d), dtype=torch.float32, device=dev)
    dlse = torch.empty((wd.B, wd.H, wd.Nq), dtype=torch.float32, device=dev)
    kv_bytes = 2 * wd.B * wd.H * wd.Nk * wd.d * 2
    part_bytes = S * wd.B * wd.H * wd.Nq * (wd.d + 1) * 4
    split_bytes = kv_bytes + dq.numel() * 2 + bt.size * 4 + part_bytes
    combine_bytes = part_bytes + do.numel() * 4 + dlse.numel() * 4
    decode_bytes = split_bytes + combine_bytes

    # ---- short query set with ALiBi + softcap, split 8 ways over the keys
    ws = W.WORKLOADS[5]
    log(f"generating {ws.name}")
    sq_np, sk_np, sv_np = W.gen_qkv(ws)
    sq, sk, sv = up(sq_np, ws.dtype), up(sk_np, ws.dtype), up(sv_np, ws.dtype)
    del sq_np, sk_np, sv_np
    s_slopes = torch.from_numpy(np.asarray(ws.slopes(), np.float32)).to(dev)
    SS = 8
    s_opart = torch.empty((SS, ws.B, ws.H, ws.Nq, ws.d), dtype=torch.float32, device=dev)
    s_lpart = torch.empty((SS, ws.B, ws.H, ws.Nq), dtype=torch.float32, device=dev)
    s_o = torch.empty((ws.B, ws.Nq, ws.H, ws.d), dtype=torch.float32, device=dev)
    s_lse = torch.empty((ws.B, ws.H, ws.Nq), dtype=torch.float32, device=dev)
    split_flops = 4.0 * ws.B * ws.H * ws.d * allowed_pairs(ws.Nq, ws.Nk, True, -1, -1)
    split_bytes5 = (sq.numel() + sk.numel() + sv.numel()) * 2 + s_opart.numel() * 4 + s_lpart.numel() * 4

    # ---- sliding-window prefill: 16384 rows over a 4096-key window (d = 64)
    ww = W.WORKLOADS[3]
    log(f"generating {ww.name}")
    wq_np, wk_np, wv_np = W.gen_qkv(ww)
    wq, wk, wv = up(wq_np, ww.dtype), up(wk_np, ww.dtype), up(wv_np, ww.dtype)
    del wq_np, wk_np, wv_np
    wo = torch.empty((ww.B, ww.Nq, ww.H, ww.d), dtype=torch.float32, device=dev)
    wlse = torch.empty((ww.B, ww.H, ww.Nq), dtype=torch.float32, device=dev)
    window_pairs = allowed_pairs(ww.Nq, ww.Nk, True, ww.window_left, ww.window_right)
    window_flops = 4.0 * ww.B * ww.H * ww.d * window_pairs
    window_bytes = 3 * wq.numel() * 2 + wo.numel() * 4 + wlse.numel() * 4

    # ---- tiny fp32 case (launch-bound)
    wt = W.WORKLOADS[1]
    tq_np, tk_np, tv_np = W.gen_qkv(wt)
    tq, tk, tv = up(tq_np, wt.dtype), up(tk_np, wt.dtype), up(tv_np, wt.dtype)
    to_ = torch.empty((wt.B, wt.Nq, wt.H, wt.d), dtype=torch.float32, device=dev)
    tlse = torch.empty((wt.B, wt.H, wt.Nq), dtype=torch.float32, device=dev)
    tiny_flops = 4.0 * wt.B * wt.H * wt.d * allowed_pairs(wt.Nq, wt.Nk, False, -1, -1)

    stream = torch.cuda.current_stream()

    def check(st, where):
        if st != 0:
            raise fa.FaError(st, where)

    def prefill():
        check(fa.fa_fwd(pq, pk, pv, po, plse, wp.B, wp.H, wp.Nq, wp.Nk, wp.d, wp.scale,
                        True, -1, -1, None, 0.0, stream), "fa_fwd")

    def split_pass():
        check(fa.fa_fwd_splitkv(dq, dk, dv, dbt, dbt.shape[1], wd.page_size, o_part, lse_part, S,
                                wd.B, wd.H, wd.Nq, wd.Nk, wd.d, wd.scale, True, -1, -1, None,
                                0.0, stream), "fa_fwd_splitkv")

    def combine_pass():
        check(fa.fa_splitkv_combine(o_part, lse_part, S, wd.B, wd.H, wd.Nq, wd.d, do, dlse,
                                    stream), "fa_splitkv_combine")

    def short_split_pass():
        check(fa.fa_fwd_split(sq, sk, sv, s_opart, s_lpart, SS, ws.B, ws.H, ws.Nq, ws.Nk, ws.d,
                              ws.scale, True, -1, -1, s_slopes, ws.softcap, stream),
              "fa_fwd_split")

    def short_combine():
        check(fa.fa_splitkv_combine(s_opart, s_lpart, SS, ws.B, ws.H, ws.Nq, ws.d, s_o, s_lse,
                                    stream), "fa_splitkv_combine")

    def window():
        check(fa.fa_fwd(wq, wk, wv, wo, wlse, ww.B, ww.H, ww.Nq, ww.Nk, ww.d, ww.scale, True,
                        ww.window_left, ww.window_right, None, 0.0, stream), "fa_fwd")

    def tiny():
        check(fa.fa_fwd(tq, tk, tv, to_, tlse, wt.B, wt.H, wt.Nq, wt.Nk, wt.d, wt.scale, False,
                        -1, -1, None, 0.0, stream), "fa_fwd")

    step_parts = [prefill, split_pass, combine_pass, short_split_pass, short_combine, window, tiny]
    log("warmup")
    for _ in range(args.warmup):
        for f in step_parts:
            f()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(step_parts) + 1)]
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        e = ev[s]
        e[0].record(stream)
        for i, f in enumerate(step_parts):
            f()
            e[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def part(i):
        return np.array([e[i].elapsed_time(e[i + 1]) for e in ev]) * 1e-3

    t_prefill, t_split, t_comb, t_s5, t_s5c, t_win, t_tiny = (part(i) for i in range(len(step_parts)))
    t_short = t_s5 + t_s5c

    # ---- variable sequence lengths (side measurements, after the timed steps):
    # a packed causal prefill of 8 sequences of seeded lengths in [1, 2048] at the
    # prefill head shape, and the paged decode with seeded per-sequence cache
    # lengths in [1, 32768] over the same pool.
    vl = W.varlen_lengths(91, 8, 2048)
    log(f"generating packed prefill, lengths {vl.tolist()}")
    vq_np, vk_np, vv_np, vcq, vck = W.gen_varlen(91, vl, vl, wp.H, wp.d, 1.0, "bf16")
    vq, vk, vv = up(vq_np, "bf16"), up(vk_np, "bf16"), up(vv_np, "bf16")
    del vq_np, vk_np, vv_np
    tcq, tck = torch.from_numpy(vcq).to(dev), torch.from_numpy(vck).to(dev)
    tot = int(vl.sum())
    vo = torch.empty((tot, wp.H, wp.d), dtype=torch.float32, device=dev)
    vlse = torch.empty((wp.H, tot), dtype=torch.float32, device=dev)
    var_flops = 4.0 * wp.H * wp.d * sum(allowed_pairs(int(n), int(n), True, -1, -1) for n in vl)
    dl = np.random.default_rng([92, 7]).integers(1, wd.Nk + 1, size=wd.B)
    tdl = torch.from_numpy(dl.astype(np.int32)).to(dev)
    dl_bytes = (2 * wd.H * wd.d * 2 * int(dl.sum()) + dq.numel() * 2
                + int(sum(-(-int(n) // wd.page_size) for n in dl)) * 4 + part_bytes + combine_bytes)

    # decode step with a fused append: every sequence holds 32767 cached keys and
    # appends one, so it attends over the same 32768 keys as the decode above.
    an = torch.full((wd.B,), wd.Nk - 1, dtype=torch.int32, device=dev)
    akn = up(W.gen_tensor(94, W.TENSOR_K, wd.B, 1, wd.H, wd.d, 1.0, "bf16"), "bf16")
    avn = up(W.gen_tensor(94, W.TENSOR_V, wd.B, 1, wd.H, wd.d, 1.0, "bf16"), "bf16")

    def append_decode():
        check(fa.fa_fwd_splitkv_append(dq, akn, avn, dk, dv, dbt, dbt.shape[1], wd.page_size, an,
                                       o_part, lse_part, S, wd.B, wd.H, wd.Nq, wd.Nk, wd.d,
                                       wd.scale, True, -1, -1, None, 0.0, stream),
              "fa_fwd_splitkv_append")
        combine_pass()

    def varlen_prefill():
        check(fa.fa_fwd_varlen(vq, vk, vv, vo, vlse, tcq, tck, len(vl), wp.H, tot, tot,
                               int(vl.max()), int(vl.max()), wp.d, wp.scale, True, -1, -1, None,
                               0.0, stream), "fa_fwd_varlen")

    def seqlens_decode():
        check(fa.fa_fwd_splitkv_seqlens(dq, dk, dv, dbt, dbt.shape[1], wd.page_size, tdl, o_part,
                                        lse_part, S, wd.B, wd.H, wd.Nq, wd.Nk, wd.d, wd.scale,
                                        True, -1, -1, None, 0.0, stream),
              "fa_fwd_splitkv_seqlens")
        combine_pass()

    for _ in range(args.warmup):
        varlen_prefill()
        seqlens_decode()
        append_decode()
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    for s in range(K):
        e = ev2[s]
        e[0].record(stream)
        varlen_prefill()
        e[1].record(stream)
        seqlens_decode()
        e[2].record(stream)
        append_decode()
        e[3].record(stream)
    torch.cuda.synchronize()
    t_var = np.array([e[0].elapsed_time(e[1]) for e in ev2]) * 1e-3
    t_sld = np.array([e[1].elapsed_time(e[2]) for e in ev2]) * 1e-3
    t_app = np.array([e[2].elapsed_time(e[3]) for e in ev2]) * 1e-3
    app_bytes = decode_bytes + 2 * 2 * wd.B * wd.H * wd.d * 2  # plus the new rows read and written
    assert torch.isfinite(vo).all() and torch.isfinite(do).all()
    variable = {
        "packed_prefill": {"lengths": vl.tolist(), "gflop": round(var_flops / 1e9, 4),
                           "ms": round(t_var.mean() * 1e3, 5),
                           "ms_median": round(float(np.median(t_var)) * 1e3, 5),
                           "tflops": round(var_flops / t_var.mean() / 1e12, 3),
                           "pct_peak": round(100 * var_flops / t_var.mean() / 1e12 / PEAK_BF16_TFLOPS, 2)},
        "decode_cache_seqlens": {"lengths": dl.tolist(), "gbytes": round(dl_bytes / 1e9, 5),
                                 "ms": round(t_sld.mean() * 1e3, 5),
                                 "ms_median": round(float(np.median(t_sld)) * 1e3, 5),
                                 "gbs": round(dl_bytes / t_sld.mean() / 1e9, 2),
                                 "pct_peak": round(100 * dl_bytes / t_sld.mean() / 1e9 / PEAK_HBM_GBS, 2)},
        "decode_append": {"appended_per_sequence": 1, "keys_attended": wd.Nk,
                          "gbytes": round(app_bytes / 1e9, 5), "ms": round(t_app.mean() * 1e3, 5),
                          "ms_median": round(float(np.median(t_app)) * 1e3, 5),
                          "gbs": round(app_bytes / t_app.mean() / 1e9, 2),
                          "pct_peak": round(100 * app_bytes / t_app.mean() / 1e9 / PEAK_HBM_GBS, 2)},
    }

    # ---- backward of the causal prefill (side measurement): fa_bwd from the
    # forward's O and LSE above; algorithmic work 10*d flop per visible pair
    # and head (the five products dS = ..., dV, dP, dQ, dK of the recomputation
    # scheme, 2.5x the forward's 4*d).
    bg = up(W.gen_tensor(wp.seed, 3, wp.B, wp.Nq, wp.H, wp.d, 1.0, "bf16"), "bf16")
    bdq = torch.empty((wp.B, wp.Nq, wp.H, wp.d), dtype=torch.float32, device=dev)
    bdk = torch.empty((wp.B, wp.Nk, wp.H, wp.d), dtype=torch.float32, device=dev)
    bdv = torch.empty_like(bdk)
    bws = torch.empty((fa.fa_bwd_workspace_bytes(wp.B, wp.H, wp.Nq) // 4,), dtype=torch.float32,
                      device=dev)
    bwd_flops = 2.5 * prefill_flops

    def backward():
        check(fa.fa_bwd(pq, pk, pv, po, bg, plse, bdq, bdk, bdv, bws, wp.B, wp.H, wp.Nq, wp.Nk,
                        wp.d, wp.scale, True, -1, -1, None, 0.0, stream), "fa_bwd")

    prefill()
    for _ in range(args.warmup):
        backward()
    ev3 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, e in ev3:
        a.record(stream)
        backward()
        e.record(stream)
    torch.cuda.synchronize()
    t_bwd = np.array([a.elapsed_time(e) for a, e in ev3]) * 1e-3
    assert torch.isfinite(bdq).all() and torch.isfinite(bdk).all() and torch.isfinite(bdv).all()
    # the packed prefill's backward (fa_bwd_varlen) from its forward's O and LSE above
    vg = up(W.gen_tensor(91, 3, 1, tot, wp.H, wp.d, 1.0, "bf16")[0], "bf16")
    vdq = torch.empty((tot, wp.H, wp.d), dtype=torch.float32, device=dev)
    vdk, vdv = torch.empty_like(vdq), torch.empty_like(vdq)
    vws = torch.empty((fa.fa_bwd_workspace_bytes(len(vl), wp.H, int(vl.max())) // 4,),
                      dtype=torch.float32, device=dev)

    def varlen_backward():
        check(fa.fa_bwd_varlen(vq, vk, vv, vo, vg, vlse, vdq, vdk, vdv, vws, tcq, tck, len(vl),
                               wp.H, tot, tot, int(vl.max()), int(vl.max()), wp.d, wp.scale, True,
                               -1, -1, None, 0.0, stream), "fa_bwd_varlen")

    varlen_prefill()
    for _ in range(args.warmup):
        varlen_backward()
    ev5 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, e in ev5:
        a.record(stream)
        varlen_backward()
        e.record(stream)
    torch.cuda.synchronize()
    t_vbwd = np.array([a.elapsed_time(e) for a, e in ev5]) * 1e-3
    assert torch.isfinite(vdq).all() and torch.isfinite(vdk).all() and torch.isfinite(vdv).all()
    vbwd_flops = 2.5 * var_flops
    variable["packed_backward"] = {
        "lengths": vl.tolist(), "gflop": round(vbwd_flops / 1e9, 4),
        "ms": round(t_vbwd.mean() * 1e3, 5), "ms_median": round(float(np.median(t_vbwd)) * 1e3, 5),
        "tflops": round(vbwd_flops / t_vbwd.mean() / 1e12, 3),
        "pct_peak": round(100 * vbwd_flops / t_vbwd.mean() / 1e12 / PEAK_BF16_TFLOPS, 2)}
    del vg, vdq, vdk, vdv, vws

    backward_line = {"workload": "gpt_causal_prefill backward (fa_bwd: prep, dK/dV, dQ)",
                     "gflop": round(bwd_flops / 1e9, 4), "ms": round(t_bwd.mean() * 1e3, 5),
                     "ms_median": round(float(np.median(t_bwd)) * 1e3, 5),
                     "tflops": round(bwd_flops / t_bwd.mean() / 1e12, 3),
                     "pct_peak": round(100 * bwd_flops / t_bwd.mean() / 1e12 / PEAK_BF16_TFLOPS, 2)}

    # ---- FP8 forward on the causal prefill shape (side measurement): E4M3 codes of
    # the same seeded draws, unit descales; roofline against the FP8 MFMA peak.
    f8 = [up8(W.gen_tensor(wp.seed, t, wp.B, wp.Nq, wp.H, wp.d, 1.0, "fp8"))
          for t in (W.TENSOR_Q, W.TENSOR_K, W.TENSOR_V)]
    fo = torch.empty_like(po)
    flse = torch.empty_like(plse)

    def fp8_prefill():
        check(fa.fa_fwd_fp8(f8[0], f8[1], f8[2], 1.0, 1.0, 1.0, fo, flse, wp.B, wp.H, wp.Nq,
                            wp.Nk, wp.d, wp.scale, True, -1, -1, None, 0.0, stream), "fa_fwd_fp8")

    for _ in range(args.warmup):
        fp8_prefill()
    ev4 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, e in ev4:
        a.record(stream)
        fp8_prefill()
        e.record(stream)
    torch.cuda.synchronize()
    t_f8 = np.array([a.elapsed_time(e) for a, e in ev4]) * 1e-3
    assert torch.isfinite(fo).all()
    f8_tflops = prefill_flops / t_f8.mean() / 1e12
    fp8_line = {"workload": "gpt_causal_prefill in E4M3 (fa_fwd_fp8)",
                "gflop": round(prefill_flops / 1e9, 4), "ms": round(t_f8.mean() * 1e3, 5),
                "ms_median": round(float(np.median(t_f8)) * 1e3, 5), "tflops": round(f8_tflops, 3),
                "roofline": {"bound": "mfma", "achieved": round(f8_tflops, 3), "peak": PEAK_FP8_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(f8_tflops / PEAK_FP8_TFLOPS, 4)}}

    # ---- FP8 forward on the sliding-window shape (head_dim 64; side measurement).
    f8w = [up8(W.gen_tensor(ww.seed, t, ww.B, ww.Nq, ww.H, ww.d, 1.0, "fp8"))
           for t in (W.TENSOR_Q, W.TENSOR_K, W.TENSOR_V)]

    def fp8_window():
        check(fa.fa_fwd_fp8(f8w[0], f8w[1], f8w[2], 1.0, 1.0, 1.0, wo, wlse, ww.B, ww.H, ww.Nq,
                            ww.Nk, ww.d, ww.scale, True, ww.window_left, ww.window_right, None, 0.0,
                            stream), "fa_fwd_fp8")

    for _ in range(args.warmup):
        fp8_window()
    ev8 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, e in ev8:
        a.record(stream)
        fp8_window()
        e.record(stream)
    torch.cuda.synchronize()
    t_f8w = np.array([a.elapsed_time(e) for a, e in ev8]) * 1e-3
    assert torch.isfinite(wo).all()
    f8w_tflops = window_flops / t_f8w.mean() / 1e12
    fp8_window_line = {"workload": "sliding_window_16k in E4M3 (fa_fwd_fp8, head_dim 64)",
                       "gflop": round(window_flops / 1e9, 4), "ms": round(t_f8w.mean() * 1e3, 5),
                       "ms_median": round(float(np.median(t_f8w)) * 1e3, 5),
                       "tflops": round(f8w_tflops, 3),
                       "roofline": {"bound": "mfma", "achieved": round(f8w_tflops, 3),
                                    "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                                    "frac": round(f8w_tflops / PEAK_FP8_TFLOPS, 4)}}
    del f8w

    # ---- FP8 key splits on the ALiBi + softcap set (side measurement): E4M3 inputs of
    # that shape (amplitude 2), fa_fwd_split_fp8 with the bf16 line's split count, then
    # the combine kernel into the same partial buffers.
    f8s = [up8(W.gen_tensor(ws.seed, t, ws.B, n, ws.H, ws.d, ws.amp, "fp8"))
           for t, n in ((W.TENSOR_Q, ws.Nq), (W.TENSOR_K, ws.Nk), (W.TENSOR_V, ws.Nk))]

    def fp8_short_split():
        check(fa.fa_fwd_split_fp8(f8s[0], f8s[1], f8s[2], 1.0, 1.0, 1.0, s_opart, s_lpart, SS,
                                  ws.B, ws.H, ws.Nq, ws.Nk, ws.d, ws.scale, True, -1, -1, s_slopes,
                                  ws.softcap, stream), "fa_fwd_split_fp8")
        short_combine()

    for _ in range(args.warmup):
        fp8_short_split()
    ev9 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, e in ev9:
        a.record(stream)
        fp8_short_split()
        e.record(stream)
    torch.cuda.synchronize()
    t_f8s = np.array([a.elapsed_time(e) for a, e in ev9]) * 1e-3
    assert torch.isfinite(s_o).all()
    f8s_tflops = split_flops / t_f8s.mean() / 1e12
    fp8_split_line = {"workload": "alibi_softcap_nq_ne_nk in E4M3 (fa_fwd_split_fp8, "
                                  f"{SS} splits, + fa_splitkv_combine)",
                      "num_splits": SS, "gflop": round(split_flops / 1e9, 4),
                      "ms": round(t_f8s.mean() * 1e3, 5),
                      "ms_median": round(float(np.median(t_f8s)) * 1e3, 5),
                      "tflops": round(f8s_tflops, 3),
                      "roofline": {"bound": "mfma", "achieved": round(f8s_tflops, 3),
                                   "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                                   "frac": round(f8s_tflops / PEAK_FP8_TFLOPS, 4)}}
    del f8s

    # ---- paged decode over an E4M3 cache (side measurement): the decode pool above
    # rounded to E4M3 on the device (input preparation, untimed; its NaN pages stay
    # NaN), unit descales. Half the cache bytes of the bf16 decode.
    dk8, dv8 = dk.to(torch.float8_e4m3fn), dv.to(torch.float8_e4m3fn)
    f8_split_bytes = kv_bytes // 2 + dq.numel() * 2 + bt.size * 4 + part_bytes
    f8_decode_bytes = f8_split_bytes + combine_bytes

    def fp8_decode():
        check(fa.fa_fwd_splitkv_fp8(dq, dk8, dv8, 1.0, 1.0, dbt, dbt.shape[1], wd.page_size, None,
                                    o_part, lse_part, S, wd.B, wd.H, wd.Nq, wd.Nk, wd.d, wd.scale,
                                    True, -1, -1, None, 0.0, stream), "fa_fwd_splitkv_fp8")
        combine_pass()

    for _ in range(args.warmup):
        fp8_decode()
    ev6 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, e in ev6:
        a.record(stream)
        fp8_decode()
        e.record(stream)
    torch.cuda.synchronize()
    t_d8 = np.array([a.elapsed_time(e) for a, e in ev6]) * 1e-3
    assert torch.isfinite(do).all()
    fp8_decode_line = {"workload": "paged_splitkv_decode over an E4M3 cache (fa_fwd_splitkv_fp8 + combine)",
                       "gbytes": round(f8_decode_bytes / 1e9, 5), "ms": round(t_d8.mean() * 1e3, 5),
                       "ms_median": round(float(np.median(t_d8)) * 1e3, 5),
                       "gbs": round(f8_decode_bytes / t_d8.mean() / 1e9, 2),
                       "pct_peak": round(100 * f8_decode_bytes / t_d8.mean() / 1e9 / PEAK_HBM_GBS, 2),
                       "keys_per_s_vs_bf16": round(float((t_split + t_comb).mean() / t_d8.mean()), 3)}

    # ---- a chunk of 512 query rows over the first sequence of the decode pool
    # (chunked prefill over a paged cache; side measurement): the multi-row split
    # pass, bottom-right causal over 32768 keys, then the combine.
    cq = up(W.gen_tensor(wd.seed, W.TENSOR_Q, 1, 512, wd.H, wd.d, 1.0, "bf16"), "bf16")
    CS = fa.fa_num_splits(1, wd.H, 512, wd.Nk, wd.d, wd.page_size)
    cop = torch.empty((CS, 1, wd.H, 512, wd.d), dtype=torch.float32, device=dev)
    clp = torch.empty((CS, 1, wd.H, 512), dtype=torch.float32, device=dev)
    co = torch.empty((1, 512, wd.H, wd.d), dtype=torch.float32, device=dev)
    clse = torch.empty((1, wd.H, 512), dtype=torch.float32, device=dev)
    cbt = dbt[:1].contiguous()
    chunk_flops = 4.0 * wd.H * wd.d * allowed_pairs(512, wd.Nk, True, -1, -1)

    def paged_chunk():
        check(fa.fa_fwd_splitkv(cq, dk, dv, cbt, cbt.shape[1], wd.page_size, cop, clp, CS, 1, wd.H,
                                512, wd.Nk, wd.d, wd.scale, True, -1, -1, None, 0.0, stream),
              "fa_fwd_splitkv")
        check(fa.fa_splitkv_combine(cop, clp, CS, 1, wd.H, 512, wd.d, co, clse, stream),
              "fa_splitkv_combine")

    for _ in range(args.warmup):
        paged_chunk()
    ev7 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for a, e in ev7:
        a.record(stream)
        paged_chunk()
        e.record(stream)
    torch.cuda.synchronize()
    t_pc = np.array([a.elapsed_time(e) for a, e in ev7]) * 1e-3
    assert torch.isfinite(co).all()
    chunk_line = {"workload": "512-row chunk over a 32768-key paged sequence, H32 d128, 256-key "
                              "pages (fa_fwd_splitkv multi-row + combine)",
                  "num_splits": CS, "gflop": round(chunk_flops / 1e9, 4),
                  "ms": round(t_pc.mean() * 1e3, 5), "ms_median": round(float(np.median(t_pc)) * 1e3, 5),
                  "tflops": round(chunk_flops / t_pc.mean() / 1e12, 3),
                  "pct_peak": round(100 * chunk_flops / t_pc.mean() / 1e12 / PEAK_BF16_TFLOPS, 2)}

    # ---- the same chunk in E4M3 (side measurement): 512 E4M3 query rows over the
    # E4M3 copy of the pool's first sequence, fa_fwd_paged_fp8 with the same split
    # count, then the combine into the same buffers.
    cq8 = up8(W.gen_tensor(wd.seed, W.TENSOR_Q, 1, 512, wd.H, wd.d, 1.0, "fp8"))

    def paged_chunk_fp8():
        check(fa.fa_fwd_paged_fp8(cq8, dk8, dv8, 1.0, 1.0, 1.0, cbt, cbt.shape[1], wd.page_size,
                                  None, cop, clp, CS, 1, wd.H, 512, wd.Nk, wd.d, wd.scale, True,
                                  -1, -1, None, 0.0, stream), "fa_fwd_paged_fp8")
        check(fa.fa_splitkv_combine(cop, clp, CS, 1, wd.H, 512, wd.d, co, clse, stream),
              "fa_splitkv_combine")

    for _ in range(args.warmup):
        paged_chunk_fp8()
    ev10 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(K)]
    for a, e in ev10:
        a.record(stream)
        paged_chunk_fp8()
        e.record(stream)
    torch.cuda.synchronize()
    t_pc8 = np.array([a.elapsed_time(e) for a, e in ev10]) * 1e-3
    assert torch.isfinite(co).all()
    pc8_tflops = chunk_flops / t_pc8.mean() / 1e12
    chunk8_line = {"workload": "the 512-row chunk in E4M3 over an E4M3 copy of the paged sequence "
                               "(fa_fwd_paged_fp8 + combine)",
                   "num_splits": CS, "gflop": round(chunk_flops / 1e9, 4),
                   "ms": round(t_pc8.mean() * 1e3, 5),
                   "ms_median": round(float(np.median(t_pc8)) * 1e3, 5),
                   "tflops": round(pc8_tflops, 3),
                   "roofline": {"bound": "mfma", "achieved": round(pc8_tflops, 3),
                                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(pc8_tflops / PEAK_FP8_TFLOPS, 4)}}
    del cop, clp, co, clse, cq8, dk8, dv8

    # ---- one decode step of a small serving batch (side measurement): append of
    # the step's key and value, split pass and combine for 1 sequence of 4096
    # cached keys (32 heads, 256-key pages, the split count fa_num_splits picks),
    # 100 steps back to back, eager against a HIP graph of the step replayed.
    gw = W.Workload(0, "serving_step", B=1, H=32, Nq=1, Nk=4097, d=128, dtype="bf16",
                    causal=True, paged=True, page_size=256, pool_factor=1.0, num_splits=4,
                    seed=wd.seed)
    gq_np, gk_np, gv_np, gbt_np = W.gen_paged(gw, seqlens=[4096])
    gq, gk, gv = up(gq_np, "bf16"), up(gk_np, "bf16"), up(gv_np, "bf16")
    gkn = up(W.gen_tensor(gw.seed, W.TENSOR_K, 1, 1, gw.H, gw.d, 1.0, "bf16"), "bf16")
    gvn = up(W.gen_tensor(gw.seed, W.TENSOR_V, 1, 1, gw.H, gw.d, 1.0, "bf16"), "bf16")
    gbt = torch.from_numpy(gbt_np).to(dev)
    gsl = torch.full((1,), 4096, dtype=torch.int32, device=dev)
    GS = fa.fa_num_splits(1, gw.H, 1, gw.Nk, gw.d, gw.page_size)
    gop = torch.empty((GS, 1, gw.H, 1, gw.d), dtype=torch.float32, device=dev)
    glp = torch.empty((GS, 1, gw.H, 1), dtype=torch.float32, device=dev)
    go = torch.empty((1, 1, gw.H, gw.d), dtype=torch.bfloat16, device=dev)
    glse = torch.empty((1, gw.H, 1), dtype=torch.float32, device=dev)
    gstream = torch.cuda.Stream()  # capture needs a stream other than the default one

    def serving_step():
        check(fa.fa_fwd_splitkv_append(gq, gkn, gvn, gk, gv, gbt, gbt.shape[1], gw.page_size, gsl,
                                       gop, glp, GS, 1, gw.H, 1, gw.Nk, gw.d, gw.scale, True,
                                       stream=gstream), "fa_fwd_splitkv_append")
        check(fa.fa_splitkv_combine(gop, glp, GS, 1, gw.H, 1, gw.d, go, glse, gstream),
              "fa_splitkv_combine")

    n_steps = 100
    for _ in range(3):
        serving_step()
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(gstream)
    for _ in range(n_steps):
        serving_step()
    e.record(gstream)
    torch.cuda.synchronize()
    t_eager = a.elapsed_time(e) * 1e-3 / n_steps
    # One graph launch costs more host time than the two kernel launches of a step,
    # so a graph holds several steps (the same step repeated, as in the eager loop).
    per_graph = 10
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gstream):
        for _ in range(per_graph):
            serving_step()
    torch.cuda.synchronize()
    with torch.cuda.stream(gstream):
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        a.record(gstream)
        for _ in range(n_steps // per_graph):
            graph.replay()
        e.record(gstream)
    torch.cuda.synchronize()
    t_graph = a.elapsed_time(e) * 1e-3 / n_steps
    assert torch.isfinite(go.float()).all()
    serving_line = {"workload": "decode step with a cache append, 1 sequence x 32 heads, 4097 keys "
                                "(fa_fwd_splitkv_append + fa_splitkv_combine)",
                    "num_splits": GS, "steps": n_steps, "steps_per_graph": per_graph,
                    "eager_us_per_step": round(t_eager * 1e6, 2),
                    "hip_graph_us_per_step": round(t_graph * 1e6, 2)}
    del graph

    pre_tflops = prefill_flops / t_prefill.mean() / 1e12
    dec_time = (t_split + t_comb).mean()
    dec_gbs = decode_bytes / dec_time / 1e9
    split_gbs = split_bytes / t_split.mean() / 1e9
    short_tflops = split_flops / t_short.mean() / 1e12
    short_kernel_tflops = split_flops / t_s5.mean() / 1e12
    win_tflops = window_flops / t_win.mean() / 1e12
    tiny_tflops = tiny_flops / t_tiny.mean() / 1e12
    assert torch.isfinite(po).all() and torch.isfinite(do).all() and torch.isfinite(s_o).all()
    assert torch.isfinite(wo).all() and torch.isfinite(to_).all()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        from threadpoolctl import threadpool_info, threadpool_limits
        log("cpu baseline: oracle on the full causal-prefill batch")
        q, k, v = W.gen_qkv(wp)
        qf, kf, vf = (W.to_float(x, wp.dtype) for x in (q, k, v))
        usable = len(os.sched_getaffinity(0))
        with threadpool_limits(limits=usable):
            t = time.perf_counter()
            O.attention_ref(qf, kf, vf, wp.scale, True)
            dt = time.perf_counter() - t
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        cpu = {"value": round(prefill_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle",
               "sample": f"whole causal-prefill batch B4 H16 N2048 d128 (fp64 numpy, {dt:.1f} s; "
                         f"BLAS threads {threads}, usable cpus {usable}, os.cpu_count "
                         f"{os.cpu_count()}, {cpu_model()})"}

    line = {
        "metric": "attn fwd TFLOP/s (% bf16 MFMA peak); decode split-KV GB/s (% HBM peak)",
        "value": round(pre_tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 inputs, seeded block-table permutation)",
        "config": {"workload": "gpt_causal_prefill B4 H16 Nq=Nk=2048 d128 bf16 causal "
                               "+ paged_splitkv_decode B8 H32 Nq1 Nk32768 d128 page256 S16 "
                               "+ alibi_softcap_nq_ne_nk B2 H8 Nq512 Nk4096 d128 split8 "
                               "+ sliding_window_16k B1 H16 Nq=Nk=16384 d64 bf16 causal wl4096 "
                               "+ tiny_fp32_noncausal B1 H2 Nq=Nk=128 d64 fp32",
                   "prefill_gflop": round(prefill_flops / 1e9, 4),
                   "decode_gbytes": round(decode_bytes / 1e9, 5)},
        "device": device_info(torch, dev),
        "prefill": {"ms": round(t_prefill.mean() * 1e3, 5), "ms_min": round(t_prefill.min() * 1e3, 5),
                    "ms_median": round(float(np.median(t_prefill)) * 1e3, 5),
                    "tflops": round(pre_tflops, 3), "pct_peak": round(100 * pre_tflops / PEAK_BF16_TFLOPS, 2)},
        "decode": {"ms": round(dec_time * 1e3, 5),
                   "ms_median": round(float(np.median(t_split + t_comb)) * 1e3, 5),
                   "ms_min": round(float((t_split + t_comb).min()) * 1e3, 5),
                   "split_ms": round(t_split.mean() * 1e3, 5),
                   "combine_ms": round(t_comb.mean() * 1e3, 5), "gbs": round(dec_gbs, 2),
                   "pct_peak": round(100 * dec_gbs / PEAK_HBM_GBS, 2),
                   "roofline": {"bound": "hbm", "achieved": round(split_gbs, 2), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(split_gbs / PEAK_HBM_GBS, 4),
                                "traffic": measured_traffic("decode_split"),
                                "algorithmic_bytes": int(split_bytes)}},
        "short_query_split": {"ms": round(t_short.mean() * 1e3, 5),
                              "ms_min": round(t_short.min() * 1e3, 5),
                              "ms_median": round(float(np.median(t_short)) * 1e3, 5),
                              "split_ms": round(t_s5.mean() * 1e3, 5),
                              "split_ms_min": round(t_s5.min() * 1e3, 5),
                              "split_ms_max": round(t_s5.max() * 1e3, 5),
                              "combine_ms": round(t_s5c.mean() * 1e3, 5),
                              "tflops": round(short_tflops, 3),
                              "pct_peak": round(100 * short_tflops / PEAK_BF16_TFLOPS, 2),
                              "num_splits": SS, "gflop": round(split_flops / 1e9, 4),
                              "roofline": {"bound": "mfma", "achieved": round(short_kernel_tflops, 3),
                                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                           "frac": round(short_kernel_tflops / PEAK_BF16_TFLOPS, 4),
                                           "traffic": measured_traffic("short_split"),
                                           "algorithmic_bytes": int(split_bytes5),
                                           "kernel": "fwd_bf16_kernel<128, true, true, FWD_CONTIG_SPLIT>"}},
        "sliding_window": {"workload": "sliding_window_16k B1 H16 Nq=Nk=16384 d64 causal wl4096",
                           "in_window_pairs_per_head": int(window_pairs),
                           "dense_fraction": round(window_pairs / (ww.Nq * ww.Nk), 4),
                           "gflop": round(window_flops / 1e9, 4),
                           "ms": round(t_win.mean() * 1e3, 5), "ms_min": round(t_win.min() * 1e3, 5),
                           "ms_median": round(float(np.median(t_win)) * 1e3, 5),
                           "tflops": round(win_tflops, 3),
                           "pct_peak": round(100 * win_tflops / PEAK_BF16_TFLOPS, 2),
                           "roofline": {"bound": "mfma", "achieved": round(win_tflops, 3),
                                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(win_tflops / PEAK_BF16_TFLOPS, 4),
                                        "traffic": measured_traffic("window"),
                                        "algorithmic_bytes": int(window_bytes),
                                        "kernel": "fwd_bf16_kernel<64, false, false, FWD_CONTIG>"}},
        "tiny_fp32": {"workload": "tiny_fp32_noncausal B1 H2 Nq=Nk=128 d64 fp32 (launch-bound)",
                      "us": round(t_tiny.mean() * 1e6, 2), "us_min": round(t_tiny.min() * 1e6, 2),
                      "us_median": round(float(np.median(t_tiny)) * 1e6, 2),
                      "tflops": round(tiny_tflops, 4),
                      "pct_fp32_peak": round(100 * tiny_tflops / PEAK_FP32_TFLOPS, 3)},
        "variable_lengths": variable,
        "backward": backward_line,
        "fp8_prefill": fp8_line,
        "fp8_window": fp8_window_line,
        "fp8_short_split": fp8_split_line,
        "fp8_decode": fp8_decode_line,
        "serving_step": serving_line,
        "paged_prefill_chunk": chunk_line,
        "fp8_paged_prefill_chunk": chunk8_line,
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("prefill"),
                     "algorithmic_bytes": int(prefill_bytes), "kernel": "fwd_bf16_kernel<128, false, false, FWD_CONTIG>"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
