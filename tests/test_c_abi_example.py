"""The C ABI used from plain C: tests/c_abi/fa_c_example (built with the library)
allocates its own device memory through the HIP runtime, calls fa_fwd and the
paged split pass + combine on a stream of its own, and writes raw outputs that
are checked here against the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_common import check, say

EXAMPLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "fa_c_example")


def run_example(args, tmp_path):
    assert os.path.exists(EXAMPLE), "build the library first (it builds the C example too)"
    r = subprocess.run([EXAMPLE, *map(str, args)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr


@pytest.mark.gpu
def test_c_example_prefill(tmp_path):
    B, H, N, D = 2, 3, 300, 128
    say("C example: prefill")
    q, k, v = (W.gen_tensor(14400, t, B, N, H, D, 1.0, "bf16") for t in (W.TENSOR_Q, W.TENSOR_K, W.TENSOR_V))
    paths = {n: tmp_path / f"{n}.bin" for n in ("q", "k", "v", "o", "lse")}
    for n, x in (("q", q), ("k", k), ("v", v)):
        np.ascontiguousarray(x).tofile(paths[n])
    run_example(["prefill", B, H, N, D, paths["q"], paths["k"], paths["v"], paths["o"],
                 paths["lse"]], tmp_path)
    o = np.fromfile(paths["o"], dtype=np.float32).reshape(B, N, H, D)
    lse = np.fromfile(paths["lse"], dtype=np.float32).reshape(B, H, N)
    ro, rl = O.attention_ref(W.to_float(q, "bf16"), W.to_float(k, "bf16"), W.to_float(v, "bf16"),
                             1.0 / np.sqrt(D), True)
    check(o, lse, ro, rl, "bf16", "C example prefill")


@pytest.mark.gpu
def test_c_example_paged_decode(tmp_path):
    w = W.Workload(0, "c_decode", B=3, H=4, Nq=1, Nk=1500, d=128, dtype="bf16", causal=True,
                   paged=True, page_size=64, pool_factor=1.3, num_splits=6, seed=14401)
    say("C example: paged decode")
    q, kc, vc, bt = W.gen_paged(w)
    paths = {n: tmp_path / f"{n}.bin" for n in ("q", "kc", "vc", "bt", "o", "lse")}
    for n, x in (("q", q), ("kc", kc), ("vc", vc), ("bt", bt.astype(np.int32))):
        np.ascontiguousarray(x).tofile(paths[n])
    run_example(["decode", w.B, w.H, w.Nk, w.d, w.page_size, kc.shape[0], bt.shape[1],
                 w.num_splits, paths["q"], paths["kc"], paths["vc"], paths["bt"], paths["o"],
                 paths["lse"]], tmp_path)
    o = np.fromfile(paths["o"], dtype=np.float32).reshape(w.B, 1, w.H, w.d)
    lse = np.fromfile(paths["lse"], dtype=np.float32).reshape(w.B, w.H, 1)
    kf = np.stack([O.paged_gather_ref(W.to_float(kc, "bf16"), bt, b, w.Nk) for b in range(w.B)])
    vf = np.stack([O.paged_gather_ref(W.to_float(vc, "bf16"), bt, b, w.Nk) for b in range(w.B)])
    ro, rl = O.attention_ref(W.to_float(q, "bf16"), kf, vf, w.scale, True)
    check(o, lse, ro, rl, "bf16", "C example decode")
