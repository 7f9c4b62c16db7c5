"""fa_bwd_noalloc (the backward with the library's static row-term buffer) against fa_bwd
(the same kernels with a caller workspace): identical gradients, call after call on one
GPU, with a smaller problem after a larger one (the buffer keeps the last call's
contents) and a problem that fills the buffer to its last row block."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_05_amd as fa
import workloads as W
from gpu_common import say, to_dev

pytestmark = pytest.mark.gpu


def both(seed, B, H, nq, nk, d, causal, wl, wr, alibi, cap, grad_dtype=torch.float32):
    q = W.gen_tensor(seed, W.TENSOR_Q, B, nq, H, d, 1.0, "bf16")
    k = W.gen_tensor(seed, W.TENSOR_K, B, nk, H, d, 1.0, "bf16")
    v = W.gen_tensor(seed, W.TENSOR_V, B, nk, H, d, 1.0, "bf16")
    g = W.gen_tensor(seed, 3, B, nq, H, d, 1.0, "bf16")
    tq, tk, tv, tg = (to_dev(x, "bf16") for x in (q, k, v, g))
    scale = 1.0 / np.sqrt(d)
    ts = torch.from_numpy(W.alibi_slopes(H)).cuda() if alibi else None
    o, lse = fa.attention(tq, tk, tv, scale, causal, wl, wr, ts, cap)
    ref = fa.attention_backward(tq, tk, tv, o, lse, tg, scale, causal, wl, wr, ts, cap,
                                grad_dtype=grad_dtype)
    got = [torch.full_like(x, float("nan")) for x in ref]
    st = fa.fa_bwd_noalloc(tq, tk, tv, o, tg, lse, *got, B, H, nq, nk, d, scale, causal, wl, wr,
                           ts, cap)
    assert st == 0, fa.fa_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{name}: max |diff| {(a.float() - b.float()).abs().max().item()}"


def test_noalloc_backward_equals_the_workspace_backward():
    say("noalloc: larger problem, then a smaller one, then the full buffer")
    both(9100, 2, 4, 300, 400, 128, True, -1, -1, True, 20.0)
    both(9101, 1, 2, 70, 90, 64, False, 30, 10, False, 0.0, grad_dtype=torch.bfloat16)
    # batch * heads * ceil(seqlen_q / 32) = 64 * 32 * 32 = 65536 row blocks: the whole buffer.
    assert fa.fa_bwd_workspace_bytes(64, 32, 1024) == 16 << 20
    both(9102, 64, 32, 1024, 64, 64, True, -1, -1, False, 0.0)
    both(9103, 1, 3, 33, 17, 128, True, -1, -1, False, 0.0)


def test_noalloc_refuses_a_problem_past_the_buffer():
    t = torch.zeros(1, device="cuda")
    st = fa.fa_bwd_noalloc(t.bfloat16(), t.bfloat16(), t.bfloat16(), t, t.bfloat16(), t, t, t, t,
                           64, 32, 1025, 64, 64, 0.125, True)
    assert st == 7 and "static buffer" in fa.fa_status_string(st)
