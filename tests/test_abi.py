"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, imports no device allocator, and rejects bad arguments with
the documented status codes before making any HIP call.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

import exact_tiled_attention_05_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# FA_ABI_TEST_LIB names a host-only build of the C ABI (the same fa_api.cpp with stub
# launchers, compiled under AddressSanitizer and UndefinedBehaviorSanitizer by
# tests/test_abi_sanitized.py); when it is set, every call below goes to that build.
SANITIZED_LIB = os.environ.get("FA_ABI_TEST_LIB")
if SANITIZED_LIB:
    fa._lib = fa.declare(ctypes.CDLL(SANITIZED_LIB))
    fa._lib.fa_stub_launches.restype = ctypes.c_longlong

pytestmark = pytest.mark.skipif(not SANITIZED_LIB and not os.path.exists(fa.library_path()),
                                reason="libfa.so not built (run __graft_entry__.build())")
real_library_only = pytest.mark.skipif(bool(SANITIZED_LIB), reason="inspects the built libfa.so")
stub_launchers_only = pytest.mark.skipif(
    not SANITIZED_LIB, reason="passes valid sizes with placeholder pointers: host-only build only")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
OK, NULL, SHAPE, UNSUP, MASK, HIP, VALUE, SCRATCH = range(8)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:\w+\s+)*\w+\s*\*?\s*(fa_\w+)\s*\(", text,
                                 re.M)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_split", "fa_fwd_splitkv", "fa_fwd_splitkv_seqlens",
              "fa_fwd_varlen", "fa_splitkv_combine", "fa_status_string", "fa_split_chunk_len"):
        assert n in names
    assert set(fa.EXPORTED) == set(names)


@real_library_only
def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in declared_functions():
        assert n in exported, n


@real_library_only
def test_library_never_allocates_device_memory():
    out = subprocess.run(["nm", "-D", "--undefined-only", fa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    bad = [s for s in out.split() if re.match(r"hip(Ext)?Malloc|hipFree|hipMemAlloc|hipHostMalloc", s)]
    assert bad == []


def test_status_strings():
    for s in range(8):
        assert fa.fa_status_string(s)
    assert fa.fa_status_string(99) == "unknown status"


def test_split_chunk_len():
    assert fa.fa_split_chunk_len(32768, 16, 256) == 2048
    assert fa.fa_split_chunk_len(2000, 2, 1) == 1000
    assert fa.fa_split_chunk_len(100, 3, 16) == 48
    assert fa.fa_split_chunk_len(5, 8, 1) == 1
    assert fa.fa_split_chunk_len(0, 1, 1) == -1


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=1, o=FAKE, o_dtype=0, lse=None, batch=1, heads=1,
             seqlen_q=4, seqlen_k=4, head_dim=64, scale=0.125, causal=0, wl=-1, wr=-1,
             alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd(a["q"], a["k"], a["v"], a["in_dtype"], a["o"], a["o_dtype"],
                                    a["lse"], a["batch"], a["heads"], a["seqlen_q"], a["seqlen_k"],
                                    a["head_dim"], a["scale"], a["causal"], a["wl"], a["wr"],
                                    a["alibi"], a["softcap"], a["stream"])


def split(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=1, bt=FAKE, maxp=4, ps=16, op=FAKE, lp=FAKE, S=2,
             batch=1, heads=1, seqlen_q=1, seqlen_k=64, head_dim=128, scale=0.1, causal=1,
             wl=-1, wr=-1, alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_splitkv(
        a["q"], a["k"], a["v"], a["in_dtype"], a["bt"], a["maxp"], a["ps"], a["op"], a["lp"],
        a["S"], a["batch"], a["heads"], a["seqlen_q"], a["seqlen_k"], a["head_dim"], a["scale"],
        a["causal"], a["wl"], a["wr"], a["alibi"], a["softcap"], a["stream"])


def fsplit(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=1, op=FAKE, lp=FAKE, S=4, batch=1, heads=1,
             seqlen_q=8, seqlen_k=256, head_dim=128, scale=0.1, causal=1, wl=-1, wr=-1,
             alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_split(
        a["q"], a["k"], a["v"], a["in_dtype"], a["op"], a["lp"], a["S"], a["batch"], a["heads"],
        a["seqlen_q"], a["seqlen_k"], a["head_dim"], a["scale"], a["causal"], a["wl"], a["wr"],
        a["alibi"], a["softcap"], a["stream"])


def comb(**kw):
    a = dict(op=FAKE, lp=FAKE, S=2, batch=1, heads=1, seqlen_q=1, head_dim=128, o=FAKE,
             o_dtype=0, lse=None, stream=None)
    a.update(kw)
    return fa.load_library().fa_splitkv_combine(a["op"], a["lp"], a["S"], a["batch"], a["heads"],
                                                a["seqlen_q"], a["head_dim"], a["o"],
                                                a["o_dtype"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL),
    (dict(batch=0), SHAPE), (dict(heads=-1), SHAPE), (dict(seqlen_q=0), SHAPE),
    (dict(seqlen_k=0), SHAPE), (dict(seqlen_k=(1 << 28) + 1), SHAPE),
    (dict(head_dim=96), UNSUP), (dict(head_dim=256), UNSUP), (dict(in_dtype=2), UNSUP),
    (dict(o_dtype=5), UNSUP),
    (dict(wl=-2), MASK), (dict(wr=-3), MASK), (dict(causal=1, wr=1), MASK),
    (dict(scale=0.0), VALUE), (dict(scale=-1.0), VALUE), (dict(scale=math.inf), VALUE),
    (dict(scale=math.nan), VALUE), (dict(softcap=-1.0), VALUE), (dict(softcap=math.nan), VALUE),
])
def test_fa_fwd_rejects(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(bt=None), NULL), (dict(op=None), NULL), (dict(lp=None), NULL), (dict(q=None), NULL),
    (dict(S=0), SHAPE), (dict(ps=0), SHAPE), (dict(maxp=0), SHAPE),
    (dict(maxp=3, ps=16, seqlen_k=64), SHAPE),
    (dict(head_dim=32), UNSUP), (dict(in_dtype=7), UNSUP),
    (dict(causal=1, wr=2), MASK), (dict(wl=-5), MASK), (dict(softcap=-0.5), VALUE),
])
def test_fa_fwd_splitkv_rejects(kw, code):
    assert split(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(op=None), NULL),
    (dict(lp=None), NULL), (dict(S=0), SHAPE), (dict(S=(1 << 16) + 1), SHAPE),
    (dict(batch=0), SHAPE), (dict(seqlen_k=0), SHAPE),
    (dict(in_dtype=0), UNSUP), (dict(in_dtype=3), UNSUP), (dict(head_dim=96), UNSUP),
    (dict(causal=1, wr=1), MASK), (dict(wl=-2), MASK), (dict(scale=0.0), VALUE),
    (dict(softcap=math.inf), VALUE),
])
def test_fa_fwd_split_rejects(kw, code):
    assert fsplit(**kw) == code


def test_split_chunk_len_for_contiguous_splits():
    # fa_fwd_split cuts the keys in chunks that are whole 64-key tiles.
    assert fa.fa_split_chunk_len(4096, 4, 64) == 1024
    assert fa.fa_split_chunk_len(4096, 3, 64) == 1408
    assert fa.fa_split_chunk_len(100, 8, 64) == 64
    assert fa.fa_split_chunk_len(2000, 7, 64) == 320


@pytest.mark.parametrize("kw,code", [
    (dict(op=None), NULL), (dict(lp=None), NULL), (dict(o=None), NULL),
    (dict(S=0), SHAPE), (dict(batch=0), SHAPE), (dict(seqlen_q=-1), SHAPE),
    (dict(head_dim=80), UNSUP), (dict(o_dtype=3), UNSUP),
])
def test_fa_splitkv_combine_rejects(kw, code):
    assert comb(**kw) == code


def split_seqlens(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=1, bt=FAKE, maxp=4, ps=16, sl=FAKE, op=FAKE, lp=FAKE,
             S=2, batch=1, heads=1, seqlen_q=1, max_k=64, head_dim=128, scale=0.1, causal=1,
             wl=-1, wr=-1, alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_splitkv_seqlens(
        a["q"], a["k"], a["v"], a["in_dtype"], a["bt"], a["maxp"], a["ps"], a["sl"], a["op"],
        a["lp"], a["S"], a["batch"], a["heads"], a["seqlen_q"], a["max_k"], a["head_dim"],
        a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"], a["softcap"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(sl=None), NULL), (dict(bt=None), NULL), (dict(op=None), NULL), (dict(k=None), NULL),
    (dict(S=0), SHAPE), (dict(max_k=0), SHAPE), (dict(maxp=3, ps=16, max_k=64), SHAPE),
    (dict(seqlen_q=0), SHAPE), (dict(head_dim=32), UNSUP), (dict(in_dtype=9), UNSUP),
    (dict(causal=1, wr=3), MASK), (dict(scale=-2.0), VALUE),
])
def test_fa_fwd_splitkv_seqlens_rejects(kw, code):
    assert split_seqlens(**kw) == code


def varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, in_dtype=1, o=FAKE, o_dtype=0, lse=None, cq=FAKE, ck=FAKE,
             batch=2, heads=1, total_q=10, total_k=12, max_q=6, max_k=8, head_dim=64, scale=0.125,
             causal=0, wl=-1, wr=-1, alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_varlen(
        a["q"], a["k"], a["v"], a["in_dtype"], a["o"], a["o_dtype"], a["lse"], a["cq"], a["ck"],
        a["batch"], a["heads"], a["total_q"], a["total_k"], a["max_q"], a["max_k"],
        a["head_dim"], a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"], a["softcap"],
        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cq=None), NULL), (dict(ck=None), NULL), (dict(q=None), NULL), (dict(o=None), NULL),
    (dict(k=None), NULL), (dict(v=None), NULL),
    (dict(batch=0), SHAPE), (dict(heads=0), SHAPE), (dict(total_q=-1), SHAPE),
    (dict(total_k=-1), SHAPE), (dict(max_q=0), SHAPE), (dict(max_k=-1), SHAPE),
    (dict(max_q=(1 << 28) + 1), SHAPE),
    (dict(head_dim=96), UNSUP), (dict(in_dtype=4), UNSUP), (dict(o_dtype=2), UNSUP),
    (dict(wl=-2), MASK), (dict(causal=1, wr=1), MASK), (dict(scale=math.nan), VALUE),
])
def test_fa_fwd_varlen_rejects(kw, code):
    assert varlen(**kw) == code


def test_fa_fwd_varlen_empty_pack_launches_nothing():
    # No query row: the call returns before any HIP call (so it runs without a GPU),
    # and tensors of zero rows may be NULL.
    assert varlen(total_q=0, q=None, o=None) == OK
    assert varlen(total_q=0, total_k=0, q=None, o=None, k=None, v=None, max_k=0) == OK


def split_fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kd=1.0, vd=1.0, bt=FAKE, maxp=4, ps=16, sl=None, op=FAKE,
             lp=FAKE, S=2, batch=1, heads=1, seqlen_q=1, nk=64, head_dim=128, scale=0.1, causal=1,
             wl=-1, wr=-1, alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_splitkv_fp8(
        a["q"], a["k"], a["v"], a["kd"], a["vd"], a["bt"], a["maxp"], a["ps"], a["sl"], a["op"],
        a["lp"], a["S"], a["batch"], a["heads"], a["seqlen_q"], a["nk"], a["head_dim"],
        a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"], a["softcap"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(bt=None), NULL),
    (dict(op=None), NULL), (dict(lp=None), NULL),
    (dict(S=0), SHAPE), (dict(batch=0), SHAPE), (dict(nk=0), SHAPE), (dict(maxp=3), SHAPE),
    (dict(seqlen_q=2), UNSUP), (dict(head_dim=96), UNSUP),
    (dict(kd=0.0), VALUE), (dict(vd=-1.0), VALUE), (dict(kd=math.inf), VALUE),
    (dict(vd=math.nan), VALUE), (dict(kd=1e30, scale=1e30), VALUE), (dict(scale=0.0), VALUE),
    (dict(causal=1, wr=2), MASK), (dict(softcap=-1.0), VALUE),
])
def test_fa_fwd_splitkv_fp8_rejects(kw, code):
    assert split_fp8(**kw) == code


def split_append(**kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, k=FAKE, v=FAKE, in_dtype=1, bt=FAKE, maxp=4, ps=16, sl=FAKE,
             op=FAKE, lp=FAKE, S=2, batch=1, heads=1, seqlen_q=1, max_k=64, head_dim=128,
             scale=0.1, causal=1, wl=-1, wr=-1, alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_splitkv_append(
        a["q"], a["kn"], a["vn"], a["k"], a["v"], a["in_dtype"], a["bt"], a["maxp"], a["ps"],
        a["sl"], a["op"], a["lp"], a["S"], a["batch"], a["heads"], a["seqlen_q"], a["max_k"],
        a["head_dim"], a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"], a["softcap"],
        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), NULL), (dict(vn=None), NULL), (dict(sl=None), NULL), (dict(k=None), NULL),
    (dict(bt=None), NULL), (dict(op=None), NULL),
    (dict(seqlen_q=5, max_k=4), SHAPE), (dict(S=0), SHAPE), (dict(maxp=3, ps=16, max_k=64), SHAPE),
    (dict(batch=0), SHAPE), (dict(head_dim=80), UNSUP), (dict(in_dtype=3), UNSUP),
    (dict(wl=-4), MASK), (dict(softcap=-1.0), VALUE),
])
def test_fa_fwd_splitkv_append_rejects(kw, code):
    assert split_append(**kw) == code



def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, in_dtype=1, o_dtype=0, dq=FAKE,
             dk=FAKE, dv=FAKE, g_dtype=0, ws=FAKE, batch=1, heads=2, seqlen_q=8, seqlen_k=8,
             head_dim=128, scale=0.1, causal=1, wl=-1, wr=-1, alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_bwd(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["in_dtype"], a["o_dtype"], a["dq"],
        a["dk"], a["dv"], a["g_dtype"], a["ws"], a["batch"], a["heads"], a["seqlen_q"],
        a["seqlen_k"], a["head_dim"], a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"],
        a["softcap"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(o=None), NULL), (dict(do=None), NULL), (dict(lse=None), NULL),
    (dict(dq=None), NULL), (dict(dk=None), NULL), (dict(dv=None), NULL), (dict(ws=None), NULL),
    (dict(batch=0), SHAPE), (dict(seqlen_q=0), SHAPE), (dict(seqlen_k=-1), SHAPE),
    (dict(in_dtype=0), UNSUP), (dict(head_dim=96), UNSUP), (dict(o_dtype=4), UNSUP),
    (dict(g_dtype=2), UNSUP), (dict(causal=1, wr=2), MASK), (dict(wl=-3), MASK),
    (dict(scale=0.0), VALUE), (dict(softcap=math.inf), VALUE),
])
def test_fa_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def bwd_noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, in_dtype=1, o_dtype=0, dq=FAKE,
             dk=FAKE, dv=FAKE, g_dtype=0, batch=1, heads=2, seqlen_q=8, seqlen_k=8,
             head_dim=128, scale=0.1, causal=1, wl=-1, wr=-1, alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_bwd_noalloc(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["in_dtype"], a["o_dtype"], a["dq"],
        a["dk"], a["dv"], a["g_dtype"], a["batch"], a["heads"], a["seqlen_q"], a["seqlen_k"],
        a["head_dim"], a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"], a["softcap"],
        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(lse=None), NULL), (dict(dv=None), NULL),
    (dict(batch=0), SHAPE), (dict(seqlen_k=-1), SHAPE), (dict(in_dtype=0), UNSUP),
    (dict(head_dim=96), UNSUP), (dict(causal=1, wr=2), MASK), (dict(scale=0.0), VALUE),
    # the static buffer holds 65536 blocks of 32 rows: one block more is refused
    (dict(batch=2, heads=32, seqlen_q=32 * 1024 + 1), SCRATCH),
    (dict(batch=1, heads=1, seqlen_q=32 * 65536 + 1), SCRATCH),
])
def test_fa_bwd_noalloc_rejects(kw, code):
    assert bwd_noalloc(**kw) == code


def test_noalloc_limit_matches_the_workspace_rule():
    """FA_NOALLOC_SCRATCH_BYTES (the header's figure) against fa_bwd_workspace_bytes at the
    edge: 65536 blocks of 32 rows fit, one more does not."""
    text = open(HEADER).read()
    limit = int(re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+) \* 1024 \* 1024\)", text).group(1)) << 20
    assert fa.fa_bwd_workspace_bytes(2, 32, 32 * 1024) == limit
    assert fa.fa_bwd_workspace_bytes(2, 32, 32 * 1024 + 1) > limit


def test_bwd_workspace_bytes():
    assert fa.fa_bwd_workspace_bytes(4, 16, 2048) == 2 * 4 * 16 * 2048 * 4
    assert fa.fa_bwd_workspace_bytes(1, 2, 33) == 2 * 2 * 64 * 4  # rows padded to 32 per head
    assert fa.fa_bwd_workspace_bytes(0, 1, 1) == -1


def bwd_varlen(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, in_dtype=1, o_dtype=0, dq=FAKE,
             dk=FAKE, dv=FAKE, g_dtype=0, ws=FAKE, cq=FAKE, ck=FAKE, batch=2, heads=2,
             total_q=8, total_k=8, max_q=4, max_k=4, head_dim=128, scale=0.1, causal=1, wl=-1,
             wr=-1, alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_bwd_varlen(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["in_dtype"], a["o_dtype"], a["dq"],
        a["dk"], a["dv"], a["g_dtype"], a["ws"], a["cq"], a["ck"], a["batch"], a["heads"],
        a["total_q"], a["total_k"], a["max_q"], a["max_k"], a["head_dim"], a["scale"],
        a["causal"], a["wl"], a["wr"], a["alibi"], a["softcap"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cq=None), NULL), (dict(ck=None), NULL), (dict(ws=None), NULL), (dict(q=None), NULL),
    (dict(o=None), NULL), (dict(do=None), NULL), (dict(lse=None), NULL), (dict(dq=None), NULL),
    (dict(k=None), NULL), (dict(v=None), NULL), (dict(dk=None), NULL), (dict(dv=None), NULL),
    (dict(batch=0), SHAPE), (dict(heads=0), SHAPE), (dict(total_q=-1), SHAPE),
    (dict(total_k=-1), SHAPE), (dict(max_q=0), SHAPE), (dict(max_k=-1), SHAPE),
    (dict(max_q=(1 << 28) + 1), SHAPE),
    (dict(in_dtype=0), UNSUP), (dict(head_dim=96), UNSUP), (dict(o_dtype=4), UNSUP),
    (dict(g_dtype=2), UNSUP), (dict(causal=1, wr=2), MASK), (dict(wl=-3), MASK),
    (dict(scale=0.0), VALUE), (dict(softcap=math.inf), VALUE),
])
def test_fa_bwd_varlen_rejects(kw, code):
    assert bwd_varlen(**kw) == code


def test_fa_bwd_varlen_empty_pack_launches_nothing():
    # No row on either side: the call returns before any HIP call, and the
    # tensors of zero rows may be NULL.
    assert bwd_varlen(total_q=0, total_k=0, q=None, o=None, do=None, lse=None, dq=None, k=None,
                      v=None, dk=None, dv=None) == OK
    assert bwd_varlen(total_q=0, total_k=0, in_dtype=0) == UNSUP  # still validated


def fp8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, qd=1.0, kd=1.0, vd=1.0, o=FAKE, o_dtype=0, lse=None, batch=1,
             heads=1, seqlen_q=4, seqlen_k=4, head_dim=128, scale=0.125, causal=0, wl=-1, wr=-1,
             alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_fp8(
        a["q"], a["k"], a["v"], a["qd"], a["kd"], a["vd"], a["o"], a["o_dtype"], a["lse"],
        a["batch"], a["heads"], a["seqlen_q"], a["seqlen_k"], a["head_dim"], a["scale"],
        a["causal"], a["wl"], a["wr"], a["alibi"], a["softcap"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL),
    (dict(batch=0), SHAPE), (dict(seqlen_k=0), SHAPE), (dict(head_dim=96), UNSUP),
    (dict(o_dtype=3), UNSUP), (dict(causal=1, wr=2), MASK), (dict(qd=0.0), VALUE),
    (dict(kd=-1.0), VALUE), (dict(vd=math.inf), VALUE), (dict(qd=math.nan), VALUE),
    (dict(qd=1e30, kd=1e30), VALUE), (dict(scale=0.0), VALUE),
])
def test_fa_fwd_fp8_rejects(kw, code):
    assert fp8(**kw) == code


def split8(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, qd=1.0, kd=1.0, vd=1.0, op=FAKE, lp=FAKE, S=4, batch=1,
             heads=1, seqlen_q=4, seqlen_k=1000, head_dim=128, scale=0.125, causal=0, wl=-1, wr=-1,
             alibi=None, softcap=0.0, stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_split_fp8(
        a["q"], a["k"], a["v"], a["qd"], a["kd"], a["vd"], a["op"], a["lp"], a["S"], a["batch"],
        a["heads"], a["seqlen_q"], a["seqlen_k"], a["head_dim"], a["scale"], a["causal"], a["wl"],
        a["wr"], a["alibi"], a["softcap"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(op=None), NULL),
    (dict(lp=None), NULL), (dict(batch=0), SHAPE), (dict(seqlen_q=0), SHAPE), (dict(S=0), SHAPE),
    (dict(S=(1 << 16) + 1), SHAPE), (dict(head_dim=96), UNSUP), (dict(causal=1, wr=2), MASK),
    (dict(wl=-2), MASK), (dict(qd=0.0), VALUE), (dict(vd=math.nan), VALUE),
    (dict(qd=1e30, kd=1e30), VALUE), (dict(scale=-1.0), VALUE), (dict(softcap=-1.0), VALUE),
])
def test_fa_fwd_split_fp8_rejects(kw, code):
    assert split8(**kw) == code


def paged8(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, qd=1.0, kd=1.0, vd=1.0, bt=FAKE, maxp=8, page=128,
             seqlens=None, op=FAKE, lp=FAKE, S=4, batch=1, heads=1, seqlen_q=300, seqlen_k=1000,
             head_dim=128, scale=0.125, causal=1, wl=-1, wr=-1, alibi=None, softcap=0.0,
             stream=None)
    a.update(kw)
    return fa.load_library().fa_fwd_paged_fp8(
        a["q"], a["kc"], a["vc"], a["qd"], a["kd"], a["vd"], a["bt"], a["maxp"], a["page"],
        a["seqlens"], a["op"], a["lp"], a["S"], a["batch"], a["heads"], a["seqlen_q"],
        a["seqlen_k"], a["head_dim"], a["scale"], a["causal"], a["wl"], a["wr"], a["alibi"],
        a["softcap"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(kc=None), NULL), (dict(vc=None), NULL), (dict(bt=None), NULL),
    (dict(op=None), NULL), (dict(lp=None), NULL), (dict(batch=0), SHAPE),
    (dict(seqlen_q=0), SHAPE), (dict(seqlen_k=0), SHAPE), (dict(S=0), SHAPE),
    (dict(S=(1 << 16) + 1), SHAPE), (dict(maxp=0), SHAPE), (dict(page=0), SHAPE),
    (dict(maxp=7), SHAPE),                                   # 7 pages of 128 < 1000 keys
    (dict(page=1 << 20, heads=1 << 4), SHAPE),               # a page of >= 2^31 bytes
    (dict(head_dim=96), UNSUP), (dict(causal=1, wr=2), MASK), (dict(wl=-2), MASK),
    (dict(qd=0.0), VALUE), (dict(kd=math.inf), VALUE), (dict(vd=math.nan), VALUE),
    (dict(qd=1e30, kd=1e30), VALUE), (dict(scale=-1.0), VALUE), (dict(softcap=-1.0), VALUE),
])
def test_fa_fwd_paged_fp8_rejects(kw, code):
    assert paged8(**kw) == code


def test_fp8_split_chunks_are_multiples_of_the_fp8_key_tile():
    assert fa.fa_split_chunk_len(1000, 4, 128) == 256
    assert fa.fa_split_chunk_len(4096, 8, 128) == 512
    assert fa.fa_split_chunk_len(100, 3, 128) == 128


def test_num_splits_heuristic():
    # One query row: at least two workgroups per compute unit (256 here), head
    # groups of 256-byte segments (512 at head_dim 128: the wide groups), at most
    # one split per page and 64 splits.
    ns = fa.fa_num_splits
    assert ns(1, 32, 1, 4096, 128, 256, num_cus=256) == 16
    assert ns(4, 32, 1, 8192, 128, 256, num_cus=256) == 8
    assert ns(1, 8, 1, 16384, 128, 256, num_cus=256) == 64
    assert ns(16, 32, 1, 2048, 128, 256, num_cus=256) == 2
    assert ns(64, 32, 1, 2048, 128, 256, num_cus=256) == 1
    assert ns(8, 32, 1, 32768, 128, 256, fp8_cache=True, num_cus=256) == 8  # 4 heads per group
    assert ns(1, 32, 1, 4096, 128, 256, fp8_cache=True, num_cus=256) == 16  # capped: 16 pages
    assert ns(1, 32, 1, 4096, 64, 256, fp8_cache=True, num_cus=256) == 16   # capped: 16 pages
    assert ns(1, 1, 1, 300, 128, 256, num_cus=256) == 2                      # 2 pages
    assert ns(1, 1, 1, 1 << 20, 128, 16, num_cus=256) == 64                  # at most 64
    # Several rows: two workgroups per compute unit (128-row query tiles).
    assert ns(2, 8, 512, 4096, 128, 64, num_cus=256) == 8
    assert ns(4, 16, 2048, 2048, 128, 64, num_cus=256) == 1
    for bad in [(0, 1, 1, 1, 128, 64), (1, 0, 1, 1, 128, 64), (1, 1, 0, 1, 128, 64),
                (1, 1, 1, 0, 128, 64), (1, 1, 1, 1, 96, 64), (1, 1, 1, 1, 128, 0)]:
        assert ns(*bad, num_cus=256) == -1


def test_binding_checks_alibi_slopes():
    """The binding passes slopes as a raw pointer the kernels read as float32 [heads]:
    anything else (another dtype, another length, another device) is refused before
    the call."""
    import torch
    h = 4
    assert fa._slopes_ptr(None, h, None) is None
    with pytest.raises(TypeError):
        fa._slopes_ptr([0.5] * h, h, None)
    with pytest.raises(TypeError):
        fa._slopes_ptr(torch.ones(h, dtype=torch.float64), h, None)
    with pytest.raises(ValueError):
        fa._slopes_ptr(torch.ones(h - 1, dtype=torch.float32), h, None)
    with pytest.raises(ValueError):
        fa._slopes_ptr(torch.ones(1, h, dtype=torch.float32), h, None)
    with pytest.raises(ValueError):  # host memory, never a device pointer
        fa._slopes_ptr(torch.ones(h, dtype=torch.float32), h, None)
    with pytest.raises(ValueError):  # q on another device
        fa._slopes_ptr(torch.ones(h, dtype=torch.float32), h, torch.empty(1, device="meta"))



def test_binding_combine_checks_partials():
    """combine() takes its sizes from o_part, so a log-sum-exp buffer of another
    shape or dtype (which the kernel would read past its end) is refused first."""
    import torch
    op = torch.zeros(3, 2, 4, 5, 64)
    with pytest.raises(ValueError):
        fa.combine(op, torch.zeros(3, 2, 4, 6))
    with pytest.raises(ValueError):
        fa.combine(op, torch.zeros(3, 2, 4, 5, dtype=torch.float64))
    with pytest.raises(ValueError):
        fa.combine(op.double(), torch.zeros(3, 2, 4, 5))
    with pytest.raises(ValueError):
        fa.combine(op[0], torch.zeros(2, 4, 5))
    with pytest.raises(ValueError):  # lse_part on another device
        fa.combine(op, torch.zeros(3, 2, 4, 5, device="meta"))

def launches():
    return fa.load_library().fa_stub_launches()


@stub_launchers_only
@pytest.mark.parametrize("call,kw", [
    (lambda **kw: fwd(**kw), dict()),
    (lambda **kw: fwd(**kw), dict(batch=1 << 24, heads=1, seqlen_q=1, seqlen_k=1 << 28)),
    (lambda **kw: fwd(**kw), dict(batch=1, heads=1 << 16, seqlen_q=1 << 14, seqlen_k=7)),
    (lambda **kw: split(**kw), dict()),
    (lambda **kw: split(**kw), dict(S=1 << 16, seqlen_k=1 << 28, maxp=(1 << 28) // 16)),
    (lambda **kw: fsplit(**kw), dict()),
    (lambda **kw: comb(**kw), dict()),
    (lambda **kw: varlen(**kw), dict()),
    (lambda **kw: split_fp8(**kw), dict()),
    (lambda **kw: split_append(**kw), dict()),
    (lambda **kw: split_append(**kw), dict(seqlen_q=8)),             # append launch, then slabs
    (lambda **kw: split_append(**kw), dict(seqlen_q=8, ps=7, maxp=10)),  # rows gathered
    (lambda **kw: fp8(**kw), dict()),
    (lambda **kw: split8(**kw), dict()),
    (lambda **kw: split8(**kw), dict(S=1 << 16, seqlen_k=1 << 28)),
    (lambda **kw: paged8(**kw), dict()),
    (lambda **kw: paged8(**kw), dict(page=384, maxp=3)),   # a page size that is no power of two
    (lambda **kw: paged8(**kw), dict(page=16, maxp=63)),   # rows gathered page by page
    (lambda **kw: paged8(**kw), dict(page=7, maxp=143)),
    (lambda **kw: paged8(**kw), dict(seqlen_q=1, S=1 << 16, seqlen_k=1 << 28, page=128,
                                     maxp=1 << 21)),
    (lambda **kw: bwd(**kw), dict()),
    (lambda **kw: bwd(**kw), dict(batch=1 << 10, heads=1 << 10, seqlen_q=1 << 11, seqlen_k=1)),
    (lambda **kw: bwd_noalloc(**kw), dict()),
])
def test_valid_calls_reach_the_launchers(call, kw):
    """Valid sizes, up to the stated limits, pass validation and reach the launchers with
    parameters the kernels can run (the stubs check them); run under the sanitizers, the
    size arithmetic on the way is free of overflow and out-of-bounds access."""
    n = launches()
    assert call(**kw) == OK
    assert launches() > n


@stub_launchers_only
def test_refused_and_empty_calls_launch_nothing():
    n = launches()
    assert fwd(batch=0) == SHAPE and fwd(head_dim=96) == UNSUP and bwd(ws=None) == NULL
    assert varlen(total_q=0, total_k=0, q=None, o=None, k=None, v=None, max_k=0) == OK
    assert bwd_noalloc(batch=2, heads=32, seqlen_q=32 * 1024 + 1) == SCRATCH
    assert launches() == n
