"""Python binding of libfa, the gfx950 exact tiled attention library.

The functions named like the C ABI (``fa_fwd``, ``fa_fwd_split``,
``fa_fwd_splitkv``, ``fa_fwd_splitkv_seqlens``, ``fa_fwd_splitkv_append``, ``fa_fwd_varlen``,
``fa_fwd_fp8``, ``fa_fwd_split_fp8``, ``fa_fwd_splitkv_fp8``, ``fa_fwd_paged_fp8``, ``fa_bwd``, ``fa_bwd_workspace_bytes``, ``fa_splitkv_combine``, ``fa_status_string``,
``fa_split_chunk_len``) only
marshal arguments: torch tensors become device pointers, the current torch
stream becomes the HIP stream, and every step of the computation runs in the
library's kernels. ``attention``, ``attention_fp8``, ``attention_split_fp8``, ``attention_varlen``, ``attention_split``,
``attention_paged_splitkv``, ``attention_paged_fp8``, ``attention_paged_append``, ``attention_backward``,
``combine`` and ``decode_paged`` add output allocation (torch.empty) on top of them.

The library must be built (``python -m exact_tiled_attention_05_amd.build``);
importing works without it, but every call raises if libfa.so is missing.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "FA_FP32", "FA_BF16", "FaError", "library_path", "load_library",
    "fa_fwd", "fa_fwd_split", "fa_fwd_splitkv", "fa_fwd_splitkv_seqlens",
    "fa_fwd_splitkv_append", "fa_fwd_varlen", "fa_fwd_fp8", "fa_fwd_split_fp8", "fa_fwd_splitkv_fp8",
    "fa_fwd_paged_fp8", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_workspace_bytes", "fa_bwd_varlen", "fa_splitkv_combine", "fa_status_string",
    "fa_split_chunk_len", "fa_num_splits",
    "attention", "attention_fp8", "attention_split_fp8", "attention_split_partials_fp8",
    "attention_varlen", "attention_split", "attention_split_partials",
    "attention_paged_splitkv", "attention_paged_splitkv_fp8", "attention_paged_fp8",
    "attention_paged_append",
    "attention_backward", "attention_varlen_backward", "combine", "decode_paged",
]

FA_FP32, FA_BF16 = 0, 1
FA_OK = 0
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
_lib = None

EXPORTED = ("fa_fwd", "fa_fwd_split", "fa_fwd_splitkv", "fa_fwd_splitkv_seqlens",
            "fa_fwd_splitkv_append", "fa_fwd_varlen", "fa_fwd_fp8", "fa_fwd_split_fp8",
            "fa_fwd_splitkv_fp8", "fa_fwd_paged_fp8", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_workspace_bytes", "fa_bwd_varlen", "fa_splitkv_combine", "fa_status_string",
            "fa_split_chunk_len", "fa_num_splits")


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {fa_status_string(status)}")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libfa.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m exact_tiled_attention_05_amd.build`")
    _lib = declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def declare(lib):
    """Set the ctypes signatures of the C ABI's functions on a loaded library."""
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, i, vp, i, vp, i, i, i, i, i, f, i, i, i, vp, f, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, i, vp, i, i, vp, vp, i, i, i, i, i, i, f, i, i, i,
                                   vp, f, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_split.argtypes = [vp, vp, vp, i, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, f, vp]
    lib.fa_fwd_split.restype = i
    lib.fa_fwd_splitkv_seqlens.argtypes = [vp, vp, vp, i, vp, i, i, vp, vp, vp, i, i, i, i, i, i,
                                           f, i, i, i, vp, f, vp]
    lib.fa_fwd_splitkv_seqlens.restype = i
    lib.fa_fwd_splitkv_append.argtypes = [vp, vp, vp, vp, vp, i, vp, i, i, vp, vp, vp, i, i, i,
                                          i, i, i, f, i, i, i, vp, f, vp]
    lib.fa_fwd_splitkv_append.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, f, f, f, vp, i, vp, i, i, i, i, i, f, i, i, i, vp, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_split_fp8.argtypes = [vp, vp, vp, f, f, f, vp, vp, i, i, i, i, i, i, f, i, i, i, vp,
                                     f, vp]
    lib.fa_fwd_split_fp8.restype = i
    lib.fa_fwd_splitkv_fp8.argtypes = [vp, vp, vp, f, f, vp, i, i, vp, vp, vp, i, i, i, i, i, i,
                                       f, i, i, i, vp, f, vp]
    lib.fa_fwd_splitkv_fp8.restype = i
    lib.fa_fwd_paged_fp8.argtypes = [vp, vp, vp, f, f, f, vp, i, i, vp, vp, vp, i, i, i, i, i, i,
                                     f, i, i, i, vp, f, vp]
    lib.fa_fwd_paged_fp8.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, i, vp, i, i, i, i, i, f, i,
                           i, i, vp, f, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, i, i, i, i, i, i,
                                   f, i, i, i, vp, f, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, vp, vp, vp, i, vp, vp, vp, i, i,
                                  i, i, i, i, i, f, i, i, i, vp, f, vp]
    lib.fa_bwd_varlen.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_longlong
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, i, vp, i, vp, vp, vp, i, i, i, i, i, i, i, f, i, i,
                                  i, vp, f, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_splitkv_combine.argtypes = [vp, vp, i, i, i, i, i, vp, i, vp, vp]
    lib.fa_splitkv_combine.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_split_chunk_len.argtypes = [i, i, i]
    lib.fa_split_chunk_len.restype = i
    lib.fa_num_splits.argtypes = [i, i, i, i, i, i, i, i]
    lib.fa_num_splits.restype = i
    return lib


# --------------------------------------------------------------------------
# marshalling helpers
# --------------------------------------------------------------------------
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _slopes_ptr(slopes, heads, like):
    """ALiBi slopes as the C ABI reads them: float32 [heads], contiguous, on q's device
    (a wrong dtype or a short tensor would be read past its end on the device)."""
    if slopes is None:
        return None
    if not isinstance(slopes, torch.Tensor):
        raise TypeError("alibi_slopes must be a torch.Tensor (float32 [heads]) or None")
    if slopes.dtype != torch.float32:
        raise TypeError(f"alibi_slopes must be float32, got {slopes.dtype}")
    if slopes.dim() != 1 or slopes.shape[0] != int(heads):
        raise ValueError(f"alibi_slopes must have shape ({int(heads)},), got {tuple(slopes.shape)}")
    if like is not None and slopes.device != like.device:
        raise ValueError(f"alibi_slopes lives on {slopes.device}, q on {like.device}")
    return _ptr(slopes)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != FA_OK:
        raise FaError(status, where)


# --------------------------------------------------------------------------
# C ABI, same names
# --------------------------------------------------------------------------
def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_num_splits(batch: int, heads: int, seqlen_q: int, seqlen_k: int, head_dim: int,
                  page_size: int = 64, fp8_cache: bool = False, num_cus: int = 0) -> int:
    """Split count for the split passes (fa_num_splits); -1 on bad sizes."""
    return int(load_library().fa_num_splits(int(batch), int(heads), int(seqlen_q), int(seqlen_k),
                                            int(head_dim), int(page_size), int(bool(fp8_cache)),
                                            int(num_cus)))


def _splits(num_splits, *args, **kw) -> int:
    if num_splits is not None:
        return int(num_splits)
    s = fa_num_splits(*args, **kw)
    if s <= 0:
        raise ValueError(f"fa_num_splits{args}: bad sizes, or no HIP device to ask for its "
                         "compute-unit count; pass num_splits explicitly")
    return s


def fa_split_chunk_len(seqlen_k: int, num_splits: int, page_size: int) -> int:
    return load_library().fa_split_chunk_len(int(seqlen_k), int(num_splits), int(page_size))


def fa_fwd(q, k, v, o, lse, batch, heads, seqlen_q, seqlen_k, head_dim, softmax_scale,
           causal=False, window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
           stream=None) -> int:
    """Call fa_fwd on caller-allocated tensors; returns the status code."""
    return load_library().fa_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(o), _dtype_code(o), _ptr(lse),
        int(batch), int(heads), int(seqlen_q), int(seqlen_k), int(head_dim),
        float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
        _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_fwd_splitkv(q, k_cache, v_cache, block_table, max_pages_per_seq, page_size, o_part,
                   lse_part, num_splits, batch, heads, seqlen_q, seqlen_k, head_dim,
                   softmax_scale, causal=False, window_left=-1, window_right=-1,
                   alibi_slopes=None, softcap=0.0, stream=None) -> int:
    """Call fa_fwd_splitkv on caller-allocated tensors; returns the status code."""
    return load_library().fa_fwd_splitkv(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q), _ptr(block_table),
        int(max_pages_per_seq), int(page_size), _ptr(o_part), _ptr(lse_part), int(num_splits),
        int(batch), int(heads), int(seqlen_q), int(seqlen_k), int(head_dim),
        float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
        _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_fwd_splitkv_seqlens(q, k_cache, v_cache, block_table, max_pages_per_seq, page_size,
                           cache_seqlens, o_part, lse_part, num_splits, batch, heads, seqlen_q,
                           max_seqlen_k, head_dim, softmax_scale, causal=False, window_left=-1,
                           window_right=-1, alibi_slopes=None, softcap=0.0, stream=None) -> int:
    """Call fa_fwd_splitkv_seqlens on caller-allocated tensors; returns the status code."""
    return load_library().fa_fwd_splitkv_seqlens(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _dtype_code(q), _ptr(block_table),
        int(max_pages_per_seq), int(page_size), _ptr(cache_seqlens), _ptr(o_part), _ptr(lse_part),
        int(num_splits), int(batch), int(heads), int(seqlen_q), int(max_seqlen_k), int(head_dim),
        float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
        _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_fwd_splitkv_append(q, k_new, v_new, k_cache, v_cache, block_table, max_pages_per_seq,
                          page_size, cache_seqlens, o_part, lse_part, num_splits, batch, heads,
                          seqlen_q, max_seqlen_k, head_dim, softmax_scale, causal=False,
                          window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                          stream=None) -> int:
    """Call fa_fwd_splitkv_append on caller-allocated tensors; returns the status code."""
    return load_library().fa_fwd_splitkv_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _dtype_code(q),
        _ptr(block_table), int(max_pages_per_seq), int(page_size), _ptr(cache_seqlens),
        _ptr(o_part), _ptr(lse_part), int(num_splits), int(batch), int(heads), int(seqlen_q),
        int(max_seqlen_k), int(head_dim), float(softmax_scale), int(bool(causal)),
        int(window_left), int(window_right), _slopes_ptr(alibi_slopes, heads, q), float(softcap),
        _stream(stream))


def _ptr_fp8(t):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("fp8 inputs must be uint8 codes or torch.float8_e4m3fn")
    return _ptr(t)


def fa_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, batch, heads, seqlen_q,
               seqlen_k, head_dim, softmax_scale, causal=False, window_left=-1, window_right=-1,
               alibi_slopes=None, softcap=0.0, stream=None) -> int:
    """Call fa_fwd_fp8 on caller-allocated tensors (q, k, v: E4M3 codes); returns the status."""
    return load_library().fa_fwd_fp8(
        _ptr_fp8(q), _ptr_fp8(k), _ptr_fp8(v), float(q_descale), float(k_descale),
        float(v_descale), _ptr(o), _dtype_code(o), _ptr(lse), int(batch), int(heads),
        int(seqlen_q), int(seqlen_k), int(head_dim), float(softmax_scale), int(bool(causal)),
        int(window_left), int(window_right), _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_fwd_split_fp8(q, k, v, q_descale, k_descale, v_descale, o_part, lse_part, num_splits,
                     batch, heads, seqlen_q, seqlen_k, head_dim, softmax_scale, causal=False,
                     window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                     stream=None) -> int:
    """Call fa_fwd_split_fp8 on caller-allocated tensors (q, k, v: E4M3 codes); returns the status."""
    return load_library().fa_fwd_split_fp8(
        _ptr_fp8(q), _ptr_fp8(k), _ptr_fp8(v), float(q_descale), float(k_descale),
        float(v_descale), _ptr(o_part), _ptr(lse_part), int(num_splits), int(batch), int(heads),
        int(seqlen_q), int(seqlen_k), int(head_dim), float(softmax_scale), int(bool(causal)),
        int(window_left), int(window_right), _slopes_ptr(alibi_slopes, heads, q), float(softcap),
        _stream(stream))


def fa_fwd_splitkv_fp8(q, k_cache, v_cache, k_descale, v_descale, block_table,
                       max_pages_per_seq, page_size, cache_seqlens, o_part, lse_part, num_splits,
                       batch, heads, seqlen_q, seqlen_k, head_dim, softmax_scale, causal=False,
                       window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                       stream=None) -> int:
    """Call fa_fwd_splitkv_fp8 on caller-allocated tensors; returns the status code."""
    return load_library().fa_fwd_splitkv_fp8(
        _ptr(q), _ptr_fp8(k_cache), _ptr_fp8(v_cache), float(k_descale), float(v_descale),
        _ptr(block_table), int(max_pages_per_seq), int(page_size), _ptr(cache_seqlens),
        _ptr(o_part), _ptr(lse_part), int(num_splits), int(batch), int(heads), int(seqlen_q),
        int(seqlen_k), int(head_dim), float(softmax_scale), int(bool(causal)), int(window_left),
        int(window_right), _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_fwd_paged_fp8(q, k_cache, v_cache, q_descale, k_descale, v_descale, block_table,
                     max_pages_per_seq, page_size, cache_seqlens, o_part, lse_part, num_splits,
                     batch, heads, seqlen_q, seqlen_k, head_dim, softmax_scale, causal=False,
                     window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                     stream=None) -> int:
    """Call fa_fwd_paged_fp8 on caller-allocated tensors (q and the caches: E4M3 codes);
    returns the status code."""
    return load_library().fa_fwd_paged_fp8(
        _ptr_fp8(q), _ptr_fp8(k_cache), _ptr_fp8(v_cache), float(q_descale), float(k_descale),
        float(v_descale), _ptr(block_table), int(max_pages_per_seq), int(page_size),
        _ptr(cache_seqlens), _ptr(o_part), _ptr(lse_part), int(num_splits), int(batch),
        int(heads), int(seqlen_q), int(seqlen_k), int(head_dim), float(softmax_scale),
        int(bool(causal)), int(window_left), int(window_right),
        _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, batch, heads, seqlen_q, seqlen_k,
           head_dim, softmax_scale, causal=False, window_left=-1, window_right=-1,
           alibi_slopes=None, softcap=0.0, stream=None) -> int:
    """Call fa_bwd on caller-allocated tensors; returns the status code."""
    return load_library().fa_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _dtype_code(q), _dtype_code(o),
        _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq), _ptr(workspace), int(batch), int(heads),
        int(seqlen_q), int(seqlen_k), int(head_dim), float(softmax_scale), int(bool(causal)),
        int(window_left), int(window_right), _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, batch, heads, seqlen_q, seqlen_k,
                   head_dim, softmax_scale, causal=False, window_left=-1, window_right=-1,
                   alibi_slopes=None, softcap=0.0, stream=None) -> int:
    """Call fa_bwd_noalloc (fa_bwd with the library's static row-term buffer); returns the
    status code."""
    return load_library().fa_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _dtype_code(q), _dtype_code(o),
        _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq), int(batch), int(heads), int(seqlen_q),
        int(seqlen_k), int(head_dim), float(softmax_scale), int(bool(causal)), int(window_left),
        int(window_right), _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_bwd_workspace_bytes(batch: int, heads: int, seqlen_q: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(int(batch), int(heads), int(seqlen_q)))


def fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, workspace, cu_seqlens_q, cu_seqlens_k,
                  batch, heads, total_q, total_k, max_seqlen_q, max_seqlen_k, head_dim,
                  softmax_scale, causal=False, window_left=-1, window_right=-1,
                  alibi_slopes=None, softcap=0.0, stream=None) -> int:
    """Call fa_bwd_varlen on caller-allocated tensors; returns the status code."""
    return load_library().fa_bwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _dtype_code(q), _dtype_code(o),
        _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq), _ptr(workspace), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), int(batch), int(heads), int(total_q), int(total_k),
        int(max_seqlen_q), int(max_seqlen_k), int(head_dim), float(softmax_scale),
        int(bool(causal)), int(window_left), int(window_right), _slopes_ptr(alibi_slopes, heads, q),
        float(softcap), _stream(stream))


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, heads, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, head_dim, softmax_scale, causal=False,
                  window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                  stream=None) -> int:
    """Call fa_fwd_varlen on caller-allocated tensors; returns the status code."""
    return load_library().fa_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(o), _dtype_code(o), _ptr(lse),
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(batch), int(heads), int(total_q),
        int(total_k), int(max_seqlen_q), int(max_seqlen_k), int(head_dim),
        float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
        _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_fwd_split(q, k, v, o_part, lse_part, num_splits, batch, heads, seqlen_q, seqlen_k,
                 head_dim, softmax_scale, causal=False, window_left=-1, window_right=-1,
                 alibi_slopes=None, softcap=0.0, stream=None) -> int:
    """Call fa_fwd_split on caller-allocated tensors; returns the status code."""
    return load_library().fa_fwd_split(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(o_part), _ptr(lse_part),
        int(num_splits), int(batch), int(heads), int(seqlen_q), int(seqlen_k), int(head_dim),
        float(softmax_scale), int(bool(causal)), int(window_left), int(window_right),
        _slopes_ptr(alibi_slopes, heads, q), float(softcap), _stream(stream))


def fa_splitkv_combine(o_part, lse_part, num_splits, batch, heads, seqlen_q, head_dim, o, lse,
                       stream=None) -> int:
    """Call fa_splitkv_combine on caller-allocated tensors; returns the status code."""
    return load_library().fa_splitkv_combine(
        _ptr(o_part), _ptr(lse_part), int(num_splits), int(batch), int(heads), int(seqlen_q),
        int(head_dim), _ptr(o), _dtype_code(o), _ptr(lse), _stream(stream))


# --------------------------------------------------------------------------
# Allocating conveniences
# --------------------------------------------------------------------------
def _same_dtype(*ts):
    d = ts[0].dtype
    for t in ts[1:]:
        if t.dtype != d:
            raise TypeError("q, k and v must share one dtype")


def attention(q, k, v, softmax_scale=None, causal=False, window_left=-1, window_right=-1,
              alibi_slopes=None, softcap=0.0, out_dtype=torch.float32, stream=None):
    """O [B, Nq, H, d] (out_dtype) and LSE [B, H, Nq] fp32 for q [B,Nq,H,d], k/v [B,Nk,H,d]."""
    _same_dtype(q, k, v)
    B, nq, H, d = q.shape
    nk = k.shape[1]
    if tuple(k.shape) != (B, nk, H, d) or tuple(v.shape) != (B, nk, H, d):
        raise ValueError("k and v must be [B, Nk, H, d] matching q")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, nq, H, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=q.device)
    _check(fa_fwd(q, k, v, o, lse, B, H, nq, nk, d, softmax_scale, causal, window_left,
                  window_right, alibi_slopes, softcap, stream), "fa_fwd")
    return o, lse


def attention_fp8(q, k, v, q_descale=1.0, k_descale=1.0, v_descale=1.0, softmax_scale=None,
                  causal=False, window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                  out_dtype=torch.float32, stream=None):
    """O [B, Nq, H, d] and LSE [B, H, Nq] for E4M3 q [B,Nq,H,d], k/v [B,Nk,H,d] (uint8 codes
    or float8_e4m3fn) with per-tensor descale factors."""
    B, nq, H, d = q.shape
    nk = k.shape[1]
    if tuple(k.shape) != (B, nk, H, d) or tuple(v.shape) != (B, nk, H, d):
        raise ValueError("k and v must be [B, Nk, H, d] matching q")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, nq, H, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=q.device)
    _check(fa_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, nq, nk, d,
                      softmax_scale, causal, window_left, window_right, alibi_slopes, softcap,
                      stream), "fa_fwd_fp8")
    return o, lse


def attention_split_partials_fp8(q, k, v, num_splits=None, q_descale=1.0, k_descale=1.0,
                                 v_descale=1.0, softmax_scale=None, causal=False, window_left=-1,
                                 window_right=-1, alibi_slopes=None, softcap=0.0, stream=None):
    """Split partials o_part [S,B,H,Nq,d] and lse_part [S,B,H,Nq] of the FP8 forward over
    E4M3 q [B,Nq,H,d], k/v [B,Nk,H,d] (uint8 codes or float8_e4m3fn)."""
    B, nq, H, d = q.shape
    nk = k.shape[1]
    if tuple(k.shape) != (B, nk, H, d) or tuple(v.shape) != (B, nk, H, d):
        raise ValueError("k and v must be [B, Nk, H, d] matching q")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_splits = _splits(num_splits, B, H, nq, nk, d, 128)
    o_part = torch.empty((num_splits, B, H, nq, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((num_splits, B, H, nq), dtype=torch.float32, device=q.device)
    _check(fa_fwd_split_fp8(q, k, v, q_descale, k_descale, v_descale, o_part, lse_part,
                            num_splits, B, H, nq, nk, d, softmax_scale, causal, window_left,
                            window_right, alibi_slopes, softcap, stream), "fa_fwd_split_fp8")
    return o_part, lse_part


def attention_split_fp8(q, k, v, num_splits=None, out_dtype=torch.float32, stream=None, **kw):
    """fa_fwd_split_fp8 followed by the combine kernel."""
    o_part, lse_part = attention_split_partials_fp8(q, k, v, num_splits, stream=stream, **kw)
    return combine(o_part, lse_part, out_dtype=out_dtype, stream=stream)


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                     softmax_scale=None, causal=False, window_left=-1, window_right=-1,
                     alibi_slopes=None, softcap=0.0, out_dtype=torch.float32, stream=None):
    """O [total_q, H, d] (out_dtype) and LSE [H, total_q] fp32 for a packed batch.

    q [total_q, H, d], k/v [total_k, H, d]; cu_seqlens_q/k are int32 [B + 1]
    device offsets. max_seqlen_q/k are host ints bounding the lengths.
    """
    _same_dtype(q, k, v)
    total_q, H, d = q.shape
    total_k = k.shape[0]
    if tuple(k.shape) != (total_k, H, d) or tuple(v.shape) != (total_k, H, d):
        raise ValueError("k and v must be [total_k, H, d] matching q")
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or cu.dim() != 1:
            raise ValueError("cu_seqlens must be int32 [B + 1]")
    if cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    B = cu_seqlens_q.shape[0] - 1
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    o = torch.empty((total_q, H, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    _check(fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k,
                         max_seqlen_q, max_seqlen_k, d, softmax_scale, causal, window_left,
                         window_right, alibi_slopes, softcap, stream), "fa_fwd_varlen")
    return o, lse


def attention_paged_splitkv(q, k_cache, v_cache, block_table, seqlen_k, num_splits=None,
                            softmax_scale=None, causal=False, window_left=-1, window_right=-1,
                            alibi_slopes=None, softcap=0.0, stream=None, cache_seqlens=None):
    """Split partials o_part [S,B,H,Nq,d] and lse_part [S,B,H,Nq] over a paged cache
    (num_splits None: fa_num_splits' choice for the current device).

    With cache_seqlens (int32 [B] on the device), sequence b uses its first
    cache_seqlens[b] keys and seqlen_k is the maximum length.
    """
    _same_dtype(q, k_cache, v_cache)
    B, nq, H, d = q.shape
    _, page_size, Hc, dc = k_cache.shape
    if (Hc, dc) != (H, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache must be [num_pages, page_size, H, d] matching q")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages_per_seq]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_splits = _splits(num_splits, B, H, nq, seqlen_k, d, page_size)
    o_part = torch.empty((num_splits, B, H, nq, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((num_splits, B, H, nq), dtype=torch.float32, device=q.device)
    if cache_seqlens is None:
        _check(fa_fwd_splitkv(q, k_cache, v_cache, block_table, block_table.shape[1], page_size,
                              o_part, lse_part, num_splits, B, H, nq, seqlen_k, d, softmax_scale,
                              causal, window_left, window_right, alibi_slopes, softcap, stream),
               "fa_fwd_splitkv")
    else:
        if cache_seqlens.dtype != torch.int32 or tuple(cache_seqlens.shape) != (B,):
            raise ValueError("cache_seqlens must be int32 [B]")
        _check(fa_fwd_splitkv_seqlens(q, k_cache, v_cache, block_table, block_table.shape[1],
                                      page_size, cache_seqlens, o_part, lse_part, num_splits, B,
                                      H, nq, seqlen_k, d, softmax_scale, causal, window_left,
                                      window_right, alibi_slopes, softcap, stream),
               "fa_fwd_splitkv_seqlens")
    return o_part, lse_part


def attention_paged_splitkv_fp8(q, k_cache, v_cache, k_descale, v_descale, block_table, seqlen_k,
                                num_splits=None, softmax_scale=None, causal=False, window_left=-1,
                                window_right=-1, alibi_slopes=None, softcap=0.0, stream=None,
                                cache_seqlens=None):
    """Split partials o_part [S,B,H,1,d] and lse_part [S,B,H,1] of one bf16 query row per
    (b, h) over a paged cache of E4M3 codes [num_pages, page_size, H, d] (uint8 or
    float8_e4m3fn) valued k_descale / v_descale times their decoded value."""
    if q.dtype != torch.bfloat16:
        raise TypeError("q must be bfloat16")
    B, nq, H, d = q.shape
    _, page_size, Hc, dc = k_cache.shape
    if (Hc, dc) != (H, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache must be [num_pages, page_size, H, d] matching q")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages_per_seq]")
    if cache_seqlens is not None and (cache_seqlens.dtype != torch.int32
                                      or tuple(cache_seqlens.shape) != (B,)):
        raise ValueError("cache_seqlens must be int32 [B]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_splits = _splits(num_splits, B, H, nq, seqlen_k, d, page_size, fp8_cache=True)
    o_part = torch.empty((num_splits, B, H, nq, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((num_splits, B, H, nq), dtype=torch.float32, device=q.device)
    _check(fa_fwd_splitkv_fp8(q, k_cache, v_cache, k_descale, v_descale, block_table,
                              block_table.shape[1], page_size, cache_seqlens, o_part, lse_part,
                              num_splits, B, H, nq, seqlen_k, d, softmax_scale, causal,
                              window_left, window_right, alibi_slopes, softcap, stream),
           "fa_fwd_splitkv_fp8")
    return o_part, lse_part


def attention_paged_fp8(q, k_cache, v_cache, block_table, seqlen_k, num_splits=None,
                        q_descale=1.0, k_descale=1.0, v_descale=1.0, softmax_scale=None,
                        causal=False, window_left=-1, window_right=-1, alibi_slopes=None,
                        softcap=0.0, stream=None, cache_seqlens=None):
    """Split partials o_part [S,B,H,Nq,d] and lse_part [S,B,H,Nq] of the FP8 forward of E4M3
    q [B,Nq,H,d] over a paged E4M3 cache [num_pages, page_size, H, d] (page_size a multiple
    of 128; uint8 codes or float8_e4m3fn)."""
    B, nq, H, d = q.shape
    _, page_size, Hc, dc = k_cache.shape
    if (Hc, dc) != (H, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache must be [num_pages, page_size, H, d] matching q")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages_per_seq]")
    if cache_seqlens is not None and (cache_seqlens.dtype != torch.int32
                                      or tuple(cache_seqlens.shape) != (B,)):
        raise ValueError("cache_seqlens must be int32 [B]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_splits = _splits(num_splits, B, H, nq, seqlen_k, d, page_size)
    o_part = torch.empty((num_splits, B, H, nq, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((num_splits, B, H, nq), dtype=torch.float32, device=q.device)
    _check(fa_fwd_paged_fp8(q, k_cache, v_cache, q_descale, k_descale, v_descale, block_table,
                            block_table.shape[1], page_size, cache_seqlens, o_part, lse_part,
                            num_splits, B, H, nq, seqlen_k, d, softmax_scale, causal,
                            window_left, window_right, alibi_slopes, softcap, stream),
           "fa_fwd_paged_fp8")
    return o_part, lse_part


def attention_backward(q, k, v, o, lse, dout, softmax_scale=None, causal=False, window_left=-1,
                       window_right=-1, alibi_slopes=None, softcap=0.0,
                       grad_dtype=torch.float32, stream=None):
    """dq, dk, dv (grad_dtype) for q [B,Nq,H,d], k/v [B,Nk,H,d], the forward's o and lse,
    and dout [B,Nq,H,d] (same dtype as q)."""
    _same_dtype(q, k, v, dout)
    B, nq, H, d = q.shape
    nk = k.shape[1]
    if tuple(k.shape) != (B, nk, H, d) or tuple(v.shape) != (B, nk, H, d):
        raise ValueError("k and v must be [B, Nk, H, d] matching q")
    if tuple(o.shape) != (B, nq, H, d) or tuple(dout.shape) != (B, nq, H, d):
        raise ValueError("o and dout must be [B, Nq, H, d]")
    if tuple(lse.shape) != (B, H, nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, H, Nq]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    dq = torch.empty((B, nq, H, d), dtype=grad_dtype, device=q.device)
    dk = torch.empty((B, nk, H, d), dtype=grad_dtype, device=q.device)
    dv = torch.empty((B, nk, H, d), dtype=grad_dtype, device=q.device)
    ws = torch.empty((fa_bwd_workspace_bytes(B, H, nq) // 4,), dtype=torch.float32,
                     device=q.device)
    _check(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, nq, nk, d, softmax_scale, causal,
                  window_left, window_right, alibi_slopes, softcap, stream), "fa_bwd")
    return dq, dk, dv


def attention_varlen_backward(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                              max_seqlen_k, softmax_scale=None, causal=False, window_left=-1,
                              window_right=-1, alibi_slopes=None, softcap=0.0,
                              grad_dtype=torch.float32, stream=None):
    """dq [total_q,H,d], dk, dv [total_k,H,d] (grad_dtype) for a packed batch, from
    attention_varlen's o and lse [H, total_q] and dout [total_q,H,d] (same dtype as q)."""
    _same_dtype(q, k, v, dout)
    total_q, H, d = q.shape
    total_k = k.shape[0]
    if tuple(k.shape) != (total_k, H, d) or tuple(v.shape) != (total_k, H, d):
        raise ValueError("k and v must be [total_k, H, d] matching q")
    if tuple(o.shape) != (total_q, H, d) or tuple(dout.shape) != (total_q, H, d):
        raise ValueError("o and dout must be [total_q, H, d]")
    if tuple(lse.shape) != (H, total_q) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [H, total_q]")
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or cu.dim() != 1:
            raise ValueError("cu_seqlens must be int32 [B + 1]")
    if cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    B = cu_seqlens_q.shape[0] - 1
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    dq = torch.empty((total_q, H, d), dtype=grad_dtype, device=q.device)
    dk = torch.empty((total_k, H, d), dtype=grad_dtype, device=q.device)
    dv = torch.empty((total_k, H, d), dtype=grad_dtype, device=q.device)
    ws = torch.empty((fa_bwd_workspace_bytes(B, H, max_seqlen_q) // 4,), dtype=torch.float32,
                     device=q.device)
    _check(fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, ws, cu_seqlens_q, cu_seqlens_k, B, H,
                         total_q, total_k, max_seqlen_q, max_seqlen_k, d, softmax_scale, causal,
                         window_left, window_right, alibi_slopes, softcap, stream),
           "fa_bwd_varlen")
    return dq, dk, dv


def attention_paged_append(q, k_new, v_new, k_cache, v_cache, block_table, cache_seqlens,
                           max_seqlen_k, num_splits=None, softmax_scale=None, causal=False,
                           window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                           stream=None):
    """Append k_new/v_new [B,Nq,H,d] to the paged cache behind cache_seqlens[b] keys and
    return the split partials over the joined keys (o_part [S,B,H,Nq,d], lse_part
    [S,B,H,Nq]). The caches are updated in place; cache_seqlens is not."""
    _same_dtype(q, k_new, v_new, k_cache, v_cache)
    B, nq, H, d = q.shape
    _, page_size, Hc, dc = k_cache.shape
    if (Hc, dc) != (H, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("cache must be [num_pages, page_size, H, d] matching q")
    if tuple(k_new.shape) != (B, nq, H, d) or tuple(v_new.shape) != (B, nq, H, d):
        raise ValueError("k_new and v_new must be [B, Nq, H, d] matching q")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages_per_seq]")
    if cache_seqlens.dtype != torch.int32 or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("cache_seqlens must be int32 [B]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_splits = _splits(num_splits, B, H, nq, max_seqlen_k, d, page_size)
    o_part = torch.empty((num_splits, B, H, nq, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((num_splits, B, H, nq), dtype=torch.float32, device=q.device)
    _check(fa_fwd_splitkv_append(q, k_new, v_new, k_cache, v_cache, block_table,
                                 block_table.shape[1], page_size, cache_seqlens, o_part, lse_part,
                                 num_splits, B, H, nq, max_seqlen_k, d, softmax_scale, causal,
                                 window_left, window_right, alibi_slopes, softcap, stream),
           "fa_fwd_splitkv_append")
    return o_part, lse_part


def attention_split_partials(q, k, v, num_splits=None, softmax_scale=None, causal=False,
                             window_left=-1, window_right=-1, alibi_slopes=None, softcap=0.0,
                             stream=None):
    """Split partials o_part [S,B,H,Nq,d] and lse_part [S,B,H,Nq] over contiguous K/V."""
    _same_dtype(q, k, v)
    B, nq, H, d = q.shape
    nk = k.shape[1]
    if tuple(k.shape) != (B, nk, H, d) or tuple(v.shape) != (B, nk, H, d):
        raise ValueError("k and v must be [B, Nk, H, d] matching q")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    num_splits = _splits(num_splits, B, H, nq, nk, d, 64)
    o_part = torch.empty((num_splits, B, H, nq, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((num_splits, B, H, nq), dtype=torch.float32, device=q.device)
    _check(fa_fwd_split(q, k, v, o_part, lse_part, num_splits, B, H, nq, nk, d, softmax_scale,
                        causal, window_left, window_right, alibi_slopes, softcap, stream),
           "fa_fwd_split")
    return o_part, lse_part


def attention_split(q, k, v, num_splits=None, out_dtype=torch.float32, stream=None, **kw):
    """fa_fwd_split followed by the combine kernel: the same result as attention()."""
    o_part, lse_part = attention_split_partials(q, k, v, num_splits, stream=stream, **kw)
    return combine(o_part, lse_part, out_dtype=out_dtype, stream=stream)


def combine(o_part, lse_part, out_dtype=torch.float32, stream=None):
    """Merge split partials into O [B, Nq, H, d] and LSE [B, H, Nq]."""
    if o_part.dim() != 5 or o_part.dtype != torch.float32:
        raise ValueError("o_part must be float32 [S, B, H, Nq, d]")
    S, B, H, nq, d = o_part.shape
    if tuple(lse_part.shape) != (S, B, H, nq) or lse_part.dtype != torch.float32:
        raise ValueError(f"lse_part must be float32 {(S, B, H, nq)} to match o_part, "
                         f"got {lse_part.dtype} {tuple(lse_part.shape)}")
    if lse_part.device != o_part.device:
        raise ValueError(f"lse_part lives on {lse_part.device}, o_part on {o_part.device}")
    o = torch.empty((B, nq, H, d), dtype=out_dtype, device=o_part.device)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=o_part.device)
    _check(fa_splitkv_combine(o_part, lse_part, S, B, H, nq, d, o, lse, stream),
           "fa_splitkv_combine")
    return o, lse


def decode_paged(q, k_cache, v_cache, block_table, seqlen_k, num_splits=None,
                 out_dtype=torch.float32, **kw):
    """Split-KV pass followed by the combine kernel, both on the current stream."""
    o_part, lse_part = attention_paged_splitkv(q, k_cache, v_cache, block_table, seqlen_k,
                                               num_splits, **kw)
    return combine(o_part, lse_part, out_dtype=out_dtype, stream=kw.get("stream"))
