"""MI355X (gfx950) attention forward: Python binding of the C ABI in
``include/attn_mi355x.h``.

The functions here carry the C entry points' names and do argument marshalling
only: they check dtype, device, shape and contiguity of torch tensors, pass
their device pointers and the current HIP stream to ``libattn_mi355x.so``, and
raise :class:`AttnError` on a non-zero status. Every step of the computation
runs in the library's HIP kernels; there is no other code path. If the library
has not been built, importing works but every call raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

__all__ = [
    "AttnError",
    "load_library",
    "exported_symbols",
    "attn_abi_version",
    "attn_status_string",
    "attn_varlen_fwd",
    "attn_paged_decode_workspace_size",
    "attn_paged_decode",
    "attn_paged_decode_sliding_window",
    "attn_paged_decode_scratch",
    "attn_padded_fwd_workspace_size",
    "attn_padded_fwd",
    "attn_masked_fwd_workspace_size",
    "attn_masked_fwd",
    "attn_paged_kv_write",
    "attn_paged_prefill",
    "attn_paged_prefill_workspace_size",
    "attn_block_map_to_index",
    "attn_block_sparse_workspace_size",
    "attn_block_sparse_fwd",
    "attn_vsa_tile_gather",
    "attn_vsa_h3_num_tiles",
    "attn_vsa_h3_tile_gather",
    "attn_vsa_h3_untile",
    "attn_vsa_h3_block_map",
    "attn_vsa_h3_gather_block_map",
    "vsa_h3_prepare",
    "attn_vsa_untile",
    "attn_vsa_block_map_workspace_size",
    "attn_vsa_block_map",
    "attn_vsa_compressed_workspace_size",
    "attn_vsa_compressed_add",
    "vsa_num_tiles",
    "vsa_prepare",
    "SUPPORTED_HEAD_DIMS",
]

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libattn_mi355x.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "attn_mi355x.h")
SUPPORTED_HEAD_DIMS = (64, 96, 128, 192, 256)

_i32, _f32, _sz, _p = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
_SIGS = {
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_abi_version": (ctypes.c_int, []),
    "attn_varlen_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                       _i32, _p, _p, _p]),
    "attn_paged_decode_workspace_size": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "attn_paged_decode": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _p,
                                         _p, _p, _sz, _p]),
    "attn_paged_decode_sliding_window": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                        _i32, _i32, _f32, _p, _p, _p, _sz, _p]),
    "attn_paged_decode_scratch": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                 _f32, _p, _p, _p]),
    "attn_padded_fwd_workspace_size": (ctypes.c_int, [_i32, ctypes.POINTER(_sz)]),
    "attn_padded_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _p, _p,
                                       _sz, _p]),
    "attn_masked_fwd_workspace_size": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                      ctypes.POINTER(_sz)]),
    "attn_masked_fwd": (ctypes.c_int, [_p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _i32, _p, _p,
                                       _p, _sz, _p]),
    "attn_paged_kv_write": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p, _p]),
    "attn_paged_prefill": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          _i32, _f32, _p, _p, _p, _sz, _p]),
    "attn_paged_prefill_workspace_size": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "attn_block_map_to_index": (ctypes.c_int, [_p, _i32, _i32, _p, _p, _p]),
    "attn_block_sparse_workspace_size": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "attn_block_sparse_fwd": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p,
                                             _sz, _p]),
    "attn_vsa_tile_gather": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p]),
    "attn_vsa_untile": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p]),
    "attn_vsa_block_map_workspace_size": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "attn_vsa_block_map": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _p, _sz, _p]),
    "attn_vsa_h3_num_tiles": (ctypes.c_int, [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                             ctypes.POINTER(_i32), ctypes.POINTER(_i32)]),
    "attn_vsa_h3_tile_gather": (ctypes.c_int, [_p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p,
                                               _p]),
    "attn_vsa_h3_untile": (ctypes.c_int, [_p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p]),
    "attn_vsa_h3_block_map": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _p, _p, _sz,
                                             _p]),
    "attn_vsa_h3_gather_block_map": (ctypes.c_int, [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                    _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _p, _p, _sz, _p]),
    "attn_vsa_compressed_workspace_size": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "attn_vsa_compressed_add": (ctypes.c_int, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _sz,
                                               _p]),
}

_lib = None


class AttnError(RuntimeError):
    """A library call returned a non-zero attn_status_t."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built HIP library once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as e; e.build()')")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols(header: str = HEADER) -> list[str]:
    """Names of the functions the C header declares."""
    with open(header) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_abi_version() -> int:
    return int(load_library().attn_abi_version())


def _check(fn: str, status: int):
    if status != 0:
        raise AttnError(fn, status, attn_status_string(status))


def _stream_ptr(t: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, device=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shape(t: torch.Tensor, name: str, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def attn_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    softmax_scale: float, causal: bool, out=None, lse=None, return_lse: bool = False, stream=None):
    """Packed varlen attention forward. q [Tq, Hq, D], k/v [Tk, Hkv, D] bf16;
    cu_seqlens int32 [B+1]. Returns out (and lse [Hq, Tq] fp32 if requested)."""
    dev = q.device
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    batch = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    _shape(v, "v", (tk, hkv, dk))
    if dk != d:
        raise ValueError("q and k head sizes differ")
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", q.shape)
    if lse is None and return_lse:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=dev)
    if lse is not None:
        _shape(lse, "lse", (hq, tq))
    lib = load_library()
    st = lib.attn_varlen_fwd(
        _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16, dev), _dev(v, "v", torch.bfloat16, dev),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev), _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, dev),
        batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, float(softmax_scale), int(bool(causal)),
        _dev(out, "out", torch.bfloat16, dev), _dev(lse, "lse", torch.float32, dev) if lse is not None else None,
        _stream_ptr(q, stream))
    _check("attn_varlen_fwd", st)
    return (out, lse) if (return_lse or lse is not None) else out


def attn_paged_decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                     max_context_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check("attn_paged_decode_workspace_size",
           load_library().attn_paged_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                           max_context_len, ctypes.byref(n)))
    return int(n.value)


def attn_paged_decode(q, kv_cache, block_tables, context_lens, max_context_len: int, softmax_scale: float,
                      out=None, lse=None, return_lse: bool = False, workspace=None, stream=None, window=None):
    """Single-token decode over a paged cache [2, NB, 128, Hkv, D]. q [S, Hq, D].
    With ``window`` (>= 0) the call goes to attn_paged_decode_sliding_window."""
    dev = q.device
    nseq, hq, d = q.shape
    two, nblocks, bs, hkv, dk = kv_cache.shape
    if two != 2 or dk != d:
        raise ValueError("kv_cache must be [2, num_blocks, block_size, num_kv_heads, head_dim]")
    mbps = block_tables.shape[1] if block_tables.dim() == 2 else 0
    _shape(block_tables, "block_tables", (nseq, mbps))
    _shape(context_lens, "context_lens", (nseq,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", q.shape)
    if lse is None and return_lse:
        lse = torch.empty((hq, nseq), dtype=torch.float32, device=dev)
    if lse is not None:
        _shape(lse, "lse", (hq, nseq))
    need = attn_paged_decode_workspace_size(nseq, hq, hkv, d, int(max_context_len))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    lib = load_library()
    head = (_dev(q, "q", torch.bfloat16), _dev(kv_cache, "kv_cache", torch.bfloat16, dev),
            _dev(block_tables, "block_tables", torch.int32, dev), _dev(context_lens, "context_lens", torch.int32, dev),
            nseq, nblocks, mbps, int(max_context_len), hq, hkv, d, bs)
    tail = (float(softmax_scale), _dev(out, "out", torch.bfloat16, dev),
            _dev(lse, "lse", torch.float32, dev) if lse is not None else None,
            _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(), _stream_ptr(q, stream))
    if window is None:
        _check("attn_paged_decode", lib.attn_paged_decode(*head, *tail))
    else:
        _check("attn_paged_decode_sliding_window", lib.attn_paged_decode_sliding_window(*head, int(window), *tail))
    return (out, lse) if (return_lse or lse is not None) else out


def attn_paged_decode_scratch(q, kv_cache, block_tables, context_lens, max_context_len: int, softmax_scale: float,
                              out=None, lse=None, return_lse: bool = False, stream=None):
    """attn_paged_decode without a workspace: its prefix sums and partials go to
    the library's fixed per-GPU device array (ATTN_DECODE_SCRATCH_BYTES); nothing is
    allocated by the library. Calls that overlap on one GPU race."""
    dev = q.device
    nseq, hq, d = q.shape
    two, nblocks, bs, hkv, dk = kv_cache.shape
    if two != 2 or dk != d:
        raise ValueError("kv_cache must be [2, num_blocks, block_size, num_kv_heads, head_dim]")
    mbps = block_tables.shape[1] if block_tables.dim() == 2 else 0
    _shape(block_tables, "block_tables", (nseq, mbps))
    _shape(context_lens, "context_lens", (nseq,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", q.shape)
    if lse is None and return_lse:
        lse = torch.empty((hq, nseq), dtype=torch.float32, device=dev)
    if lse is not None:
        _shape(lse, "lse", (hq, nseq))
    st = load_library().attn_paged_decode_scratch(
        _dev(q, "q", torch.bfloat16), _dev(kv_cache, "kv_cache", torch.bfloat16, dev),
        _dev(block_tables, "block_tables", torch.int32, dev), _dev(context_lens, "context_lens", torch.int32, dev),
        nseq, nblocks, mbps, int(max_context_len), hq, hkv, d, bs, float(softmax_scale),
        _dev(out, "out", torch.bfloat16, dev), _dev(lse, "lse", torch.float32, dev) if lse is not None else None,
        _stream_ptr(q, stream))
    _check("attn_paged_decode_scratch", st)
    return (out, lse) if (return_lse or lse is not None) else out


def attn_paged_decode_sliding_window(q, kv_cache, block_tables, context_lens, max_context_len: int, window: int,
                                     softmax_scale: float, **kw):
    """Decode where the query at position L - 1 sees keys L - 1 - window .. L - 1."""
    return attn_paged_decode(q, kv_cache, block_tables, context_lens, max_context_len, softmax_scale,
                             window=window, **kw)


def attn_padded_fwd_workspace_size(batch: int) -> int:
    n = _sz(0)
    _check("attn_padded_fwd_workspace_size", load_library().attn_padded_fwd_workspace_size(batch, ctypes.byref(n)))
    return n.value


def attn_padded_fwd(q, k, v, q_lens, k_lens, softmax_scale: float, causal: bool = False, out=None, lse=None,
                    return_lse: bool = False, workspace=None, stream=None):
    """Attention over valid prefixes of a padded batch: q [B, Sq, Hq, D],
    k/v [B, Sk, Hkv, D], q_lens/k_lens [B] int32 on the device. Rows past
    q_lens[b] come back as zeros; lse is [Hq, B * Sq]."""
    dev = q.device
    b, sq, hq, d = q.shape
    _, sk, hkv, _ = k.shape
    _shape(k, "k", (b, sk, hkv, d))
    _shape(v, "v", (b, sk, hkv, d))
    _shape(q_lens, "q_lens", (b,))
    _shape(k_lens, "k_lens", (b,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", q.shape)
    if lse is None and return_lse:
        lse = torch.empty((hq, b * sq), dtype=torch.float32, device=dev)
    if lse is not None:
        _shape(lse, "lse", (hq, b * sq))
    if workspace is None:
        workspace = torch.empty(max(attn_padded_fwd_workspace_size(b), 1), dtype=torch.uint8, device=dev)
    st = load_library().attn_padded_fwd(
        _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16, dev), _dev(v, "v", torch.bfloat16, dev),
        _dev(q_lens, "q_lens", torch.int32, dev), _dev(k_lens, "k_lens", torch.int32, dev), b, sq, sk, hq, hkv, d,
        float(softmax_scale), int(bool(causal)), _dev(out, "out", torch.bfloat16, dev),
        _dev(lse, "lse", torch.float32, dev) if lse is not None else None,
        _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(), _stream_ptr(q, stream))
    _check("attn_padded_fwd", st)
    return (out, lse) if (return_lse or lse is not None) else out


def attn_masked_fwd_workspace_size(batch: int, seqlen_q: int, seqlen_k: int, num_heads: int, num_kv_heads: int,
                                   head_dim: int, mask_queries: bool) -> int:
    n = _sz(0)
    _check("attn_masked_fwd_workspace_size",
           load_library().attn_masked_fwd_workspace_size(batch, seqlen_q, seqlen_k, num_heads, num_kv_heads,
                                                         head_dim, int(bool(mask_queries)), ctypes.byref(n)))
    return n.value


def attn_masked_fwd(q, k, v, key_mask, softmax_scale: float, causal: bool = False, mask_queries=None, out=None,
                    lse=None, return_lse: bool = False, workspace=None, stream=None):
    """Attention under a key-padding mask [B, Sk] (nonzero = real token).
    mask_queries defaults to self-attention when Sq == Sk (the mask then also
    selects the query rows; padding rows come back as zeros); pass False for
    cross-attention. lse is [Hq, B * Sq]."""
    dev = q.device
    b, sq, hq, d = q.shape
    _, sk, hkv, _ = k.shape
    _shape(k, "k", (b, sk, hkv, d))
    _shape(v, "v", (b, sk, hkv, d))
    _shape(key_mask, "key_mask", (b, sk))
    if mask_queries is None:
        mask_queries = sq == sk
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", q.shape)
    if lse is None and return_lse:
        lse = torch.empty((hq, b * sq), dtype=torch.float32, device=dev)
    if lse is not None:
        _shape(lse, "lse", (hq, b * sq))
    if workspace is None:
        need = attn_masked_fwd_workspace_size(b, sq, sk, hq, hkv, d, mask_queries)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load_library().attn_masked_fwd(
        _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16, dev), _dev(v, "v", torch.bfloat16, dev),
        _dev(key_mask, "key_mask", torch.uint8, dev), b, sq, sk, hq, hkv, d, float(softmax_scale),
        int(bool(causal)), int(bool(mask_queries)), _dev(out, "out", torch.bfloat16, dev),
        _dev(lse, "lse", torch.float32, dev) if lse is not None else None,
        _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(), _stream_ptr(q, stream))
    _check("attn_masked_fwd", st)
    return (out, lse) if (return_lse or lse is not None) else out


def attn_paged_kv_write(k, v, slot_mapping, kv_cache, stream=None):
    """Store new tokens' K/V [N, Hkv, D] at their cache slots (negative slots are
    skipped); kv_cache [2, NB, 128, Hkv, D] is written in place and returned."""
    dev = kv_cache.device
    n, hkv, d = k.shape
    two, nblocks, bs, hkv_c, dk = kv_cache.shape
    if two != 2 or hkv_c != hkv or dk != d:
        raise ValueError("kv_cache must be [2, num_blocks, block_size, num_kv_heads, head_dim] matching k")
    _shape(v, "v", (n, hkv, d))
    _shape(slot_mapping, "slot_mapping", (n,))
    st = load_library().attn_paged_kv_write(
        _dev(k, "k", torch.bfloat16, dev), _dev(v, "v", torch.bfloat16, dev),
        _dev(slot_mapping, "slot_mapping", torch.int32, dev), n, hkv, d, nblocks, bs,
        _dev(kv_cache, "kv_cache", torch.bfloat16), _stream_ptr(kv_cache, stream))
    _check("attn_paged_kv_write", st)
    return kv_cache


def attn_paged_prefill_workspace_size(batch: int, num_heads: int, num_kv_heads: int, head_dim: int,
                                      max_seqlen_q: int, max_context_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check("attn_paged_prefill_workspace_size",
           load_library().attn_paged_prefill_workspace_size(batch, num_heads, num_kv_heads, head_dim, max_seqlen_q,
                                                            max_context_len, ctypes.byref(n)))
    return n.value


def attn_paged_prefill(q, kv_cache, block_tables, cu_seqlens_q, context_lens, max_seqlen_q: int,
                       max_context_len: int, softmax_scale: float, out=None, lse=None, return_lse: bool = False,
                       workspace=None, stream=None):
    """Multi-token queries (packed [Tq, Hq, D] by cu_seqlens_q) over a paged
    cache [2, NB, 128, Hkv, D], bottom-right causal against context_lens keys."""
    dev = q.device
    total_q, hq, d = q.shape
    two, nblocks, bs, hkv, dk = kv_cache.shape
    if two != 2 or dk != d:
        raise ValueError("kv_cache must be [2, num_blocks, block_size, num_kv_heads, head_dim]")
    batch = cu_seqlens_q.numel() - 1
    mbps = block_tables.shape[1] if block_tables.dim() == 2 else 0
    _shape(block_tables, "block_tables", (batch, mbps))
    _shape(context_lens, "context_lens", (batch,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", q.shape)
    if lse is None and return_lse:
        lse = torch.empty((hq, total_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _shape(lse, "lse", (hq, total_q))
    need = attn_paged_prefill_workspace_size(batch, hq, hkv, d, int(max_seqlen_q), int(max_context_len))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = load_library().attn_paged_prefill(
        _dev(q, "q", torch.bfloat16), _dev(kv_cache, "kv_cache", torch.bfloat16, dev),
        _dev(block_tables, "block_tables", torch.int32, dev), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, dev),
        _dev(context_lens, "context_lens", torch.int32, dev), batch, total_q, int(max_seqlen_q),
        int(max_context_len), nblocks, mbps, hq, hkv, d, bs, float(softmax_scale),
        _dev(out, "out", torch.bfloat16, dev), _dev(lse, "lse", torch.float32, dev) if lse is not None else None,
        _dev(workspace, "workspace", torch.uint8, dev) if workspace is not None else None,
        workspace.numel() if workspace is not None else 0, _stream_ptr(q, stream))
    _check("attn_paged_prefill", st)
    return (out, lse) if (return_lse or lse is not None) else out


def attn_block_map_to_index(block_map, idx=None, num=None, stream=None):
    """uint8/bool [..., n_cols] map -> (idx int32 [..., n_cols], num int32 [...])."""
    if block_map.dtype == torch.bool:
        block_map = block_map.view(torch.uint8)
    n_cols = block_map.shape[-1]
    rows = block_map.numel() // n_cols if n_cols else 0
    dev = block_map.device
    if idx is None:
        idx = torch.full(block_map.shape, -1, dtype=torch.int32, device=dev)
    if num is None:
        num = torch.empty(block_map.shape[:-1], dtype=torch.int32, device=dev)
    _shape(idx, "idx", block_map.shape)
    _shape(num, "num", block_map.shape[:-1])
    st = load_library().attn_block_map_to_index(
        _dev(block_map, "block_map", torch.uint8), rows, n_cols, _dev(idx, "idx", torch.int32, dev),
        _dev(num, "num", torch.int32, dev), _stream_ptr(block_map, stream))
    _check("attn_block_map_to_index", st)
    return idx, num


def attn_block_sparse_workspace_size(batch: int, num_heads: int, num_tiles: int) -> int:
    n = ctypes.c_size_t(0)
    _check("attn_block_sparse_workspace_size",
           load_library().attn_block_sparse_workspace_size(batch, num_heads, num_tiles, ctypes.byref(n)))
    return int(n.value)


def attn_block_sparse_fwd(q, k, v, block_map, tile_sizes, softmax_scale: float, out=None, lse=None,
                          return_lse: bool = False, workspace=None, stream=None):
    """Block-sparse attention over 64-row tiles in tile order. q [B, T*64, H, D]."""
    dev = q.device
    b, s, hq, d = q.shape
    hkv = k.shape[2]
    if s % 64 != 0:
        raise ValueError("sequence length must be a multiple of the 64-row tile")
    nt = s // 64
    _shape(k, "k", (b, s, hkv, d))
    _shape(v, "v", (b, s, hkv, d))
    if block_map.dtype == torch.bool:
        block_map = block_map.view(torch.uint8)
    _shape(block_map, "block_map", (b, hq, nt, nt))
    _shape(tile_sizes, "tile_sizes", (nt,))
    if out is None:
        out = torch.empty_like(q)
    _shape(out, "out", q.shape)
    if lse is None and return_lse:
        lse = torch.empty((b, hq, s), dtype=torch.float32, device=dev)
    if lse is not None:
        _shape(lse, "lse", (b, hq, s))
    need = attn_block_sparse_workspace_size(b, hq, nt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load_library().attn_block_sparse_fwd(
        _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16, dev), _dev(v, "v", torch.bfloat16, dev),
        _dev(block_map, "block_map", torch.uint8, dev), _dev(tile_sizes, "tile_sizes", torch.int32, dev),
        b, nt, hq, hkv, d, float(softmax_scale), _dev(out, "out", torch.bfloat16, dev),
        _dev(lse, "lse", torch.float32, dev) if lse is not None else None,
        _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(), _stream_ptr(q, stream))
    _check("attn_block_sparse_fwd", st)
    return (out, lse) if (return_lse or lse is not None) else out


def vsa_num_tiles(video_shape, tile_shape) -> int:
    """Number of (clipped) boxes a raster shape is cut into."""
    n = 1
    for s_, t_ in zip(video_shape, tile_shape):
        n *= -(-int(s_) // int(t_))
    return n


def attn_vsa_tile_gather(x, video_shape, tile_shape, x_tiled=None, tile_sizes=None, stream=None):
    """Raster [B, t*h*w, H, D] bf16 -> padded tile order [B, n_tiles*64, H, D] (+ int32 tile sizes)."""
    b, n = x.shape[:2]
    row = int(x[0, 0].numel()) if n else int(torch.tensor(x.shape[2:]).prod())
    nt = vsa_num_tiles(video_shape, tile_shape)
    dev = x.device
    if x_tiled is None:
        x_tiled = torch.empty((b, nt * 64) + tuple(x.shape[2:]), dtype=x.dtype, device=dev)
    _shape(x_tiled, "x_tiled", (b, nt * 64) + tuple(x.shape[2:]))
    if tile_sizes is None:
        tile_sizes = torch.empty(nt, dtype=torch.int32, device=dev)
    _shape(tile_sizes, "tile_sizes", (nt,))
    t, h, w = (int(v) for v in video_shape)
    if n != t * h * w:
        raise ValueError("x's sequence length must equal t*h*w")
    st = load_library().attn_vsa_tile_gather(
        _dev(x, "x", torch.bfloat16), b, t, h, w, *(int(v) for v in tile_shape), row,
        _dev(x_tiled, "x_tiled", torch.bfloat16, dev), _dev(tile_sizes, "tile_sizes", torch.int32, dev),
        _stream_ptr(x, stream))
    _check("attn_vsa_tile_gather", st)
    return x_tiled, tile_sizes


def attn_vsa_untile(x_tiled, video_shape, tile_shape, out=None, stream=None):
    """Padded tile order [B, n_tiles*64, H, D] -> raster [B, t*h*w, H, D]."""
    b = x_tiled.shape[0]
    t, h, w = (int(v) for v in video_shape)
    nt = vsa_num_tiles(video_shape, tile_shape)
    _shape(x_tiled, "x_tiled", (b, nt * 64) + tuple(x_tiled.shape[2:]))
    row = 1
    for v_ in x_tiled.shape[2:]:
        row *= int(v_)
    dev = x_tiled.device
    if out is None:
        out = torch.empty((b, t * h * w) + tuple(x_tiled.shape[2:]), dtype=x_tiled.dtype, device=dev)
    _shape(out, "out", (b, t * h * w) + tuple(x_tiled.shape[2:]))
    st = load_library().attn_vsa_untile(
        _dev(x_tiled, "x_tiled", torch.bfloat16), b, t, h, w, *(int(v) for v in tile_shape), row,
        _dev(out, "out", torch.bfloat16, dev), _stream_ptr(x_tiled, stream))
    _check("attn_vsa_untile", st)
    return out


def attn_vsa_block_map_workspace_size(batch: int, num_heads: int, num_kv_heads: int, num_tiles: int,
                                      head_dim: int) -> int:
    n = ctypes.c_size_t(0)
    _check("attn_vsa_block_map_workspace_size",
           load_library().attn_vsa_block_map_workspace_size(batch, num_heads, num_kv_heads, num_tiles, head_dim,
                                                            ctypes.byref(n)))
    return int(n.value)


def attn_vsa_block_map(q_tiled, k_tiled, tile_sizes, softmax_scale: float, topk: int, block_map=None,
                       workspace=None, stream=None):
    """Top-k per query tile of scale * mean(q_tile) . mean(k_tile) -> uint8 [B, H, nT, nT]."""
    b, s, hq, d = q_tiled.shape
    hkv = k_tiled.shape[2]
    nt = s // 64
    _shape(k_tiled, "k_tiled", (b, s, hkv, d))
    _shape(tile_sizes, "tile_sizes", (nt,))
    dev = q_tiled.device
    if block_map is None:
        block_map = torch.empty((b, hq, nt, nt), dtype=torch.uint8, device=dev)
    _shape(block_map, "block_map", (b, hq, nt, nt))
    need = attn_vsa_block_map_workspace_size(b, hq, hkv, nt, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load_library().attn_vsa_block_map(
        _dev(q_tiled, "q_tiled", torch.bfloat16), _dev(k_tiled, "k_tiled", torch.bfloat16, dev),
        _dev(tile_sizes, "tile_sizes", torch.int32, dev), b, nt, hq, hkv, d, float(softmax_scale), int(topk),
        _dev(block_map, "block_map", torch.uint8, dev), _dev(workspace, "workspace", torch.uint8, dev),
        workspace.numel(), _stream_ptr(q_tiled, stream))
    _check("attn_vsa_block_map", st)
    return block_map


def attn_vsa_compressed_workspace_size(batch: int, num_heads: int, num_kv_heads: int, num_tiles: int,
                                       head_dim: int) -> int:
    n = ctypes.c_size_t(0)
    _check("attn_vsa_compressed_workspace_size",
           load_library().attn_vsa_compressed_workspace_size(batch, num_heads, num_kv_heads, num_tiles, head_dim,
                                                             ctypes.byref(n)))
    return n.value


def attn_vsa_compressed_add(q_tiled, k_tiled, v_tiled, tile_sizes, gate_tiled, softmax_scale: float, out,
                            workspace=None, stream=None):
    """out (tile order) += broadcast_rows(softmax(pooled scores) @ value tile means) * gate; returns out."""
    dev = q_tiled.device
    b, s, hq, d = q_tiled.shape
    hkv = k_tiled.shape[2]
    if s % 64 != 0:
        raise ValueError("sequence length must be a multiple of the 64-row tile")
    nt = s // 64
    _shape(k_tiled, "k_tiled", (b, s, hkv, d))
    _shape(v_tiled, "v_tiled", (b, s, hkv, d))
    _shape(gate_tiled, "gate_tiled", q_tiled.shape)
    _shape(out, "out", q_tiled.shape)
    _shape(tile_sizes, "tile_sizes", (nt,))
    need = attn_vsa_compressed_workspace_size(b, hq, hkv, nt, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = load_library().attn_vsa_compressed_add(
        _dev(q_tiled, "q_tiled", torch.bfloat16), _dev(k_tiled, "k_tiled", torch.bfloat16, dev),
        _dev(v_tiled, "v_tiled", torch.bfloat16, dev), _dev(tile_sizes, "tile_sizes", torch.int32, dev),
        _dev(gate_tiled, "gate_tiled", torch.bfloat16, dev), b, nt, hq, hkv, d, float(softmax_scale),
        _dev(out, "out", torch.bfloat16, dev), _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
        _stream_ptr(q_tiled, stream))
    _check("attn_vsa_compressed_add", st)
    return out


def _segments(prefix_segments):
    segs = (ctypes.c_int32 * max(len(prefix_segments), 1))(*[int(x) for x in prefix_segments])
    return segs, len(prefix_segments)


def attn_vsa_h3_num_tiles(prefix_segments, video_shape, tile_shape=(4, 4, 4)):
    """(prefix tiles, all tiles) of the H3 layout: prefix segments cut into 64-row
    tiles, then the video's boxes."""
    segs, n = _segments(prefix_segments)
    a, b = _i32(0), _i32(0)
    _check("attn_vsa_h3_num_tiles",
           load_library().attn_vsa_h3_num_tiles(segs, n, *(int(x) for x in video_shape),
                                                *(int(x) for x in tile_shape), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def attn_vsa_h3_tile_gather(x, prefix_segments, video_shape, tile_shape=(4, 4, 4), x_tiled=None, tile_sizes=None,
                            stream=None):
    """Raster [B, prefix + t*h*w, H, D] -> H3 tile order [B, n_tiles*64, H, D] (+ int32 tile sizes)."""
    b, n = x.shape[:2]
    row = 1
    for v_ in x.shape[2:]:
        row *= int(v_)
    _, nt = attn_vsa_h3_num_tiles(prefix_segments, video_shape, tile_shape)
    if n != sum(int(v) for v in prefix_segments) + int(np.prod([int(v) for v in video_shape])):
        raise ValueError("x's sequence length must equal the prefix rows plus t*h*w")
    dev = x.device
    if x_tiled is None:
        x_tiled = torch.empty((b, nt * 64) + tuple(x.shape[2:]), dtype=x.dtype, device=dev)
    _shape(x_tiled, "x_tiled", (b, nt * 64) + tuple(x.shape[2:]))
    if tile_sizes is None:
        tile_sizes = torch.empty(nt, dtype=torch.int32, device=dev)
    _shape(tile_sizes, "tile_sizes", (nt,))
    segs, ns = _segments(prefix_segments)
    st = load_library().attn_vsa_h3_tile_gather(
        _dev(x, "x", torch.bfloat16), segs, ns, b, *(int(v) for v in video_shape), *(int(v) for v in tile_shape), row,
        _dev(x_tiled, "x_tiled", torch.bfloat16, dev), _dev(tile_sizes, "tile_sizes", torch.int32, dev),
        _stream_ptr(x, stream))
    _check("attn_vsa_h3_tile_gather", st)
    return x_tiled, tile_sizes


def attn_vsa_h3_untile(x_tiled, prefix_segments, video_shape, tile_shape=(4, 4, 4), out=None, stream=None):
    """H3 tile order [B, n_tiles*64, H, D] -> raster [B, prefix + t*h*w, H, D]."""
    b = x_tiled.shape[0]
    _, nt = attn_vsa_h3_num_tiles(prefix_segments, video_shape, tile_shape)
    _shape(x_tiled, "x_tiled", (b, nt * 64) + tuple(x_tiled.shape[2:]))
    row = 1
    for v_ in x_tiled.shape[2:]:
        row *= int(v_)
    n = sum(int(v) for v in prefix_segments) + int(np.prod([int(v) for v in video_shape]))
    dev = x_tiled.device
    if out is None:
        out = torch.empty((b, n) + tuple(x_tiled.shape[2:]), dtype=x_tiled.dtype, device=dev)
    _shape(out, "out", (b, n) + tuple(x_tiled.shape[2:]))
    segs, ns = _segments(prefix_segments)
    st = load_library().attn_vsa_h3_untile(
        _dev(x_tiled, "x_tiled", torch.bfloat16), segs, ns, b, *(int(v) for v in video_shape),
        *(int(v) for v in tile_shape), row, _dev(out, "out", torch.bfloat16, dev), _stream_ptr(x_tiled, stream))
    _check("attn_vsa_h3_untile", st)
    return out


def attn_vsa_h3_block_map(q_tiled, k_tiled, tile_sizes, num_prefix_tiles: int, softmax_scale: float, topk: int,
                          block_map=None, workspace=None, stream=None):
    """H3 map: prefix rows and columns kept, top-k over the video columns -> uint8 [B, H, nT, nT]."""
    b, s_, hq, d = q_tiled.shape
    hkv = k_tiled.shape[2]
    nt = s_ // 64
    _shape(k_tiled, "k_tiled", (b, s_, hkv, d))
    _shape(tile_sizes, "tile_sizes", (nt,))
    dev = q_tiled.device
    if block_map is None:
        block_map = torch.empty((b, hq, nt, nt), dtype=torch.uint8, device=dev)
    _shape(block_map, "block_map", (b, hq, nt, nt))
    if workspace is None:
        workspace = torch.empty(max(attn_vsa_block_map_workspace_size(b, hq, hkv, nt, d), 1), dtype=torch.uint8,
                                device=dev)
    st = load_library().attn_vsa_h3_block_map(
        _dev(q_tiled, "q_tiled", torch.bfloat16), _dev(k_tiled, "k_tiled", torch.bfloat16, dev),
        _dev(tile_sizes, "tile_sizes", torch.int32, dev), b, nt, int(num_prefix_tiles), hq, hkv, d,
        float(softmax_scale), int(topk), _dev(block_map, "block_map", torch.uint8, dev),
        _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(), _stream_ptr(q_tiled, stream))
    _check("attn_vsa_h3_block_map", st)
    return block_map


def attn_vsa_h3_gather_block_map(q, k, prefix_segments, video_shape, softmax_scale: float, topk: int,
                                 tile_shape=(4, 4, 4), q_tiled=None, k_tiled=None, tile_sizes=None, block_map=None,
                                 workspace=None, stream=None):
    """Raster [B, prefix + t*h*w, H, D] q and k -> their (H3) tile order and the block
    map in one call (empty prefix_segments: the plain video layout). Returns
    (q_tiled, k_tiled, tile_sizes, block_map)."""
    b, n, hq, d = q.shape
    hkv = k.shape[2]
    _shape(k, "k", (b, n, hkv, d))
    _, nt = attn_vsa_h3_num_tiles(prefix_segments, video_shape, tile_shape)
    if n != sum(int(v) for v in prefix_segments) + int(np.prod([int(v) for v in video_shape])):
        raise ValueError("q's sequence length must equal the prefix rows plus t*h*w")
    dev = q.device
    if q_tiled is None:
        q_tiled = torch.empty((b, nt * 64, hq, d), dtype=q.dtype, device=dev)
    if k_tiled is None:
        k_tiled = torch.empty((b, nt * 64, hkv, d), dtype=k.dtype, device=dev)
    if tile_sizes is None:
        tile_sizes = torch.empty(nt, dtype=torch.int32, device=dev)
    if block_map is None:
        block_map = torch.empty((b, hq, nt, nt), dtype=torch.uint8, device=dev)
    _shape(q_tiled, "q_tiled", (b, nt * 64, hq, d))
    _shape(k_tiled, "k_tiled", (b, nt * 64, hkv, d))
    _shape(tile_sizes, "tile_sizes", (nt,))
    _shape(block_map, "block_map", (b, hq, nt, nt))
    if workspace is None:
        workspace = torch.empty(max(attn_vsa_block_map_workspace_size(b, hq, hkv, nt, d), 1), dtype=torch.uint8,
                                device=dev)
    segs, ns = _segments(prefix_segments)
    st = load_library().attn_vsa_h3_gather_block_map(
        _dev(q, "q", torch.bfloat16), _dev(k, "k", torch.bfloat16, dev), segs, ns, b,
        *(int(v) for v in video_shape), *(int(v) for v in tile_shape), hq, hkv, d, float(softmax_scale), int(topk),
        _dev(q_tiled, "q_tiled", torch.bfloat16, dev), _dev(k_tiled, "k_tiled", torch.bfloat16, dev),
        _dev(tile_sizes, "tile_sizes", torch.int32, dev), _dev(block_map, "block_map", torch.uint8, dev),
        _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(), _stream_ptr(q, stream))
    _check("attn_vsa_h3_gather_block_map", st)
    return q_tiled, k_tiled, tile_sizes, block_map


def vsa_h3_prepare(q, k, v, prefix_segments, video_shape, topk: int, softmax_scale: float, tile_shape=(4, 4, 4),
                   stream=None):
    """Raster [prefix + video] q/k/v -> H3 tile order plus the H3 block map, all in
    the library's kernels. Returns a dict like vsa_prepare's plus num_prefix_tiles."""
    qt, kt, sizes, bmap = attn_vsa_h3_gather_block_map(q, k, prefix_segments, video_shape, softmax_scale, topk,
                                                       tile_shape, stream=stream)
    vt, _ = attn_vsa_h3_tile_gather(v, prefix_segments, video_shape, tile_shape, stream=stream)
    n_pre, _ = attn_vsa_h3_num_tiles(prefix_segments, video_shape, tile_shape)
    return {"q": qt, "k": kt, "v": vt, "block_map": bmap, "tile_sizes": sizes, "num_prefix_tiles": n_pre}


def vsa_prepare(q, k, v, video_shape, tile_shape, topk: int, softmax_scale: float, stream=None):
    """Raster q/k/v -> tile order plus the top-k block map, all in the library's
    kernels. Returns a dict with q, k, v (tile order), block_map and tile_sizes."""
    qt, kt, sizes, bmap = attn_vsa_h3_gather_block_map(q, k, [], video_shape, softmax_scale, topk, tile_shape,
                                                       stream=stream)
    vt, _ = attn_vsa_tile_gather(v, video_shape, tile_shape, stream=stream)
    return {"q": qt, "k": kt, "v": vt, "block_map": bmap, "tile_sizes": sizes}
