"""Exact softmax attention for MI355X (gfx950): thin Python binding.

The functions here only marshal arguments: they check dtypes, devices and
contiguity, allocate outputs with torch, and call the C ABI of libattn.so
(``include/attn.h``) on torch's current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.

    attn_fwd(q, k, v, causal=False, window=0, scale=None)        bf16 prefill
    attn_fwd_f32(q, k, v, causal=False, window=0, scale=None)    fp32 prefill
    attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, ...)   bf16, packed sequences
    attn_decode_paged(q, kcache, vcache, block_table, seq_lens, ...)
    attn_decode_paged_workspace_size(B, Hq, d, block_size, max_blocks_per_seq)
    attn_prefill_paged(q, kcache, vcache, block_table, seq_lens, cu_seqlens_q, ...)
    attn_bwd(q, k, v, out, dout, lse, causal=False, window=0, scale=None)
    attn_bwd_workspace_size(B, Hq, Nq)
    attn_bwd_varlen(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, ...)
    attn_merge(o_a, lse_a, o_b, lse_b, out=None, lse=None)     merge of two partials
    attn_status_str(code)

Layouts: q [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d]; out like q; lse [B, Hq, Nq]
float32.  Packed sequences: q [total_q, Hq, d]; k, v [total_k, Hkv, d];
cu_seqlens_q, cu_seqlens_k [num_seqs + 1] int32 on the GPU; lse [Hq, total_q].  Decode: q [B, Hq, d]; caches [num_blocks, block_size, Hkv, d];
block_table [B, max_blocks] int32; seq_lens [B] int32; out [B, Hq, d];
lse [B, Hq].
"""
from __future__ import annotations

import math

import torch

from . import _lib

__all__ = [
    "attn_fwd",
    "attn_fwd_f32",
    "attn_fwd_varlen",
    "attn_decode_paged",
    "attn_decode_paged_noalloc",
    "attn_decode_paged_workspace_size",
    "attn_prefill_paged",
    "attn_prefill_paged_workspace_size",
    "attn_bwd",
    "attn_bwd_workspace_size",
    "attn_bwd_varlen",
    "attn_merge",
    "attn_status_str",
    "AttnError",
]


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_lib.status_str(code)} (status {code})")


def attn_status_str(code: int) -> str:
    return _lib.status_str(code)


def _check(code: int, where: str):
    if code == _lib.ATTN_OK:
        return
    if code in (_lib.ATTN_E_SHAPE, _lib.ATTN_E_HEADDIM, _lib.ATTN_E_MASK, _lib.ATTN_E_NULL,
                _lib.ATTN_E_WORKSPACE):
        raise ValueError(f"{where}: {_lib.status_str(code)} (status {code})")
    raise AttnError(code, where)


def _dev(t: torch.Tensor, name: str, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _fwd(fn_name, dtype, q, k, v, causal, window, scale, out, lse, return_lse):
    _dev(q, "q", dtype)
    _dev(k, "k", dtype)
    _dev(v, "v", dtype)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d]")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q and k disagree on batch or head dimension")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", dtype)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
        if lse.shape != (B, Hq, Nq):
            raise ValueError("lse must be [B, Hq, Nq]")
    fn = getattr(_lib.lib(), fn_name)
    code = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
              lse.data_ptr() if lse is not None else None,
              B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), int(window), float(scale),
              _stream(q.device))
    _check(code, fn_name)
    return out, lse


def attn_fwd(q, k, v, causal: bool = False, window: int = 0, scale=None, out=None, lse=None,
             return_lse: bool = True):
    """bf16 attention forward.  Returns (out, lse); lse is None if not requested."""
    return _fwd("attn_fwd", torch.bfloat16, q, k, v, causal, window, scale, out, lse, return_lse)


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, causal: bool = False, window: int = 0,
                    scale=None, out=None, lse=None, return_lse: bool = True):
    """bf16 forward over packed sequences.  Returns (out, lse); lse is None if not requested.

    Sequence s owns rows cu_seqlens_q[s]:cu_seqlens_q[s+1] of q/out and rows
    cu_seqlens_k[s]:cu_seqlens_k[s+1] of k/v, and attends only within itself.
    """
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, name, torch.bfloat16)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("expected q [total_q,Hq,d], k and v [total_k,Hkv,d]")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    if dk != d:
        raise ValueError("q and k disagree on the head dimension")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape or \
            cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be [num_seqs + 1]")
    if not (q.device == k.device == v.device == cu_seqlens_q.device == cu_seqlens_k.device):
        raise ValueError("all tensors must be on one device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
        if lse.shape != (Hq, total_q):
            raise ValueError("lse must be [Hq, total_q]")
    code = _lib.lib().attn_fwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1, total_q, total_k, Hq, Hkv, d,
        int(bool(causal)), int(window), float(scale), _stream(q.device))
    _check(code, "attn_fwd_varlen")
    return out, lse


def attn_fwd_f32(q, k, v, causal: bool = False, window: int = 0, scale=None, out=None, lse=None,
                 return_lse: bool = True):
    """float32 attention forward.  Returns (out, lse)."""
    return _fwd("attn_fwd_f32", torch.float32, q, k, v, causal, window, scale, out, lse,
                return_lse)


def attn_decode_paged_workspace_size(B: int, Hq: int, d: int, block_size: int,
                                     max_blocks_per_seq: int) -> int:
    return int(_lib.lib().attn_decode_paged_workspace_size(B, Hq, d, block_size,
                                                           max_blocks_per_seq))


def attn_decode_paged(q, kcache, vcache, block_table, seq_lens, scale=None, window: int = 0,
                      out=None, lse=None, workspace=None, return_lse: bool = True):
    """Single-query decode over a paged cache.  Returns (out, lse)."""
    _dev(q, "q", torch.bfloat16)
    _dev(kcache, "kcache", torch.bfloat16)
    _dev(vcache, "vcache", torch.bfloat16)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or kcache.dim() != 4 or vcache.shape != kcache.shape:
        raise ValueError("expected q [B,Hq,d] and caches [num_blocks,block_size,Hkv,d]")
    B, Hq, d = q.shape
    num_blocks, block_size, Hkv, dk = kcache.shape
    if dk != d:
        raise ValueError("q and the cache disagree on the head dimension")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    need = attn_decode_paged_workspace_size(B, Hq, d, block_size, max_blocks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device.type != "cuda":
        raise ValueError("workspace must be on the GPU")
    code = _lib.lib().attn_decode_paged(
        q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, Hq, Hkv, d, block_size, max_blocks, num_blocks, int(window), float(scale),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "attn_decode_paged")
    return out, lse


def attn_decode_paged_noalloc(q, kcache, vcache, block_table, seq_lens, scale=None,
                              window: int = 0, out=None, lse=None, return_lse: bool = True):
    """attn_decode_paged with the library's own scratch array (no workspace).

    Calls that overlap in time on one GPU must not be made (they share it).
    """
    _dev(q, "q", torch.bfloat16)
    _dev(kcache, "kcache", torch.bfloat16)
    _dev(vcache, "vcache", torch.bfloat16)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    if q.dim() != 3 or kcache.dim() != 4 or vcache.shape != kcache.shape:
        raise ValueError("expected q [B,Hq,d] and caches [num_blocks,block_size,Hkv,d]")
    B, Hq, d = q.shape
    num_blocks, block_size, Hkv, dk = kcache.shape
    if dk != d:
        raise ValueError("q and the cache disagree on the head dimension")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
    code = _lib.lib().attn_decode_paged_noalloc(
        q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, Hq, Hkv, d, block_size, block_table.shape[1], num_blocks, int(window), float(scale),
        _stream(q.device))
    _check(code, "attn_decode_paged_noalloc")
    return out, lse


def attn_prefill_paged_workspace_size(num_seqs: int, total_q: int, Hq: int, d: int,
                                      block_size: int, max_blocks_per_seq: int) -> int:
    return int(_lib.lib().attn_prefill_paged_workspace_size(num_seqs, total_q, Hq, d, block_size,
                                                            max_blocks_per_seq))


def attn_prefill_paged(q, kcache, vcache, block_table, seq_lens, cu_seqlens_q, scale=None,
                       window: int = 0, out=None, lse=None, return_lse: bool = True,
                       workspace=None):
    """Chunked prefill over a paged cache (always causal).  Returns (out, lse).

    Sequence s owns rows cu_seqlens_q[s]:cu_seqlens_q[s+1] of q/out: its new
    tokens, the last of its seq_lens[s] cached tokens.  ``workspace`` (uint8 on
    the GPU, at least attn_prefill_paged_workspace_size(...) bytes) holds the
    partial results of query tiles split along the keys; one is allocated per
    call when it is not given.
    """
    _dev(q, "q", torch.bfloat16)
    _dev(kcache, "kcache", torch.bfloat16)
    _dev(vcache, "vcache", torch.bfloat16)
    _dev(block_table, "block_table", torch.int32)
    _dev(seq_lens, "seq_lens", torch.int32)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    if q.dim() != 3 or kcache.dim() != 4 or vcache.shape != kcache.shape:
        raise ValueError("expected q [total_q,Hq,d] and caches [num_blocks,block_size,Hkv,d]")
    total_q, Hq, d = q.shape
    num_blocks, block_size, Hkv, dk = kcache.shape
    if dk != d:
        raise ValueError("q and the cache disagree on the head dimension")
    S = seq_lens.numel()
    if block_table.dim() != 2 or block_table.shape[0] != S or seq_lens.dim() != 1 or \
            cu_seqlens_q.shape != (S + 1,):
        raise ValueError("block_table must be [S, max_blocks], seq_lens [S], cu_seqlens_q [S+1]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
        if lse.shape != (Hq, total_q):
            raise ValueError("lse must be [Hq, total_q]")
    need = attn_prefill_paged_workspace_size(S, total_q, Hq, d, block_size, block_table.shape[1])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device.type != "cuda":
        raise ValueError("workspace must be on the GPU")
    code = _lib.lib().attn_prefill_paged(
        q.data_ptr(), kcache.data_ptr(), vcache.data_ptr(), block_table.data_ptr(),
        seq_lens.data_ptr(), cu_seqlens_q.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, S, total_q, Hq, Hkv, d, block_size,
        block_table.shape[1], num_blocks, int(window), float(scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "attn_prefill_paged")
    return out, lse


def attn_bwd_workspace_size(B: int, Hq: int, Nq: int) -> int:
    return int(_lib.lib().attn_bwd_workspace_size(B, Hq, Nq))


def attn_bwd(q, k, v, out, dout, lse, causal: bool = False, window: int = 0, scale=None,
             dq=None, dk=None, dv=None, workspace=None):
    """bf16 backward of attn_fwd.  Returns (dq, dk, dv)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _dev(t, name, torch.bfloat16)
    _dev(lse, "lse", torch.float32)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Nq,Hq,d], k and v [B,Nk,Hkv,d]")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have q's shape")
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk_ = k.shape
    if Bk != B or dk_ != d:
        raise ValueError("q and k disagree on batch or head dimension")
    if lse.shape != (B, Hq, Nq):
        raise ValueError("lse must be [B, Hq, Nq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for t, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if t is None:
            t = torch.empty_like(like)
        else:
            _dev(t, name, torch.bfloat16)
            if t.shape != like.shape:
                raise ValueError(f"{name} has the wrong shape")
        outs.append(t)
    dq, dk, dv = outs
    need = attn_bwd_workspace_size(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device.type != "cuda":
        raise ValueError("workspace must be on the GPU")
    code = _lib.lib().attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
        B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), int(window), float(scale),
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "attn_bwd")
    return dq, dk, dv


def attn_bwd_varlen(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, causal: bool = False,
                    window: int = 0, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """bf16 backward of attn_fwd_varlen (packed sequences).  Returns (dq, dk, dv)."""
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _dev(t, name, torch.bfloat16)
    _dev(lse, "lse", torch.float32)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("expected q [total_q,Hq,d], k and v [total_k,Hkv,d]")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have q's shape")
    total_q, Hq, d = q.shape
    total_k, Hkv, dk_ = k.shape
    if dk_ != d:
        raise ValueError("q and k disagree on the head dimension")
    if lse.shape != (Hq, total_q):
        raise ValueError("lse must be [Hq, total_q]")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape or \
            cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be [num_seqs + 1]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for t, like, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if t is None:
            t = torch.empty_like(like)
        else:
            _dev(t, name, torch.bfloat16)
            if t.shape != like.shape:
                raise ValueError(f"{name} has the wrong shape")
        outs.append(t)
    dq, dk, dv = outs
    need = attn_bwd_workspace_size(1, Hq, total_q)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device.type != "cuda":
        raise ValueError("workspace must be on the GPU")
    code = _lib.lib().attn_bwd_varlen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1, total_q, total_k, Hq, Hkv, d,
        int(bool(causal)), int(window), float(scale), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "attn_bwd_varlen")
    return dq, dk, dv


def attn_merge(o_a, lse_a, o_b, lse_b, out=None, lse=None, return_lse: bool = True):
    """Exact merge of two partial results (O [B, N, H, d] bf16, LSE [B, H, N]
    float32) of the same query rows over disjoint key sets.  out / lse may be
    o_a / lse_a for an in-place merge.  Returns (out, lse)."""
    for t, name in ((o_a, "o_a"), (o_b, "o_b")):
        _dev(t, name, torch.bfloat16)
    for t, name in ((lse_a, "lse_a"), (lse_b, "lse_b")):
        _dev(t, name, torch.float32)
    if o_a.dim() != 4 or o_b.shape != o_a.shape:
        raise ValueError("o_a and o_b must be [B, N, H, d] of one shape")
    B, N, H, d = o_a.shape
    if lse_a.shape != (B, H, N) or lse_b.shape != (B, H, N):
        raise ValueError("lse_a and lse_b must be [B, H, N]")
    if out is None:
        out = torch.empty_like(o_a)
    else:
        _dev(out, "out", torch.bfloat16)
        if out.shape != o_a.shape:
            raise ValueError("out must have o_a's shape")
    if lse is None and return_lse:
        lse = torch.empty_like(lse_a)
    elif lse is not None:
        _dev(lse, "lse", torch.float32)
        if lse.shape != lse_a.shape:
            raise ValueError("lse must be [B, H, N]")
    code = _lib.lib().attn_merge(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(),
                                 lse_b.data_ptr(), out.data_ptr(),
                                 lse.data_ptr() if lse is not None else None, B, N, H, d,
                                 _stream(o_a.device))
    _check(code, "attn_merge")
    return out, lse

