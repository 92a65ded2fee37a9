"""Python binding of libfa.so (include/fa.h): argument marshalling only.

Tensors come from PyTorch (device memory and the current HIP stream); every
step of the computation runs in the library's HIP kernels.  If the library is
not built, or no GPU is present, calls raise — there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

from ._build import LIB_PATH

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_F32, FA_BF16 = 0, 1

# Every symbol include/fa.h declares, with its ctypes signature.
_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fa_abi_version": ([], _I),
    "fa_status_string": ([_I], ctypes.c_char_p),
    "fa_last_error": ([], ctypes.c_char_p),
    "fa_prefill": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P], _I),
    "fa_decode_workspace_bytes": ([_I, _I, _I, _I, _I, _I, _I], _S),
    "fa_decode_split_tokens": ([_I, _I, _I, _I, _I, _I], _I),
    "fa_decode": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P, _S, _P], _I),
    "fa_kv_append": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P], _I),
    "fa_chunked_prefill": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P], _I),
    "fa_decode_noalloc": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P], _I),
    "fa_decode_fp8": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _F, _F, _F, _I, _P, _S, _P], _I),
    "fa_kv_append_fp8": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F, _P], _I),
    "fa_mla_decode": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _F, _I, _P, _S, _P], _I),
    "fa_mla_decode_split_tokens": ([_I, _I, _I, _I, _I], _I),
    "fa_mla_decode_workspace_bytes": ([_I, _I, _I, _I, _I, _I], _S),
}

_lib: Optional[ctypes.CDLL] = None


class FAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run flashattention_kv_cache_amd._build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().fa_status_string(s).decode()


def _check(status: int):
    if status != FA_OK:
        raise FAError(status, lib().fa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out_tensor(out: Optional[torch.Tensor], shape, dtype, device, name: str) -> torch.Tensor:
    """A caller-supplied output must be exactly what the kernel writes: the
    library receives only its address, so a smaller or differently typed
    buffer would be written past its end."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not isinstance(out, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {out.dtype} {tuple(out.shape)}")
    if out.device != device:
        raise ValueError(f"{name} must be on {device}, got {out.device}")
    if not out.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return out


def _lse_tensor(lse: Optional[torch.Tensor], want: bool, shape, device) -> Optional[torch.Tensor]:
    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=device) if want else None
    return _out_tensor(lse, shape, torch.float32, device, "lse")


def _workspace_bytes(ws: Optional[torch.Tensor], device) -> int:
    if ws is None:
        return 0
    if ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    return ws.numel() * ws.element_size()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Prepared:
    """One library call with its arguments checked and marshalled once
    (pointers, sizes and the stream fixed): calling it only enqueues the
    kernels again, for loops that repeat the same call on the same buffers."""

    def __init__(self, name: str, args, keep):
        self._fn = getattr(lib(), name)
        self._args = args
        self._keep = keep  # the tensors the pointers refer to stay alive

    def __call__(self):
        status = self._fn(*self._args)
        if status != FA_OK:
            _check(status)


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
            scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, want_lse: bool = True, window: int = 0,
            stream=None, prepare: bool = False):
    """fa_prefill: q (B, Hq, Nq, d), k/v (B, Hkv, Nk, d) -> (o, lse).
    ``window`` > 0: causal sliding window of that many keys.  With
    ``prepare``, nothing is launched: returns (call, o, lse), where call()
    enqueues this prefill on the given (or current) stream."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q (B,Hq,Nq,d) and k, v (B,Hkv,Nk,d)")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, dk = k.shape
    if k.shape[0] != B or dk != d or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v disagree in batch, head dim or dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_tensor(out, q.shape, q.dtype, q.device, "out")
    lse = _lse_tensor(lse, want_lse, (B, Hq, Nq), q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), int(window),
            float(scale), _dtype_code(q), _stream(stream))
    if prepare:
        return Prepared("fa_prefill", args, (q, k, v, out, lse)), out, lse
    _check(lib().fa_prefill(*args))
    return out, lse


class _Cache:
    """Layout of a KV cache as the C ABI takes it."""

    def __init__(self, Hkv, paged, block_size, capacity, max_blocks, bound):
        self.Hkv, self.paged, self.block_size = Hkv, paged, block_size
        self.capacity, self.max_blocks, self.bound = capacity, max_blocks, bound


def _cache_layout(ref, k_cache, v_cache, seq_lens, block_table, block_size, B, d, cache_dtype=None) -> _Cache:
    """Check a contiguous cache (B, Hkv, S_cap, d) or a paged pool
    (num_blocks, block_size, Hkv, d) with its block table (B, max_blocks)."""
    for t, n in ((ref, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (seq_lens, "seq_lens")):
        _dev(t, n)
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("seq_lens must be int32 with one entry per sequence")
    if k_cache.dim() != 4:
        raise ValueError("cache must be 4-d")
    if block_table is not None:
        _dev(block_table, "block_table")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be int32 (B, max_blocks)")
        nblk, bs, Hkv, dk = k_cache.shape
        if block_size and block_size != bs:
            raise ValueError("block_size disagrees with the pool shape")
        c = _Cache(Hkv, True, bs, nblk, block_table.shape[1], block_table.shape[1] * bs)
    else:
        Bc, Hkv, cap, dk = k_cache.shape
        if Bc != B:
            raise ValueError("cache batch != q batch")
        c = _Cache(Hkv, False, 0, cap, 0, cap)
    want = ref.dtype if cache_dtype is None else cache_dtype
    if dk != d or v_cache.shape != k_cache.shape or k_cache.dtype != want or v_cache.dtype != want:
        raise ValueError("inputs and caches disagree in head dim, shape or dtype")
    return c


def _fp8_cache(t: torch.Tensor) -> torch.Tensor:
    """E4M3 caches are passed as uint8 codes or as torch.float8_e4m3fn."""
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def decode_fp8(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
               k_scale: float, v_scale: float, block_table: Optional[torch.Tensor] = None, block_size: int = 0,
               max_seq_len: Optional[int] = None, scale: Optional[float] = None, split_tokens: int = 0,
               workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True, window: int = 0,
               stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fa_decode_fp8: bf16 q (B, Hq, d) against an FP8 E4M3 cache (uint8 codes
    or float8_e4m3fn), contiguous or paged as for ``decode``; a code stands
    for value(code) * k_scale (keys) or * v_scale (values)."""
    k_cache, v_cache = _fp8_cache(k_cache), _fp8_cache(v_cache)
    if q.dtype != torch.bfloat16:
        raise TypeError("fa_decode_fp8 takes bf16 queries")
    B, Hq, d = q.shape
    c = _cache_layout(q, k_cache, v_cache, seq_lens, block_table, block_size, B, d, torch.uint8)
    if max_seq_len is None:
        max_seq_len = c.bound
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(B, Hq, c.Hkv, d, max_seq_len, split_tokens, window)
    if need and _workspace_bytes(workspace, q.device) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = _out_tensor(out, q.shape, q.dtype, q.device, "out")
    lse = _lse_tensor(lse, want_lse, (B, Hq), q.device)
    ws_bytes = _workspace_bytes(workspace, q.device)
    _check(lib().fa_decode_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(block_table),
                               c.block_size, c.max_blocks, c.capacity, int(max_seq_len), int(window),
                               _ptr(out), _ptr(lse), B, Hq, c.Hkv, d, float(scale), float(k_scale),
                               float(v_scale), int(split_tokens), _ptr(workspace) if need else None, ws_bytes,
                               _stream(stream)))
    return out, lse


def kv_append_fp8(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  seq_lens: torch.Tensor, k_scale: float, v_scale: float,
                  block_table: Optional[torch.Tensor] = None, block_size: int = 0, stream=None) -> None:
    """fa_kv_append_fp8: quantise bf16 k_new/v_new (B, Hkv, n_new, d) into an
    FP8 E4M3 cache at positions seq_lens[b] - n_new .. seq_lens[b] - 1."""
    k_cache, v_cache = _fp8_cache(k_cache), _fp8_cache(v_cache)
    _dev(v_new, "v_new")
    if k_new.dim() != 4 or v_new.shape != k_new.shape or k_new.dtype != torch.bfloat16 or \
            v_new.dtype != torch.bfloat16:
        raise ValueError("expected bf16 k_new, v_new (B, Hkv, n_new, d)")
    B, Hkv, n_new, d = k_new.shape
    c = _cache_layout(k_new, k_cache, v_cache, seq_lens, block_table, block_size, B, d, torch.uint8)
    if c.Hkv != Hkv:
        raise ValueError("new rows and cache disagree in KV heads")
    _check(lib().fa_kv_append_fp8(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                  _ptr(block_table), c.block_size, c.max_blocks, c.capacity,
                                  B, Hkv, n_new, d, float(k_scale), float(v_scale), _stream(stream)))


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              seq_lens: torch.Tensor, block_table: Optional[torch.Tensor] = None, block_size: int = 0,
              stream=None, prepare: bool = False):
    """fa_kv_append: write k_new/v_new (B, Hkv, n_new, d) into the cache at
    positions seq_lens[b] - n_new .. seq_lens[b] - 1 (seq_lens = lengths after
    the append), in place.  With ``prepare``, nothing is launched: returns a
    call that enqueues this append."""
    _dev(v_new, "v_new")
    if k_new.dim() != 4 or v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise ValueError("expected k_new, v_new (B, Hkv, n_new, d) of one dtype")
    B, Hkv, n_new, d = k_new.shape
    c = _cache_layout(k_new, k_cache, v_cache, seq_lens, block_table, block_size, B, d)
    if c.Hkv != Hkv:
        raise ValueError("new rows and cache disagree in KV heads")
    args = (_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(block_table),
            c.block_size, c.max_blocks, c.capacity, B, Hkv, n_new, d, _dtype_code(k_new), _stream(stream))
    if prepare:
        return Prepared("fa_kv_append", args, (k_new, v_new, k_cache, v_cache, seq_lens, block_table))
    _check(lib().fa_kv_append(*args))


def chunked_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                    block_table: Optional[torch.Tensor] = None, block_size: int = 0,
                    max_seq_len: Optional[int] = None, causal: bool = True, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    want_lse: bool = True, window: int = 0, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fa_chunked_prefill: the Nq newest tokens of each sequence, q
    (B, Hq, Nq, d), against its whole cache (contiguous (B, Hkv, S_cap, d) or a
    paged pool with ``block_table``); seq_lens count the cached tokens, the Nq
    new ones included.  ``max_seq_len`` defaults to the layout's capacity."""
    if q.dim() != 4:
        raise ValueError("expected q (B, Hq, Nq, d)")
    B, Hq, Nq, d = q.shape
    c = _cache_layout(q, k_cache, v_cache, seq_lens, block_table, block_size, B, d)
    if max_seq_len is None:
        max_seq_len = c.bound
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_tensor(out, q.shape, q.dtype, q.device, "out")
    lse = _lse_tensor(lse, want_lse, (B, Hq, Nq), q.device)
    _check(lib().fa_chunked_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(block_table),
                                    c.block_size, c.max_blocks, c.capacity, int(max_seq_len),
                                    _ptr(out), _ptr(lse), B, Hq, c.Hkv, Nq, d, int(bool(causal)), int(window),
                                    float(scale),
                                    _dtype_code(q), _stream(stream)))
    return out, lse


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, max_seq_len: int, split_tokens: int = 0,
                           window: int = 0) -> int:
    return int(lib().fa_decode_workspace_bytes(B, Hq, Hkv, d, max_seq_len, window, split_tokens))


def decode_split_tokens(B: int, Hq: int, Hkv: int, d: int, max_seq_len: int, window: int = 0) -> int:
    return int(lib().fa_decode_split_tokens(B, Hq, Hkv, d, max_seq_len, window))


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
           block_table: Optional[torch.Tensor] = None, block_size: int = 0,
           max_seq_len: Optional[int] = None, scale: Optional[float] = None,
           split_tokens: int = 0, workspace: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           want_lse: bool = True, window: int = 0, stream=None, prepare: bool = False):
    """fa_decode: q (B, Hq, d) against a contiguous cache (B, Hkv, S_cap, d) or,
    with ``block_table`` (B, max_blocks) int32, a paged pool
    (num_blocks, block_size, Hkv, d).  ``max_seq_len`` bounds seq_lens; it
    defaults to the capacity of the layout (no device read-back).  ``window``
    > 0 attends only the last ``window`` keys.  ``prepare``: as for
    ``prefill``, returns (call, o, lse) without launching."""
    B, Hq, d = q.shape
    c = _cache_layout(q, k_cache, v_cache, seq_lens, block_table, block_size, B, d)
    Hkv, paged, block_size, capacity, max_blocks = c.Hkv, c.paged, c.block_size, c.capacity, c.max_blocks
    if max_seq_len is None:
        max_seq_len = c.bound
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(B, Hq, Hkv, d, max_seq_len, split_tokens, window)
    if need and _workspace_bytes(workspace, q.device) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = _out_tensor(out, q.shape, q.dtype, q.device, "out")
    lse = _lse_tensor(lse, want_lse, (B, Hq), q.device)
    ws_bytes = _workspace_bytes(workspace, q.device)
    args = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(block_table),
            block_size if paged else 0, max_blocks, capacity, int(max_seq_len), int(window),
            _ptr(out), _ptr(lse), B, Hq, Hkv, d, float(scale), _dtype_code(q),
            int(split_tokens), _ptr(workspace) if need else None, ws_bytes, _stream(stream))
    if prepare:
        return Prepared("fa_decode", args, (q, k_cache, v_cache, seq_lens, block_table, out, lse, workspace)), out, lse
    _check(lib().fa_decode(*args))
    return out, lse


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                   block_table: Optional[torch.Tensor] = None, block_size: int = 0,
                   max_seq_len: Optional[int] = None, scale: Optional[float] = None, split_tokens: int = 0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   want_lse: bool = True, window: int = 0, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fa_decode_noalloc: ``decode`` without a workspace; the library keeps
    the split partials in a fixed scratch array on each GPU (no device
    allocation by the library).  Pass ``out`` (and ``lse``) to allocate nothing
    here either."""
    B, Hq, d = q.shape
    c = _cache_layout(q, k_cache, v_cache, seq_lens, block_table, block_size, B, d)
    if max_seq_len is None:
        max_seq_len = c.bound
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _out_tensor(out, q.shape, q.dtype, q.device, "out")
    lse = _lse_tensor(lse, want_lse, (B, Hq), q.device)
    _check(lib().fa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(block_table),
                                   c.block_size if c.paged else 0, c.max_blocks, c.capacity, int(max_seq_len),
                                   int(window), _ptr(out), _ptr(lse), B, Hq, c.Hkv, d, float(scale), _dtype_code(q),
                                   int(split_tokens), _stream(stream)))
    return out, lse


MLA_DC, MLA_DR = 512, 64


def mla_decode_split_tokens(B: int, Hq: int, max_seq_len: int) -> int:
    return int(lib().fa_mla_decode_split_tokens(B, Hq, MLA_DC, MLA_DR, max_seq_len))


def mla_decode_workspace_bytes(B: int, Hq: int, max_seq_len: int, split_tokens: int = 0) -> int:
    return int(lib().fa_mla_decode_workspace_bytes(B, Hq, MLA_DC, MLA_DR, max_seq_len, split_tokens))


def mla_decode(q: torch.Tensor, kv_cache: torch.Tensor, seq_lens: torch.Tensor, scale: float,
               block_table: Optional[torch.Tensor] = None, max_seq_len: Optional[int] = None,
               split_tokens: int = 0, workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, want_lse: bool = True,
               stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fa_mla_decode: bf16 q (B, Hq, 576) = [absorbed latent query ; position
    query] against cache rows [latent (512) ; position key (64)], contiguous
    (B, S_cap, 576) or a paged pool (num_blocks, block_size, 576) with
    ``block_table``.  Returns the latent-space output (B, Hq, 512) and LSE."""
    for t, n in ((q, "q"), (kv_cache, "kv_cache"), (seq_lens, "seq_lens")):
        _dev(t, n)
    if q.dtype != torch.bfloat16 or kv_cache.dtype != torch.bfloat16:
        raise TypeError("fa_mla_decode takes bf16 queries and cache")
    if q.dim() != 3 or kv_cache.dim() != 3 or q.shape[2] != MLA_DC + MLA_DR or kv_cache.shape[2] != q.shape[2]:
        raise ValueError("expected q (B, Hq, 576) and a cache of 576-wide rows")
    B, Hq, _ = q.shape
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("seq_lens must be int32 with one entry per sequence")
    if block_table is not None:
        _dev(block_table, "block_table")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be int32 (B, max_blocks)")
        nblk, bs, _ = kv_cache.shape
        capacity, max_blocks, bound = nblk, block_table.shape[1], block_table.shape[1] * bs
    else:
        if kv_cache.shape[0] != B:
            raise ValueError("cache batch != q batch")
        bs, capacity, max_blocks, bound = 0, kv_cache.shape[1], 0, kv_cache.shape[1]
    if max_seq_len is None:
        max_seq_len = bound
    need = mla_decode_workspace_bytes(B, Hq, max_seq_len, split_tokens)
    if need and _workspace_bytes(workspace, q.device) < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = _out_tensor(out, (B, Hq, MLA_DC), torch.bfloat16, q.device, "out")
    lse = _lse_tensor(lse, want_lse, (B, Hq), q.device)
    ws_bytes = _workspace_bytes(workspace, q.device)
    _check(lib().fa_mla_decode(_ptr(q), _ptr(kv_cache), _ptr(seq_lens), _ptr(block_table), bs, max_blocks, capacity,
                               int(max_seq_len), _ptr(out), _ptr(lse), B, Hq, MLA_DC, MLA_DR, float(scale),
                               int(split_tokens), _ptr(workspace) if need else None, ws_bytes, _stream(stream)))
    return out, lse
