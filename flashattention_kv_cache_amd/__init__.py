"""Exact softmax attention for AMD Instinct MI355X (gfx950).

``prefill``, ``decode`` (``decode_fp8``), ``chunked_prefill`` and ``kv_append``
(``kv_append_fp8``) and ``mla_decode`` call the C-ABI
library libfa.so (include/fa.h), whose hand-written HIP kernels do all of the
arithmetic; PyTorch supplies device memory and streams.  ``workloads`` holds
the seeded synthetic inputs.
"""
from .binding import (FAError, chunked_prefill, decode, decode_fp8, decode_split_tokens,  # noqa: F401
                      decode_workspace_bytes, kv_append, kv_append_fp8, lib, mla_decode,
                      mla_decode_split_tokens, mla_decode_workspace_bytes, prefill)

__all__ = ["prefill", "decode", "decode_fp8", "chunked_prefill", "kv_append", "kv_append_fp8", "mla_decode",
           "decode_workspace_bytes", "decode_split_tokens", "mla_decode_workspace_bytes", "mla_decode_split_tokens",
           "FAError", "lib"]
