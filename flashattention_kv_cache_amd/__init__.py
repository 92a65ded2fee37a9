"""Exact softmax attention for AMD Instinct MI355X (gfx950).

``prefill`` and ``decode`` call the C-ABI library libfa.so (include/fa.h),
whose hand-written HIP kernels do all of the arithmetic; PyTorch supplies
device memory and streams.  ``workloads`` holds the seeded synthetic inputs.
"""
from .binding import (FAError, decode, decode_split_tokens, decode_workspace_bytes, lib,  # noqa: F401
                      prefill)

__all__ = ["prefill", "decode", "decode_workspace_bytes", "decode_split_tokens", "FAError", "lib"]
