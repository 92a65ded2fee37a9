"""Running the fp64 oracle over whole full-size outputs in reasonable time
(test helper; not a test module).

Nothing here computes attention: every value comes from the oracle's own
functions.  The helpers only choose what to hand it and run independent parts
in a thread pool (NumPy releases the GIL in its matrix products and
exponentials):

* ``prefill_heads``: whole query heads of a prefill, one 1024-row block at a
  time.  A block of rows [r0, r1) is given only the keys that any of its rows
  can see under the bottom-right causal mask (and the sliding window): keys
  [lo, r1) with lo = max(0, r0 - W + 1) when a window W is set, else 0.  With
  those slices the oracle's own bottom-right alignment puts key j of the slice
  at position lo + j and query i at r0 + i, so every row sees exactly the keys
  it sees in the full problem; the masked-out keys it no longer gets would
  have had weight exactly zero.
* ``decode_batches``: the decode oracles over chunks of sequences.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle

try:
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover
    threadpool_limits = None

ROW_BLOCK = 1024


def workers() -> int:
    return max(1, min(8, (os.cpu_count() or 2) // 2))


def _limited(fn):
    """Run fn with the BLAS thread count capped (the pool supplies the parallelism)."""
    def run(*a):
        if threadpool_limits is None:
            return fn(*a)
        with threadpool_limits(limits=2):
            return fn(*a)
    return run


def prefill_heads(q, k, v, scale: float, causal: bool, heads, window: int = 0):
    """Oracle output rows of the given (b, h) heads of a prefill with Nq = Nk.
    Returns {(b, h): (O (Nq, d), LSE (Nq,))} in fp64."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    assert Nq == Nk, "row-block key slicing assumes Nq == Nk"

    def block(job):
        b, h, r0 = job
        r1 = min(Nq, r0 + ROW_BLOCK)
        g = oracle.kv_head_of(h, Hq, Hkv)
        if causal:
            lo = max(0, r0 - window + 1) if window > 0 else 0
            hi = r1
        else:
            lo, hi = 0, Nk
        O, L = oracle.prefill(q[b:b + 1, h:h + 1, r0:r1], k[b:b + 1, g:g + 1, lo:hi], v[b:b + 1, g:g + 1, lo:hi],
                              scale, causal, window=window if causal else 0)
        return (b, h, r0), O[0, 0], L[0, 0]

    jobs = [(b, h, r0) for b, h in heads for r0 in range(0, Nq, ROW_BLOCK)]
    out = {bh: (np.zeros((Nq, v.shape[3])), np.zeros(Nq)) for bh in heads}
    with cf.ThreadPoolExecutor(workers()) as ex:
        for (b, h, r0), O, L in ex.map(_limited(block), jobs):
            out[(b, h)][0][r0:r0 + O.shape[0]] = O
            out[(b, h)][1][r0:r0 + O.shape[0]] = L
    return out


def decode_batches(fn, B: int, Hq: int, chunk: int = 4):
    """Whole-batch decode through ``fn(heads) -> (O, LSE)`` (an oracle decode
    with its inputs bound), chunk sequences at a time.  Returns O (B, Hq, d)
    and LSE (B, Hq)."""
    parts = [list(range(s, min(B, s + chunk))) for s in range(0, B, chunk)]

    def run(bs):
        O, L = fn([(b, h) for b in bs for h in range(Hq)])
        return bs, O[bs], L[bs]

    O_all, L_all = None, np.zeros((B, Hq))
    with cf.ThreadPoolExecutor(workers()) as ex:
        for bs, O, L in ex.map(_limited(run), parts):
            if O_all is None:
                O_all = np.zeros((B, Hq, O.shape[-1]))
            O_all[bs], L_all[bs] = O, L
    return O_all, L_all
