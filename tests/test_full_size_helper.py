"""The full-size test helper hands the oracle row blocks with only the keys
those rows can see, and chunks of a decode batch; this checks (CPU only, on
small shapes with a small row block) that the pieces put back together equal
the oracle run on the whole problem."""
import numpy as np
import pytest

import full_size as FS
import oracle
from flashattention_kv_cache_amd.workloads import make_decode_inputs, make_prefill_inputs


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 37), (False, 0)])
def test_prefill_heads_equals_whole_problem(monkeypatch, causal, window):
    monkeypatch.setattr(FS, "ROW_BLOCK", 64)
    q, k, v = make_prefill_inputs(2, 4, 2, 300, 300, 64, "bf16", seed=31)
    O, L = oracle.prefill(q, k, v, 0.125, causal, window=window)
    heads = [(0, 1), (1, 2), (1, 3)]
    got = FS.prefill_heads(q, k, v, 0.125, causal, heads, window=window)
    for b, h in heads:
        assert np.allclose(got[(b, h)][0], O[b, h], rtol=0, atol=1e-12)
        assert np.allclose(got[(b, h)][1], L[b, h], rtol=0, atol=1e-12)


def test_decode_batches_equals_whole_batch():
    di = make_decode_inputs(7, 8, 2, 64, "bf16", seed=32, len_range=(1, 90), paged=True, block_size=4)
    fn = lambda heads: oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, 4, 0.125,  # noqa: E731
                                           heads=heads)
    O, L = fn(None)
    O2, L2 = FS.decode_batches(fn, 7, 8, chunk=3)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
