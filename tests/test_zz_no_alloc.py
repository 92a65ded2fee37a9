"""fa_decode_noalloc (the decode entry point that allocates nothing) against
fa_decode, through the C ABI.

Both run the same kernels with the same split length, so the outputs must be
equal bit for bit; both are also held to the oracle's bf16 bar.  Two calls in
a row, the second with a smaller batch and shorter sequences, check that the
shared scratch array carries nothing from one call into the next.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from flashattention_kv_cache_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(fa, B, Hq, Hkv, d, lens, paged, split, seed):
    di = W.make_decode_inputs(B, Hq, Hkv, d, "bf16", seed=seed, seq_lens=lens, paged=paged,
                              s_cap=max(lens) + 3, spare_blocks=2 if paged else 0)
    scale = 1 / math.sqrt(d)
    args = (di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.seq_lens.to(DEV))
    kw = dict(max_seq_len=di.max_seq_len, split_tokens=split)
    if paged:
        kw["block_table"] = di.block_table.to(DEV)
    assert fa.decode_workspace_bytes(B, Hq, Hkv, d, di.max_seq_len, split) > 0  # the partials are used
    o_ref, l_ref = fa.decode(*args, **kw)
    o, lse = fa.decode_noalloc(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32))
    if paged:
        O, L = oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, di.block_size, scale)
    else:
        O, L = oracle.decode_contiguous(di.q, di.k_cache, di.v_cache, di.seq_lens, scale)
    err = np.abs(o.cpu().double().numpy() - O)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    assert np.abs(lse.cpu().double().numpy() - L).max() <= 1e-4


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contiguous"])
def test_noalloc_decode_matches_decode_twice(fa, paged):
    # a larger call, then a smaller one: fewer sequences, fewer splits
    _case(fa, 6, 16, 4, 128, [3000, 17, 1290, 2049, 700, 2500], paged, 256, seed=21)
    _case(fa, 2, 8, 2, 128, [600, 300], paged, 256, seed=22)


def test_noalloc_rejects_partials_larger_than_its_array(fa):
    di = W.make_decode_inputs(2, 8, 2, 128, "bf16", seed=23, seq_lens=[5, 9])
    big = 1 << 20  # a max_seq_len whose 256-token splits would need more than the array holds
    q = di.q.to(DEV).repeat(64, 1, 1)
    lens = torch.full((128,), 5, dtype=torch.int32, device=DEV)
    kc = torch.zeros((128, 2, 8, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fa.FAError, match="scratch"):
        # contiguous capacity is checked against max_seq_len first: use a paged layout
        table = torch.zeros((128, big // 16), dtype=torch.int32, device=DEV)
        pool = torch.zeros((1, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
        fa.decode_noalloc(q, pool, pool, lens, block_table=table, max_seq_len=big, split_tokens=256)
    del kc
