"""The work list of split-K decode (through the C ABI): every (sequence,
split) item once, longest first, and the outputs it leads to against the fp64
oracle (bf16 tolerances: max-abs 2e-2, mean-abs 2e-3 on O; LSE 1e-4).

Many sequences over a tiny pool (block ids repeat), so that lengths up to
20000 tokens cost little memory and the split lengths spread over many of the
sort's 64-token buckets; the edge lengths 0, 1, the maximum and an invalid -1
are included.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"
B, HQ, HKV, D, BS, NBLK, MAX_LEN = 300, 8, 2, 128, 16, 32, 20000
SCALE = 1 / math.sqrt(D)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _expected(lens, st, ns_max):
    """Item id -> split length of every split the list must hold: a valid
    length L gives ceil(L / st) splits of st tokens (the last one shorter), an
    invalid one a single item; ids are b * ns_max + s."""
    items = {}
    for b, L in enumerate(lens):
        if L < 0 or L > MAX_LEN:
            items[b * ns_max] = 0
            continue
        ns = max(1, -(-L // st))
        for s in range(ns):
            items[b * ns_max + s] = min(L, (s + 1) * st) - s * st
    return items


@pytest.mark.parametrize("st", [512, 1536])
def test_decode_work_list_longest_first(fa, st):
    note(f"decode work list B={B} split_tokens={st}")
    g = torch.Generator().manual_seed(1400 + st)
    lens = torch.randint(0, MAX_LEN + 1, (B,), generator=g, dtype=torch.int32)
    lens[:4] = torch.tensor([0, 1, MAX_LEN, -1], dtype=torch.int32)
    table = torch.randint(0, NBLK, (B, -(-MAX_LEN // BS)), generator=g, dtype=torch.int32)
    q = torch.randn((B, HQ, D), generator=g).to(torch.bfloat16)
    k = torch.randn((NBLK, BS, HKV, D), generator=g).to(torch.bfloat16)
    v = torch.randn((NBLK, BS, HKV, D), generator=g).to(torch.bfloat16)
    need = fa.decode_workspace_bytes(B, HQ, HKV, D, MAX_LEN, st)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    o, lse = fa.decode(q.to(DEV), k.to(DEV), v.to(DEV), lens.to(DEV), block_table=table.to(DEV), max_seq_len=MAX_LEN,
                       scale=SCALE, split_tokens=st, workspace=ws)
    torch.cuda.synchronize()

    ns_max = -(-MAX_LEN // st)
    items = _expected(lens.tolist(), st, ns_max)
    slots = B * HQ * ns_max
    # workspace: fp32 partial outputs, fp32 partial LSEs, then the list (each 256-byte aligned)
    off = -(-slots * D * 4 // 256) * 256 + -(-slots * 4 // 256) * 256
    plan = ws[off:off + 4 * (1 + len(items))].cpu().view(torch.int32).tolist()
    assert plan[0] == len(items)
    order = plan[1:]
    assert sorted(order) == sorted(items), "the list is not a permutation of the work items"
    buckets = [-(-items[i] // 64) for i in order]
    assert all(x >= y for x, y in zip(buckets, buckets[1:])), "work list not longest first"

    lse_h = lse.cpu()
    assert torch.isnan(lse_h[3]).all(), "an invalid length must give NaN"
    assert torch.isfinite(lse_h[4:]).all()
    assert (o.cpu()[0] == 0).all() and torch.isinf(lse_h[0]).all()
    # sampled sequences, several splits each, against the oracle
    pick = [1, 2] + [int(b) for b in torch.randperm(B - 4, generator=g)[:6] + 4]
    O_ref, lse_ref = oracle.decode_paged(q[pick], k, v, table[pick], lens[pick], BS, SCALE)
    O = o.cpu()[pick].to(torch.float64).numpy()
    err = np.abs(O - np.asarray(O_ref))
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    assert np.abs(lse_h[pick].to(torch.float64).numpy() - np.asarray(lse_ref)).max() <= 1e-4
