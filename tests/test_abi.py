"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects every contract violation with a status code before any
HIP call (so none of these tests needs a GPU)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "fa.h")
FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
F32, BF16 = 0, 1
A = 1 << 20            # a fake, 16-byte aligned "device" address: never dereferenced
MIS = A + 8            # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("fa_prefill", "fa_decode", "fa_decode_workspace_bytes", "fa_status_string",
                 "fa_last_error", "fa_abi_version", "fa_decode_split_tokens", "fa_kv_append",
                 "fa_chunked_prefill", "fa_decode_fp8", "fa_kv_append_fp8", "fa_mla_decode",
                 "fa_mla_decode_split_tokens", "fa_mla_decode_workspace_bytes"):
        assert want in names


def test_library_exports_every_declared_symbol(fa):
    L = fa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(fa.SIGNATURES) == set(declared_functions())
    assert L.fa_abi_version() == 7


def test_status_strings(fa):
    assert fa.status_string(FA_OK) == "ok"
    assert "invalid" in fa.status_string(FA_ERR_INVALID)
    assert "unsupported" in fa.status_string(FA_ERR_UNSUPPORTED)
    assert "HIP" in fa.status_string(FA_ERR_HIP)


def prefill(fa, q=A, k=A, v=A, o=A, lse=A, B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=64, causal=1, window=0, scale=0.125,
            dtype=BF16):
    P = ctypes.c_void_p
    return fa.lib().fa_prefill(P(q), P(k), P(v), P(o), P(lse), B, Hq, Hkv, Nq, Nk, d, causal, window, scale, dtype,
                               None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Hkv=3), FA_ERR_INVALID, "divide"),
    (dict(Hq=0), FA_ERR_INVALID, "heads"),
    (dict(B=-1), FA_ERR_INVALID, ">= 0"),
    (dict(d=96), FA_ERR_UNSUPPORTED, "head dim"),
    (dict(d=256), FA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=7), FA_ERR_INVALID, "dtype"),
    (dict(causal=2), FA_ERR_INVALID, "causal"),
    (dict(Nq=9, Nk=8), FA_ERR_INVALID, "Nq=9 > Nk=8"),
    (dict(window=-1), FA_ERR_INVALID, "window"),
    (dict(window=4, causal=0), FA_ERR_INVALID, "sliding window needs causal"),
    (dict(scale=0.0), FA_ERR_INVALID, "scale"),
    (dict(scale=float("inf")), FA_ERR_INVALID, "scale"),
    (dict(scale=float("nan")), FA_ERR_INVALID, "scale"),
    (dict(q=0), FA_ERR_INVALID, "null"),
    (dict(o=0), FA_ERR_INVALID, "null"),
    (dict(k=MIS), FA_ERR_INVALID, "aligned"),
    (dict(lse=MIS), FA_ERR_INVALID, "aligned"),
])
def test_prefill_rejects(fa, kw, status, msg):
    assert prefill(fa, **kw) == status
    assert msg in fa.lib().fa_last_error().decode()


def test_prefill_empty_is_a_noop(fa):
    # nothing is launched, so no GPU is needed and null pointers are fine
    assert prefill(fa, q=0, k=0, v=0, o=0, lse=0, B=0) == FA_OK
    assert prefill(fa, q=0, k=0, v=0, o=0, lse=0, Nq=0, Nk=0) == FA_OK
    assert fa.lib().fa_last_error().decode() == ""


def decode(fa, q=A, k=A, v=A, lens=A, table=None, bs=16, mbps=4, cap=64, maxlen=64, window=0, o=A, lse=A,
           B=2, Hq=8, Hkv=2, d=128, scale=0.1, dtype=BF16, split=0, ws=None, ws_bytes=0):
    P = ctypes.c_void_p
    return fa.lib().fa_decode(P(q), P(k), P(v), P(lens), P(table), bs, mbps, cap, maxlen, window, P(o), P(lse),
                              B, Hq, Hkv, d, scale, dtype, split, P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Hkv=3), FA_ERR_INVALID, "divide"),
    (dict(d=80), FA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=5), FA_ERR_INVALID, "dtype"),
    (dict(scale=-1.0), FA_ERR_INVALID, "scale"),
    (dict(split=100), FA_ERR_INVALID, "multiple of 256"),
    (dict(maxlen=-1), FA_ERR_INVALID, "max_seq_len"),
    (dict(window=-3), FA_ERR_INVALID, "window"),
    (dict(cap=32, maxlen=64), FA_ERR_INVALID, "capacity"),                 # contiguous S_cap < max len
    (dict(table=A, bs=12), FA_ERR_INVALID, "power of two"),
    (dict(table=A, bs=2048, mbps=1), FA_ERR_INVALID, "power of two"),
    (dict(table=A, bs=16, mbps=3, maxlen=64), FA_ERR_INVALID, "max_blocks_per_seq"),
    (dict(table=A, cap=0), FA_ERR_INVALID, "at least one block"),
    (dict(q=0), FA_ERR_INVALID, "null"),
    (dict(lens=0), FA_ERR_INVALID, "null"),
    (dict(k=MIS), FA_ERR_INVALID, "aligned"),
    (dict(lens=A + 2), FA_ERR_INVALID, "4-byte"),
    (dict(table=A + 2), FA_ERR_INVALID, "4-byte"),
    (dict(B=70000), FA_ERR_UNSUPPORTED, "grid"),
])
def test_decode_rejects(fa, kw, status, msg):
    assert decode(fa, **kw) == status
    assert msg in fa.lib().fa_last_error().decode()


def test_decode_workspace_contract(fa):
    L = fa.lib()
    # one split per sequence needs no workspace
    assert L.fa_decode_workspace_bytes(2, 8, 2, 128, 256, 0, 256) == 0
    n = L.fa_decode_workspace_bytes(2, 8, 2, 128, 1024, 0, 256)
    slots = 2 * 8 * 4
    # partial outputs, partial LSEs, then the work list (count + one entry per (sequence, split))
    assert n == ((slots * 128 * 4 + 255) // 256) * 256 + ((slots * 4 + 255) // 256) * 256 + \
        ((1 + 2 * 4) * 4 + 255) // 256 * 256
    # a call that needs it without one, or with too little, is rejected
    assert decode(fa, maxlen=1024, cap=1024, split=256) == FA_ERR_INVALID
    assert "workspace" in L.fa_last_error().decode()
    assert decode(fa, maxlen=1024, cap=1024, split=256, ws=A, ws_bytes=n - 1) == FA_ERR_INVALID
    assert decode(fa, maxlen=1024, cap=1024, split=256, ws=A + 16, ws_bytes=n) == FA_ERR_INVALID
    # rejected sizes report 0
    assert L.fa_decode_workspace_bytes(2, 8, 3, 128, 1024, 0, 0) == 0
    assert L.fa_decode_workspace_bytes(2, 8, 2, 128, 1024, -1, 0) == 0
    # a window caps the keys a query sees, and with them the splits
    assert L.fa_decode_workspace_bytes(2, 8, 2, 128, 1024, 256, 256) == 0
    assert L.fa_decode_workspace_bytes(2, 8, 2, 128, 1024, 512, 256) == \
        ((2 * 8 * 2 * 128 * 4 + 255) // 256) * 256 + 256 + 256


def test_decode_split_choice(fa):
    L = fa.lib()
    for args in [(64, 32, 8, 128, 8192), (128, 32, 8, 128, 32768), (1, 32, 8, 128, 4096), (4, 8, 8, 64, 100)]:
        st = L.fa_decode_split_tokens(*args, 0)
        assert st >= 256 and st % 256 == 0 and st <= 16384
    assert L.fa_decode_split_tokens(2, 8, 3, 128, 100, 0) == 0
    # a window shorter than the longest sequence sizes the splits by the window
    assert L.fa_decode_split_tokens(128, 32, 8, 128, 32768, 1024) == L.fa_decode_split_tokens(128, 32, 8, 128, 1024, 0)


def decode_noalloc(fa, q=A, k=A, v=A, lens=A, table=None, bs=16, mbps=4, cap=64, maxlen=64, window=0, o=A, lse=A,
                   B=2, Hq=8, Hkv=2, d=128, scale=0.1, dtype=BF16, split=0):
    P = ctypes.c_void_p
    return fa.lib().fa_decode_noalloc(P(q), P(k), P(v), P(lens), P(table), bs, mbps, cap, maxlen, window, P(o),
                                      P(lse), B, Hq, Hkv, d, scale, dtype, split, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Hkv=3), FA_ERR_INVALID, "divide"),
    (dict(d=80), FA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=5), FA_ERR_INVALID, "dtype"),
    (dict(split=100), FA_ERR_INVALID, "multiple of 256"),
    (dict(table=A, bs=12), FA_ERR_INVALID, "power of two"),
    (dict(q=0), FA_ERR_INVALID, "null"),
    (dict(k=MIS), FA_ERR_INVALID, "aligned"),
    # split partials larger than the scratch array: 128 x 32 heads x 128 splits x 129 floats
    (dict(B=128, Hq=32, Hkv=8, maxlen=32768, cap=32768, split=256), FA_ERR_UNSUPPORTED, "scratch"),
])
def test_decode_noalloc_rejects(fa, kw, status, msg):
    """The no-allocation decode checks its arguments like fa_decode (before
    any HIP call), and refuses sizes whose partials exceed its scratch array."""
    assert decode_noalloc(fa, **kw) == status
    assert msg in fa.lib().fa_last_error().decode()


def test_decode_noalloc_scratch_limit_matches_header(fa):
    text = open(HEADER).read()
    m = re.search(r"#define FA_DECODE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    limit = int(m.group(1)) << int(m.group(2))
    L = fa.lib()
    # the benchmark's paged decode batch fits (128 x 32 heads, up to 32768 tokens, library split)
    st = L.fa_decode_split_tokens(128, 32, 8, 128, 32768, 0)
    assert 0 < L.fa_decode_workspace_bytes(128, 32, 8, 128, 32768, 0, st) <= limit
    assert L.fa_decode_workspace_bytes(128, 32, 8, 128, 32768, 0, 256) > limit


def test_decode_empty_batch_is_a_noop(fa):
    assert decode(fa, q=0, k=0, v=0, lens=0, o=0, lse=0, B=0) == FA_OK


def chunked(fa, q=A, k=A, v=A, lens=A, table=None, bs=16, mbps=4, cap=64, maxlen=64, o=A, lse=A,
            B=2, Hq=8, Hkv=2, Nq=16, d=128, causal=1, window=0, scale=0.1, dtype=BF16):
    P = ctypes.c_void_p
    return fa.lib().fa_chunked_prefill(P(q), P(k), P(v), P(lens), P(table), bs, mbps, cap, maxlen, P(o), P(lse),
                                       B, Hq, Hkv, Nq, d, causal, window, scale, dtype, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Hkv=3), FA_ERR_INVALID, "divide"),
    (dict(Nq=-1), FA_ERR_INVALID, ">= 0"),
    (dict(d=96), FA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=9), FA_ERR_INVALID, "dtype"),
    (dict(causal=3), FA_ERR_INVALID, "causal"),
    (dict(window=-1), FA_ERR_INVALID, "window"),
    (dict(window=8, causal=0), FA_ERR_INVALID, "sliding window needs causal"),
    (dict(scale=0.0), FA_ERR_INVALID, "scale"),
    (dict(maxlen=-1), FA_ERR_INVALID, "max_seq_len"),
    (dict(Nq=65, maxlen=64), FA_ERR_INVALID, "exceeds max_seq_len"),
    (dict(cap=32, maxlen=64), FA_ERR_INVALID, "capacity"),
    (dict(table=A, bs=24), FA_ERR_INVALID, "power of two"),
    (dict(table=A, bs=16, mbps=3), FA_ERR_INVALID, "max_blocks_per_seq"),
    (dict(table=A, cap=0), FA_ERR_INVALID, "at least one block"),
    (dict(table=A + 2), FA_ERR_INVALID, "4-byte"),
    (dict(lens=A + 2), FA_ERR_INVALID, "4-byte"),
    (dict(q=0), FA_ERR_INVALID, "null"),
    (dict(lens=0), FA_ERR_INVALID, "null"),
    (dict(o=MIS), FA_ERR_INVALID, "aligned"),
])
def test_chunked_prefill_rejects(fa, kw, status, msg):
    assert chunked(fa, **kw) == status
    assert msg in fa.lib().fa_last_error().decode()


def test_chunked_prefill_empty_is_a_noop(fa):
    assert chunked(fa, q=0, k=0, v=0, lens=0, o=0, lse=0, B=0) == FA_OK
    assert chunked(fa, q=0, k=0, v=0, lens=0, o=0, lse=0, Nq=0) == FA_OK
    # a non-causal chunk may be longer than any cached sequence
    assert chunked(fa, q=0, k=0, v=0, lens=0, o=0, lse=0, Nq=0, causal=0, maxlen=8) == FA_OK


def append(fa, kn=A, vn=A, k=A, v=A, lens=A, table=None, bs=16, mbps=4, cap=64, B=2, Hkv=2, n=4, d=128,
           dtype=BF16):
    P = ctypes.c_void_p
    return fa.lib().fa_kv_append(P(kn), P(vn), P(k), P(v), P(lens), P(table), bs, mbps, cap, B, Hkv, n, d,
                                 dtype, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(B=-1), FA_ERR_INVALID, "B=-1"),
    (dict(Hkv=0), FA_ERR_INVALID, "Hkv"),
    (dict(n=-2), FA_ERR_INVALID, "n_new"),
    (dict(dtype=4), FA_ERR_INVALID, "dtype"),
    (dict(d=12), FA_ERR_UNSUPPORTED, "multiple of 16"),
    (dict(d=6, dtype=F32), FA_ERR_UNSUPPORTED, "multiple of 16"),
    (dict(cap=0), FA_ERR_INVALID, "capacity"),
    (dict(table=A, bs=3), FA_ERR_INVALID, "power of two"),
    (dict(table=A, mbps=0), FA_ERR_INVALID, "max_blocks_per_seq"),
    (dict(table=A, cap=0), FA_ERR_INVALID, "at least one block"),
    (dict(kn=0), FA_ERR_INVALID, "null"),
    (dict(lens=0), FA_ERR_INVALID, "null"),
    (dict(v=MIS), FA_ERR_INVALID, "aligned"),
    (dict(lens=A + 1), FA_ERR_INVALID, "4-byte"),
    (dict(B=40000, Hkv=2), FA_ERR_UNSUPPORTED, "65535"),
])
def test_kv_append_rejects(fa, kw, status, msg):
    assert append(fa, **kw) == status
    assert msg in fa.lib().fa_last_error().decode()


def test_kv_append_empty_is_a_noop(fa):
    assert append(fa, kn=0, vn=0, k=0, v=0, lens=0, B=0) == FA_OK
    assert append(fa, kn=0, vn=0, k=0, v=0, lens=0, n=0) == FA_OK
    # d = 8 fp32 is 32 bytes a row: accepted (any d whose row is whole 16-byte chunks)
    assert append(fa, kn=0, vn=0, k=0, v=0, lens=0, n=0, d=8, dtype=F32) == FA_OK


def decode_fp8(fa, q=A, k=A, v=A, lens=A, table=None, bs=16, mbps=4, cap=64, maxlen=64, window=0, o=A, lse=A,
               B=2, Hq=8, Hkv=2, d=128, scale=0.1, ks=0.5, vs=0.5, split=0, ws=None, ws_bytes=0):
    P = ctypes.c_void_p
    return fa.lib().fa_decode_fp8(P(q), P(k), P(v), P(lens), P(table), bs, mbps, cap, maxlen, window, P(o), P(lse),
                                  B, Hq, Hkv, d, scale, ks, vs, split, P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Hkv=3), FA_ERR_INVALID, "divide"),
    (dict(d=96), FA_ERR_UNSUPPORTED, "head dim"),
    (dict(ks=0.0), FA_ERR_INVALID, "k_scale"),
    (dict(vs=float("inf")), FA_ERR_INVALID, "v_scale"),
    (dict(ks=float("nan")), FA_ERR_INVALID, "k_scale"),
    (dict(scale=-1.0), FA_ERR_INVALID, "scale"),
    (dict(window=-1), FA_ERR_INVALID, "window"),
    (dict(table=A, bs=6), FA_ERR_INVALID, "power of two"),
    (dict(q=0), FA_ERR_INVALID, "null"),
    (dict(v=MIS), FA_ERR_INVALID, "aligned"),
    (dict(maxlen=1024, cap=1024, split=256), FA_ERR_INVALID, "workspace"),
])
def test_decode_fp8_rejects(fa, kw, status, msg):
    assert decode_fp8(fa, **kw) == status
    assert msg in fa.lib().fa_last_error().decode()


def append_fp8(fa, kn=A, vn=A, k=A, v=A, lens=A, table=None, bs=16, mbps=4, cap=64, B=2, Hkv=2, n=4, d=128,
               ks=1.0, vs=1.0):
    P = ctypes.c_void_p
    return fa.lib().fa_kv_append_fp8(P(kn), P(vn), P(k), P(v), P(lens), P(table), bs, mbps, cap, B, Hkv, n, d,
                                     ks, vs, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(B=-1), FA_ERR_INVALID, "B=-1"),
    (dict(d=40), FA_ERR_UNSUPPORTED, "multiple of 16"),
    (dict(ks=-2.0), FA_ERR_INVALID, "k_scale"),
    (dict(vs=0.0), FA_ERR_INVALID, "v_scale"),
    (dict(table=A, bs=5), FA_ERR_INVALID, "power of two"),
    (dict(k=0), FA_ERR_INVALID, "null"),
    (dict(kn=MIS), FA_ERR_INVALID, "aligned"),
    (dict(B=70000, Hkv=1), FA_ERR_UNSUPPORTED, "65535"),
])
def test_kv_append_fp8_rejects(fa, kw, status, msg):
    assert append_fp8(fa, **kw) == status
    assert msg in fa.lib().fa_last_error().decode()


def test_fp8_empty_calls_are_noops(fa):
    assert decode_fp8(fa, q=0, k=0, v=0, lens=0, o=0, lse=0, B=0) == FA_OK
    assert append_fp8(fa, kn=0, vn=0, k=0, v=0, lens=0, n=0) == FA_OK


def mla(fa, q=A, kv=A, lens=A, table=None, bs=64, mbps=4, cap=256, maxlen=256, o=A, lse=A, B=2, Hq=128, dc=512,
        dr=64, scale=0.07, split=0, ws=None, ws_bytes=0):
    P = ctypes.c_void_p
    return fa.lib().fa_mla_decode(P(q), P(kv), P(lens), P(table), bs, mbps, cap, maxlen, P(o), P(lse), B, Hq, dc,
                                  dr, scale, split, P(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dc=256), FA_ERR_UNSUPPORTED, "512 + 64"),
    (dict(dr=32), FA_ERR_UNSUPPORTED, "512 + 64"),
    (dict(Hq=0), FA_ERR_INVALID, "Hq"),
    (dict(B=-3), FA_ERR_INVALID, "B=-3"),
    (dict(split=100), FA_ERR_INVALID, "multiple of 32"),
    (dict(scale=0.0), FA_ERR_INVALID, "scale"),
    (dict(table=A, bs=48), FA_ERR_INVALID, "power of two"),
    (dict(table=A, bs=64, mbps=3), FA_ERR_INVALID, "max_blocks_per_seq"),
    (dict(cap=100), FA_ERR_INVALID, "capacity"),
    (dict(q=0), FA_ERR_INVALID, "null"),
    (dict(kv=MIS), FA_ERR_INVALID, "aligned"),
    (dict(maxlen=4096, cap=4096, split=256), FA_ERR_INVALID, "workspace"),
])
def test_mla_decode_rejects(fa, kw, status, msg):
    assert mla(fa, **kw) == status
    assert msg in fa.lib().fa_last_error().decode()


def test_mla_workspace_and_split_contract(fa):
    L = fa.lib()
    assert L.fa_mla_decode_workspace_bytes(2, 128, 512, 64, 256, 256) == 0
    n = L.fa_mla_decode_workspace_bytes(2, 128, 512, 64, 1024, 256)
    slots = 2 * 128 * 4
    plan = (1 + 2 * 4) * 4  # item count, then one entry per (sequence, split)
    assert n == sum((x + 255) // 256 * 256 for x in (slots * 512 * 2, slots * 4, plan))  # bf16 partials
    assert L.fa_mla_decode_workspace_bytes(2, 128, 256, 64, 1024, 256) == 0
    st = L.fa_mla_decode_split_tokens(128, 128, 512, 64, 16384)
    assert st >= 1024 and st % 256 == 0
    assert L.fa_mla_decode_split_tokens(128, 128, 500, 64, 16384) == 0
    assert mla(fa, q=0, kv=0, lens=0, o=0, lse=0, B=0) == FA_OK


def test_no_cpu_fallback_without_gpu(fa):
    """On a machine without a GPU the binding raises instead of computing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.prefill(q, q, q)
    lens = torch.ones(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.chunked_prefill(q, q, q, lens)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.kv_append(q, q, q, q, lens)
    qb = torch.zeros(1, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.decode_fp8(qb, q.to(torch.uint8), q.to(torch.uint8), lens, 1.0, 1.0)
