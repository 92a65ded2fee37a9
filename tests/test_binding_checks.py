"""The Python binding refuses caller-supplied outputs, log-sum-exps and
workspaces that do not match what the kernels write (CPU only).

The C ABI receives raw addresses, so it cannot see the size of a buffer; the
binding is where a mis-shaped or mis-typed ``out``/``lse`` is caught.  Here the
device check is lifted (CPU tensors stand in for GPU ones) and the library is
replaced by a stub that fails the test if any entry point is reached: every
case must raise ValueError before a call into the library.
"""
import pytest
import torch

from flashattention_kv_cache_amd import binding


class _NoLibrary:
    def __getattr__(self, name):
        raise AssertionError(f"the library was called ({name}) although the arguments are invalid")


@pytest.fixture
def cpu_binding(monkeypatch):
    monkeypatch.setattr(binding, "_dev", lambda t, n: None)
    monkeypatch.setattr(binding, "lib", lambda: _NoLibrary())
    monkeypatch.setattr(binding, "_stream", lambda stream: None)  # no device to ask for its stream
    # the workspace size is a library query: answer it without the library
    monkeypatch.setattr(binding, "decode_workspace_bytes", lambda *a, **k: 0)
    monkeypatch.setattr(binding, "mla_decode_workspace_bytes", lambda *a, **k: 0)
    return binding


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


PREFILL_BAD = {
    "out_short": dict(out=bf16(1, 4, 7, 64)),
    "out_dtype": dict(out=f32(1, 4, 8, 64)),
    "out_noncontig": dict(out=bf16(1, 4, 64, 8).transpose(2, 3)),
    "lse_shape": dict(lse=f32(1, 4, 9)),
    "lse_dtype": dict(lse=bf16(1, 4, 8)),
    "lse_noncontig": dict(lse=f32(1, 8, 4).transpose(1, 2)),
}


@pytest.mark.parametrize("kind", sorted(PREFILL_BAD))
def test_prefill_rejects_bad_outputs(cpu_binding, kind):
    q, k, v = bf16(1, 4, 8, 64), bf16(1, 2, 8, 64), bf16(1, 2, 8, 64)
    with pytest.raises(ValueError):
        cpu_binding.prefill(q, k, v, causal=True, **PREFILL_BAD[kind])


@pytest.mark.parametrize("kind", ["out_short", "out_dtype", "lse_shape"])
def test_chunked_prefill_rejects_bad_outputs(cpu_binding, kind):
    q = bf16(2, 4, 8, 64)
    kc, vc = bf16(2, 2, 32, 64), bf16(2, 2, 32, 64)
    lens = torch.full((2,), 20, dtype=torch.int32)
    bad = {"out_short": dict(out=bf16(2, 4, 8, 32)), "out_dtype": dict(out=f32(2, 4, 8, 64)),
           "lse_shape": dict(lse=f32(2, 4))}[kind]
    with pytest.raises(ValueError):
        cpu_binding.chunked_prefill(q, kc, vc, lens, **bad)


DECODE_BAD = {
    "out_shape": dict(out=bf16(3, 8, 64)),
    "out_dtype": dict(out=f32(3, 8, 128)),
    "lse_shape": dict(lse=f32(3, 4)),
    "lse_dtype": dict(lse=bf16(3, 8)),
    "workspace_noncontig": dict(workspace=torch.zeros(64, 64, dtype=torch.uint8).t()),
}


@pytest.mark.parametrize("kind", sorted(DECODE_BAD))
def test_decode_rejects_bad_outputs(cpu_binding, kind):
    q = bf16(3, 8, 128)
    kc, vc = bf16(3, 2, 100, 128), bf16(3, 2, 100, 128)
    lens = torch.full((3,), 50, dtype=torch.int32)
    with pytest.raises(ValueError):
        cpu_binding.decode(q, kc, vc, lens, **DECODE_BAD[kind])


@pytest.mark.parametrize("kind", ["out_shape", "out_dtype", "lse_shape"])
def test_decode_fp8_rejects_bad_outputs(cpu_binding, kind):
    q = bf16(3, 8, 128)
    kc, vc = torch.zeros(3, 2, 100, 128, dtype=torch.uint8), torch.zeros(3, 2, 100, 128, dtype=torch.uint8)
    lens = torch.full((3,), 50, dtype=torch.int32)
    with pytest.raises(ValueError):
        cpu_binding.decode_fp8(q, kc, vc, lens, 1.0, 1.0, **DECODE_BAD[kind])


@pytest.mark.parametrize("bad", [dict(out=bf16(2, 16, 576)), dict(out=f32(2, 16, 512)), dict(lse=f32(2, 15))],
                         ids=["out_shape", "out_dtype", "lse_shape"])
def test_mla_decode_rejects_bad_outputs(cpu_binding, bad):
    q = bf16(2, 16, 576)
    kv = bf16(2, 64, 576)
    lens = torch.full((2,), 30, dtype=torch.int32)
    with pytest.raises(ValueError):
        cpu_binding.mla_decode(q, kv, lens, 0.07, **bad)


def test_matching_outputs_reach_the_library(cpu_binding):
    """The checks pass a correct ``out``/``lse``: the call gets as far as the
    (stubbed) library."""
    q, k, v = bf16(1, 4, 8, 64), bf16(1, 2, 8, 64), bf16(1, 2, 8, 64)
    with pytest.raises(AssertionError, match="library was called"):
        cpu_binding.prefill(q, k, v, out=bf16(1, 4, 8, 64), lse=f32(1, 4, 8))
