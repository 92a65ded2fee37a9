"""Throughput of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over resident synthetic inputs:
  * paged KV-cache decode, bf16: B=128, Hq=32, Hkv=8, d=128, block 16, cached
    lengths uniform in [512, 32768] (the metric's decode half), then
  * causal GQA prefill, bf16 in / fp32 accumulate: B=1, Hq=32, Hkv=8,
    N=4096, d=128 (the workload the metric is quoted on).
Inputs are generated once with the seeded recipe of
flashattention_kv_cache_amd.workloads and copied to HBM before timing.

Printed: one JSON line.  ``value`` is prefill TFLOP/s (algorithmic flops:
2 per multiply-add, QK^T and PV over unmasked pairs only); the ``decode``
object holds the decode KV GB/s (algorithmic bytes: every cached K/V byte once,
plus q, o, lse and the block-table entries read).  Kernel durations come from
HIP events recorded around each launch on the stream the kernels run on.
``extras`` (outside the step, skipped with --no-extras; run before the
warm-up, see ``preconditioning``) times the KV append,
the chunked prefill against a paged cache, sliding-window prefill and decode,
decode against an FP8 cache, the long-context prefill (N = 32768) and decode
against a contiguous cache, and MLA decode, each on its own.
``--power-seconds S`` (outside the step, after the timing) runs the step's
prefill and then its decode back to back for S seconds each and reports the
board power and the per-XCD shader clocks amd-smi reads meanwhile
(``power_clock``).
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
_CSRC = "flashattention_kv_cache_amd/csrc/"
_PREFILL_SRC = [_CSRC + "prefill_bf16.hip", _CSRC + "fa_internal.h"]
_DECODE_SRC = [_CSRC + "decode.hip", _CSRC + "fa_internal.h", _CSRC + "fa_api.cpp"]  # fa_api.cpp: the split length
# The files whose kernels (and launch choices) each traffic record in
# profiles/traffic.json was measured on.
KERNEL_SOURCES = {
    "prefill": _PREFILL_SRC, "prefill_long": _PREFILL_SRC, "chunked_prefill": _PREFILL_SRC,
    "window_prefill": _PREFILL_SRC,
    "decode": _DECODE_SRC, "decode_contiguous": _DECODE_SRC, "fp8_decode": _DECODE_SRC, "window_decode": _DECODE_SRC,
    "mla": [_CSRC + "mla_decode.hip", _CSRC + "fa_internal.h", _CSRC + "fa_api.cpp"],
    "kv_append": [_CSRC + "kv_append.hip", _CSRC + "fa_internal.h"],
}
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "prefill TFLOP/s & decode KV GB/s (% of MI355X peak), GQA d=128 bf16"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # ~0.4 s of untimed work: the GPU clock ramps up over the first few
    # hundred milliseconds of load, and prefill throughput follows it.
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--split-tokens", type=int, default=0, help="decode tokens per split (0 = library choice)")
    p.add_argument("--copy-calib-mib", type=int, default=0,
                   help="after timing, run one device copy of this many MiB (a known-size kernel for HBM counters)")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the measurements outside the step (KV append, chunked prefill)")
    p.add_argument("--power-seconds", type=float, default=0.0,
                   help="after timing, run the prefill and then the decode alone for this many seconds each "
                        "while sampling board power and shader clocks with amd-smi (0 = off)")
    return p.parse_args()


def source_sha(kind: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (already scaled by the copy-kernel calibration), or None when the
    kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kind]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kind):
        return None
    return int(rec["fetch_bytes"] + rec["write_bytes"])


def time_launches(fn, steps: int, warmup: int, back_to_back: bool = False):
    """Average and median kernel time (ms) of fn() over `steps` launches, from
    HIP events recorded around each launch on the current stream.  With
    back_to_back, also the average over `steps` launches issued between one
    pair of events (for kernels of a few microseconds, where the per-launch
    events' own cost shows)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    if not back_to_back:
        return sum(ms) / steps, ms[steps // 2]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return sum(ms) / steps, ms[steps // 2], a.elapsed_time(b) / steps


def extras(dev, steps: int, dec):
    """Measurements outside the step, each kernel on its own, in this order:
      * causal GQA prefill at N = 32768 with 64 query heads;
      * the KV append and the chunked prefill against a paged cache: 1024-token
        chunks of 4 sequences appended to paged caches holding 1024..7168
        tokens, then attended causally against the whole sequences;
      * sliding-window attention (W = 4096): a causal GQA prefill of 32768
        tokens, and the resident paged decode batch with the window applied;
      * the resident paged decode batch against an FP8 (E4M3) copy of its cache;
      * decode against a contiguous cache (64 sequences of 1024..8192 tokens);
      * MLA decode (absorbed latent form), last: it runs right before the
        step's warm-up, with nothing freed or computed on the host after it.
    ``dec`` holds the decode batch already in HBM."""
    import torch
    from flashattention_kv_cache_amd import binding
    from flashattention_kv_cache_amd import workloads as W
    out = {}
    # long-context causal GQA prefill (N = 32768, 64 query heads), first: after
    # this much MFMA load the clocks take a while to recover, which the decode
    # kernels measured right after it would pay for (measured on MI355X: the
    # contiguous decode batch 8% slower)
    w4 = W.C4
    q, k, v = (t.to(dev) for t in W.prefill_inputs(w4))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    p_avg, p_med = time_launches(lambda: binding.prefill(q, k, v, causal=True, scale=w4.scale, out=o, lse=lse),
                                 max(5, steps // 5), 3)
    tf = w4.flops() / (p_avg * 1e-3) / 1e12
    out["prefill_long"] = {"workload": w4.name, "value": round(tf, 3), "unit": "TFLOP/s", "kernel_ms": round(p_avg, 5),
                           "kernel_ms_median": round(p_med, 5), "flops": w4.flops(),
                           "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
                                        "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                        "kernel": "prefill_bf16_kernel<128, contiguous, no window>",
                                        "traffic": measured_traffic("prefill_long")}}
    del q, k, v, o, lse
    w = W.CHUNKED
    ci = W.chunked_inputs(w)
    q, kn, vn = ci.q.to(dev), ci.k_new.to(dev), ci.v_new.to(dev)
    kc, vc = ci.k_cache.to(dev), ci.v_cache.to(dev)
    lens, table = ci.seq_lens.to(dev), ci.block_table.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    # checked and marshalled once: a launch then costs the host a few
    # microseconds, less than the kernel, so back-to-back launches time the GPU
    append = binding.kv_append(kn, vn, kc, vc, lens, block_table=table, prepare=True)

    def chunk():
        binding.chunked_prefill(q, kc, vc, lens, block_table=table, max_seq_len=ci.max_seq_len,
                                scale=w.scale, out=o, lse=lse)

    append()
    a_avg, a_med, a_b2b = time_launches(append, steps, 20, back_to_back=True)
    c_avg, c_med = time_launches(chunk, steps, 50)
    flops = w.flops(ci.seq_lens.tolist())
    # new K/V read and written once, plus seq_lens and the table entries of the written blocks
    ents = sum((int(L) + w.block_size - 1) // w.block_size - (int(L) - w.chunk) // w.block_size
               for L in ci.seq_lens.tolist())
    abytes = w.append_bytes() + w.B * 4 + ents * 4
    tf = flops / (c_avg * 1e-3) / 1e12
    # a ~10 us kernel: rated on back-to-back launches (the per-launch events'
    # own cost is a sizeable part of each bracketed interval)
    gbs = abytes / (a_b2b * 1e-3) / 1e9
    out.update({
        "chunked_prefill": {"workload": w.name, "value": round(tf, 3), "unit": "TFLOP/s",
                            "kernel_ms": round(c_avg, 5), "kernel_ms_median": round(c_med, 5), "flops": flops,
                            "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
                                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                         "kernel": "prefill_bf16_kernel<128, paged, no window>",
                                         "traffic": measured_traffic("chunked_prefill")}},
        "kv_append": {"workload": f"append of the same chunks ({w.B} x {w.chunk} tokens, {w.Hkv} KV heads, "
                                  f"d={w.d}, bf16) into the paged pool",
                      "value": round(gbs, 2), "unit": "GB/s", "kernel_ms": round(a_b2b, 5),
                      "kernel_ms_per_launch_events": round(a_avg, 5), "kernel_ms_median": round(a_med, 5),
                      "bytes": abytes,
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "kv_append_kernel",
                                   "traffic": measured_traffic("kv_append")}},
    })
    del q, kn, vn, kc, vc, o, lse, ci

    # sliding window: prefill
    wp = W.WINDOW_PREFILL
    q, k, v = (t.to(dev) for t in W.prefill_inputs(wp))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    p_avg, p_med = time_launches(lambda: binding.prefill(q, k, v, causal=True, scale=wp.scale, window=wp.window,
                                                         out=o, lse=lse), steps, 20)
    tf = wp.flops() / (p_avg * 1e-3) / 1e12
    out["window_prefill"] = {"workload": wp.name, "value": round(tf, 3), "unit": "TFLOP/s",
                             "kernel_ms": round(p_avg, 5), "kernel_ms_median": round(p_med, 5), "flops": wp.flops(),
                             "roofline": {"bound": "mfma", "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
                                          "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                          "kernel": "prefill_bf16_kernel<128, contiguous, window>",
                                          "traffic": measured_traffic("window_prefill")}}
    del q, k, v, o, lse

    # sliding window: decode over the resident batch
    wd = W.WINDOW_DECODE
    Wn = wd.window
    lens = dec["seq_lens_cpu"].to(torch.int64).clamp(max=Wn)
    first = dec["seq_lens_cpu"].to(torch.int64) - lens
    ents = int(((first + lens + wd.block_size - 1) // wd.block_size - first // wd.block_size).sum())
    nbytes = int(lens.sum()) * 2 * wd.Hkv * wd.d * 2 + dec["q"].numel() * 2 * 2 + dec["q"].shape[0] * wd.Hq * 4 \
        + ents * 4 + wd.B * 4
    st = binding.decode_split_tokens(wd.B, wd.Hq, wd.Hkv, wd.d, dec["max_seq_len"], Wn)
    ws = torch.empty(max(1, binding.decode_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.d, dec["max_seq_len"], st, Wn)),
                     dtype=torch.uint8, device=dev)
    do = torch.empty_like(dec["q"])
    dl = torch.empty(dec["q"].shape[:2], dtype=torch.float32, device=dev)
    d_avg, d_med = time_launches(lambda: binding.decode(dec["q"], dec["k"], dec["v"], dec["lens"],
                                                        block_table=dec["table"], max_seq_len=dec["max_seq_len"],
                                                        scale=wd.scale, split_tokens=st, workspace=ws, out=do,
                                                        lse=dl, window=Wn), steps, 20)
    gbs = nbytes / (d_avg * 1e-3) / 1e9
    out_window = {"workload": wd.name, "value": round(gbs, 2), "unit": "GB/s", "kernel_ms": round(d_avg, 5),
                            "kernel_ms_median": round(d_med, 5), "bytes": nbytes, "split_tokens": st,
                            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                         "kernel": "decode_split_kernel<bf16,128,4,paged> (one split per sequence)",
                                         "traffic": measured_traffic("window_decode")}}
    out["window_decode"] = out_window

    # FP8 (E4M3) cache: the resident batch's cache rounded to E4M3 codes on the
    # GPU (times 64, scale 1/64), same lengths and block table
    wf = W.FP8_DECODE
    fk = torch.empty(dec["k"].shape, dtype=torch.uint8, device=dev)
    fv = torch.empty_like(fk)
    step = 4096
    for i in range(0, fk.shape[0], step):
        fk[i:i + step] = (dec["k"][i:i + step].float() * W.FP8_SIGMA).to(torch.float8_e4m3fn).view(torch.uint8)
        fv[i:i + step] = (dec["v"][i:i + step].float() * W.FP8_SIGMA).to(torch.float8_e4m3fn).view(torch.uint8)
    tokens = int(dec["seq_lens_cpu"].to(torch.int64).sum())
    nblk = int(((dec["seq_lens_cpu"].to(torch.int64) + wf.block_size - 1) // wf.block_size).sum())
    fbytes = tokens * 2 * wf.Hkv * wf.d + dec["q"].numel() * 2 * 2 + wf.B * wf.Hq * 4 + nblk * 4 + wf.B * 4
    st = binding.decode_split_tokens(wf.B, wf.Hq, wf.Hkv, wf.d, dec["max_seq_len"])
    ws = torch.empty(max(1, binding.decode_workspace_bytes(wf.B, wf.Hq, wf.Hkv, wf.d, dec["max_seq_len"], st)),
                     dtype=torch.uint8, device=dev)
    f_avg, f_med = time_launches(lambda: binding.decode_fp8(dec["q"], fk, fv, dec["lens"], W.FP8_SCALE, W.FP8_SCALE,
                                                            block_table=dec["table"], max_seq_len=dec["max_seq_len"],
                                                            scale=wf.scale, split_tokens=st, workspace=ws, out=do,
                                                            lse=dl), steps, 20)
    gbs = fbytes / (f_avg * 1e-3) / 1e9
    out["fp8_decode"] = {"workload": wf.name, "value": round(gbs, 2), "unit": "GB/s", "kernel_ms": round(f_avg, 5),
                         "kernel_ms_median": round(f_med, 5), "bytes": fbytes, "split_tokens": st,
                         "tokens_per_s": round(tokens / (f_avg * 1e-3), 1),
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                      "kernel": "decode_plan_kernel + decode_split_kernel<fp8,128,4,paged> + decode_merge_kernel",
                                      "traffic": measured_traffic("fp8_decode")}}
    del fk, fv

    # decode against a contiguous cache (64 sequences, S_cap 8192)
    w3 = W.C3
    di = W.decode_inputs(w3)
    cq, ck, cv, cl = di.q.to(dev), di.k_cache.to(dev), di.v_cache.to(dev), di.seq_lens.to(dev)
    st = binding.decode_split_tokens(w3.B, w3.Hq, w3.Hkv, w3.d, di.max_seq_len)
    ws = torch.empty(max(1, binding.decode_workspace_bytes(w3.B, w3.Hq, w3.Hkv, w3.d, di.max_seq_len, st)),
                     dtype=torch.uint8, device=dev)
    co = torch.empty_like(cq)
    cls = torch.empty(cq.shape[:2], dtype=torch.float32, device=dev)
    d_avg, d_med = time_launches(lambda: binding.decode(cq, ck, cv, cl, max_seq_len=di.max_seq_len, scale=w3.scale,
                                                        split_tokens=st, workspace=ws, out=co, lse=cls), steps, 20)
    cbytes = di.kv_bytes() + cq.numel() * 2 * 2 + cls.numel() * 4 + w3.B * 4
    gbs = cbytes / (d_avg * 1e-3) / 1e9
    out["decode_contiguous"] = {"workload": w3.name, "value": round(gbs, 2), "unit": "GB/s",
                                "kernel_ms": round(d_avg, 5), "kernel_ms_median": round(d_med, 5), "bytes": cbytes,
                                "split_tokens": st,
                                "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                                             "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                             "kernel": "decode_plan_kernel + decode_split_kernel<bf16,128,4,contiguous> + decode_merge_kernel",
                                             "traffic": measured_traffic("decode_contiguous")}}
    del cq, ck, cv, co, di

    # MLA decode (absorbed latent form), DeepSeek-V3-shaped batch
    wm = W.MLA_DECODE
    mi = W.mla_inputs(wm)
    mq, mkv = mi.q.to(dev), mi.kv.to(dev)
    ml, mt = mi.seq_lens.to(dev), mi.block_table.to(dev)
    mo = torch.empty((wm.B, wm.Hq, wm.d_c), dtype=torch.bfloat16, device=dev)
    mlse = torch.empty((wm.B, wm.Hq), dtype=torch.float32, device=dev)
    mmax = mi.max_seq_len
    st = binding.mla_decode_split_tokens(wm.B, wm.Hq, mmax)
    ws = torch.empty(max(1, binding.mla_decode_workspace_bytes(wm.B, wm.Hq, mmax, st)),
                     dtype=torch.uint8, device=dev)
    mflops = wm.flops(mi.seq_lens.tolist())
    mbytes = mi.kv_bytes() + mq.numel() * 2 + mo.numel() * 2 + mlse.numel() * 4 + \
        int(((mi.seq_lens.to(torch.int64) + wm.block_size - 1) // wm.block_size).sum()) * 4 + wm.B * 4
    # This is the last kernel before the step's warm-up: the host copies of its
    # inputs (1.3 GB) are freed before it is timed, not after, since freeing
    # them takes tens of milliseconds, and an idle GPU of that length before the
    # warm-up makes the first ~15 timed steps run up to 30% slower while the
    # clocks recover (measured on MI355X).
    del mi
    gc.collect()
    m_avg, m_med = time_launches(lambda: binding.mla_decode(mq, mkv, ml, wm.scale, block_table=mt,
                                                            max_seq_len=mmax, split_tokens=st,
                                                            workspace=ws, out=mo, lse=mlse), steps, 20)
    tf = mflops / (m_avg * 1e-3) / 1e12
    gbs = mbytes / (m_avg * 1e-3) / 1e9
    out["mla_decode"] = {"workload": wm.name, "value": round(tf, 3), "unit": "TFLOP/s", "kernel_ms": round(m_avg, 5),
                         "kernel_ms_median": round(m_med, 5), "flops": mflops, "bytes": mbytes, "split_tokens": st,
                         "hbm_GBps": round(gbs, 2),
                         # 1152 B and 278528 flop per cached token (242 flop/B) sit below the
                         # ridge point (2.5e15 / 8e12 = 312 flop/B): the floor is HBM time
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                      "kernel": "mla_plan_kernel + mla_split_kernel + mla_merge_kernel",
                                      "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                      "traffic": measured_traffic("mla")}}
    del mq, mkv, mo
    return out


def parse_smi_metric(text: str):
    """(socket power in W, [shader clock of each XCD in MHz]) from the text of
    ``amd-smi metric -p -c``; None where the field is absent."""
    watts, gfx, block = None, [], None
    for line in text.splitlines():
        t = line.strip()
        if t.startswith("SOCKET_POWER:"):
            try:
                watts = float(t.split(":")[1].split()[0])
            except ValueError:
                watts = None
        elif t.endswith(":") and " " not in t:
            block = t[:-1]
        elif t.startswith("CLK:") and block is not None and block.startswith("GFX_"):
            try:
                gfx.append(float(t.split(":")[1].split()[0]))
            except ValueError:
                pass
    return watts, gfx


def power_clock(torch, calls, seconds: float):
    """Board power and shader clocks while each call runs back to back for
    `seconds`: the power the board draws under that kernel and the clock it
    holds there.  amd-smi refreshes its readings about every 0.75 s, so the
    first second of each run is skipped and the rest sampled every 0.25 s."""
    import shutil
    import subprocess
    import threading
    smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(smi):
        return {"error": "amd-smi not found"}
    res = {}
    for name, call, batch in calls:
        samples = []
        stop = threading.Event()

        def sample():
            time.sleep(1.0)
            while not stop.is_set():
                r = subprocess.run([smi, "metric", "-p", "-c", "-g", "0"], capture_output=True, text=True)
                samples.append(parse_smi_metric(r.stdout))
                time.sleep(0.25)

        th = threading.Thread(target=sample)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 0
        t_end = time.perf_counter() + seconds
        e0.record()
        th.start()
        while time.perf_counter() < t_end:
            for _ in range(batch):
                call()
            n += batch
            torch.cuda.synchronize()
        e1.record()
        stop.set()
        th.join()
        torch.cuda.synchronize()
        watts = [w for w, _ in samples if w is not None]
        clocks = [sum(g) / len(g) for _, g in samples if g]
        res[name] = {"launches": n, "kernel_us": round(e0.elapsed_time(e1) / n * 1000, 2), "samples": len(samples),
                     "socket_w_mean": round(sum(watts) / len(watts), 1) if watts else None,
                     "socket_w_max": max(watts) if watts else None,
                     "gfx_mhz_mean": round(sum(clocks) / len(clocks), 1) if clocks else None,
                     "gfx_mhz_min_xcd": min(min(g) for _, g in samples if g) if clocks else None,
                     "gfx_mhz_max_xcd": max(max(g) for _, g in samples if g) if clocks else None}
    return res


def cpu_baseline(budget_s: float = 12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same workloads:
    whole (b, h) heads of the prefill until about budget_s seconds have passed,
    then a few decode sequences."""
    import numpy as np
    import oracle
    from flashattention_kv_cache_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    w = W.C2
    q, k, v = W.prefill_inputs(w)
    n_rep = w.Hq // w.Hkv
    heads, t0 = 0, time.perf_counter()
    while heads < w.Hq and time.perf_counter() - t0 < budget_s:
        h = heads
        g = h // n_rep
        oracle.prefill(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], w.scale, True)
        heads += 1
    dt = time.perf_counter() - t0
    flops_per_head = 4 * w.d * w.unmasked_pairs()
    pre = flops_per_head * heads / dt / 1e12
    # decode: a handful of whole sequences of the paged workload (all heads)
    wd = W.C5
    di = W.make_decode_inputs(8, wd.Hq, wd.Hkv, wd.d, "bf16", seed=wd.seed, len_range=(wd.len_lo, wd.len_hi),
                              paged=True, block_size=wd.block_size)
    t1 = time.perf_counter()
    oracle.decode_paged(di.q, di.k_cache, di.v_cache, di.block_table, di.seq_lens, di.block_size, wd.scale)
    ddt = time.perf_counter() - t1
    dec = di.kv_bytes() / ddt / 1e9
    return {"value": round(pre, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 NumPy oracle, causal prefill of {heads} of {w.Hq} query heads of the "
                      f"N=4096 workload ({dt:.1f} s); decode of 8 paged sequences of the B=128 workload, "
                      f"{int(di.seq_lens.sum())} tokens x 32 heads ({ddt:.1f} s)",
            "decode_value": round(dec, 4), "decode_unit": "GB/s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from flashattention_kv_cache_amd import _build, binding
    from flashattention_kv_cache_amd import workloads as W
    if not os.path.exists(_build.LIB_PATH):
        _build.build()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs, resident in HBM before timing
    wp = W.C2
    q, k, v = W.prefill_inputs(wp)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((wp.B, wp.Hq, wp.Nq), dtype=torch.float32, device=dev)
    flops = wp.flops()

    wd = W.C5
    di = W.decode_inputs(wd)
    dq, dk, dv = di.q.to(dev), di.k_cache.to(dev), di.v_cache.to(dev)
    dl, dt_ = di.seq_lens.to(dev), di.block_table.to(dev)
    do = torch.empty_like(dq)
    dlse = torch.empty((wd.B, wd.Hq), dtype=torch.float32, device=dev)
    split = args.split_tokens or binding.decode_split_tokens(wd.B, wd.Hq, wd.Hkv, wd.d, di.max_seq_len)
    ws_bytes = binding.decode_workspace_bytes(wd.B, wd.Hq, wd.Hkv, wd.d, di.max_seq_len, split)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    nblk_read = int(((di.seq_lens.to(torch.int64) + wd.block_size - 1) // wd.block_size).sum())
    kv_bytes = di.kv_bytes()
    dec_bytes = kv_bytes + dq.numel() * 2 + do.numel() * 2 + dlse.numel() * 4 + nblk_read * 4 + wd.B * 4
    dec = {"q": dq, "k": dk, "v": dv, "lens": dl, "table": dt_, "max_seq_len": wd.len_hi,
           "seq_lens_cpu": di.seq_lens.clone()}
    del di

    # the two calls of a step, checked and marshalled once (the timed loop only enqueues)
    prefill = binding.prefill(q, k, v, causal=True, scale=wp.scale, out=o, lse=lse, prepare=True)[0]
    decode = binding.decode(dq, dk, dv, dl, block_table=dt_, max_seq_len=wd.len_hi, scale=wd.scale,
                            split_tokens=split, workspace=ws, out=do, lse=dlse, prepare=True)[0]

    # The measurements outside the step run first and end right before the
    # warm-up: they keep the GPU busy for two seconds, so the timed steps see
    # the clocks a GPU under continuous load holds.  Measured on MI355X: after
    # an idle gap of 30 ms or more, the prefill launches of the next ~15 steps
    # run up to 30% slower while the clocks recover (5% on the average of 20
    # steps); straight from other work they run at the steady rate from the
    # first step.  With --no-extras, the W warm-up steps are all the warm-up.
    extra = None
    busy_s = 0.0
    # the timed region's events exist before any of it, so that nothing but a
    # synchronisation separates the extras, the warm-up and the timed steps
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not args.no_extras:
        t0 = time.perf_counter()
        extra = extras(dev, max(10, min(args.steps, 50)), dec)
        torch.cuda.synchronize()
        busy_s = time.perf_counter() - t0

    for _ in range(args.warmup):
        decode()
        prefill()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    # A step is the decode batch, then the prefill.  The first launch after
    # the synchronisation starts only when the host has enqueued it (~15 us
    # with the GPU idle); in this order that lands on a 1.4 ms decode rather
    # than on a 0.13 ms prefill, and every prefill is enqueued while the GPU
    # is still busy with the decode before it, as in the warm-up.
    t_start.record()
    for i in range(K):
        ev[i][2].record()
        decode()
        ev[i][3].record()
        ev[i][0].record()
        prefill()
        ev[i][1].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    pre_steps = [e[0].elapsed_time(e[1]) for e in ev]
    pre_ms = sorted(pre_steps)
    dec_ms = sorted(e[2].elapsed_time(e[3]) for e in ev)
    pre_avg = sum(pre_ms) / K
    dec_avg = sum(dec_ms) / K
    tflops = flops / (pre_avg * 1e-3) / 1e12
    gbs = dec_bytes / (dec_avg * 1e-3) / 1e9

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal GQA prefill bf16 B=1 Hq=32 Hkv=8 N=4096 d=128 + paged decode bf16 B=128 "
                        "Hq=32 Hkv=8 d=128 block 16 L~U[512,32768]",
            "prefill": {"B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "N": wp.Nq, "d": wp.d, "causal": True,
                        "seed": wp.seed, "flops": flops},
            "decode": {"B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "d": wd.d, "block_size": wd.block_size,
                       "len_range": [wd.len_lo, wd.len_hi], "seed": wd.seed, "tokens": kv_bytes // wd.kv_bytes_per_token(),
                       "split_tokens": split, "bytes": dec_bytes},
        },
        "prefill": {"value": round(tflops, 3), "unit": "TFLOP/s", "kernel_ms": round(pre_avg, 5),
                    "kernel_ms_median": round(pre_ms[K // 2], 5), "frac_of_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
                    "kernel_ms_by_step": [round(x, 4) for x in pre_steps]},
        "decode": {"value": round(gbs, 2), "unit": "GB/s", "kernel_ms": round(dec_avg, 5),
                   "kernel_ms_median": round(dec_ms[K // 2], 5), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic("prefill"),
                     "algorithmic_bytes": wp.algorithmic_bytes(), "kernel": "prefill_bf16_kernel<128, contiguous, no window>"},
        "roofline_decode": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode"),
                            "algorithmic_bytes": dec_bytes,
                            "kernel": "decode_plan_kernel + decode_split_kernel<bf16,128,4,paged> + decode_merge_kernel"},
        "wall_s_timed": round(wall, 4),
    }
    if args.power_seconds > 0:
        # the step's two kernels, then the prefill's per-workgroup work on half
        # and a quarter of the CUs (C2's sequence length and head layout per
        # KV head, fewer KV heads): does the clock, and with it the
        # per-workgroup time, rise when fewer CUs draw power?
        calls = [("prefill", prefill, 2000), ("decode", decode, 200)]
        keep = []
        for hq, hkv in ((16, 4), (8, 2)):
            pq, pk, pv = (t.to(dev) for t in W.make_prefill_inputs(1, hq, hkv, wp.Nq, wp.Nk, wp.d, "bf16", wp.seed))
            c = binding.prefill(pq, pk, pv, causal=True, scale=wp.scale, prepare=True)[0]
            keep.append((pq, pk, pv))
            calls.append((f"prefill_Hq{hq}_Hkv{hkv}", c, 2000))
        out["power_clock"] = power_clock(torch, calls, args.power_seconds)
        # Hq / Hkv = 4: a workgroup holds 64 positions of 4 heads, two tiles
        for name, hkv in (("prefill", wp.Hkv), ("prefill_Hq16_Hkv4", 4), ("prefill_Hq8_Hkv2", 2)):
            if name in out["power_clock"]:
                out["power_clock"][name]["workgroups"] = hkv * wp.Nq // 64 // 2
        del keep
    out["preconditioning"] = {"extras_first": extra is not None, "gpu_busy_s_before_warmup": round(busy_s, 2),
                              "warmup_steps": args.warmup}
    if extra is not None:
        out["extras"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
