"""Benchmark of the Lynx split-stream KV codec on one MI355X.

One step = the whole hot path over the Qwen-32B-shaped KV set at 16K
context (64 layers x {K, V} x 16384 tokens x 1024 channels, bf16, 4 GiB,
seeded synthetic values, resident in HBM before timing):
    quantize + split (lynx_quantize_pages)
 -> anchor-only reconstruction (lynx_dequant_anchor)
 -> anchor + residual reconstruction (lynx_dequant_full)

Prints ONE JSON line.  value = bf16 KV bytes through the whole path per
second (2 bytes x elements / step time).  Per-kernel times come from HIP
events recorded on the launch stream around every launch of the timed
steps; `roofline` reports the dominant kernel's algorithmic bytes per launch
over its average launch time against the 8 TB/s HBM peak.  `cpu_baseline`
times the CPU oracle (test infrastructure, never tuned) on a bounded sample
of the same workload on this host.

`transfer` reports the split-stream transfer of the same set through
pinned host memory (lynx_split_stream_transfer, objects of 4096 page
blocks, the anchor queue drained first on both hops): the link alone and
the pipelined quantize -> link out -> link in -> rebuild, as medians of
alternating runs, and how much of the codec time the pipeline hides.

`split_variants` reports the other splits of the 8-bit code (3 + 5, 5 + 3,
6 + 2 beside the paper's 4 + 4), the single streams of the paper's
Lynx-INT4 and Lynx-INT8 (4 + 0, 8 + 0) and the 4 + 4 split with bfloat16
metadata on the same set: stream bytes, kernel times and the
reconstruction error (NMSE) of the anchor alone and of the full code.

`large_set` reports the three codec kernels over the whole 23.5 GiB
Qwen3-235B-A22B-shaped KV set at 128K context, resident in HBM, one launch
each per pass.

`verify` reports the speculative verification (lynx_spec_verify) of 8
drafts over a 151936-token vocabulary: time per call and logit bytes per
second.

`single_page` reports the latency of each codec kernel on the single-page
workload (one K and one V page block), over 2048 rotating copies.

`attention` reports, beside the step, the fused dequant + attention calls
(lynx_decode_attn_dequant) on their own workloads: decode (1 query token,
64 q-heads over 8 KV heads, 32768 tokens; anchor-only and full codes) and
draft verification (8 query tokens, 32 q-heads over 4 KV heads, 131072
tokens, full codes, causal tail): average time per call over rotating copies
of the codes (so the codes come from HBM, not the 256 MiB last-level
cache), algorithmic code + metadata bytes per second against the HBM peak,
and QK + PV flops per second.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --profile-run      # the codec steps only, for rocprofv3
    python bench.py --attention-only [--attention-case NAME]   # attention calls only
    python bench.py --large-only       # the 23.5 GiB set's three kernels only
    python bench.py --transfer-only packed|separate   # the codec steps, then one layout's transfer
    python bench.py --copy-probe       # plain 1 GiB copy, PMC scale factor
    python bench.py --hbm-probe        # plain streaming ceilings (torch + csrc/stream_ceiling.hip)
"""
from __future__ import annotations

import argparse
import json
import statistics
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "quantize+split and dequant GB/s of bf16 KV (1 GPU) + % of HBM peak"
WORKLOAD = "qwen32b_16k"

# Algorithmic HBM bytes per bf16 element (one page block of 32768 elements
# moves 64 KiB of bf16, 16 KiB per 4-bit stream and 9 KiB of metadata).
BYTES_PER_ELEM = {
    "quantize": 2.0 + 0.5 + 0.5 + 0.28125,
    "dequant_anchor": 0.5 + 0.28125 + 2.0,
    "dequant_full": 0.5 + 0.5 + 0.28125 + 2.0,
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_qwen32b_16k.md")


def load_traffic(kernel: str):
    """Measured HBM bytes per launch from the committed PMC summary, or
    None if absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
        t = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, ValueError, IndexError):
        return None
    from progressive_kv_transfer_amd.profiling import kernel_source_hash
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def load_counters():
    """VALU figures of the quantize kernel from the committed SQ-counter
    summary, or None if absent or taken on different kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles", "counters_qwen32b_16k.md")) as f:
            text = f.read()
        t = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, ValueError, IndexError):
        return None
    from progressive_kv_transfer_amd.profiling import kernel_source_hash
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("quantize")


# Host threads of one GPU's share of the host (one job runs per GPU and each
# is given 16 host threads, whatever os.cpu_count() reports).
CPU_SHARE = 16


def cpu_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(CPU_SHARE, n))


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, vendor, family /
    model / stepping and the number of logical CPUs listed."""
    fields, n = {}, 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k = k.strip()
                if k == "processor":
                    n += 1
                if k in ("model name", "vendor_id", "cpu family", "model", "stepping") \
                        and k not in fields:
                    fields[k] = v.strip()
    except OSError:
        return "unknown"
    return (f"{fields.get('model name', 'unknown')} ({fields.get('vendor_id', '?')}, family "
            f"{fields.get('cpu family', '?')} model {fields.get('model', '?')} stepping "
            f"{fields.get('stepping', '?')}; {n} logical CPUs listed)")


def run_cpu_baseline(cfg, kv_dev, budget_s: float):
    """Oracle quantize + both dequants, tensor by tensor, until ~budget_s, on
    a pool of threads over page blocks; then the same steps on one thread
    over the first 256 blocks of the first tensor."""
    import oracle
    from progressive_kv_transfer_amd import kvgen

    th = cpu_threads()
    oracle.lib()
    done, elems, t_total = 0, 0, 0.0
    while done < kv_dev.shape[0]:
        xb = kvgen.bf16_bits(kv_dev[done:done + 1])
        t0 = time.perf_counter()
        c = oracle.quantize(xb, threads=th)
        oracle.dequant(c, xb.shape, False, threads=th)
        oracle.dequant(c, xb.shape, True, threads=th)
        t_total += time.perf_counter() - t0
        done += 1
        elems += xb.size
        if t_total >= budget_s:
            break
    gbps = 2.0 * elems / t_total / 1e9

    one_blocks = 256
    xb = kvgen.bf16_bits(kv_dev[0:1])
    t0 = time.perf_counter()
    c = oracle.quantize(xb, threads=1, blocks=(0, one_blocks))
    oracle.dequant(c, xb.shape, False, threads=1, blocks=(0, one_blocks))
    oracle.dequant(c, xb.shape, True, threads=1, blocks=(0, one_blocks))
    t_one = time.perf_counter() - t0
    one_elems = one_blocks * 32768
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": th, "kind": "oracle",
            "host_threads": {"os_cpu_count": os.cpu_count(), "affinity": affinity,
                             "used": th, "share_per_gpu": CPU_SHARE},
            "sample": (f"first {done} of {kv_dev.shape[0]} tensors (K/V of layers "
                       f"0..{(done - 1) // 2}) of {cfg.name}: {elems} elements, "
                       f"{t_total:.1f} s wall, quantize + anchor dequant + full dequant"),
            "cpu_model": cpu_model(), "wall_s": round(t_total, 2),
            "elements_per_s": round(elems / t_total, 1),
            "single_thread": {"value": round(2.0 * one_elems / t_one / 1e9, 4),
                              "unit": "GB/s", "elements": one_elems,
                              "wall_s": round(t_one, 2),
                              "elements_per_s": round(one_elems / t_one, 1),
                              "sample": f"page blocks 0..{one_blocks - 1} of tensor 0"}}


def copy_probe(timed: bool = False):
    """A plain device copy of 1 GiB (PMC byte-counter scale factor); with
    `timed`, also the achieved copy, read-only and write-only bandwidths on
    4 GiB buffers (a practical streaming ceiling beside the 8 TB/s peak)."""
    import torch
    n = 1 << 29  # 1 GiB of int16
    a = torch.ones(n, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    out = {"copy_probe_bytes_read": 2 * n, "copy_probe_bytes_written": 2 * n}
    if timed:
        del a, b
        m = 1 << 31  # 4 GiB of int16
        a = torch.ones(m, dtype=torch.int16, device="cuda")
        b = torch.empty_like(a)

        def timeit(fn, reps=10):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps * 1e-3

        t = timeit(lambda: b.copy_(a))
        out["copy_GBps"] = round(2 * 2 * m / t / 1e9, 1)
        t = timeit(lambda: b.fill_(3))
        out["write_GBps"] = round(2 * m / t / 1e9, 1)
        del a, b
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        # plain HIP streams of several read / write mixes (a child process)
        from progressive_kv_transfer_amd import build as B
        if not os.path.exists(B.PROBE):
            raise RuntimeError(f"{B.PROBE} is not built: run "
                               "`python -m progressive_kv_transfer_amd.build`")
        r = subprocess.run([B.PROBE], capture_output=True, text=True, timeout=300)
        if r.returncode != 0:
            raise RuntimeError("stream probe failed: " + r.stderr[-2000:])
        out["streams"] = [json.loads(l) for l in r.stdout.splitlines() if l.strip()]
    print(json.dumps(out))


# (name, KV workload, t_q, q-heads, KV heads, full codes, causal tail, q seed)
ATTENTION_CASES = [
    ("decode_32k_anchor", "decode_attn_32k", 1, 64, 8, False, False, 3000),
    ("decode_32k_full", "decode_attn_32k", 1, 64, 8, True, False, 3000),
    ("verify_128k_full", "verify_attn_128k", 8, 32, 4, True, True, 4000),
]
ROTATE_BYTES = 640 << 20  # > the 256 MiB last-level cache


def measure_attention(torch, kvgen, lynx, calls: int, warmup: int, only=None):
    """Average time of lynx_decode_attn_dequant per call on each attention
    workload (or only the named one), cycling over copies of the codes:
    us_per_call from replaying the calls captured in one HIP graph (device
    time), us_per_call_eager from issuing them one by one from Python."""
    stream = torch.cuda.current_stream()
    res = {}
    built = {}
    for name, wl, t_q, nqh, nkvh, full, causal, qseed in ATTENTION_CASES:
        if only and name != only:
            continue
        cfg = kvgen.CONFIGS[wl]
        if wl not in built:
            kv = cfg.make("cuda")
            built.clear()
            built[wl] = lynx.quantize_pages(kv)
            del kv
        codes = built[wl]
        ctx = cfg.num_tokens
        nb = codes.anchor.shape[0]
        per_copy = sum(t.numel() * t.element_size() for t in (codes.anchor, codes.gamma_min,
                                                              codes.gamma_scale, codes.mu,
                                                              codes.sigma))
        if full:
            per_copy += codes.residual.numel()
        copies = [codes] + [lynx.Codes(*(t.clone() for t in (
            codes.anchor, codes.residual, codes.gamma_min, codes.gamma_scale, codes.mu,
            codes.sigma))) for _ in range(max(0, -(-ROTATE_BYTES // per_copy) - 1))]
        views = [(lynx.CodeView(c, 0, nb // 2, full), lynx.CodeView(c, nb // 2, nb, full))
                 for c in copies]
        q = kvgen.queries(qseed, t_q, nqh, device="cuda")
        out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(lynx.attn_workspace_bytes(t_q, nqh, nkvh, ctx), dtype=torch.uint8,
                         device="cuda")
        scale = 1.0 / 128 ** 0.5
        for i in range(warmup):
            k, v = views[i % len(views)]
            lynx.decode_attn_dequant(q, k, v, ctx, nkvh, scale, causal, out=out, workspace=ws,
                                     stream=stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(calls):
            k, v = views[i % len(views)]
            lynx.decode_attn_dequant(q, k, v, ctx, nkvh, scale, causal, out=out, workspace=ws,
                                     stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        us_eager = ev[0].elapsed_time(ev[1]) / calls * 1e3
        ref = out.clone()
        # The same calls captured once in a HIP graph and replayed: the device
        # time per call without the Python / launch cost of each call (how a
        # decode loop runs them).  Each replay's output must equal the eager
        # result of the last call bit for bit.
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            for i in range(calls):
                k, v = views[i % len(views)]
                lynx.decode_attn_dequant(q, k, v, ctx, nkvh, scale, causal, out=out,
                                         workspace=ws, stream=cap)
        stream.wait_stream(cap)
        times = []
        for r in range(3):
            out.zero_()
            torch.cuda.synchronize()
            ev[0].record(stream)
            graph.replay()
            ev[1].record(stream)
            torch.cuda.synchronize()
            times.append(ev[0].elapsed_time(ev[1]) / calls * 1e3)
            if not torch.equal(out, ref):
                raise RuntimeError(f"{name}: graph replay {r} differs from the eager result")
        us = min(times)
        del graph
        algo = per_copy + q.numel() * 2 + out.numel() * 2
        flops = 4.0 * t_q * nqh * 128 * ctx
        res[name] = {"workload": wl, "t_q": t_q, "q_heads": nqh, "kv_heads": nkvh,
                     "context": ctx, "codes": "anchor+residual" if full else "anchor",
                     "causal_tail": causal, "us_per_call": round(us, 2),
                     "us_per_call_eager": round(us_eager, 2),
                     "algorithmic_bytes": int(algo),
                     "GBps": round(algo / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "TFLOPs": round(flops / (us * 1e-6) / 1e12, 2),
                     "rotating_copies": len(copies)}
        del views, copies
    built.clear()
    torch.cuda.synchronize()
    return res


def measure_single_page(torch, kvgen, lynx, copies: int = 2048):
    """The single-page workload (one K and one V page block, 2 x 256 x 128):
    latency of each codec kernel per call, cycling over `copies` copies of
    input and outputs (more bytes than the last-level cache), from a HIP
    graph of the calls replayed (device time; every replay must reproduce
    the eager outputs bit for bit) and issued one by one (eager)."""
    cfg = kvgen.CONFIGS["single_page"]
    base = cfg.make("cuda")
    kvs = base.unsqueeze(0).repeat(copies, 1, 1, 1)
    nb = base.numel() // 32768
    codes = [lynx.alloc_codes(nb, "cuda") for _ in range(copies)]
    outs = torch.empty_like(kvs)
    p = lynx.params()
    stream = torch.cuda.current_stream()
    calls = {
        "quantize": lambda i, s: lynx.quantize_pages(kvs[i], p, out=codes[i], stream=s),
        "dequant_anchor": lambda i, s: lynx.dequant_anchor(codes[i], outs[i], p, stream=s),
        "dequant_full": lambda i, s: lynx.dequant_full(codes[i], outs[i], p, stream=s),
    }
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"workload": cfg.name, "blocks": nb, "copies": copies,
           "us_per_call": {}, "us_per_call_eager": {}}
    for name, fn in calls.items():
        for i in range(copies):
            fn(i, stream)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(copies):
            fn(i, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        res["us_per_call_eager"][name] = round(e0.elapsed_time(e1) / copies * 1e3, 2)
        ref = (torch.cat([c.anchor.view(-1) for c in codes[:4]]).clone(), outs[:4].clone())
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            for i in range(copies):
                fn(i, cap)
        stream.wait_stream(cap)
        times = []
        for r in range(3):
            torch.cuda.synchronize()
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / copies * 1e3)
            got = (torch.cat([c.anchor.view(-1) for c in codes[:4]]), outs[:4])
            if not (torch.equal(got[0], ref[0]) and
                    torch.equal(got[1].view(torch.int16), ref[1].view(torch.int16))):
                raise RuntimeError(f"single page {name}: graph replay {r} differs")
        del graph
        res["us_per_call"][name] = round(min(times), 2)
    return res


def measure_verify(torch, kvgen, lynx, calls: int = 200, sets: int = 32):
    """Speculative verification of 8 drafts over a Qwen-sized vocabulary:
    average time per call over `sets` different input sets (more bytes than
    the last-level cache), from a replayed HIP graph of the calls (device
    time) and issued one by one (eager); algorithmic bytes = the 2T + 1
    logit rows once plus the two rows of the correction pass."""
    T, V = kvgen.VERIFY_T, kvgen.VERIFY_VOCAB
    inputs = []
    for i in range(sets):
        d, t, s, u, us = kvgen.verify_inputs(7000 + i, T, V, 0.3)
        inputs.append((d.cuda(), t.cuda(), s.cuda(), u.cuda(), us))
    ws = torch.empty(lynx.spec_verify_workspace_bytes(T, V), dtype=torch.uint8, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(10):
        lynx.spec_verify(*inputs[i % sets], out=out, workspace=ws, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(calls):
        lynx.spec_verify(*inputs[i % sets], out=out, workspace=ws, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us_eager = e0.elapsed_time(e1) / calls * 1e3
    ref = out.clone()
    # Device time: the same calls captured once in a HIP graph and replayed;
    # each replay must end with the eager result of the last call.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(graph, stream=cap):
        for i in range(calls):
            lynx.spec_verify(*inputs[i % sets], out=out, workspace=ws, stream=cap)
    stream.wait_stream(cap)
    times = []
    for r in range(3):
        out.fill_(-7)
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / calls * 1e3)
        if not torch.equal(out, ref):
            raise RuntimeError(f"verify: graph replay {r} differs from the eager result")
    del graph
    us_call = min(times)
    algo = (2 * T + 1 + 2) * V * 4
    return {"drafts": T, "vocab": V, "us_per_call": round(us_call, 2),
            "us_per_call_eager": round(us_eager, 2),
            "algorithmic_bytes": algo, "GBps": round(algo / (us_call * 1e-6) / 1e9, 1),
            "hbm_frac": round(algo / (us_call * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "input_sets": sets}


# (anchor bits, residual bits, metadata bits): the splits of the 8-bit code
# (4 + 4 = the paper's), the single streams of the paper's Lynx-INT4 /
# Lynx-INT8, and the paper's split with bfloat16 metadata
FORMATS = ((3, 5, 32), (4, 4, 32), (5, 3, 32), (6, 2, 32), (4, 0, 32), (8, 0, 32),
           (4, 4, 16))


def measure_splits(torch, lynx, kv, out, reps: int = 5, acc_tensors: int = 8):
    """The splits of the 8-bit code and the single streams (the paper's
    Lynx-INT4 / Lynx-INT8) on the same set, each at its own code range
    (128 - 2^(b - 1) for a split, 2^(a - 1) - 1 for a single stream,
    nothing clipped): bytes per element of the streams (+ metadata), kernel
    times (HIP events, average of `reps` launches, best of 3 rounds), and the
    reconstruction error of the first `acc_tensors` tensors as NMSE =
    sum (x^ - x)^2 / sum x^2 for the anchor alone and for anchor + residual."""
    stream = torch.cuda.current_stream()
    nb = kv.numel() // (256 * 128)
    res = {}
    for a, b, mb in FORMATS:
        p = lynx.params(code_scale=float(lynx.code_max(a, b)), anchor_bits=a, residual_bits=b,
                        meta_bits=mb)
        codes = lynx.alloc_codes(nb, "cuda", anchor_bits=a, residual_bits=b, meta_bits=mb)
        calls = {"quantize": lambda: lynx.quantize_pages(kv, p, out=codes, stream=stream),
                 "dequant_anchor": lambda: lynx.dequant_anchor(codes, out, p, stream=stream)}
        if b:
            calls["dequant_full"] = lambda: lynx.dequant_full(codes, out, p, stream=stream)
        times = {}
        for name, fn in calls.items():
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            best = float("inf")
            for _ in range(3):
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                best = min(best, e0.elapsed_time(e1) / reps)
            times[name + "_ms"] = round(best, 4)
        err = {}
        for full in (False, True) if b else (False,):
            (lynx.dequant_full if full else lynx.dequant_anchor)(codes, out, p, stream=stream)
            num = den = 0.0
            for t in range(acc_tensors):
                x = kv[t].float()
                num += float(((out[t].float() - x) ** 2).sum())
                den += float((x ** 2).sum())
            err["full_nmse" if full else "anchor_nmse"] = float(f"{num / den:.4g}")
        res[f"{a}+{b}" + ("" if mb == 32 else "/bf16-metadata")] = {
            "code_scale": p.code_scale, "anchor_bytes_per_elem": a / 8,
            "residual_bytes_per_elem": b / 8, "metadata_bytes_per_elem": 0.28125 * mb / 32,
            **times, **err}
        del codes
    torch.cuda.synchronize()
    return {"workload": WORKLOAD, "accuracy_tensors": acc_tensors, "splits": res}


LARGE_WORKLOAD = "qwen3_235b_128k"


def measure_large(torch, kvgen, lynx, reps: int = 10):
    """The Qwen3-235B-A22B-shaped set at 128K context (94 layers x {K, V} x
    131072 tokens x 512 channels, 23.5 GiB of bf16) resident on the GPU:
    quantize + split and both reconstructions over the whole set in one
    launch each, HIP events around `reps` launches after one warm-up, with
    the step's algorithmic bytes per element."""
    cfg = kvgen.CONFIGS[LARGE_WORKLOAD]
    kv = cfg.make("cuda")
    n_elem = kv.numel()
    nb = n_elem // (256 * 128)
    codes = lynx.alloc_codes(nb, "cuda")
    out = torch.empty_like(kv)
    p = lynx.params()
    stream = torch.cuda.current_stream()
    calls = {"quantize": lambda: lynx.quantize_pages(kv, p, out=codes, stream=stream),
             "dequant_anchor": lambda: lynx.dequant_anchor(codes, out, p, stream=stream),
             "dequant_full": lambda: lynx.dequant_full(codes, out, p, stream=stream)}
    res = {}
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        algo = BYTES_PER_ELEM[name] * n_elem / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "bf16_GBps": round(2.0 * n_elem / (ms * 1e-3) / 1e9, 1),
                     "algo_GBps": round(algo, 1), "hbm_frac": round(algo / HBM_PEAK_GBPS, 4)}
    del kv, codes, out
    torch.cuda.empty_cache()
    return {"workload": LARGE_WORKLOAD, "kv_bf16_bytes": 2 * n_elem, "blocks": nb,
            "launches_timed": reps, "kernels": res}


TRANSFER_OBJECT_BLOCKS = 4096  # 256 MiB of bf16 KV per transfer object (16 objects)
TRANSFER_REPS = 9              # alternating link-only / pipeline runs (medians reported)
TRANSFER_RESERVED_CUS = 32     # compute units the codec streams leave to copy kernels


def measure_transfer(torch, lynx, kv, codes, out_a, out_f, kern_ms, layout,
                     reserved_cus=TRANSFER_RESERVED_CUS):
    """Split-stream transfer of the whole set through pinned host memory:
    the link alone (codes already made) and the full pipeline (quantize,
    two link streams, rebuild from anchor, refine).  layout: the code
    layout (packed = the pages' transmission buffer, one copy per hop for an
    object's anchor + metadata; separate = stream and four metadata arrays,
    five copies).  The sender and receiver run on codec streams that leave
    reserved_cus compute units to the runtime's copy kernels; the same
    measurement on four plain streams is reported beside it."""
    shape = lynx.shape_of(kv)
    nb = lynx.num_blocks(shape)
    p = lynx.params(layout=layout)
    if layout == lynx.LAYOUT_PACKED:
        codes = lynx.quantize_pages(kv, p)
    rx = lynx.alloc_codes(nb, "cuda", layout=layout)
    wire = lynx.alloc_codes(nb, "cpu", pin_memory=True, layout=layout)
    # Sender and receiver: codec streams leaving TRANSFER_RESERVED_CUS compute
    # units to the runtime's device-to-host copy kernels; the same run with
    # four plain streams follows for comparison.
    sender, receiver = lynx.CodecStream(reserved_cus), lynx.CodecStream(reserved_cus)
    streams = (sender.stream, torch.cuda.Stream(), torch.cuda.Stream(), receiver.stream)
    plain = tuple(torch.cuda.Stream() for _ in range(4))
    # Raw PCIe rates of one 1 GiB pinned copy each way (the link's floor).
    pcie = {}
    for name, src, dst in (("d2h", codes.residual, wire.residual),
                           ("h2d", wire.residual, rx.residual)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(streams[1]):
            for rep in range(2):
                e0.record()
                dst.copy_(src, non_blocking=True)
                e1.record()
        streams[1].synchronize()
        pcie[name] = src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    ob = TRANSFER_OBJECT_BLOCKS
    codec_ms = kern_ms["quantize"] + kern_ms["dequant_anchor"]

    def runs(sts):
        lynx.split_stream_transfer(None, shape, ob, codes, wire, rx, copies_only=True, p=p,
                                   streams=sts)  # warm-up
        # Pinned copies of ~90 ms vary by a few ms from run to run, more than
        # the codec time whose hiding is measured: alternate link-only and
        # pipeline runs and take the median of each time.
        links, pipes = [], []
        for _ in range(TRANSFER_REPS):
            links.append(lynx.split_stream_transfer(None, shape, ob, codes, wire, rx,
                                                    copies_only=True, p=p, streams=sts))
            pipes.append(lynx.split_stream_transfer(kv, shape, ob, codes, wire, rx, out_a,
                                                    out_f, p=p, streams=sts))
        link = {k: statistics.median(r[k] for r in links) for k in links[0]}
        pipe = {k: statistics.median(r[k] for r in pipes) for k in pipes[0]}
        return links, pipes, link, pipe

    def hidden(exposed_ms):
        # share of quantize + anchor rebuild time that does not show up after
        # the link (1 when the pipeline is no slower than the link)
        return round(min(1.0, max(0.0, 1.0 - max(exposed_ms, 0.0) / codec_ms)), 4)

    links, pipes, link, pipe = runs(streams)
    _, _, link_p, pipe_p = runs(plain)
    sender.close()
    receiver.close()
    anchor_bytes = nb * (16384 + 9216)
    residual_bytes = nb * 16384
    serial_anchor = kern_ms["quantize"] + link["anchor_arrived"] + kern_ms["dequant_anchor"]
    exposed = pipe["anchor_ready"] - link["anchor_arrived"]
    exposed_p = pipe_p["anchor_ready"] - link_p["anchor_arrived"]
    del rx, wire
    return {
        "workload": WORKLOAD, "object_blocks": ob, "objects": -(-nb // ob),
        "layout": "packed" if layout == lynx.LAYOUT_PACKED else "separate",
        "copies_per_object_per_hop": 2 if layout == lynx.LAYOUT_PACKED else 6,
        "wire": "pinned host memory (device -> host -> device per object)",
        "pcie_GBps": {k: round(v, 1) for k, v in pcie.items()},
        "link_floor_ms": round((anchor_bytes + residual_bytes) / 1e9 / min(pcie.values()) * 1e3,
                               2),
        "anchor_metadata_bytes": anchor_bytes, "residual_bytes": residual_bytes,
        "runs": TRANSFER_REPS,
        "link_only_ms": {k: round(v, 3) for k, v in link.items()},
        "pipeline_ms": {k: round(v, 3) for k, v in pipe.items()},
        "anchor_ready_runs_ms": {"link_only": [round(r["anchor_ready"], 2) for r in links],
                                 "pipeline": [round(r["anchor_ready"], 2) for r in pipes]},
        "link_anchor_GBps": round(anchor_bytes / (link["anchor_arrived"] * 1e-3) / 1e9, 2),
        "serial_anchor_ready_ms": round(serial_anchor, 3),
        "codec_streams_reserved_cus": reserved_cus,
        "exposed_anchor_overhead_ms": round(exposed, 3),
        "hidden_fraction_of_codec_time": hidden(exposed),
        "plain_streams": {"link_anchor_arrived_ms": round(link_p["anchor_arrived"], 3),
                          "pipeline_anchor_ready_ms": round(pipe_p["anchor_ready"], 3),
                          "pipeline_full_ready_ms": round(pipe_p["full_ready"], 3),
                          "exposed_anchor_overhead_ms": round(exposed_p, 3),
                          "hidden_fraction_of_codec_time": hidden(exposed_p)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--hbm-probe", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-transfer", action="store_true")
    ap.add_argument("--no-large", action="store_true")
    ap.add_argument("--attention-only", action="store_true")
    ap.add_argument("--large-only", action="store_true")
    ap.add_argument("--transfer-only", choices=["packed", "separate"], default=None)
    ap.add_argument("--transfer-reserved-cus", type=int, default=TRANSFER_RESERVED_CUS)
    ap.add_argument("--attention-calls", type=int, default=50)
    ap.add_argument("--attention-case", default=None,
                    choices=[c[0] for c in ATTENTION_CASES])
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one MI355X: the codec's page blocks are independent and "
              "this build runs on a single GPU only (--gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe or args.hbm_probe:
        copy_probe(timed=args.hbm_probe)
        return
    if args.profile_run or args.transfer_only:  # the timed steps only (same steps and warm-up)
        args.no_cpu_baseline = True

    import torch
    from progressive_kv_transfer_amd import kvgen, lynx

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lynx.lib()
    if args.large_only:
        print(json.dumps({"large_set": measure_large(torch, kvgen, lynx)}), flush=True)
        return
    if args.attention_only:
        print(json.dumps({"attention": measure_attention(
            torch, kvgen, lynx, args.attention_calls, 5, args.attention_case)}), flush=True)
        return
    cfg = kvgen.CONFIGS[WORKLOAD]
    dev = "cuda"
    kv = cfg.make(dev)
    n_elem = kv.numel()
    nb = n_elem // (256 * 128)
    codes = lynx.alloc_codes(nb, dev)
    out_a = torch.empty_like(kv)
    out_f = torch.empty_like(kv)
    p = lynx.params()
    stream = torch.cuda.current_stream()

    names = ["quantize", "dequant_anchor", "dequant_full"]

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        lynx.quantize_pages(kv, p, out=codes, stream=stream)
        if evs:
            evs[1].record(stream)
        lynx.dequant_anchor(codes, out_a, p, stream=stream)
        if evs:
            evs[2].record(stream)
        lynx.dequant_full(codes, out_f, p, stream=stream)
        if evs:
            evs[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {n: [] for n in names}
    for ev in events:
        for i, n in enumerate(names):
            per[n].append(ev[i].elapsed_time(ev[i + 1]))
    kern = {}
    for n in names:
        # the mean matches the profiler's average duration; the median and
        # the minimum show the spread over the timed steps
        ms = sum(per[n]) / len(per[n])
        algo = BYTES_PER_ELEM[n] * n_elem / (ms * 1e-3) / 1e9
        kern[n] = {"ms": round(ms, 4), "ms_median": round(statistics.median(per[n]), 4),
                   "ms_min": round(min(per[n]), 4),
                   "bf16_GBps": round(2.0 * n_elem / (ms * 1e-3) / 1e9, 1),
                   "algo_GBps": round(algo, 1), "hbm_frac": round(algo / HBM_PEAK_GBPS, 4)}
    ms_step = wall / args.steps * 1e3
    value = 2.0 * n_elem / (wall / args.steps) / 1e9
    dom = max(names, key=lambda n: kern[n]["ms"])
    achieved = kern[dom]["algo_GBps"]
    traffic = load_traffic(dom)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded per-channel Laplacian KV with x100 outlier channels and "
                "x20 bursts, bf16)",
        "config": {"workload": WORKLOAD, "layers": cfg.layers, "tensors": cfg.num_tensors,
                   "tokens": cfg.num_tokens, "channels": cfg.num_channels,
                   "page_tokens": 256, "chunk_tokens": 32, "head_channels": 128,
                   "alpha": p.alpha, "eps": p.eps, "code_scale": p.code_scale,
                   "kv_bf16_bytes": 2 * n_elem, "step": "quantize+anchor_dequant+full_dequant"},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "algorithmic_bytes_per_launch": int(BYTES_PER_ELEM[dom] * n_elem),
                     # share of the kernel's cycles the SIMDs spend issuing
                     # VALU work, from the committed rocprofv3 SQ counters
                     # (null when the kernel sources changed since)
                     "valu_busy": (load_counters() or {}).get("valu_busy")
                     if dom == "quantize" else None},
        "kernels": kern,
    }
    if args.transfer_only:  # the codec steps, then one layout's transfer alone
        kms = {n: kern[n]["ms"] for n in names}
        layout = lynx.LAYOUT_PACKED if args.transfer_only == "packed" else lynx.LAYOUT_SEPARATE
        print(json.dumps({"transfer": measure_transfer(torch, lynx, kv, codes, out_a, out_f, kms,
                                                       layout, args.transfer_reserved_cus)}),
              flush=True)
        return
    if not args.no_transfer and not args.profile_run:
        kms = {n: kern[n]["ms"] for n in names}
        # the pages' transmission buffer (anchor + scalars per block, one copy
        # per hop and object), then the separate arrays for comparison
        out["transfer"] = measure_transfer(torch, lynx, kv, codes, out_a, out_f, kms,
                                           lynx.LAYOUT_PACKED, args.transfer_reserved_cus)
        out["transfer_separate"] = measure_transfer(torch, lynx, kv, codes, out_a, out_f, kms,
                                                    lynx.LAYOUT_SEPARATE,
                                                    args.transfer_reserved_cus)
    if not args.profile_run:
        out["split_variants"] = measure_splits(torch, lynx, kv, out_a)
    if not args.no_attention and not args.profile_run:
        del out_a, out_f
        out["attention"] = measure_attention(torch, kvgen, lynx, args.attention_calls, 5)
    if not args.profile_run:
        out["verify"] = measure_verify(torch, kvgen, lynx)
        out["single_page"] = measure_single_page(torch, kvgen, lynx)
    if not args.no_large and not args.profile_run:
        out["large_set"] = measure_large(torch, kvgen, lynx)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = run_cpu_baseline(cfg, kv, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
