#!/usr/bin/env python3
"""Benchmark of libgdn on one MI355X.

Headline: chunked prefill tokens/s on n_seqs=1, n_tokens=4096, n_heads=32,
head_dim=128, bf16 q/k/v, fp32 g/beta/state (one GDN layer of a 4B hybrid
model; "ggml attention kernels" model card, section "Measured").  A step is one
gdn_forward call over that batch: every stage of the chunked path runs inside
it.  Also reported (extra keys on the same JSON line): single-token decode
microseconds per layer over 24 sequential layer calls, batched decode, and the
long batched prefill (4 x 32768 tokens, 16 heads).

Cold-cache protocol: MI355X has 256 MB of Infinity Cache in front of HBM and
every workload here except the long prefill would fit in it, so timed loops
rotate through enough input copies (or scrub a 1 GiB buffer first) that each
call reads inputs the cache no longer holds.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
CHUNK = 64


def algorithmic_bytes(S, T, H, D, esz, state_read=True, key_heads=None):
    """Each input read once, each output written once, the state read+written once
    (q and k hold key_heads heads when given)."""
    tok = S * T * H * D * esz
    tok_kq = S * T * (H if key_heads is None else key_heads) * D * esz
    gate = S * T * H * 4
    st = S * H * D * D * 4
    return 2 * tok_kq + 2 * tok + 2 * gate + st * (2 if state_read else 1)


def algorithmic_flops_chunked(S, T, H, D, C=CHUNK):
    """Per token-head 5 C d + 6 d^2 + C^2/3 (triangular work the chunked form needs)."""
    return S * T * H * (5 * C * D + 6 * D * D + C * C / 3.0)


def _code_tokens(text):
    """C/C++/HIP source with comments removed and whitespace runs collapsed, so that
    the fingerprint below changes with the code only."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                        # string or character literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(read=None):
    """Fingerprint of the kernel sources (code only: comments and layout do not
    count), which the committed counter summaries record."""
    csrc = os.path.join(ROOT, "linear_attention_recurrence_03_amd", "csrc")
    if read is None:
        def read(name):
            with open(os.path.join(csrc, name), "rb") as f:
                return f.read()
        names = sorted(os.listdir(csrc))
    else:
        names = sorted(read(None))
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode() + _code_tokens(read(name).decode("utf-8")).encode())
    return h.hexdigest()[:16]


def load_traffic_record(workload_key):
    """The committed counter record of a workload (profiles/traffic.json), if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec


def load_traffic(workload_key):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    rec = load_traffic_record(workload_key)
    return rec.get("bytes_per_launch") if rec else None


def run_env(torch):
    """Where the numbers were taken: GPU, its compute units, HIP and torch builds,
    host CPU model and the cores this process may use."""
    props = torch.cuda.get_device_properties(0)
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip": torch.version.hip,
            "torch": torch.__version__, "host_cpu": cpu,
            "host_cores": len(os.sched_getaffinity(0))}


def load_mfma(workload_key):
    """Matrix-core busy share per prefill kernel from the committed counter run, if it
    was taken on the current kernel sources (else None)."""
    try:
        with open(os.path.join(ROOT, "profiles", "mfma.json")) as f:
            rec = json.load(f).get(workload_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return {k: round(v["mfma_busy_frac"], 4) for k, v in rec["kernels"].items()}


def to_dev(x, dtype, torch):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {}
    for n in ("q", "k", "v"):
        d[n] = torch.from_numpy(x[n]).to("cuda").to(tdt).contiguous()
    for n in ("g", "beta", "state"):
        d[n] = torch.from_numpy(x[n]).to("cuda").contiguous()
    return d


class Slot:
    """One resident copy of a workload's inputs plus its output buffers."""

    def __init__(self, gdn, d, torch, pre=None, algo="auto"):
        self.d = d
        self.pre = pre or {}
        v = d["v"]
        S, T, H, D = v.shape
        self.out = torch.empty_like(v)
        self.state_out = torch.empty((S, H, D, D), dtype=torch.float32, device="cuda")
        need = gdn.workspace_size("bf16" if v.dtype == torch.bfloat16 else "f32", S, T, H, D,
                                  algo)
        self.ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        # arguments validated and marshalled once; each run re-issues the C call
        self.call = gdn.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                algo=algo, out=self.out, state_out=self.state_out,
                                workspace=self.ws, **self.pre)

    def run(self, gdn, stream=None):
        """One gdn_forward call on the prepared arguments (on ``stream`` if given, else
        on the stream current when the slot was made)."""
        self.call(stream)


def clone_dev(d):
    return {n: t.clone() for n, t in d.items()}


def time_loop(torch, fn, n):
    """HIP-event time of n calls of fn() on the current stream, in ms per call."""
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def moved(torch, t, off_bytes):
    """A copy of t that starts off_bytes past a 2 MiB boundary inside a buffer of its
    own (torch puts large tensors on such a boundary); returns (copy, buffer)."""
    n = t.numel() * t.element_size()
    buf = torch.empty(n + off_bytes + (4 << 20), dtype=torch.uint8, device=t.device)
    base = (-buf.data_ptr()) % (2 << 20) + off_bytes
    view = buf[base:base + n].view(t.dtype).view(t.shape)
    view.copy_(t)
    return view, buf


def bench_prefill(gdn, torch, wl, steps, warmup, nbuf, pre=None, algo="auto", placement=None):
    from linear_attention_recurrence_03_amd import inputs
    x = inputs.make(wl)
    base = to_dev(x, wl.dtype, torch)
    copies = [base if i == 0 else clone_dev(base) for i in range(nbuf)]
    keep = []
    if placement is not None:   # {name: bytes past a 2 MiB boundary}
        for d in copies:
            bufs = []
            for name, off in placement.items():
                d[name], buf = moved(torch, d[name], off)
                bufs.append(buf)
            keep.append(bufs)
    slots = [Slot(gdn, d, torch, pre, algo) for d in copies]
    for s, bufs in zip(slots, keep):
        s.keep = bufs
    del x
    for i in range(warmup):
        slots[i % nbuf].run(gdn)
    ms = time_loop(torch, lambda i: slots[i % nbuf].run(gdn), steps)
    return ms, slots


def bench_decode_layers(gdn, torch, wl, reps, n_layers=24):
    """24 sequential single-token layer calls, each with its own inputs and state.

    Device time comes from replaying the 24 calls captured in one HIP graph
    (so host-side Python overhead does not starve the GPU), with a 1 GiB scrub
    before each timed replay; host time is the wall time of eager calls.
    Median over reps."""
    from linear_attention_recurrence_03_amd import inputs
    slots = [Slot(gdn, to_dev(inputs.make(wl, layer=l), wl.dtype, torch), torch)
             for l in range(n_layers)]
    scrub = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm up outside capture
        for s in slots:
            s.run(gdn, side)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for s in slots:
            s.run(gdn, cap)
    dev_us, host_us = [], []
    for _ in range(reps):
        scrub.fill_(1.0)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        dev_us.append(a.elapsed_time(b) * 1e3 / n_layers)
        scrub.fill_(1.0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in slots:
            s.run(gdn)
        host_us.append((time.perf_counter() - t0) * 1e6 / n_layers)
        torch.cuda.synchronize()
    return statistics.median(dev_us), min(dev_us), max(dev_us), statistics.median(host_us)


def bench_dispatch_floor(torch, n=24, reps=30):
    """Device time per dispatch of n dependent one-element kernels (torch add_ on a
    single float) replayed from one HIP graph: the floor any one-kernel layer call
    pays on this machine, against which the single-token decode is read."""
    x = torch.zeros(1, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        x.add_(1.0)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n):
            x.add_(1.0)
    us = []
    for _ in range(reps):
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3 / n)
    return statistics.median(us)


def bench_state_copy_floor(gdn, torch, wl, reps=30, n_layers=24):
    """Device time per layer of 24 zero-token gdn_forward calls on the single-token
    decode's states (each launches the library's plain state copy: the same 2 MB
    read and written, no token arithmetic), replayed from one HIP graph after the
    same 1 GiB scrub as the decode timing: what reading and writing a layer's state
    costs on this machine, between the dispatch floor and the decode."""
    from linear_attention_recurrence_03_amd import inputs
    S, _, H, D = wl.shape()
    states = [torch.from_numpy(inputs.make(wl, layer=l)["state"]).cuda() for l in range(n_layers)]
    outs = [torch.empty_like(st) for st in states]
    empty = torch.empty((S, 0, H, D), dtype=torch.float32, device="cuda")
    gates = torch.empty((S, 0, H), dtype=torch.float32, device="cuda")
    calls = [gdn.prepare(empty, empty, empty, gates, gates, st, out=empty, state_out=o)
             for st, o in zip(states, outs)]
    scrub = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c(side)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for c in calls:
            c(cap)
    us = []
    for _ in range(reps):
        scrub.fill_(1.0)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3 / n_layers)
    assert all(torch.equal(o, st) for o, st in zip(outs, states))
    return statistics.median(us)


def bench_attn(gdn, torch, n_calls=40, reps=7):
    """Decode attention, one query per head: the card's shape (16 query heads over 4
    key/value heads, head_dim 256, 141 and 512 cached positions; warm, as a decode
    loop re-reads its cache) and 32 sequences x 32 query heads over 8 key/value heads
    x d128 x 4096 positions (0.5 GB of cache, 4 rotating copies: HBM-bound).  Device
    time from replaying n_calls calls captured in one HIP graph (median of reps);
    host time from eager calls."""
    res = {}
    for (S, H, HKV, NKV, D, nbuf) in ((1, 16, 4, 141, 256, 1), (1, 16, 4, 512, 256, 1),
                                      (32, 32, 8, 4096, 128, 4)):
        g = torch.Generator(device="cuda")
        g.manual_seed(S * 100000 + NKV)
        sets = []
        for _ in range(nbuf):
            q = torch.randn((S, H, 1, D), device="cuda", generator=g).to(torch.bfloat16)
            k = torch.randn((S, HKV, NKV, D), device="cuda", generator=g).to(torch.bfloat16)
            v = torch.randn((S, HKV, NKV, D), device="cuda", generator=g).to(torch.bfloat16)
            out = torch.empty((S, 1, H, D), dtype=torch.bfloat16, device="cuda")
            sets.append((q, k, v, out))
        ws = torch.empty(max(gdn.workspace_size_flash_attn(S, H, HKV, 1, NKV, D), 1),
                         dtype=torch.uint8, device="cuda")

        def call(i):
            q, k, v, out = sets[i % nbuf]
            gdn.flash_attn(q, k, v, None, out=out, workspace=ws)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):       # warm up outside capture
            for i in range(2 * nbuf):
                call(i)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_calls):
                call(i)
        dev = []
        for _ in range(reps):
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            graph.replay()
            b.record()
            torch.cuda.synchronize()
            dev.append(a.elapsed_time(b) * 1e3 / n_calls)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n_calls):
            call(i)
        torch.cuda.synchronize()
        host = (time.perf_counter() - t0) * 1e6 / n_calls
        us = statistics.median(dev)
        nbytes = 2 * S * HKV * NKV * D * 2 + 2 * S * H * D * 2
        res["S%d_H%d_Hkv%d_nkv%d_d%d" % (S, H, HKV, NKV, D)] = {
            "us_per_call_device": round(us, 2), "us_per_call_host_eager": round(host, 2),
            "bytes_per_call": nbytes,
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "inputs": "bf16, warm" if nbuf == 1 else "bf16, %d rotating copies" % nbuf}
        del sets, ws, graph
        torch.cuda.empty_cache()
    return res


def profile_pass(gdn, torch, wl, launches=10):
    """Short run for hardware-counter passes: an elementwise multiply by one over
    512 MiB (known bytes: reads 512 MiB, writes 512 MiB; it calibrates FETCH_SIZE
    and WRITE_SIZE), a few launches of the headline workload, then of the batched
    decode (rotating input copies) and of the single-token decode (24 layers, each
    with its own inputs and state)."""
    from linear_attention_recurrence_03_amd import inputs
    src = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)          # the calibration kernel: 512 MiB in, 512 MiB out
    torch.cuda.synchronize()
    _, slots = bench_prefill(gdn, torch, wl, steps=launches, warmup=0, nbuf=4)
    del slots
    _, slots = bench_prefill(gdn, torch, inputs.WORKLOADS[3], steps=launches, warmup=0, nbuf=3)
    del slots
    wl2 = inputs.WORKLOADS[2]
    for layer in range(24):
        Slot(gdn, to_dev(inputs.make(wl2, layer=layer), wl2.dtype, torch), torch).run(gdn)
    torch.cuda.synchronize()
    print("profile pass done: copy %d bytes, %d launches" % (src.numel() * 4, launches), flush=True)


def traffic_records(fetch_dir, write_dir):
    """Turn two rocprofv3 --pmc runs of --profile-pass (FETCH_SIZE, WRITE_SIZE, in
    KiB per dispatch) into HBM bytes per launch of each libgdn kernel.  Each counter
    is scaled by what it reads for the 512 MiB elementwise kernel, whose reads and
    writes are known (512 MiB each)."""
    import csv
    copy_bytes = 512 * 1024 * 1024       # read, and written, by the calibration kernel

    def kernel_key(name):
        return ("copy" if "MulFunctor" in name else
                "chunk_scan" if "chunk_scan" in name else
                "chunk_prep" if "chunk_prep" in name else
                # the profile pass runs the token recurrence twice: the batched decode
                # (32 lanes per row, eight rows per wave: recurrent_kernel<128, 32, 4, ...>)
                # and the single-token layer calls (fewer rows per wave)
                "decode_batched" if "recurrent_kernel<128, 32, 4," in name else
                "decode_1tok" if "recurrent_kernel<128, " in name else None)

    def per_kernel(d, counter, dur):
        vals = {}
        path = os.path.join(d, "run_counter_collection.csv")
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = kernel_key(r["Kernel_Name"])
            if key:
                vals.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
                dur.setdefault(key, {})[(d, r["Dispatch_Id"])] = (
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        return {k: statistics.median(v) for k, v in vals.items()}

    dur = {}
    f = per_kernel(fetch_dir, "FETCH_SIZE", dur)
    w = per_kernel(write_dir, "WRITE_SIZE", dur)
    fs, ws = copy_bytes / f["copy"], copy_bytes / w["copy"]
    kernels = {k: {"fetch_bytes": f.get(k, 0) * fs, "write_bytes": w.get(k, 0) * ws}
               for k in ("chunk_prep", "chunk_scan")}
    total = sum(v["fetch_bytes"] + v["write_bytes"] for v in kernels.values())
    note = ("FETCH_SIZE and WRITE_SIZE per dispatch (medians), each scaled by the factor that "
            "maps its reading for the 512 MiB elementwise kernel to the kernel's known 512 MiB "
            "of reads or writes")
    factors = {"fetch": fs, "write": ws}
    rec = {"prefill_bf16": {"source_hash": kernel_source_hash(), "bytes_per_launch": round(total),
                            "kernels": kernels, "calibration_factors": factors, "note": note}}
    # decode: one kernel per call; counted bytes over the dispatch's own duration
    for key, shape in (("decode_batched", (64, 1, 32, 128)), ("decode_1tok", (1, 1, 32, 128))):
        if key not in f or key not in w:
            continue
        nb = f[key] * fs + w[key] * ws
        t = statistics.median(dur[key].values())
        rec[key] = {"source_hash": kernel_source_hash(), "bytes_per_launch": round(nb),
                    "fetch_bytes": round(f[key] * fs), "write_bytes": round(w[key] * ws),
                    "algorithmic_bytes": algorithmic_bytes(*shape, 4),
                    "seconds_under_counters": t, "counted_GBs": round(nb / t / 1e9, 1),
                    "counted_hbm_frac": round(nb / t / 1e9 / HBM_PEAK_GBS, 4),
                    "calibration_factors": factors, "note": note}
    return rec


def summarize_pmc(fetch_dir, write_dir):
    """traffic_records of two counter runs, written to profiles/traffic.json."""
    rec = traffic_records(fetch_dir, write_dir)
    out = os.path.join(ROOT, "profiles", "traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def summarize_mfma(pmc_dir):
    """Matrix-core counters of one rocprofv3 --pmc run of --profile-pass
    (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) per
    launch of each prefill kernel: bf16 MFMA FLOP (MOPS x 512, the counter's unit);
    the share of SIMD cycles with the matrix core busy while the kernel ran (busy
    cycles summed over SIMDs, over active cycles x SIMDs; GRBM_GUI_ACTIVE comes summed
    over the XCDs, so it is divided by their count from the agent table); and the
    MFMA rate over the dispatch's own duration against the dense bf16 peak.  Writes
    profiles/mfma.json."""
    import csv
    agent = next(r for r in csv.DictReader(open(os.path.join(pmc_dir, "run_agent_info.csv")))
                 if r.get("Agent_Type", "").upper().endswith("GPU") or r.get("Name") == "gfx950")
    n_xcc, n_simd = int(agent["Num_Xcc"]), int(agent["Simd_Count"])
    vals, dur = {}, {}
    for r in csv.DictReader(open(os.path.join(pmc_dir, "run_counter_collection.csv"))):
        name = r["Kernel_Name"]
        key = ("chunk_scan" if "chunk_scan" in name else
               "chunk_prep" if "chunk_prep" in name else None)
        if key:
            vals.setdefault((key, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
            dur.setdefault(key, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) -
                                                         int(r["Start_Timestamp"])) * 1e-9
    rec = {"source_hash": kernel_source_hash(), "xcds": n_xcc, "simds": n_simd, "kernels": {}}
    for k in ("chunk_prep", "chunk_scan"):
        flop = statistics.median(vals[(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16")]) * 512
        busy = statistics.median(vals[(k, "SQ_VALU_MFMA_BUSY_CYCLES")])
        gui = statistics.median(vals[(k, "GRBM_GUI_ACTIVE")]) / n_xcc
        t = statistics.median(dur[k].values())
        rec["kernels"][k] = {"mfma_flop_bf16": flop, "mfma_busy_cycles": busy,
                             "active_cycles": gui, "mfma_busy_frac": busy / (gui * n_simd),
                             "seconds_under_counters": t,
                             "mfma_frac_of_bf16_peak": flop / t / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    out = os.path.join(ROOT, "profiles", "mfma.json")
    with open(out, "w") as fh:
        json.dump({"prefill_bf16": rec}, fh, indent=1)
    print(json.dumps(rec, indent=1))


def _oracle_seconds(x, threads, min_seconds, min_reps=1, sub=None):
    """Mean wall seconds of one oracle pass over x (or x restricted by ``sub``, a
    (seq slice, head slice) pair), repeated until min_seconds have passed."""
    import oracle
    if sub is not None:
        ss, hs = sub
        x = {n: (x[n][ss, :, hs] if n in ("q", "k", "v", "g", "beta") else x[n][ss, hs])
             for n in ("q", "k", "v", "g", "beta", "state")}
        x = {n: np.ascontiguousarray(a) for n, a in x.items()}
    reps, total = 0, 0.0
    while total < min_seconds or reps < min_reps:
        t0 = time.perf_counter()
        oracle.gdn_recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], x["state"],
                             threads=threads)
        total += time.perf_counter() - t0
        reps += 1
    return total / reps, reps


def cpu_baseline(wl, budget=1.0):
    """The fp64 oracle (plain token recurrence, OpenMP over (seq, head)) timed on this
    host's cores, at 1 thread and at all the cores this process may use, for each
    workload: microseconds per layer call for the decodes (the single-token decode
    as its 24 sequential layer calls) and tokens/s for the prefills.  Where a whole
    workload would take more than a few seconds of CPU time, a stated sample of its
    (sequence, head) units is timed and scaled to the whole workload by the unit count
    (the units are independent and equally long).  ``budget`` scales the repeat
    times (about 25 s in all at 1.0)."""
    from linear_attention_recurrence_03_amd import inputs
    cores = len(os.sched_getaffinity(0))
    legs = {}

    # single-token decode: 24 layers, each its own inputs and state
    wl2 = inputs.WORKLOADS[2]
    xs = [inputs.make(wl2, layer=l) for l in range(24)]
    for label, th in (("threads_1", 1), ("threads_all", cores)):
        t_all, reps = 0.0, 0
        while t_all < 1.0 * budget or reps < 3:
            t0 = time.perf_counter()
            for x in xs:
                _oracle_seconds(x, th, 0.0)
            t_all += time.perf_counter() - t0
            reps += 1
        legs.setdefault("decode_1tok", {})[label] = {
            "us_per_layer": round(t_all / reps / 24 * 1e6, 2), "threads": th,
            "sample": "all 24 layer calls, %d times" % reps}
    del xs
    # batched decode: 64 seqs x 32 heads, one token
    wl3 = inputs.WORKLOADS[3]
    x3 = inputs.make(wl3)
    for label, th in (("threads_1", 1), ("threads_all", cores)):
        sec, reps = _oracle_seconds(x3, th, 1.5 * budget, min_reps=3)
        legs.setdefault("decode_batched", {})[label] = {
            "us_per_call": round(sec * 1e6, 1), "threads": th,
            "sample": "the whole call, %d times" % reps}
    del x3
    # prefill 1 x 4096 x 32 heads: all cores on the whole workload, 1 thread on 4 heads
    x4 = inputs.make(wl)
    sec, reps = _oracle_seconds(x4, cores, 6.0 * budget, min_reps=3)
    legs["prefill_bf16"] = {"threads_all": {
        "tokens_per_s": round(wl.n_seqs * wl.n_tokens / sec, 1), "threads": cores,
        "sample": "the whole workload, %d times" % reps}}
    h1 = 4
    sec1, reps1 = _oracle_seconds(x4, 1, 4.0 * budget, sub=(slice(0, 1), slice(0, h1)))
    whole1 = sec1 * wl.n_heads / h1
    legs["prefill_bf16"]["threads_1"] = {
        "tokens_per_s": round(wl.n_seqs * wl.n_tokens / whole1, 1), "threads": 1,
        "sample": "heads 0-%d of the sequence (%d of %d (seq, head) units), %d times, "
                  "scaled by %d" % (h1 - 1, h1, wl.n_heads, reps1, wl.n_heads // h1)}
    headline = {"value": legs["prefill_bf16"]["threads_all"]["tokens_per_s"],
                "seconds": round(sec * reps, 3), "reps": reps}
    del x4
    # long prefill 4 x 32768 x 16 heads: sequence 0 only (all cores), one head (1 thread)
    wl5 = inputs.WORKLOADS[5]
    x5 = inputs.make(wl5, seq=0)
    units = wl5.n_seqs * wl5.n_heads
    sec, reps = _oracle_seconds(x5, cores, 4.0 * budget)
    legs["prefill_long"] = {"threads_all": {
        "tokens_per_s": round(wl5.n_seqs * wl5.n_tokens / (sec * wl5.n_seqs), 1),
        "threads": cores,
        "sample": "sequence 0, all %d heads (%d of %d units), %d times, scaled by %d" % (
            wl5.n_heads, wl5.n_heads, units, reps, wl5.n_seqs)}}
    sec1, reps1 = _oracle_seconds(x5, 1, 2.0 * budget, sub=(slice(0, 1), slice(0, 1)))
    legs["prefill_long"]["threads_1"] = {
        "tokens_per_s": round(wl5.n_seqs * wl5.n_tokens / (sec1 * units), 1), "threads": 1,
        "sample": "sequence 0, head 0 (1 of %d units), %d times, scaled by %d" % (
            units, reps1, units)}
    del x5
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                       None)
    except OSError:
        pass
    return {"value": headline["value"], "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu,
            "sample": "the headline workload (%d seq x %d tokens x %d heads, d=%d) %d times on "
                      "%d threads, fp64 token recurrence, OpenMP over (seq, head); every "
                      "workload at 1 thread and at all cores in legs" % (
                          wl.n_seqs, wl.n_tokens, wl.n_heads, wl.head_dim, headline["reps"],
                          cores),
            "seconds": headline["seconds"], "legs": legs}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="time only the oracle legs (no GPU needed)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the decode and long-prefill extras")
    ap.add_argument("--profile-pass", action="store_true",
                    help="short run for rocprofv3 --pmc passes (copy calibration, 10 prefill and "
                         "10 batched-decode launches, 24 single-token decode calls)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two --pmc runs of --profile-pass")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="write profiles/mfma.json from a --pmc run of --profile-pass with "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.cpu_baseline_only:
        from linear_attention_recurrence_03_amd import inputs
        print(json.dumps(cpu_baseline(inputs.WORKLOADS[4])), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs on exactly one GPU; --gpus %d (WORLD_SIZE=%d) is not "
              "supported.  Each (sequence, head) is independent, so a multi-GPU run would "
              "shard heads with no communication; it is not measured here." % (args.gpus, world),
              file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_recurrence_03_amd as gdn
    from linear_attention_recurrence_03_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    gdn._lib()

    wl = inputs.WORKLOADS[4]
    if args.profile_pass:
        profile_pass(gdn, torch, wl)
        return
    S, T, H, D = wl.shape()
    ms, _ = bench_prefill(gdn, torch, wl, args.steps, args.warmup, nbuf=4)
    tok_s = S * T / (ms * 1e-3)
    nbytes = algorithmic_bytes(S, T, H, D, 2)
    flops = algorithmic_flops_chunked(S, T, H, D)
    achieved = nbytes / (ms * 1e-3) / 1e9
    traffic = load_traffic("prefill_bf16")
    line = {
        "metric": "GDN prefill tokens/s @T=4096,H=32,d=128",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_bf16: n_seqs=1 n_tokens=4096 n_heads=32 head_dim=128, "
                               "bf16 q/k/v/out, fp32 g/beta/state, chunk 64",
                   "n_seqs": S, "n_tokens": T, "n_heads": H, "head_dim": D},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": nbytes,
                     "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "mfma_busy_counters": load_mfma("prefill_bf16"),
                     "scope": "one gdn_forward call (all kernels of the chunked path)"},
    }

    if not args.headline_only:
        extras = {}
        # single-token decode, 24 layers
        wl2 = inputs.WORKLOADS[2]
        med, lo, hi, host = bench_decode_layers(gdn, torch, wl2, reps=30)
        b2 = algorithmic_bytes(*wl2.shape(), 4)
        extras["decode_1tok"] = {
            "us_per_layer_device": round(med, 3), "us_min": round(lo, 3), "us_max": round(hi, 3),
            "us_per_layer_host": round(host, 3), "bytes_per_call": b2,
            "hbm_frac": round(b2 / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "counters": load_traffic_record("decode_1tok"),
            "dispatch_floor_us": round(bench_dispatch_floor(torch), 3),
            "state_copy_us": round(bench_state_copy_floor(gdn, torch, wl2), 3),
            "host_path": "prepared call (arguments validated once, C call re-issued)",
            "workload": "1 seq x 1 token x 32 heads x d128 fp32, 24 sequential layer calls "
                        "replayed from one HIP graph, 1 GiB scrub before each replay"}
        # batched decode
        wl3 = inputs.WORKLOADS[3]
        ms3, _ = bench_prefill(gdn, torch, wl3, steps=50, warmup=5, nbuf=3)
        b3 = algorithmic_bytes(*wl3.shape(), 4)
        extras["decode_batched"] = {
            "us_per_call": round(ms3 * 1e3, 3), "bytes_per_call": b3,
            "achieved_GBs": round(b3 / (ms3 * 1e-3) / 1e9, 1),
            "hbm_frac": round(b3 / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "counters": load_traffic_record("decode_batched"),
            "workload": "64 seqs x 1 token x 32 heads x d128 fp32, 3 rotating input copies"}
        torch.cuda.empty_cache()
        # long prefill
        wl5 = inputs.WORKLOADS[5]
        ms5, slots = bench_prefill(gdn, torch, wl5, steps=10, warmup=2, nbuf=1)
        del slots
        torch.cuda.empty_cache()
        S5, T5, H5, D5 = wl5.shape()
        b5 = algorithmic_bytes(S5, T5, H5, D5, 2)
        f5 = algorithmic_flops_chunked(S5, T5, H5, D5)
        extras["prefill_long"] = {
            "tokens_per_s": round(S5 * T5 / (ms5 * 1e-3), 1), "ms_per_call": round(ms5, 4),
            "hbm_frac": round(b5 / (ms5 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(f5 / (ms5 * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "workload": "4 seqs x 32768 tokens x 16 heads x d128 bf16, carried N(0,0.1) state"}
        # prefill with 16 query/key heads tiled over 32 value heads (no expanded copy)
        wlt = inputs.GQA_PREFILL
        mst, slots = bench_prefill(gdn, torch, wlt, steps=100, warmup=10, nbuf=4)
        del slots
        torch.cuda.empty_cache()
        St, Tt, Ht, Dt = wlt.shape()
        bt = algorithmic_bytes(St, Tt, Ht, Dt, 2, key_heads=wlt.key_heads)
        extras["prefill_tiled"] = {
            "tokens_per_s": round(St * Tt / (mst * 1e-3), 1), "us_per_call": round(mst * 1e3, 2),
            "bytes_per_call": bt,
            "hbm_frac": round(bt / (mst * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "workload": "1 seq x 4096 tokens x 32 value heads (16 query/key heads, tiled) x "
                        "d128 bf16, zero state, 4 rotating input copies"}
        # the same with raw inputs: q/k rows normalised and gates activated inside the op
        wlr = dataclasses.replace(wlt, raw=True)
        msr, slots = bench_prefill(gdn, torch, wlr, steps=100, warmup=10, nbuf=4,
                                   pre={"l2norm_qk": True, "raw_gates": True})
        del slots
        torch.cuda.empty_cache()
        extras["prefill_tiled_raw"] = {
            "tokens_per_s": round(St * Tt / (msr * 1e-3), 1), "us_per_call": round(msr * 1e3, 2),
            "bytes_per_call": bt,
            "hbm_frac": round(bt / (msr * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "workload": "as prefill_tiled, with unnormalised q/k rows and raw gate "
                        "pre-activations transformed inside the op"}
        # a batch of prefills with a (seq, head) pair per compute unit: AUTO (the
        # whole-head pass) against the per-tile pass forced
        wlb = inputs.BATCHED_PREFILL
        Sb, Tb, Hb, Db = wlb.shape()
        bb = algorithmic_bytes(Sb, Tb, Hb, Db, 2)
        rec = {"workload": "8 seqs x 2048 tokens x 32 heads x d128 bf16, zero state, "
                           "2 rotating input copies", "bytes_per_call": bb}
        for key, algo in (("auto", "auto"), ("per_tile", "chunked")):
            msb, slots = bench_prefill(gdn, torch, wlb, steps=20, warmup=3, nbuf=2, algo=algo)
            del slots
            torch.cuda.empty_cache()
            rec[key] = {"us_per_call": round(msb * 1e3, 2),
                        "tokens_per_s": round(Sb * Tb / (msb * 1e-3), 1),
                        "hbm_frac": round(bb / (msb * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        extras["prefill_batched"] = rec
        # the headline workload through the two-chunk-lag form of the chunked pass
        msl, slots = bench_prefill(gdn, torch, wl, steps=50, warmup=5, nbuf=4,
                                   algo="chunked_lag")
        del slots
        torch.cuda.empty_cache()
        extras["prefill_lag"] = {
            "tokens_per_s": round(S * T / (msl * 1e-3), 1), "us_per_call": round(msl * 1e3, 2),
            "hbm_frac": round(nbytes / (msl * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "workload": "the headline workload with algo chunked_lag (two-chunk-lag chunk "
                        "pass), 4 rotating input copies"}
        # the headline workload with q and k placed explicitly: where k lies relative to q
        # decides which heads' rows share a memory hot spot that sets the pass's end (with
        # q and k a multiple of 2 MiB apart, as torch's 32 MiB allocations here are, heads
        # h = 1 (mod 4)); the headline keeps torch's own placement
        rec = {"workload": "the headline workload, 4 rotating input copies, each q and k copy "
                           "placed the given number of bytes past a 2 MiB boundary"}
        for key, place in (("q0_k0", {"q": 0, "k": 0}), ("q0_k768", {"q": 0, "k": 768})):
            msk, slots = bench_prefill(gdn, torch, wl, steps=100, warmup=10, nbuf=4,
                                       placement=place)
            del slots
            torch.cuda.empty_cache()
            rec[key] = {"us_per_call": round(msk * 1e3, 2),
                        "tokens_per_s": round(S * T / (msk * 1e-3), 1),
                        "hbm_frac": round(nbytes / (msk * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        extras["prefill_placement"] = rec
        # decode flash attention: the card's measured shape, and a bandwidth-sized cache
        extras["flash_attn_decode"] = bench_attn(gdn, torch)
        line["extras"] = extras

    line["env"] = run_env(torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
