"""Per-wave timing of the chunk-to-chunk passes, from the trace build.

The trace build (``python -m linear_attention_recurrence_03_amd.build --trace``,
which writes libgdn_trace.so next to libgdn.so) has the first eight workgroups of
a chunk-to-chunk pass record the shader clock (s_memtime ticks) at fixed points of
every chunk step.  This script runs the prefill of 1 x 4096 tokens x 32 heads,
d=128, bf16 (four rotating input copies, as the benchmark does) on that build and
prints medians and 10th/90th percentiles over the steady chunks.

``--pass scan`` (default): the per-tile pass that AUTO runs for this shape, waves
X (K M^T, E, Delta = T E), U (the state update) and O (the output) of value tile
0, two workgroup barriers (A, B) per chunk:

  step        from leaving barrier A to leaving it again (X's stamps)
  A->B, B->A  work of each wave between leaving one barrier and arriving at the next
  wait A/B    arriving at a barrier to leaving it
  last at A/B how often each wave is the last of the three to arrive

and each traced workgroup's edges (start to the first barrier, to chunk 0, the chunk
steps, after the last barrier until the state and the output are stored), then every
workgroup's start, end and life on the chip-wide 100 MHz clock (s_memrealtime), in
microseconds from the first start: the kernel ends with its slowest workgroup.

``--pass prep``: the prep kernel of the same call (the per-tile pass's variant),
wave 0 of each of its first 4,096 workgroups: the phases of a workgroup (rows
landed, products, diagonal inverses, the two levels of off-diagonal blocks, the T
stores) and when workgroups start and end relative to the first start on their XCD
(consecutive workgroups go to the eight XCDs in turn, and each XCD's shader clock
has its own origin).

``--pass lag``: the two-chunk-lag pass (algo "chunked_lag"), waves C, G, U, O and
one barrier per phase:

  work        closing stamp - opening stamp (everything the wave does in a phase)
  operands    landed stamp - opening stamp (waiting for the phase's operands)
  at barrier  next opening stamp - closing stamp (waiting for the other waves)

and the phase length (opening stamp to the next).

``--shape S,T,H`` traces another size (d=128, bf16): e.g. 2,4096,32 has more value tiles
than compute units, so the per-tile pass runs two tiles per workgroup (waves X_0, U_0,
O_0 of tile 0 are traced).

Usage: python -m linear_attention_recurrence_03_amd.phase_trace [--pass scan|prep|lag]
       [--shape S,T,H] [--json OUT]
"""
import argparse
import ctypes
import json
import os
import statistics
import sys

ROLES = ("C", "G", "U", "O")
SCAN_ROLES = ("X", "U", "O")
GROUPS, PHASES = 8, 1024


def _pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def summarize(raw, n_phases, skip=3):
    """raw: uint64 array [GROUPS][4][PHASES][3].  Returns per-role statistics over
    phases skip .. n_phases - skip - 1 of every traced workgroup."""
    out = {"phase": []}
    for r in ROLES:
        out[r] = {"work": [], "operands": [], "at_barrier": []}
    for wg in range(GROUPS):
        for p in range(skip, n_phases - skip - 1):
            out["phase"].append(int(raw[wg][0][p + 1][0]) - int(raw[wg][0][p][0]))
            for w, r in enumerate(ROLES):
                s0, s1, s2 = (int(raw[wg][w][p][i]) for i in range(3))
                nxt = int(raw[wg][w][p + 1][0])
                out[r]["work"].append(s2 - s0)
                if s0 <= s1 <= s2:
                    out[r]["operands"].append(s1 - s0)
                out[r]["at_barrier"].append(nxt - s2)

    def st(xs):
        return {"median": statistics.median(xs), "p10": _pct(xs, 0.1), "p90": _pct(xs, 0.9)} \
            if xs else None
    res = {"phase": st(out["phase"])}
    for r in ROLES:
        res[r] = {k: st(v) for k, v in out[r].items()}
    return res


def summarize_scan(raw, n_chunks, skip=3):
    """raw: uint64 array [GROUPS][4][PHASES][4] (arrive A, leave A, arrive B, leave B
    per role and chunk).  Statistics over chunks skip .. n_chunks - skip - 2."""
    out = {"step": []}
    for r in SCAN_ROLES:
        out[r] = {"A->B": [], "B->A": [], "wait A": [], "wait B": []}
    last = {"A": {r: 0 for r in SCAN_ROLES}, "B": {r: 0 for r in SCAN_ROLES}}
    release = {"A": [], "B": []}
    for wg in range(GROUPS):
        for n in range(skip, n_chunks - skip - 1):
            st = [[int(x) for x in raw[wg][w][n]] for w in range(3)]
            nx = [[int(x) for x in raw[wg][w][n + 1]] for w in range(3)]
            out["step"].append(nx[0][1] - st[0][1])
            for w, r in enumerate(SCAN_ROLES):
                out[r]["A->B"].append(st[w][2] - st[w][1])
                out[r]["B->A"].append(nx[w][0] - st[w][3])
                out[r]["wait A"].append(st[w][1] - st[w][0])
                out[r]["wait B"].append(st[w][3] - st[w][2])
            for bar, ia, il in (("A", 0, 1), ("B", 2, 3)):
                arrive = [st[w][ia] for w in range(3)]
                last[bar][SCAN_ROLES[arrive.index(max(arrive))]] += 1
                release[bar].append(min(st[w][il] for w in range(3)) - max(arrive))

    def stat(xs):
        return {"median": statistics.median(xs), "p10": _pct(xs, 0.1), "p90": _pct(xs, 0.9)} \
            if xs else None
    res = {"step": stat(out["step"]), "last_at": last,
           "release_after_last_traced_arrival": {k: stat(v) for k, v in release.items()}}
    for r in SCAN_ROLES:
        res[r] = {k: stat(v) for k, v in out[r].items()}
    # workgroup edges (row [3][0]: X starts, X leaves the first barrier, U has stored
    # the state, O has stored the last output), against X's stamps at chunk 0's
    # barrier A and the last chunk's barrier B
    edges = {k: [] for k in ("start to first barrier", "first barrier to chunk 0 A",
                             "chunk steps", "last B to state stored",
                             "last B to output stored", "span")}
    for wg in range(GROUPS):
        e = [int(x) for x in raw[wg][3][0]]
        if n_chunks > PHASES or not all(e):
            continue
        a0 = int(raw[wg][0][0][0])
        bl = int(raw[wg][0][n_chunks - 1][3])
        edges["start to first barrier"].append(e[1] - e[0])
        edges["first barrier to chunk 0 A"].append(a0 - e[1])
        edges["chunk steps"].append(bl - a0)
        edges["last B to state stored"].append(e[2] - bl)
        edges["last B to output stored"].append(e[3] - bl)
        edges["span"].append(max(e[2], e[3]) - e[0])
    res["edges"] = {k: stat(v) for k, v in edges.items()}
    return res


SPAN_GROUPS = 4096


def summarize_span(raw, n_groups):
    """raw: uint64 array [SPAN_GROUPS][4] of each per-tile-pass workgroup's start, U
    end and O end on the 100 MHz clock.  Microseconds from the earliest start."""
    rows = [[int(x) for x in raw[i][:3]] for i in range(min(n_groups, SPAN_GROUPS))]
    rows = [r for r in rows if r[0]]
    if not rows:
        return None
    t0 = min(r[0] for r in rows)
    us = lambda t: (t - t0) / 100.0
    starts = [us(r[0]) for r in rows]
    ends = [us(max(r[1], r[2])) for r in rows]
    lives = [e - s for s, e in zip(starts, ends)]
    def stat(xs):
        return {"min": min(xs), "median": statistics.median(xs), "p90": _pct(xs, 0.9),
                "max": max(xs)}
    return {"groups": len(rows), "start": stat(starts), "end": stat(ends), "life": stat(lives),
            "extent": max(ends)}


PREP_GROUPS = 4096
PREP_PHASES = ("rows landed", "products", "inverse", "level 1", "level 2", "T stored")


def summarize_prep(raw, n_groups):
    """raw: uint64 array [PREP_GROUPS][8], stamps 0..6 of each workgroup's wave 0.
    Statistics over the first n_groups workgroups."""
    n = min(n_groups, PREP_GROUPS)
    rows = [[int(x) for x in raw[i][:7]] for i in range(n)]
    # per-XCD origin: workgroup i runs on XCD i % 8
    t0 = {x: min(rows[i][0] for i in range(x, n, 8)) for x in range(min(8, n))}

    def stat(xs):
        return {"median": statistics.median(xs), "p10": _pct(xs, 0.1), "p90": _pct(xs, 0.9),
                "max": max(xs)} if xs else None
    res = {"groups": n}
    for i, name in enumerate(PREP_PHASES):
        res[name] = stat([r[i + 1] - r[i] for r in rows])
    res["total"] = stat([r[6] - r[0] for r in rows])
    res["start"] = stat([r[0] - t0[i % 8] for i, r in enumerate(rows)])
    res["end"] = stat([r[6] - t0[i % 8] for i, r in enumerate(rows)])
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--pass", dest="which", choices=("scan", "prep", "lag"), default="scan",
                    help="which chunk-to-chunk pass to trace")
    ap.add_argument("--json", help="also write the statistics to this file")
    ap.add_argument("--shape", help="n_seqs,n_tokens,n_heads (default 1,4096,32)")
    ap.add_argument("--lib", help="trace build to load (default: libgdn_trace.so here)")
    args = ap.parse_args()
    here = os.path.dirname(os.path.abspath(__file__))
    lib_path = args.lib or os.path.join(here, "libgdn_trace.so")
    if not os.path.exists(lib_path):
        sys.exit("libgdn_trace.so is not built (python -m linear_attention_recurrence_03_amd.build "
                 "--trace)")
    os.environ["LIBGDN_PATH"] = lib_path
    sys.path.insert(0, os.path.dirname(here))
    import numpy as np
    import torch
    import linear_attention_recurrence_03_amd as gdn
    from linear_attention_recurrence_03_amd import inputs

    lib = gdn._lib()
    read = {"scan": lib.gdn_scan_trace_read, "prep": lib.gdn_prep_trace_read,
            "lag": lib.gdn_phase_trace_read}[args.which]
    read.restype = ctypes.c_int
    read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    algo = "chunked_lag" if args.which == "lag" else "chunked"
    wl = inputs.WORKLOADS[4]
    if args.shape:
        s_, t_, h_ = (int(v) for v in args.shape.split(","))
        wl = inputs.Workload("traced", s_, t_, h_, 128, "bf16", "zeros", "standard", seed=11)
    x = inputs.make(wl)
    S, T, H, D = wl.shape()
    sets = []
    for i in range(4):
        d = {n: torch.from_numpy(x[n]).cuda().to(torch.bfloat16) for n in ("q", "k", "v")}
        d.update({n: torch.from_numpy(x[n]).cuda() for n in ("g", "beta")})
        sets.append(d)
    out = torch.empty_like(sets[0]["v"])
    fin = torch.empty((S, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(gdn.workspace_size("bf16", S, T, H, D, algo), dtype=torch.uint8,
                     device="cuda")
    calls = [gdn.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], None, algo=algo,
                         out=out, state_out=fin, workspace=ws) for d in sets]
    for i in range(12):
        calls[i % 4]()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    calls[1]()
    b.record()
    torch.cuda.synchronize()
    n_chunks = (T + 63) // 64
    if args.which == "scan":
        raw = np.zeros((GROUPS, 4, PHASES, 4), dtype=np.uint64)
        assert read(raw.ctypes.data, raw.nbytes) == 0
        res = summarize_scan(raw, n_chunks)
        res["call_us"] = a.elapsed_time(b) * 1e3
        res["n_chunks"] = n_chunks
        print("traced call (prep + per-tile pass): %.1f us, %d chunks" % (res["call_us"], n_chunks))
        st = res["step"]
        print("chunk step: median %d, p10 %d, p90 %d cycles" % (st["median"], st["p10"], st["p90"]))
        print("%-4s %-8s %8s %8s %8s" % ("wave", "", "median", "p10", "p90"))
        for r in SCAN_ROLES:
            for k in ("A->B", "wait B", "B->A", "wait A"):
                v = res[r][k]
                print("%-4s %-8s %8d %8d %8d" % (r, k, v["median"], v["p10"], v["p90"]))
        for bar in ("A", "B"):
            rel = res["release_after_last_traced_arrival"][bar]
            print("barrier %s: last traced arrival %s; release after it: median %d cycles" % (
                bar, ", ".join("%s %d" % kv for kv in res["last_at"][bar].items()), rel["median"]))
        for k, v in res["edges"].items():
            if v:
                print("workgroup %-27s median %8d, p10 %8d, p90 %8d cycles" % (
                    k, v["median"], v["p10"], v["p90"]))
        if hasattr(lib, "gdn_scan_span_read"):
            lib.gdn_scan_span_read.restype = ctypes.c_int
            lib.gdn_scan_span_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
            span = np.zeros((SPAN_GROUPS, 4), dtype=np.uint64)
            assert lib.gdn_scan_span_read(span.ctypes.data, span.nbytes) == 0
            res["span"] = summarize_span(span, SPAN_GROUPS)
            if res["span"]:
                sp = res["span"]
                print("all %d workgroups (100 MHz clock, us from the first start): extent %.2f"
                      % (sp["groups"], sp["extent"]))
                for k in ("start", "end", "life"):
                    print("  %-5s min %7.2f median %7.2f p90 %7.2f max %7.2f" % (
                        k, sp[k]["min"], sp[k]["median"], sp[k]["p90"], sp[k]["max"]))
    elif args.which == "prep":
        raw = np.zeros((PREP_GROUPS, 8), dtype=np.uint64)
        assert read(raw.ctypes.data, raw.nbytes) == 0
        n_groups = S * H * n_chunks
        res = summarize_prep(raw, n_groups)
        res["call_us"] = a.elapsed_time(b) * 1e3
        print("traced call (prep + per-tile pass): %.1f us, %d prep workgroups, %d traced" % (
            res["call_us"], n_groups, res["groups"]))
        print("%-12s %8s %8s %8s %8s (cycles)" % ("", "median", "p10", "p90", "max"))
        for k in PREP_PHASES + ("total", "start", "end"):
            v = res[k]
            print("%-12s %8d %8d %8d %8d" % (k, v["median"], v["p10"], v["p90"], v["max"]))
    else:
        raw = np.zeros((GROUPS, 4, PHASES, 3), dtype=np.uint64)
        assert read(raw.ctypes.data, raw.nbytes) == 0
        n_phases = n_chunks + 2
        res = summarize(raw, n_phases)
        res["call_us"] = a.elapsed_time(b) * 1e3
        res["n_phases"] = n_phases
        print("traced call (prep + lag scan): %.1f us, %d phases" % (res["call_us"], n_phases))
        ph = res["phase"]
        print("phase length: median %d, p10 %d, p90 %d cycles" % (ph["median"], ph["p10"], ph["p90"]))
        print("%-4s %-11s %8s %8s %8s" % ("wave", "", "median", "p10", "p90"))
        for r in ROLES:
            for k in ("work", "operands", "at_barrier"):
                v = res[r][k]
                if v:
                    print("%-4s %-11s %8d %8d %8d" % (r, k, v["median"], v["p10"], v["p90"]))
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()
