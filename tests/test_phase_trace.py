"""Host logic of the phase-trace summaries (no GPU): known stamps give known
statistics."""
import numpy as np

from linear_attention_recurrence_03_amd import phase_trace as pt


def test_scan_summary_of_synthetic_stamps():
    raw = np.zeros((pt.GROUPS, 4, pt.PHASES, 4), dtype=np.uint64)
    n_chunks = 20
    for wg in range(pt.GROUPS):
        for n in range(n_chunks):
            t0 = 10_000 + 2_000 * n                # every wave leaves A at t0
            # X arrives at B last (t0 + 1100), U at t0 + 300, O at t0 + 900; all leave
            # B at t0 + 1200; they arrive at the next A at t0 + 1900, 1990, 1500
            for w, (b_arr, a_next) in enumerate(((1100, 1900), (300, 1990), (900, 1500))):
                raw[wg, w, n] = [t0 - (2000 - a_next), t0, t0 + b_arr, t0 + 1200]
    last_b = 10_000 + 2_000 * (n_chunks - 1) + 1200
    for wg in range(pt.GROUPS):
        # edges: X starts, leaves the first barrier, U stores the state, O the output
        raw[wg, 3, 0] = [5_000, 6_000, last_b + 300, last_b + 500]
    res = pt.summarize_scan(raw, n_chunks)
    assert res["step"]["median"] == 2000
    e = res["edges"]
    assert e["start to first barrier"]["median"] == 1000
    assert e["first barrier to chunk 0 A"]["median"] == 9_900 - 6_000
    assert e["chunk steps"]["median"] == last_b - 9_900
    assert e["last B to state stored"]["median"] == 300
    assert e["last B to output stored"]["median"] == 500
    assert e["span"]["median"] == last_b + 500 - 5_000
    assert res["X"]["A->B"]["median"] == 1100 and res["X"]["wait B"]["median"] == 100
    assert res["U"]["B->A"]["median"] == 790 and res["O"]["wait A"]["median"] == 500
    assert res["last_at"]["B"]["X"] == res["last_at"]["B"]["X"] > 0
    assert res["last_at"]["B"]["U"] == 0 and res["last_at"]["A"]["U"] > 0
    assert res["release_after_last_traced_arrival"]["B"]["median"] == 100
    assert res["release_after_last_traced_arrival"]["A"]["median"] == 10


def test_lag_summary_of_synthetic_stamps():
    raw = np.zeros((pt.GROUPS, 4, pt.PHASES, 3), dtype=np.uint64)
    n_phases = 20
    for wg in range(pt.GROUPS):
        for p in range(n_phases):
            t0 = 5_000 + 4_000 * p
            for w in range(4):
                raw[wg, w, p] = [t0, t0 + 100 * (w + 1), t0 + 1000 * (w + 1)]
    res = pt.summarize(raw, n_phases)
    assert res["phase"]["median"] == 4000
    assert res["C"]["work"]["median"] == 1000 and res["O"]["work"]["median"] == 4000
    assert res["G"]["operands"]["median"] == 200 and res["U"]["at_barrier"]["median"] == 1000


def test_prep_summary_of_synthetic_stamps():
    raw = np.zeros((pt.PREP_GROUPS, 8), dtype=np.uint64)
    n_groups = 100
    for i in range(n_groups):
        t0 = 1_000 + 50 * i
        steps = [0, 400, 900, 1700, 1800, 1900, 2000]   # cumulative stamps
        raw[i, :7] = [t0 + x for x in steps]
    res = pt.summarize_prep(raw, n_groups)
    assert res["rows landed"]["median"] == 400 and res["inverse"]["median"] == 800
    assert res["total"]["median"] == 2000
    # starts are taken from the first start on each XCD (workgroup i on XCD i % 8)
    assert res["start"]["max"] == 50 * (99 - 3) and res["end"]["max"] == 50 * 96 + 2000


def test_span_summary_of_synthetic_stamps():
    raw = np.zeros((pt.SPAN_GROUPS, 4), dtype=np.uint64)
    for i in range(256):
        # 100 MHz ticks: starts 10 ns apart, U done after 50 us, O 1 us later
        raw[i, :3] = [1_000 + i, 1_000 + i + 5_000, 1_000 + i + 5_100]
    res = pt.summarize_span(raw, pt.SPAN_GROUPS)
    assert res["groups"] == 256
    assert res["start"]["min"] == 0 and res["start"]["max"] == 2.55
    assert res["life"]["median"] == 51.0
    assert res["extent"] == 2.55 + 51.0
    assert pt.summarize_span(np.zeros_like(raw), pt.SPAN_GROUPS) is None
