"""Host-side pieces of bench.py (no GPU): the algorithmic byte and FLOP counts the
roofline is computed from, and the code fingerprint that decides whether the
committed counter summaries still describe the current kernels."""
import bench


def test_algorithmic_bytes_per_workload():
    # each input read once, each output written once, the state read and written
    # once: q, k, v, out, g, beta, state
    assert bench.algorithmic_bytes(1, 64, 2, 32, 4) == 4 * 16384 + 2 * 512 + 2 * 8192
    assert bench.algorithmic_bytes(1, 1, 32, 128, 4) == 4_260_096
    assert bench.algorithmic_bytes(64, 1, 32, 128, 4) == 272_646_144
    assert bench.algorithmic_bytes(1, 4096, 32, 128, 2) == 139_460_608
    assert bench.algorithmic_bytes(4, 32768, 16, 128, 2) == 2_172_649_472
    # tiled key heads: q and k hold half the heads
    full = bench.algorithmic_bytes(1, 4096, 32, 128, 2)
    tiled = bench.algorithmic_bytes(1, 4096, 32, 128, 2, key_heads=16)
    assert full - tiled == 2 * 4096 * 16 * 128 * 2


def test_algorithmic_flops_chunked():
    # 5 C d + 6 d^2 + C^2 / 3 per token-head at C = 64, d = 128: 140,629 (rounded)
    per = bench.algorithmic_flops_chunked(1, 1, 1, 128)
    assert abs(per - 140_629.33) < 0.01
    assert abs(bench.algorithmic_flops_chunked(1, 4096, 32, 128) - 1.8433e10) < 1e7


def _hash(files):
    return bench.kernel_source_hash(lambda name: sorted(files) if name is None
                                    else files[name].encode())


def test_code_fingerprint_ignores_comments_and_layout():
    a = {"k.hip": 'int f(int x) { return x + 1; }  // add one\n/* note */ const char *s = "a//b";\n'}
    b = {"k.hip": '// other words\nint f(int x)\n{\n    return x + 1;\n}\nconst char *s = "a//b";'}
    c = {"k.hip": 'int f(int x) { return x + 2; }\nconst char *s = "a//b";\n'}
    d = {"k.hip": 'int f(int x) { return x + 1; }\nconst char *s = "a/*b";\n'}
    assert _hash(a) == _hash(b)
    assert _hash(a) != _hash(c)            # a code change
    assert _hash(a) != _hash(d)            # string contents are code
    assert _hash(a) != _hash({"j.hip": a["k.hip"]})   # file names count
    assert bench._code_tokens('x = "/* kept */"; /* gone */ y') == 'x = "/* kept */"; y'
    assert bench._code_tokens("c = '\"'; // q\nd") == "c = '\"'; d"


def test_fingerprint_of_the_tree_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def _counter_csv(path, counter, rows):
    import csv
    import os
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for i, (name, kib, ns) in enumerate(rows):
            w.writerow([i, name, counter, kib, 1000, 1000 + ns])


def test_traffic_records_calibrate_each_counter(tmp_path):
    """Synthetic counter files: the elementwise kernel's FETCH_SIZE reads half of its
    512 MiB of reads and WRITE_SIZE all of its writes, so fetch values scale by 2 and
    write values by 1; decode records take bytes over the dispatch's own duration."""
    mib = 1024  # KiB per MiB
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>"
    scan = "void gdn::chunk_scan_kernel<128, true, 1, false>(...)"
    prep = "void gdn::chunk_prep_kernel<128, true, false>(...)"
    dec = "void gdn::recurrent_kernel<128, 32, 4, false, true, true>(...)"
    _counter_csv(tmp_path / "f", "FETCH_SIZE",
                 [(copy, 256 * mib, 10), (prep, 10 * mib, 10), (scan, 20 * mib, 10),
                  (scan, 22 * mib, 10), (scan, 21 * mib, 10), (dec, 60 * mib, 50_000)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE",
                 [(copy, 512 * mib, 10), (prep, 5 * mib, 10), (scan, 7 * mib, 10),
                  (dec, 130 * mib, 50_000)])
    rec = bench.traffic_records(str(tmp_path / "f"), str(tmp_path / "w"))
    mb = 1024 * 1024
    p = rec["prefill_bf16"]
    assert abs(p["calibration_factors"]["fetch"] - 2.0) < 1e-12
    assert abs(p["calibration_factors"]["write"] - 1.0) < 1e-12
    assert abs(p["kernels"]["chunk_prep"]["fetch_bytes"] - 20 * mb) < 1
    assert abs(p["kernels"]["chunk_scan"]["fetch_bytes"] - 42 * mb) < 1   # median of 20, 22, 21
    assert abs(p["kernels"]["chunk_scan"]["write_bytes"] - 7 * mb) < 1
    assert p["bytes_per_launch"] == round((20 + 5 + 42 + 7) * mb)
    d = rec["decode_batched"]
    assert d["bytes_per_launch"] == round((120 + 130) * mb)
    assert abs(d["seconds_under_counters"] - 50e-6) < 1e-12
    assert abs(d["counted_GBs"] - round(250 * mb / 50e-6 / 1e9, 1)) < 0.06
    assert "decode_1tok" not in rec
    # the single-token layer calls: any other row count of the d = 128 recurrence
    one = "void gdn::recurrent_kernel<128, 32, 2, false, true, true>(...)"
    _counter_csv(tmp_path / "f1", "FETCH_SIZE", [(copy, 256 * mib, 10), (one, 2 * mib, 4_000)])
    _counter_csv(tmp_path / "w1", "WRITE_SIZE", [(copy, 512 * mib, 10), (one, 2 * mib, 4_000)])
    rec1 = bench.traffic_records(str(tmp_path / "f1"), str(tmp_path / "w1"))
    assert rec1["decode_1tok"]["bytes_per_launch"] == round((4 + 2) * mb)


def test_more_than_one_gpu_is_refused():
    """bench.py --gpus N > 1 (or a multi-rank launch) exits with a message before
    touching any GPU."""
    import os
    import subprocess
    import sys
    env = dict(os.environ)
    for args, world in ((["--gpus", "2"], "1"), ([], "2")):
        env["WORLD_SIZE"] = world
        r = subprocess.run([sys.executable, bench.__file__] + args, env=env,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2, r.stderr
        assert "exactly one GPU" in r.stderr


def test_moved_copy_starts_past_a_2mib_boundary():
    # the placement helper of the bench's prefill_placement record: a copy of the
    # tensor, equal in value, starting exactly off bytes past a 2 MiB boundary
    import torch
    t = torch.arange(3 * 1000, dtype=torch.float32).reshape(3, 1000)
    for off in (0, 256, 768):
        v, buf = bench.moved(torch, t, off)
        assert v.data_ptr() % (2 << 20) == off
        assert torch.equal(v, t) and v.is_contiguous()
        assert buf.data_ptr() <= v.data_ptr()
        assert v.data_ptr() + t.numel() * 4 <= buf.data_ptr() + buf.numel()
