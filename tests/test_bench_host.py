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
