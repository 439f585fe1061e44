"""GPU parity: libgdn (through the C-ABI) against the fp64 oracle.

Error metric, per tensor X in {out, final_state}:
    err(X) = max |X_gpu - X_oracle| / max |X_oracle|
with the limits 1e-4 for fp32 q/k/v and 2e-2 for bf16 q/k/v (fp32 state in
both cases).  The oracle always runs on exactly the values the GPU received
(bf16 inputs already rounded, widened to fp64).
"""
import numpy as np
import pytest

import oracle
from linear_attention_recurrence_03_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import linear_attention_recurrence_03_amd as m
    m._lib()   # fail loudly if the HIP library is missing
    return m


def to_dev(x, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda() for n in ("g", "beta")}
    for n in ("q", "k", "v"):
        d[n] = torch.from_numpy(np.ascontiguousarray(x[n])).to("cuda").to(tdt)
    d["state"] = None if x["state"] is None else torch.from_numpy(
        np.ascontiguousarray(x["state"])).cuda()
    return d


def run_gpu(gdn, x, dtype, algo="auto", state=True, **pre):
    d = to_dev(x, dtype)
    out, fin = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"],
                           d["state"] if state else None, algo=algo, **pre)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), fin.cpu().numpy().astype(np.float64)


def rel_err(a, b):
    den = np.max(np.abs(b))
    num = np.max(np.abs(a - b)) if a.size else 0.0
    return num / den if den > 0 else num


def check(gdn, x, dtype, algo, state=True, what="", **pre):
    print("case:", what, dtype, algo, x["q"].shape, pre, flush=True)
    out, fin = run_gpu(gdn, x, dtype, algo, state, **pre)
    ro, rf = oracle.gdn_recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                  x["state"] if state else None, **pre)
    eo, ef = rel_err(out, ro), rel_err(fin, rf)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(fin))
    assert eo <= TOL[dtype], "out err %.3e > %.1e (%s)" % (eo, TOL[dtype], what)
    assert ef <= TOL[dtype], "state err %.3e > %.1e (%s)" % (ef, TOL[dtype], what)
    return eo, ef


# ---- the five workloads -------------------------------------------------------

@pytest.mark.parametrize("algo", ["auto", "recurrent", "chunked"])
def test_workload1_tiny(gdn, algo):
    eo, ef = check(gdn, inputs.make(inputs.WORKLOADS[1]), "f32", algo, what="tiny")
    print("ERR tiny_f32 %s: out %.3e state %.3e" % (algo, eo, ef), flush=True)


def test_workload2_decode_all_layers(gdn):
    """All 24 layer calls of the single-token decode timing, each with its own seed."""
    worst = (0.0, 0.0)
    for layer in range(24):
        eo, ef = check(gdn, inputs.make(inputs.WORKLOADS[2], layer=layer), "f32", "auto",
                       what="decode layer %d" % layer)
        worst = (max(worst[0], eo), max(worst[1], ef))
    print("ERR decode_f32 (24 layers): out %.3e state %.3e" % worst, flush=True)


def test_workload3_batched_decode(gdn):
    eo, ef = check(gdn, inputs.make(inputs.WORKLOADS[3]), "f32", "auto", what="batched decode")
    print("ERR batched_decode_f32: out %.3e state %.3e" % (eo, ef), flush=True)


@pytest.mark.parametrize("algo", ["auto", "recurrent", "chunked_lag"])
def test_workload4_prefill(gdn, algo):
    eo, ef = check(gdn, inputs.make(inputs.WORKLOADS[4]), "bf16", algo, what="prefill 4096")
    print("ERR prefill_bf16 %s: out %.3e state %.3e" % (algo, eo, ef), flush=True)


@pytest.mark.parametrize("algo", ["auto", "chunked_lag"])
def test_workload5_long_prefill_all_heads(gdn, algo):
    """The full long prefill on the GPU (all 4 sequences in one call, the launch the
    benchmark times), then every (sequence, head) compared with the oracle, one
    sequence at a time so that host memory stays near half a GB of fp64."""
    wl = inputs.WORKLOADS[5]
    x = inputs.make(wl)
    print("case: long prefill full", algo, flush=True)
    d = to_dev(x, "bf16")
    out, fin = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], algo=algo)
    torch.cuda.synchronize()
    out = out.float().cpu()
    fin = fin.cpu().numpy().astype(np.float64)
    del d
    assert bool(torch.isfinite(out).all()) and np.all(np.isfinite(fin))
    worst_o, worst_f = 0.0, 0.0
    for s in range(wl.n_seqs):
        sl = slice(s, s + 1)
        ro, rf = oracle.gdn_recurrent(x["q"][sl], x["k"][sl], x["v"][sl], x["g"][sl],
                                      x["beta"][sl], x["state"][sl])
        o = out[sl].numpy().astype(np.float64)
        for h in range(wl.n_heads):
            eo = rel_err(o[:, :, h], ro[:, :, h])
            ef = rel_err(fin[sl, h], rf[:, h])
            assert eo <= TOL["bf16"] and ef <= TOL["bf16"], (s, h, eo, ef)
            worst_o, worst_f = max(worst_o, eo), max(worst_f, ef)
        del ro, rf, o
    print("ERR long_prefill_bf16 %s (64 seq-heads): out %.3e state %.3e"
          % (algo, worst_o, worst_f), flush=True)


# ---- tails, widths, decay regimes -------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 64, 96, 128])
@pytest.mark.parametrize("T", [1, 2, 63, 65, 130])
@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_tails_and_widths(gdn, dtype, D, T, algo):
    x = inputs.custom(2, T, 3, D, dtype=dtype, state="normal", seed=T * 1000 + D)
    check(gdn, x, dtype, algo, what="tail T=%d D=%d" % (T, D))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [32, 96, 128])
@pytest.mark.parametrize("rows", [4096, 8192, 16384, 65536])
@pytest.mark.parametrize("T", [2, 3, 6])
def test_recurrence_rows_per_wave(gdn, dtype, D, rows, T):
    """Several tokens through the token recurrence in each of its shapes: two, four
    and eight state rows per wave (chosen by the total row count), odd and even
    numbers of tokens (the loop takes two per pass), and widths whose lanes hold an
    odd or even number of keys (bf16 words straddle lanes at d = 32 and 96)."""
    n_heads = -(-rows // (2 * D))               # at least `rows` rows in all
    x = inputs.custom(2, T, n_heads, D, dtype=dtype, state="normal", gate="weak",
                      seed=rows + T * 10 + D)
    check(gdn, x, dtype, "recurrent", what="rows %d T=%d D=%d" % (rows, T, D))


@pytest.mark.parametrize("gate", ["weak", "mixed"])
@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_decay_regimes(gdn, gate, algo):
    """Weak decay makes the carried state matter across many chunks; the mixed
    recipe has within-chunk gate sums far below -70."""
    x = inputs.custom(1, 1000, 4, 128, dtype="bf16", state="normal", gate=gate,
                      beta_std=2.0, seed=42)
    check(gdn, x, "bf16", algo, what="gate " + gate)
    xf = inputs.custom(1, 200, 2, 64, dtype="f32", state="normal", gate=gate, seed=43)
    check(gdn, xf, "f32", algo, what="gate f32 " + gate)


def test_token_recurrence_with_65536_heads(gdn):
    """The token recurrence reads its token and head counts from arguments packed
    into the launch's preloaded registers while they fit in 32 and 16 bits; 65,536
    heads take the variant that reads the full-width counts.  Both against the
    oracle, and the packed one (65,535 heads, the largest) too."""
    for H in (65535, 65536):
        x = inputs.make(inputs.Workload("heads", 1, 2, H, 32, "f32", "normal", "standard",
                                        seed=31))
        check(gdn, x, "f32", "recurrent", what="%d heads" % H)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_row_blocks(gdn, dtype):
    """More (sequence, head, 16 value rows) blocks than compute units: the bf16 scan
    then holds 32 value rows per workgroup, the fp32 scan runs more workgroups than
    there are compute units."""
    x = inputs.custom(2, 130, 20, 128, dtype=dtype, state="normal", seed=77)
    check(gdn, x, dtype, "chunked", what="many row blocks")


# Degenerate gates and betas, where the recurrence reduces to a simpler one (the
# oracle is pinned to these closed forms in test_oracle.py): beta = 0 (no write,
# the state only decays; gates a hundredth of the standard recipe's, so that the
# state stays far above fp32's smallest normal numbers, which the kernels flush to
# zero below), g = 0 (no decay: the plain delta rule), beta = 1 with g = 0 (each
# write replaces the value stored along its key), and g = -40 (every token forgets
# all before it: exp underflows to zero inside the chunked forms).
_DEGENERATE = {
    "beta0": lambda g, b: (0.01 * g, np.zeros_like(b)),
    "g0": lambda g, b: (np.zeros_like(g), b),
    "beta1_g0": lambda g, b: (np.zeros_like(g), np.ones_like(b)),
    "forget": lambda g, b: (np.full_like(g, -40.0), b),
}


@pytest.mark.parametrize("case", sorted(_DEGENERATE))
@pytest.mark.parametrize("dtype,algo", [("f32", "recurrent"), ("f32", "chunked"),
                                        ("bf16", "recurrent"), ("bf16", "chunked"),
                                        ("bf16", "chunked_head"), ("bf16", "chunked_lag")])
def test_degenerate_gates_and_betas(gdn, case, dtype, algo):
    x = inputs.custom(1, 130, 3, 64, dtype=dtype, state="normal", seed=31)
    x["g"], x["beta"] = (np.ascontiguousarray(a, dtype=np.float32)
                         for a in _DEGENERATE[case](x["g"], x["beta"]))
    check(gdn, x, dtype, algo, what="degenerate " + case)


# ---- the two-chunk-lag form of the chunked pass (bf16 rows) ----------------------

@pytest.mark.parametrize("D", [32, 64, 96, 128])
@pytest.mark.parametrize("T", [1, 2, 63, 65, 130, 200])
def test_lag_tails_and_widths(gdn, D, T):
    """One, two and three chunks (the chain reaches back two), full and partial."""
    x = inputs.custom(2, T, 3, D, dtype="bf16", state="normal", seed=T * 1000 + D + 5)
    check(gdn, x, "bf16", "chunked_lag", what="lag tail T=%d D=%d" % (T, D))


@pytest.mark.parametrize("gate", ["weak", "mixed"])
def test_lag_decay_regimes(gdn, gate):
    """Weak decay keeps the two earlier chunks' terms large; the mixed recipe has
    chunk gate sums far below -70 (the cross-chunk factors underflow to zero)."""
    x = inputs.custom(1, 1000, 4, 128, dtype="bf16", state="normal", gate=gate,
                      beta_std=2.0, seed=42)
    check(gdn, x, "bf16", "chunked_lag", what="lag gate " + gate)


def test_lag_many_row_blocks(gdn):
    x = inputs.custom(2, 130, 20, 128, dtype="bf16", state="normal", seed=77)
    check(gdn, x, "bf16", "chunked_lag", what="lag many row blocks")


@pytest.mark.parametrize("HK", [1, 2])
def test_lag_tiled_key_heads(gdn, HK):
    x = inputs.custom(2, 200, 6, 64, dtype="bf16", state="normal", seed=950 + HK,
                      key_heads=HK)
    check(gdn, x, "bf16", "chunked_lag", what="lag tiled key heads HK=%d" % HK)


@pytest.mark.parametrize("l2,gates", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("D", [32, 128])
def test_lag_input_transforms(gdn, l2, gates, D):
    x = _mixed_raw(2, 200, 3, D, "bf16", seed=750 + D, l2=l2, gates=gates)
    check(gdn, x, "bf16", "chunked_lag", what="lag transforms D=%d" % D, l2norm_qk=l2,
          raw_gates=gates)


def test_lag_agrees_with_chunked(gdn):
    """Both chunked forms compute the same quantities: their outputs differ by no more
    than bf16 operand rounding, and each value channel depends only on its own
    channel of v (perturbing one changes nothing else)."""
    x = inputs.custom(1, 300, 4, 128, dtype="bf16", state="normal", gate="weak", seed=61)
    a = run_gpu(gdn, x, "bf16", "chunked")
    b = run_gpu(gdn, x, "bf16", "chunked_lag")
    assert rel_err(b[0], a[0]) < 2e-2 and rel_err(b[1], a[1]) < 2e-2
    y = dict(x)
    y["v"] = x["v"].copy()
    y["v"][..., 17] = inputs.bf16_round(y["v"][..., 17] + 1.0)
    c = run_gpu(gdn, y, "bf16", "chunked_lag")
    other = [j for j in range(128) if j != 17]
    assert np.array_equal(b[0][..., other], c[0][..., other])
    assert np.array_equal(b[1][:, :, other, :], c[1][:, :, other, :])


# ---- the whole-head chunk-to-chunk pass (bf16 rows) -------------------------------

@pytest.mark.parametrize("D", [32, 64, 96, 128])
@pytest.mark.parametrize("T", [1, 2, 63, 65, 130, 200])
def test_head_tails_and_widths(gdn, D, T):
    x = inputs.custom(2, T, 3, D, dtype="bf16", state="normal", seed=T * 1000 + D + 9)
    check(gdn, x, "bf16", "chunked_head", what="head tail T=%d D=%d" % (T, D))


@pytest.mark.parametrize("gate", ["weak", "mixed"])
def test_head_decay_regimes(gdn, gate):
    x = inputs.custom(1, 1000, 4, 128, dtype="bf16", state="normal", gate=gate,
                      beta_std=2.0, seed=42)
    check(gdn, x, "bf16", "chunked_head", what="head gate " + gate)


@pytest.mark.parametrize("HK", [1, 2])
def test_head_tiled_key_heads(gdn, HK):
    x = inputs.custom(2, 200, 6, 64, dtype="bf16", state="normal", seed=960 + HK,
                      key_heads=HK)
    check(gdn, x, "bf16", "chunked_head", what="head tiled key heads HK=%d" % HK)


@pytest.mark.parametrize("l2,gates", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("D", [32, 128])
def test_head_input_transforms(gdn, l2, gates, D):
    x = _mixed_raw(2, 200, 3, D, "bf16", seed=760 + D, l2=l2, gates=gates)
    check(gdn, x, "bf16", "chunked_head", what="head transforms D=%d" % D, l2norm_qk=l2,
          raw_gates=gates)


@pytest.mark.parametrize("D,pre", [(128, {}), (64, {"l2norm_qk": True, "raw_gates": True})])
def test_head_equals_per_tile_scan(gdn, D, pre):
    """The two chunk-to-chunk passes round at the same points: identical bits."""
    x = (_mixed_raw(2, 300, 4, D, "bf16", seed=71, l2=True, gates=True) if pre
         else inputs.custom(2, 300, 4, D, dtype="bf16", state="normal", gate="weak", seed=71))
    a = run_gpu(gdn, x, "bf16", "chunked", **pre)
    b = run_gpu(gdn, x, "bf16", "chunked_head", **pre)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_head_chosen_for_large_grids(gdn):
    """256 (seq, head) pairs or more: AUTO runs the whole-head pass (one pair per
    compute unit); checked against the oracle, with a ragged last chunk and key
    heads tiled over value heads."""
    x = inputs.custom(8, 130, 32, 128, dtype="bf16", state="normal", seed=88, key_heads=16)
    eo, ef = check(gdn, x, "bf16", "auto", what="large grid auto")
    a = run_gpu(gdn, x, "bf16", "auto")
    b = run_gpu(gdn, x, "bf16", "chunked_head")
    c = run_gpu(gdn, x, "bf16", "chunked")       # the per-tile pass, forced
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
    print("ERR large_grid_bf16 auto: out %.3e state %.3e" % (eo, ef), flush=True)


# ---- q and k with fewer (key) heads, tiled over the value heads ---------------------

def _carve(t, off_bytes):
    """A copy of t that starts off_bytes past a 4 KiB boundary inside a larger buffer
    (returned too, to keep it alive)."""
    n = t.numel() * t.element_size()
    buf = torch.empty(n + off_bytes + 8192, dtype=torch.uint8, device=t.device)
    base = (-buf.data_ptr()) % 4096 + off_bytes
    view = buf[base:base + n].view(t.dtype).view(t.shape)
    view.copy_(t)
    return view, buf


@pytest.mark.parametrize("dtype,algo", [("f32", "recurrent"), ("f32", "chunked"),
                                        ("bf16", "recurrent"), ("bf16", "chunked"),
                                        ("bf16", "chunked_lag"), ("bf16", "chunked_head")])
def test_any_16_byte_placement(gdn, dtype, algo):
    """The result does not depend on where the tensors lie: every input and output
    placed at a different 16-byte offset from a 4 KiB boundary gives bit for bit the
    result of the same call on torch's own (aligned) allocations.  The kernels read
    rows as 16-byte pieces at per-lane offsets from a wave-wide base, so an odd
    16-byte base takes other address paths than an aligned one."""
    x = inputs.make(inputs.Workload("placement", 2, 130, 4, 128, dtype, "normal", "mixed",
                                    seed=23))
    d = to_dev(x, dtype)
    print("case: placement", dtype, algo, flush=True)
    ref_out, ref_fin = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                   algo=algo)
    keep, c = [], {}
    for n, off in (("q", 16), ("k", 272), ("v", 4112), ("g", 48), ("beta", 80), ("state", 144)):
        c[n], b = _carve(d[n], off)
        keep.append(b)
    out, b_out = _carve(torch.zeros_like(ref_out), 528)
    fin, b_fin = _carve(torch.zeros_like(ref_fin), 1040)
    gdn.forward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["state"], algo=algo, out=out,
                state_out=fin)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "out differs with moved tensors (%s %s)" % (dtype, algo)
    assert torch.equal(fin, ref_fin), "state differs with moved tensors (%s %s)" % (dtype, algo)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("HK", [1, 2, 3])
@pytest.mark.parametrize("T,algo", [(1, "recurrent"), (7, "recurrent"), (63, "chunked"),
                                    (130, "chunked")])
def test_tiled_key_heads(gdn, dtype, HK, T, algo):
    x = inputs.custom(2, T, 6, 64, dtype=dtype, state="normal", seed=900 + 10 * HK + T,
                      key_heads=HK)
    assert x["q"].shape[2] == HK and x["v"].shape[2] == 6
    check(gdn, x, dtype, algo, what="tiled key heads HK=%d T=%d" % (HK, T))


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_tiled_equals_expanded_copy(gdn, algo):
    """The tiled call reads the same values as a call on q, k expanded to one head
    per value head (h -> h mod HK), so the results are identical bit for bit."""
    x = inputs.custom(1, 200, 8, 128, dtype="bf16", state="normal", seed=31, key_heads=2)
    a = run_gpu(gdn, x, "bf16", algo)
    y = dict(x)
    idx = [h % 2 for h in range(8)]
    y["q"], y["k"] = x["q"][:, :, idx], x["k"][:, :, idx]
    b = run_gpu(gdn, y, "bf16", algo)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_tiled_prefill_workload(gdn):
    """The full 4096-token prefill with 32 value heads over 16 query/key heads."""
    check(gdn, inputs.make(inputs.GQA_PREFILL), "bf16", "auto", what="tiled prefill 4096")


# ---- input transforms inside the op (unnormalised q/k rows, raw gates) ------------

def _mixed_raw(n_seqs, n_tokens, n_heads, head_dim, dtype, seed, l2, gates, key_heads=None):
    """Raw q/k rows and/or raw gate pre-activations, the rest from the standard
    recipe of the same draw."""
    raw = inputs.custom(n_seqs, n_tokens, n_heads, head_dim, dtype=dtype, state="normal",
                        seed=seed, raw=True, key_heads=key_heads)
    std = inputs.custom(n_seqs, n_tokens, n_heads, head_dim, dtype=dtype, state="normal",
                        seed=seed, key_heads=key_heads)
    x = dict(std)
    if l2:
        x["q"], x["k"] = raw["q"], raw["k"]
    if gates:
        x["g"], x["beta"] = raw["g"], raw["beta"]
    return x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows", [4096, 8192, 16384])
def test_tiled_key_heads_rows_per_wave(gdn, dtype, rows):
    """Query/key heads shared by four value heads each (value head h reads key head
    h mod n_k) in every several-token shape of the token recurrence."""
    n_heads = rows // (2 * 128)
    x = inputs.custom(2, 4, n_heads, 128, dtype=dtype, state="normal", seed=900 + rows // 1024,
                      key_heads=n_heads // 4)
    check(gdn, x, dtype, "recurrent", what="tiled rows %d" % rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [96, 128])
@pytest.mark.parametrize("rows", [8192, 16384])
def test_input_transforms_rows_per_wave(gdn, dtype, D, rows):
    """Normalised q/k rows and raw gates in the several-token shapes with 16 lanes
    per state row (four and eight rows per wave)."""
    n_heads = -(-rows // (2 * D))
    x = _mixed_raw(2, 5, n_heads, D, dtype, seed=800 + D + rows // 1024, l2=True, gates=True)
    check(gdn, x, dtype, "recurrent", what="transforms rows %d D=%d" % (rows, D),
          l2norm_qk=True, raw_gates=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("l2,gates", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("T,algo", [(1, "recurrent"), (9, "recurrent"), (65, "chunked"),
                                    (130, "chunked")])
def test_input_transforms(gdn, dtype, l2, gates, D, T, algo):
    x = _mixed_raw(2, T, 3, D, dtype, seed=700 + T + D, l2=l2, gates=gates)
    check(gdn, x, dtype, algo, what="transforms D=%d T=%d" % (D, T), l2norm_qk=l2,
          raw_gates=gates)


def test_input_transforms_tiled_prefill(gdn):
    """Both transforms with 16 query/key heads over 32 value heads, 4096 tokens."""
    x = _mixed_raw(1, 4096, 32, 128, "bf16", seed=6100, l2=True, gates=True, key_heads=16)
    check(gdn, x, "bf16", "auto", what="transforms, tiled prefill 4096", l2norm_qk=True,
          raw_gates=True)


@pytest.mark.parametrize("T,algo", [(1, "recurrent"), (5, "recurrent"), (130, "chunked")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_input_transforms_tiled(gdn, T, algo, dtype):
    """Both transforms with q/k of 2 heads tiled over 6 value heads (decode and prefill)."""
    x = _mixed_raw(2, T, 6, 64, dtype, seed=800 + T, l2=True, gates=True, key_heads=2)
    check(gdn, x, dtype, algo, what="transforms tiled T=%d" % T, l2norm_qk=True,
          raw_gates=True)


def test_input_transforms_zero_rows(gdn):
    """All-zero q or k rows stay finite with normalisation (epsilon in the root)."""
    x = _mixed_raw(1, 130, 2, 64, "bf16", seed=7, l2=True, gates=False)
    x["k"][0, 5] = 0.0
    x["q"][0, 70] = 0.0
    for algo in ("recurrent", "chunked"):
        check(gdn, x, "bf16", algo, what="zero rows", l2norm_qk=True)


def test_zero_initial_state_pointer(gdn):
    x = inputs.custom(1, 70, 2, 64, dtype="f32", state="zeros", seed=1)
    check(gdn, x, "f32", "auto", state=False, what="state None")


@pytest.mark.parametrize("n_seqs,n_tokens,n_heads,head_dim,dtype", [
    (1, 1, 4, 128, "bf16"),      # one token, four rows per wave
    (1, 7, 3, 96, "f32"),        # several tokens, two rows per wave
    (8, 1, 32, 128, "f32"),      # one token, eight rows per wave
    (8, 3, 32, 128, "bf16"),     # several tokens, eight rows per wave
])
def test_zero_initial_state_pointer_recurrent(gdn, n_seqs, n_tokens, n_heads, head_dim, dtype):
    """Without an initial state the token recurrence starts from zeros in every
    kernel shape (rows per wave, single and several tokens)."""
    x = inputs.custom(n_seqs, n_tokens, n_heads, head_dim, dtype=dtype, state="zeros", seed=2)
    check(gdn, x, dtype, "recurrent", state=False, what="state None")


# ---- contract properties ------------------------------------------------------

def test_in_place_state_update(gdn):
    x = inputs.custom(2, 5, 4, 128, dtype="f32", seed=3)
    d = to_dev(x, "f32")
    ref_o, ref_f = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"].clone())
    st = d["state"].clone()
    o, f = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], st, state_out=st)
    torch.cuda.synchronize()
    assert f.data_ptr() == st.data_ptr()
    assert torch.equal(o, ref_o) and torch.equal(st, ref_f)


def test_zero_tokens_copies_state(gdn):
    x = inputs.custom(2, 0, 3, 64, dtype="bf16", seed=4)
    d = to_dev(x, "bf16")
    o, f = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"])
    o2, f2 = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], None)
    torch.cuda.synchronize()
    assert o.numel() == 0 and torch.equal(f, d["state"])
    assert torch.count_nonzero(f2).item() == 0


def test_deterministic(gdn):
    x = inputs.custom(1, 300, 4, 128, dtype="bf16", seed=5)
    a = run_gpu(gdn, x, "bf16", "auto")
    b = run_gpu(gdn, x, "bf16", "auto")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("algo", ["recurrent", "chunked"])
def test_value_row_independence(gdn, algo):
    """Perturbing value channel i changes only out[..., i] and state row i."""
    x = inputs.custom(1, 130, 2, 128, dtype="bf16", seed=6)
    o1, f1 = run_gpu(gdn, x, "bf16", algo)
    y = dict(x)
    y["v"] = x["v"].copy()
    y["v"][..., 17] = inputs.bf16_round(y["v"][..., 17] + 1.0)
    o2, f2 = run_gpu(gdn, y, "bf16", algo)
    other = [j for j in range(128) if j != 17]
    assert np.array_equal(o1[..., other], o2[..., other])
    assert np.array_equal(f1[:, :, other, :], f2[:, :, other, :])
    assert not np.array_equal(o1[..., 17], o2[..., 17])


def test_runs_on_callers_stream(gdn):
    """Inputs produced by a torch op on a side stream and consumed there with no
    synchronisation in between: the library must join that stream's queue."""
    x = inputs.custom(2, 100, 8, 128, dtype="bf16", seed=7)
    ref_o, ref_f = run_gpu(gdn, x, "bf16", "auto")
    d = to_dev(x, "bf16")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        big = torch.randn(4096, 4096, device="cuda")
        for _ in range(3):
            big = big @ big * 1e-3                       # keep the stream busy
        v2 = d["v"] + (big[0, 0] * 0).to(torch.bfloat16)  # depends on the busy work
        out, fin = gdn.forward(d["q"], d["k"], v2, d["g"], d["beta"], d["state"])
    side.synchronize()
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), ref_o)
    assert np.array_equal(fin.cpu().numpy().astype(np.float64), ref_f)


def test_explicit_stream_argument(gdn):
    """stream= names a stream that is not torch's current one: outputs and the
    workspace are allocated on that stream and the call runs there, so other work
    on the current stream cannot be handed their memory while the call runs."""
    x = inputs.custom(2, 100, 8, 128, dtype="bf16", seed=7)
    ref_o, ref_f = run_gpu(gdn, x, "bf16", "auto")
    d = to_dev(x, "bf16")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        big = torch.randn(2048, 2048, device="cuda")
        for _ in range(3):
            big = big @ big * 1e-3                       # keep the side stream busy
    out, fin = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                           stream=side)
    churn = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(16)]  # current stream
    side.synchronize()
    torch.cuda.synchronize()
    del churn
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), ref_o)
    assert np.array_equal(fin.cpu().numpy().astype(np.float64), ref_f)


def test_prepared_call_repeats(gdn):
    """A prepared call re-issues the validated C call: the same results as forward,
    call after call, with the inputs' contents changed in between."""
    x = inputs.custom(1, 1, 32, 128, dtype="f32", state="normal", seed=9)
    d = to_dev(x, "f32")
    st = d["state"].clone()
    call = gdn.prepare(d["q"], d["k"], d["v"], d["g"], d["beta"], st, state_out=st)
    ref_st = d["state"].clone()
    for step in range(3):
        o_ref, f_ref = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], ref_st)
        ref_st = f_ref
        o, f = call()
        torch.cuda.synchronize()
        assert f.data_ptr() == st.data_ptr()
        assert torch.equal(o, o_ref) and torch.equal(f, f_ref), step
        d["v"].mul_(0.5)                                 # new contents, same storage


def test_flash_attn_explicit_stream(gdn):
    """flash_attn with stream=: the float32 mask copy, the output and the workspace are
    made on that stream."""
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    q = torch.randn((2, 8, 3, 128), device="cuda", generator=g)
    k = torch.randn((2, 2, 700, 128), device="cuda", generator=g)
    v = torch.randn((2, 2, 700, 128), device="cuda", generator=g)
    m = torch.randn((2, 1, 3, 700), device="cuda", generator=g).to(torch.float16)
    ref = gdn.flash_attn(q, k, v, m)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = gdn.flash_attn(q, k, v, m, stream=side)
    churn = [torch.full((1 << 20,), 3.0, device="cuda") for _ in range(16)]
    side.synchronize()
    torch.cuda.synchronize()
    del churn
    assert torch.equal(out, ref)


def test_empty_batch_noop(gdn):
    q = torch.empty((0, 5, 2, 64), device="cuda")
    g = torch.empty((0, 5, 2), device="cuda")
    o, f = gdn.forward(q, q, q, g, g, None)
    assert o.shape == q.shape and f.shape == (0, 2, 64, 64)


def test_rejects_bad_arguments(gdn):
    x = inputs.custom(1, 4, 2, 64, dtype="f32", seed=8)
    d = to_dev(x, "f32")
    with pytest.raises(gdn.GdnError):
        gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                    out=d["q"])   # output aliases an input
    q48 = torch.zeros((1, 4, 2, 48), device="cuda")
    g = torch.zeros((1, 4, 2), device="cuda")
    with pytest.raises(gdn.GdnError):
        gdn.forward(q48, q48, q48, g, g, None)
    q3 = torch.zeros((1, 4, 3, 64), device="cuda")
    v2 = torch.zeros((1, 4, 2, 64), device="cuda")
    g2 = torch.zeros((1, 4, 2), device="cuda")
    with pytest.raises(gdn.GdnError):
        gdn.forward(q3, q3, v2, g2, g2, None)   # 3 key heads do not tile 2 value heads
