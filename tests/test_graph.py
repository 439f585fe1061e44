"""HIP graph capture of the library's calls: each captured call is replayed several
times, with eager work on the inputs and synchronisations between the replays, and
every replay is compared bit for bit with an eager call on the same inputs.  None
of the library's launches records a memset, so captured calls replay correctly."""
import numpy as np
import pytest

from linear_attention_recurrence_03_amd import inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    import linear_attention_recurrence_03_amd as m
    m._lib()
    return m


def dev(x, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(tdt) for n in ("q", "k", "v")}
    for n in ("g", "beta", "state"):
        d[n] = torch.from_numpy(np.ascontiguousarray(x[n])).cuda()
    return d


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype,T,algo,pre", [("bf16", 300, "chunked", {}),
                                              ("f32", 5, "recurrent", {}),
                                              ("bf16", 200, "chunked",
                                               {"l2norm_qk": True, "raw_gates": True}),
                                              ("bf16", 300, "chunked_head", {}),
                                              ("bf16", 200, "chunked_head",
                                               {"l2norm_qk": True, "raw_gates": True}),
                                              ("bf16", 300, "chunked_lag", {}),
                                              ("f32", 200, "chunked", {})])
def test_forward_graph_replays(gdn, dtype, T, algo, pre):
    x = inputs.custom(2, T, 4, 128, dtype=dtype, state="normal", seed=T, raw=bool(pre))
    d = dev(x, dtype)
    out = torch.empty_like(d["v"])
    fin = torch.empty_like(d["state"])
    need = gdn.workspace_size(dtype, 2, T, 4, 128, algo)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    g = capture(lambda: gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                    algo=algo, out=out, state_out=fin, workspace=ws, **pre))
    for rep in range(3):
        d["v"].mul_(1.25)                      # eager work on an input between replays
        d["g"].mul_(0.9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro, rf = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                             algo=algo, **pre)
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(fin, rf), rep


def test_in_place_decode_graph_replays(gdn):
    """state_out == state_in inside the graph: each replay advances the state."""
    x = inputs.custom(1, 1, 8, 128, dtype="f32", state="normal", seed=3)
    d = dev(x, "f32")
    st = d["state"].clone()
    out = torch.empty_like(d["v"])
    g = capture(lambda: gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], st,
                                    out=out, state_out=st))
    for rep in range(3):
        before = st.clone()
        d["q"].mul_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ro, rf = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], before)
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(st, rf), rep


def test_flash_attn_graph_replays(gdn):
    rng = np.random.default_rng(5)
    q = torch.from_numpy(rng.standard_normal((1, 16, 2, 256), dtype=np.float32)).cuda()
    k = torch.from_numpy(rng.standard_normal((1, 4, 900, 256), dtype=np.float32)).cuda()
    v = torch.from_numpy(rng.standard_normal((1, 4, 900, 256), dtype=np.float32)).cuda()
    m = torch.from_numpy(rng.normal(0, 1, (1, 1, 2, 900)).astype(np.float32)).cuda()
    out = torch.empty((1, 2, 16, 256), device="cuda")
    need = gdn.workspace_size_flash_attn(1, 16, 4, 2, 900, 256)
    assert need > 0                            # the cache is split: two kernels per call
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    g = capture(lambda: gdn.flash_attn(q, k, v, m, out=out, workspace=ws))
    for rep in range(3):
        k.mul_(1.1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = gdn.flash_attn(q, k, v, m)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
