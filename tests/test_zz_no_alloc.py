"""gdn_forward_noalloc (scratch in the library's fixed per-GPU array) against
gdn_forward_ex with a caller workspace: the same kernels on the same inputs, so
the results must be identical bit for bit.  Two calls in a row, the second on a
smaller input, so that the second reuses scratch the first left behind."""
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


def _dev(x, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(tdt) for n in ("q", "k", "v")}
    for n in ("g", "beta", "state"):
        d[n] = torch.from_numpy(np.ascontiguousarray(x[n])).cuda()
    return d


@pytest.mark.parametrize("dtype,algo", [("bf16", "chunked"), ("f32", "chunked"),
                                        ("bf16", "recurrent")])
def test_noalloc_equals_workspace_call(gdn, dtype, algo):
    cases = [(1, 4096, 32, 128, None), (2, 130, 6, 64, 3)]   # second call: smaller input
    for (S, T, H, D, HK) in cases:
        print("case: noalloc", dtype, algo, (S, T, H, D, HK), flush=True)
        x = inputs.custom(S, T, H, D, dtype=dtype, state="normal", seed=S * 100 + T,
                          key_heads=HK)
        d = _dev(x, dtype)
        ref_o, ref_f = gdn.forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                   algo=algo)
        out = torch.empty_like(d["v"])
        fin = torch.empty_like(d["state"])
        got_o, got_f = gdn.forward_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                           d["state"], out, fin, algo=algo)
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o), (S, T, H, D)
        assert torch.equal(got_f, ref_f), (S, T, H, D)
