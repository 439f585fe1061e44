"""GPU check of the chunked path's intermediate values against the oracle.

The chunked algorithm first computes, for every (sequence, head, chunk), the
state-independent matrices T = (I + A)^{-1} and the decay-masked P, plus the
per-token gate factors, into the caller's workspace.  This test decodes that
workspace (its layout is internal to the library and mirrored here: per chunk
T and then P / sqrt(head_dim) (the output's factor, applied where P is formed)
as six "fragment blocks" each, then four fp32 rows of 64: beta,
e^gam, e^(gam_last - gam) and e^gam_last repeated; when the op normalises q and
k the gates take 2 KiB with a fifth row) and compares it with the
oracle's stage values, so that a parity failure can be attributed to the first
or the second half of the path.

A fragment block holds the 16 x 32 sub-matrix (row tile tt, column half h) of a
64 x 64 lower-triangular matrix as 64 units of 8 elements: the unit of row i
(0..15) and lane group g (0..3) sits at position 4 i + (g ^ (i >> 2)), and its
element j is column 32 h + 4 g + j (j < 4) or 32 h + 16 + 4 g + j - 4 (j >= 4).
The six stored blocks are (tt, h) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1); the
matrix is zero elsewhere.
"""
import numpy as np
import pytest

import oracle
from linear_attention_recurrence_03_amd import inputs

torch = pytest.importorskip("torch")
C = 64


BLOCKS = [(0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1)]


def _block_index_map():
    """(row, col) of every element of the six-block image, in storage order."""
    rows, cols = [], []
    for tt, h in BLOCKS:
        for pos in range(64):
            i = pos >> 2
            g = (pos & 3) ^ (i >> 2)
            for j in range(8):
                rows.append(16 * tt + i)
                cols.append(32 * h + (4 * g + j if j < 4 else 16 + 4 * g + j - 4))
    return np.array(rows), np.array(cols)


def _decode_ws(ws, dtype, n_units):
    esz = 2 if dtype == "bf16" else 4
    nel = 6 * 64 * 8                      # elements in six blocks
    per = 2 * nel * esz + 4 * C * 4      # gates: four rows (1 KiB) without normalisation
    raw = ws[: n_units * per].cpu().numpy().reshape(n_units, per)
    mats = raw[:, : 2 * nel * esz]
    if dtype == "bf16":
        vals = (mats.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    else:
        vals = mats.view(np.float32)
    vals = vals.reshape(n_units, 2, nel).astype(np.float64)
    rows, cols = _block_index_map()
    full = np.zeros((n_units, 2, C, C))
    full[:, :, rows, cols] = vals
    gates = raw[:, 2 * nel * esz:2 * nel * esz + 4 * C * 4].view(np.float32).reshape(
        n_units, 4, C).transpose(0, 2, 1)
    return full[:, 0], full[:, 1], gates.astype(np.float64)


def test_block_map_covers_lower_triangle():
    """The six blocks hold every element on or below the diagonal exactly once."""
    rows, cols = _block_index_map()
    assert len(set(zip(rows.tolist(), cols.tolist()))) == len(rows)
    lower = {(r, c) for r in range(C) for c in range(r + 1)}
    assert lower <= set(zip(rows.tolist(), cols.tolist()))


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,T", [("f32", 64), ("bf16", 64), ("bf16", 150), ("f32", 100)])
def test_workspace_matches_oracle_stages(dtype, T):
    import linear_attention_recurrence_03_amd as gdn
    D, H = 64, 2
    x = inputs.custom(1, T, H, D, dtype=dtype, state="normal", seed=T)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).cuda().to(tdt) for n in ("q", "k", "v"))
    g, beta, st = (torch.from_numpy(x[n]).cuda() for n in ("g", "beta", "state"))
    need = gdn.workspace_size(dtype, 1, T, H, D, "chunked")
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    gdn.forward(q, k, v, g, beta, st, algo="chunked", workspace=ws)
    torch.cuda.synchronize()
    nc = (T + C - 1) // C
    Tm, Pm, G = _decode_ws(ws, dtype, H * nc)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for h in range(H):
        for n in range(nc):
            t0, t1 = n * C, min(T, n * C + C)
            nv = t1 - t0
            r = oracle.chunk_stages(x["q"][0, t0:t1, h], x["k"][0, t0:t1, h], x["v"][0, t0:t1, h],
                                    x["g"][0, t0:t1, h], x["beta"][0, t0:t1, h], None)
            u = h * nc + n
            what = "head %d chunk %d" % (h, n)
            np.testing.assert_allclose(G[u, :nv, 0], x["beta"][0, t0:t1, h], rtol=1e-6,
                                       err_msg=what)
            np.testing.assert_allclose(G[u, :nv, 1], np.exp(r["gam"]), rtol=1e-4, atol=1e-30,
                                       err_msg=what)
            np.testing.assert_allclose(G[u, :nv, 2], np.exp(r["gam"][-1] - r["gam"]), rtol=1e-4,
                                       err_msg=what)
            np.testing.assert_allclose(G[u, 0, 3], np.exp(r["gam"][-1]), rtol=1e-4, err_msg=what)
            assert np.all(G[u, nv:, :3] == 0), what
            eT = np.max(np.abs(Tm[u, :nv, :nv] - r["T"])) / np.max(np.abs(r["T"]))
            eP = np.max(np.abs(Pm[u, :nv, :nv] * np.sqrt(D) - r["P"])) / np.max(np.abs(r["P"]))
            assert eT < tol and eP < tol, (what, eT, eP)
            assert np.all(np.triu(Tm[u], 1) == 0) and np.all(np.triu(Pm[u], 1) == 0), what
