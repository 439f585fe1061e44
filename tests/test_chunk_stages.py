"""GPU check of the chunked path's intermediate values against the oracle.

The chunked algorithm first computes, for every (sequence, head, chunk), the
state-independent matrices into the caller's workspace.  This test decodes that
workspace (its layout is internal to the library and mirrored here) and compares it
with the oracle's stage values, so that a parity failure can be attributed to the
first or the second half of the path.

Default chunked form, per chunk: T and then P / sqrt(head_dim) (the output's factor,
applied where P is formed) as six "fragment blocks" each (fp32 or bf16 like the
rows), then four fp32 rows of 64: beta, e^gam, e^(gam_last - gam) and e^gam_last
repeated.

Two-chunk-lag form (bf16 rows), per chunk of 30 KiB: T and P as above, then R1 and
R2 as eight blocks each, the full 64 x 64 matrices through which the chunk's deltas
depend on those of the two chunks before it (``oracle.chunk_lag_terms``), then
2 KiB of fp32 rows of 64: beta, e^gam, e^(gam_last - gam), e^gam_last repeated, e^gam
again (the output's row).

A fragment block holds a 16 x 32 sub-matrix (row tile tt, column half h) of a 64 x
64 matrix as 64 units of 8 elements: the unit of row i (0..15) and lane group g
(0..3) sits at position 4 i + (g ^ (i >> 2)), and its element j is column
32 h + 4 g + j (j < 4) or 32 h + 16 + 4 g + j - 4 (j >= 4).  The six stored blocks of
a lower-triangular matrix are (tt, h) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1); the
matrix is zero elsewhere.  The eight blocks of a full matrix are (tt, h) at 2 tt + h.
"""
import numpy as np
import pytest

import oracle
from linear_attention_recurrence_03_amd import inputs

torch = pytest.importorskip("torch")
C = 64


BLOCKS = [(0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1)]
FULL = [(tt, h) for tt in range(4) for h in range(2)]


def _block_index_map(blocks=BLOCKS):
    """(row, col) of every element of a block image, in storage order."""
    rows, cols = [], []
    for tt, h in blocks:
        for pos in range(64):
            i = pos >> 2
            g = (pos & 3) ^ (i >> 2)
            for j in range(8):
                rows.append(16 * tt + i)
                cols.append(32 * h + (4 * g + j if j < 4 else 16 + 4 * g + j - 4))
    return np.array(rows), np.array(cols)


def _unpack(raw, dtype, blocks):
    n_units = raw.shape[0]
    if dtype == "bf16":
        vals = (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    else:
        vals = raw.view(np.float32)
    vals = vals.reshape(n_units, -1).astype(np.float64)
    rows, cols = _block_index_map(blocks)
    full = np.zeros((n_units, C, C))
    full[:, rows, cols] = vals
    return full


def _decode_ws(ws, dtype, n_units, lag):
    """T, P, gates (n_units, 64, rows) and, for the lag form, R1, R2."""
    esz = 2 if dtype == "bf16" else 4
    blk = 64 * 8 * esz
    if lag:
        per, g0, ng = 30 * 1024, 28 * blk, 5
    else:
        per, g0, ng = 12 * blk + 4 * C * 4, 12 * blk, 4
    raw = ws[: n_units * per].cpu().numpy().reshape(n_units, per)
    out = {"T": _unpack(raw[:, :6 * blk], dtype, BLOCKS),
           "P": _unpack(raw[:, 6 * blk:12 * blk], dtype, BLOCKS),
           "gates": raw[:, g0:g0 + ng * C * 4].view(np.float32).reshape(
               n_units, ng, C).transpose(0, 2, 1).astype(np.float64)}
    if lag:
        out["R1"] = _unpack(raw[:, 12 * blk:20 * blk], dtype, FULL)
        out["R2"] = _unpack(raw[:, 20 * blk:28 * blk], dtype, FULL)
    return out


def test_block_map_covers_lower_triangle():
    """The six blocks hold every element on or below the diagonal exactly once, the
    eight blocks every element."""
    rows, cols = _block_index_map()
    assert len(set(zip(rows.tolist(), cols.tolist()))) == len(rows)
    lower = {(r, c) for r in range(C) for c in range(r + 1)}
    assert lower <= set(zip(rows.tolist(), cols.tolist()))
    rows, cols = _block_index_map(FULL)
    assert set(zip(rows.tolist(), cols.tolist())) == {(r, c) for r in range(C) for c in range(C)}


def _rel(a, b):
    den = np.max(np.abs(b))
    return np.max(np.abs(a - b)) / den if den > 0 else np.max(np.abs(a))


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,T,H,D,gate,algo", [
    ("f32", 64, 2, 64, "standard", "chunked"), ("bf16", 64, 2, 64, "standard", "chunked"),
    ("bf16", 150, 2, 64, "standard", "chunked"), ("f32", 100, 2, 64, "standard", "chunked"),
    # the headline width, and a grid of more row blocks than compute units (two value
    # tiles per scan workgroup), whose output is compared as well
    ("bf16", 260, 2, 128, "standard", "chunked"), ("bf16", 200, 2, 128, "weak", "chunked"),
    ("f32", 130, 2, 128, "weak", "chunked"), ("bf16", 130, 40, 128, "weak", "chunked"),
    ("bf16", 260, 2, 128, "standard", "chunked_lag"), ("bf16", 200, 2, 128, "weak", "chunked_lag"),
    ("bf16", 3 * 64, 2, 32, "weak", "chunked_lag"), ("bf16", 230, 2, 96, "weak", "chunked_lag")])
def test_workspace_matches_oracle_stages(dtype, T, H, D, gate, algo):
    import linear_attention_recurrence_03_amd as gdn
    lag = algo == "chunked_lag"
    x = inputs.custom(1, T, H, D, dtype=dtype, state="normal", gate=gate, seed=T + D)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).cuda().to(tdt) for n in ("q", "k", "v"))
    g, beta, st = (torch.from_numpy(x[n]).cuda() for n in ("g", "beta", "state"))
    need = gdn.workspace_size(dtype, 1, T, H, D, algo)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    print("case: stages", dtype, T, H, D, gate, algo, flush=True)
    out, s_out = gdn.forward(q, k, v, g, beta, st, algo=algo, workspace=ws)
    torch.cuda.synchronize()
    nc = (T + C - 1) // C
    w = _decode_ws(ws, dtype, H * nc, lag)
    G = w["gates"]
    tol = 2e-2 if dtype == "bf16" else 1e-5
    worst = {}
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
            if lag:
                np.testing.assert_allclose(G[u, :nv, 4], np.exp(r["gam"]), rtol=1e-4, atol=1e-30,
                                           err_msg=what)
            errs = {"T": _rel(w["T"][u, :nv, :nv], r["T"]),
                    "P": _rel(w["P"][u, :nv, :nv] * np.sqrt(D), r["P"])}
            assert np.all(np.triu(w["T"][u], 1) == 0) and np.all(np.triu(w["P"][u], 1) == 0), what
            if lag:
                r1, r2 = oracle.chunk_lag_terms(x["k"][0, :, h], x["g"][0, :, h], x["beta"][0, :, h], n)
                for name, ref in (("R1", r1), ("R2", r2)):
                    got = w[name][u]
                    assert np.all(got[nv:] == 0), (what, name)
                    if np.max(np.abs(ref)) > 0:
                        errs[name] = _rel(got[:nv], ref)
                    else:
                        assert np.all(got == 0), (what, name)
            for key, e in errs.items():
                assert e < tol, (what, key, e)
                worst[key] = max(worst.get(key, 0.0), e)
    print("stage errors", dtype, T, H, D, gate, algo, {k_: "%.2e" % e for k_, e in worst.items()},
          flush=True)
    if H > 2:
        # the call's results as well (the scan that ran on this grid)
        ref_out, ref_state = oracle.gdn_recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                  x["state"])
        eo = _rel(out.float().cpu().numpy(), ref_out)
        es = _rel(s_out.cpu().numpy(), ref_state)
        print("ERR out %.3e state %.3e" % (eo, es), flush=True)
        assert eo < tol and es < tol, (eo, es)
