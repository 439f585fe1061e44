"""Seeded synthetic inputs for the gated delta rule workloads.

This module is shared by the tests, the benchmark and the oracle's callers.  It
holds no step of the recurrence itself: only random draws and the caller-side
preparation that precedes the op (L2-normalising q and k, turning raw draws
into a log-domain gate with -softplus and into beta with a sigmoid, rounding to
bf16).  The op takes q, k, g and beta as given.

Workload shapes stand in for a GDN layer of a 4B hybrid model with 32 value
heads of width 128 over 24 GDN layers ("ggml attention kernels" model card,
section "Measured", first table) and for the 4K-context decode of the velstech
page's table (section "Why this bites AMD users specifically").  No model
weights are used; every tensor is drawn from the distributions below.

Generator: numpy PCG64 ``default_rng(seed)``, float32 draws, in the order
q, k, v, gate normals (and, for the mixed-gate workload, the strong-decay
normals and the uniform selector), beta normals, initial state.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    NaN/Inf are not expected in generated data and are not special-cased.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, storage dtype of q/k/v/out and recipe."""
    name: str
    n_seqs: int
    n_tokens: int
    n_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16" for q, k, v and out
    state: str                 # "zeros" or "normal" (std 0.1)
    gate: str                  # "standard", "mixed" (90/10 strong decay) or "weak"
    beta_std: float = 1.0      # beta = sigmoid(N(0, beta_std))
    seed: int = 0
    per_seq_seeds: bool = False  # spawn one child seed per sequence
    key_heads: Optional[int] = None  # heads of q and k (None: n_heads)
    raw: bool = False  # leave q, k unnormalised and g, beta as pre-activations

    def shape(self):
        return (self.n_seqs, self.n_tokens, self.n_heads, self.head_dim)

    def n_key_heads(self):
        return self.n_heads if self.key_heads is None else self.key_heads


# The five workloads.  Seeds follow 1000 * workload number (+ layer index for the
# 24-layer decode timing).
WORKLOADS = {
    1: Workload("tiny_f32", 1, 64, 2, 32, "f32", "zeros", "standard", seed=1000),
    2: Workload("decode_f32", 1, 1, 32, 128, "f32", "normal", "standard", seed=2000),
    3: Workload("batched_decode_f32", 64, 1, 32, 128, "f32", "normal", "standard",
                seed=3000),
    4: Workload("prefill_bf16", 1, 4096, 32, 128, "bf16", "zeros", "standard",
                seed=4000),
    5: Workload("long_prefill_bf16", 4, 32768, 16, 128, "bf16", "normal", "mixed",
                beta_std=2.0, seed=5000, per_seq_seeds=True),
}

# 32 value heads sharing 16 query/key heads (tiled order), otherwise the prefill
# workload above: the key-head count of a GQA-style GDN layer.
GQA_PREFILL = Workload("prefill_tiled_bf16", 1, 4096, 32, 128, "bf16", "zeros", "standard",
                       seed=6000, key_heads=16)

# A batch of prefills with one (seq, head) pair per compute unit of MI355X (8
# sequences x 32 heads), otherwise the prefill recipe: the size from which the
# whole-head chunk-to-chunk pass is chosen.
BATCHED_PREFILL = Workload("prefill_batched_bf16", 8, 2048, 32, 128, "bf16", "zeros",
                           "standard", seed=7000)


def _draw(rng, shape, dtype, state_kind, gate, beta_std, head_dim, key_heads=None, raw=False):
    S, T, H, d = shape
    HK = H if key_heads is None else key_heads
    q = rng.standard_normal((S, T, HK, d), dtype=np.float32)
    k = rng.standard_normal((S, T, HK, d), dtype=np.float32)
    v = rng.standard_normal((S, T, H, d), dtype=np.float32)
    zg = rng.standard_normal((S, T, H), dtype=np.float32)
    if raw and gate != "standard":
        raise ValueError("raw inputs use the standard gate recipe")
    if gate == "mixed":
        zs = rng.standard_normal((S, T, H), dtype=np.float32) + np.float32(4.0)
        sel = rng.random((S, T, H), dtype=np.float32) < np.float32(0.1)
        g = np.where(sel, -_softplus(zs), -_softplus(zg)).astype(np.float32)
    elif gate == "weak":
        # Slow decay so that the carried state matters across many chunks.
        g = (-np.float32(0.01) * _softplus(zg)).astype(np.float32)
    elif gate == "standard":
        g = -_softplus(zg)
    else:
        raise ValueError("unknown gate recipe %r" % gate)
    zb = rng.standard_normal((S, T, H), dtype=np.float32) * np.float32(beta_std)
    beta = _sigmoid(zb)
    if state_kind == "normal":
        st = rng.standard_normal((S, H, d, d), dtype=np.float32) * np.float32(0.1)
    elif state_kind == "zeros":
        st = np.zeros((S, H, d, d), dtype=np.float32)
    else:
        raise ValueError("unknown state recipe %r" % state_kind)
    if raw:
        # the pre-activations and unnormalised rows that the transforms above
        # would turn into g, beta, q and k
        g, beta = zg, zb
    else:
        q = _l2norm(q)
        k = _l2norm(k)
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    elif dtype != "f32":
        raise ValueError("dtype must be 'f32' or 'bf16'")
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "state": st}


def make(workload: Workload, layer: int = 0, seq: Optional[int] = None):
    """Draw the inputs of ``workload`` (float32 arrays; bf16 values pre-rounded).

    ``layer`` offsets the seed (independent layers of the decode timing).  For
    a workload with per-sequence seeds, ``seq`` selects one sequence (arrays
    then have n_seqs = 1); ``seq=None`` draws them all and concatenates.
    """
    shape = workload.shape()
    base = workload.seed + layer
    if workload.per_seq_seeds:
        children = np.random.SeedSequence(base).spawn(workload.n_seqs)
        seqs = range(workload.n_seqs) if seq is None else [seq]
        parts = []
        for s in seqs:
            rng = np.random.default_rng(children[s])
            parts.append(_draw(rng, (1,) + shape[1:], workload.dtype,
                               workload.state, workload.gate, workload.beta_std,
                               workload.head_dim, workload.key_heads, workload.raw))
        if len(parts) == 1:
            return parts[0]
        return {key: np.concatenate([p[key] for p in parts], axis=0)
                for key in parts[0]}
    if seq is not None:
        raise ValueError("this workload draws all sequences from one seed")
    rng = np.random.default_rng(base)
    return _draw(rng, shape, workload.dtype, workload.state, workload.gate,
                 workload.beta_std, workload.head_dim, workload.key_heads, workload.raw)


def custom(n_seqs, n_tokens, n_heads, head_dim, dtype="f32", state="normal",
           gate="standard", beta_std=1.0, seed=0, key_heads=None, raw=False):
    """Inputs of any shape with one of the recipes above (for edge cases)."""
    wl = Workload("custom", n_seqs, n_tokens, n_heads, head_dim, dtype, state,
                  gate, beta_std=beta_std, seed=seed, key_heads=key_heads, raw=raw)
    return make(wl)


def make_device(n_seqs, n_tokens, n_heads, head_dim, dtype="bf16", state="zeros",
                gate_offset=0.0, seed=0, device="cuda"):
    """The standard recipe drawn on a GPU with torch's seeded generator, for sizes
    whose host-side draw would take minutes; the tensors stay on ``device``.

    q, k: N(0,1) rows L2-normalised in fp32; v: N(0,1); g = -softplus(N(0,1)) -
    gate_offset; beta = sigmoid(N(0,1)); state: zeros or N(0, 0.1) fp32
    [value][key].  q, k, v are then stored as ``dtype`` (bf16 rounds to nearest
    even); g, beta and the state are fp32.  Draw order: q, k, v, gate normals,
    beta normals, state.  Returns a dict of torch tensors like ``make``.
    """
    import torch

    gen = torch.Generator(device=device).manual_seed(int(seed))
    S, T, H, d = n_seqs, n_tokens, n_heads, head_dim
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]

    def rows(shape, normalise):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        if normalise:
            x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min_(1e-30)
        return x.to(tdt)

    q = rows((S, T, H, d), True)
    k = rows((S, T, H, d), True)
    v = rows((S, T, H, d), False)
    zg = torch.randn((S, T, H), generator=gen, device=device, dtype=torch.float32)
    g = -torch.nn.functional.softplus(zg) - float(gate_offset)
    zb = torch.randn((S, T, H), generator=gen, device=device, dtype=torch.float32)
    beta = torch.sigmoid(zb)
    if state == "normal":
        st = torch.randn((S, H, d, d), generator=gen, device=device, dtype=torch.float32)
        st *= 0.1
    elif state == "zeros":
        st = torch.zeros((S, H, d, d), device=device, dtype=torch.float32)
    else:
        raise ValueError("unknown state recipe %r" % state)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "state": st}
